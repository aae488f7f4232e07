// Token reorder (and its inverse) of [B, S, H, D] tensors, per head.
//
// Sliding-tile attention needs the tokens of each 3D tile contiguous in the sequence
// (Sliding Tile Attention explainer, method section 3; video-DiT attention blog,
// section 7.2: a token permutation is one gather before attention and one after), and
// temporal heads want each spatial position's frames contiguous (Sparse VideoGen on
// TPU, "arranging tokens for temporal access").  Every head has its own order
// (VSA_LAYOUT_*), so a head's D channels of a token move as one unit.  Each thread
// copies one 16-byte chunk; consecutive threads take consecutive chunks of a token
// row, so loads and stores are coalesced per head segment.  Pure data movement, bound
// by HBM bandwidth (read + write of every byte once).
#include "vsa_geom.h"

namespace vsa {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kTokPerBlock = 4;

// Divisors of the position arithmetic, fixed per call (every element divides by them).
struct Divs {
  FastDiv HW, Wg, T1, vol, nHW, nW, bhw, bw, bt, bh;
};

// frame-major index of the token at tile-major position p (-1: padding of a padded grid)
__device__ __forceinline__ int tile_to_frame(const Geom& g, const Divs& dv, int p) {
  const int vol = g.bt * g.bh * g.bw;
  const int tau = fastdiv_q(p, dv.vol), io = p - tau * vol;
  const int nHW = g.nH * g.nW;
  const int tt = fastdiv_q(tau, dv.nHW), r = tau - tt * nHW;
  const int th = fastdiv_q(r, dv.nW), tw = r - th * g.nW;
  const int it = fastdiv_q(io, dv.bhw), r2 = io - it * (g.bh * g.bw);
  const int ih = fastdiv_q(r2, dv.bw), iw = r2 - ih * g.bw;
  const int t = tt * g.bt + it, y = th * g.bh + ih, x = tw * g.bw + iw;
  if (t >= g.T || y >= g.Hg || x >= g.Wg) return -1;
  return (t * g.Hg + y) * g.Wg + x;
}

// tile-major position of frame-major token p
__device__ __forceinline__ int frame_to_tile(const Geom& g, const Divs& dv, int p) {
  const int t = fastdiv_q(p, dv.HW), r = p - t * g.HW;
  const int y = fastdiv_q(r, dv.Wg), x = r - y * g.Wg;
  const int tt = fastdiv_q(t, dv.bt), ty = fastdiv_q(y, dv.bh), tx = fastdiv_q(x, dv.bw);
  const int tau = (tt * g.nH + ty) * g.nW + tx;
  const int io = ((t - tt * g.bt) * g.bh + (y - ty * g.bh)) * g.bw + (x - tx * g.bw);
  return tau * (g.bt * g.bh * g.bw) + io;
}

// frame-major index of the token at position-major position p: frame 0 leads in
// frame-major order, then spatial position s holds frames 1 .. T-1 at HW + s*(T-1)
__device__ __forceinline__ int position_to_frame(const Geom& g, const Divs& dv, int p) {
  if (p < g.HW) return p;  // (T == 1 has no position after frame 0)
  const int r = p - g.HW;
  const int s = fastdiv_q(r, dv.T1);
  return (r - s * (g.T - 1) + 1) * g.HW + s;
}

// position-major position of frame-major token p
__device__ __forceinline__ int frame_to_position(const Geom& g, const Divs& dv, int p) {
  const int t = fastdiv_q(p, dv.HW), s = p - t * g.HW;
  return t == 0 ? s : g.HW + s * (g.T - 1) + (t - 1);
}

__device__ __forceinline__ int source_position(const Geom& g, const Divs& dv, int layout, int p, int inverse) {
  if (layout == VSA_LAYOUT_TILE_MAJOR) return inverse ? frame_to_tile(g, dv, p) : tile_to_frame(g, dv, p);
  if (layout == VSA_LAYOUT_POSITION_MAJOR)
    return inverse ? frame_to_position(g, dv, p) : position_to_frame(g, dv, p);
  return p;
}

// Workgroup (x, b) writes positions [x*kTokPerBlock, (x+1)*kTokPerBlock) of batch item
// b of dst (S_dst positions per item; src has S_src).  per_head: heads differ in order,
// and a head segment is head_chunks 16-byte chunks; otherwise every head has order
// lay[0].  A padding position of a padded grid receives zeros.
__global__ __launch_bounds__(kThreads) void reorder_kernel(const u32x4* __restrict__ src,
                                                           u32x4* __restrict__ dst, Geom g, Divs dv,
                                                           HeadLayouts hl, int S_src, int S_dst,
                                                           int row_chunks, FastDiv d_row, FastDiv d_head,
                                                           int per_head, int inverse) {
  const int p0 = blockIdx.x * kTokPerBlock;
  const size_t base_s = (size_t)blockIdx.y * S_src, base_d = (size_t)blockIdx.y * S_dst;
  for (int e = threadIdx.x; e < kTokPerBlock * row_chunks; e += kThreads) {
    const int i = fastdiv_q(e, d_row);
    const int p = p0 + i;
    if (p >= S_dst) break;
    const int c = e - i * row_chunks;
    const int h = per_head ? fastdiv_q(c, d_head) : 0;
    // destination position p takes the token at position src_p of the source order
    const int src_p = source_position(g, dv, hl.lay[h], p, inverse);
    dst[(base_d + p) * row_chunks + c] = src_p < 0 ? u32x4{0u, 0u, 0u, 0u} : src[(base_s + src_p) * row_chunks + c];
  }
}

}  // namespace

hipError_t launch_reorder(const void* src, void* dst, int32_t elem_bytes, int32_t B, int32_t H, int32_t D,
                          const Geom& g, const HeadLayouts& hl, int32_t inverse, hipStream_t stream) {
  // a padded grid's executed order is longer than the frame-major sequence
  const int S_frame = g.T * g.HW;
  const int S_src = inverse ? g.S : S_frame, S_dst = inverse ? S_frame : g.S;
  const long long row_bytes = (long long)H * D * elem_bytes;
  if (row_bytes % 16 || H > VSA_MAX_HEADS || B > 65535) return hipErrorInvalidValue;
  bool uniform = true;
  for (int h = 1; h < H; ++h) uniform = uniform && hl.lay[h] == hl.lay[0];
  // a 16-byte chunk must not straddle two heads that move differently
  if (!uniform && ((long long)D * elem_bytes) % 16) return hipErrorInvalidValue;
  const int row_chunks = (int)(row_bytes / 16);
  const int head_chunks = uniform ? 1 : (int)((long long)D * elem_bytes / 16);
  const long long blocks = ((long long)S_dst + kTokPerBlock - 1) / kTokPerBlock;
  if (blocks == 0 || B == 0) return hipSuccess;
  Divs dv;
  dv.HW = fastdiv_make(g.HW);
  dv.Wg = fastdiv_make(g.Wg);
  dv.T1 = fastdiv_make(g.T - 1);
  dv.vol = fastdiv_make(g.bt * g.bh * g.bw);
  dv.nHW = fastdiv_make(g.nH * g.nW);
  dv.nW = fastdiv_make(g.nW);
  dv.bhw = fastdiv_make(g.bh * g.bw);
  dv.bw = fastdiv_make(g.bw);
  dv.bt = fastdiv_make(g.bt);
  dv.bh = fastdiv_make(g.bh);
  hipLaunchKernelGGL(reorder_kernel, dim3((unsigned)blocks, (unsigned)B), dim3(kThreads), 0, stream,
                     (const u32x4*)src, (u32x4*)dst, g, dv, hl, S_src, S_dst, row_chunks, fastdiv_make(row_chunks),
                     fastdiv_make(head_chunks), uniform ? 0 : 1, inverse);
  return hipGetLastError();
}

}  // namespace vsa
