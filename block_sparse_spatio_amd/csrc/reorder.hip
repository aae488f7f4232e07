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

// frame-major index of the token at tile-major position p
__device__ __forceinline__ int tile_to_frame(const Geom& g, int p) {
  int vol = g.bt * g.bh * g.bw;
  int tau = p / vol, io = p - tau * vol;
  int nHW = g.nH * g.nW;
  int tt = tau / nHW, r = tau - tt * nHW;
  int th = r / g.nW, tw = r - th * g.nW;
  int it = io / (g.bh * g.bw), r2 = io - it * (g.bh * g.bw);
  int ih = r2 / g.bw, iw = r2 - ih * g.bw;
  return ((tt * g.bt + it) * g.Hg + (th * g.bh + ih)) * g.Wg + (tw * g.bw + iw);
}

// tile-major position of frame-major token p
__device__ __forceinline__ int frame_to_tile(const Geom& g, int p) {
  int t = p / g.HW, r = p - t * g.HW;
  int y = r / g.Wg, x = r - y * g.Wg;
  int tau = ((t / g.bt) * g.nH + y / g.bh) * g.nW + x / g.bw;
  int io = ((t % g.bt) * g.bh + y % g.bh) * g.bw + x % g.bw;
  return tau * (g.bt * g.bh * g.bw) + io;
}

// frame-major index of the token at position-major position p: frame 0 leads in
// frame-major order, then spatial position s holds frames 1 .. T-1 at HW + s*(T-1)
__device__ __forceinline__ int position_to_frame(const Geom& g, int p) {
  if (p < g.HW) return p;
  const int Tm = imax(g.T - 1, 1);  // T == 1 has no position after frame 0
  const int r = p - g.HW;
  const int s = r / Tm;
  return (r - s * Tm + 1) * g.HW + s;
}

// position-major position of frame-major token p
__device__ __forceinline__ int frame_to_position(const Geom& g, int p) {
  const int t = p / g.HW, s = p - t * g.HW;
  return t == 0 ? s : g.HW + s * (g.T - 1) + (t - 1);
}

__device__ __forceinline__ int source_position(const Geom& g, int layout, int p, int inverse) {
  if (layout == VSA_LAYOUT_TILE_MAJOR) return inverse ? frame_to_tile(g, p) : tile_to_frame(g, p);
  if (layout == VSA_LAYOUT_POSITION_MAJOR) return inverse ? frame_to_position(g, p) : position_to_frame(g, p);
  return p;
}

// head_elems: elements per head segment (D), or 0 when every head has layout lay[0]
__global__ __launch_bounds__(kThreads) void reorder_kernel(const u32x4* __restrict__ src,
                                                           u32x4* __restrict__ dst, Geom g, HeadLayouts hl,
                                                           int B, int row_chunks, int chunk_elems,
                                                           int head_elems, int inverse) {
  const long long tok0 = (long long)blockIdx.x * kTokPerBlock;
  const long long n_tok = (long long)B * g.S;
  for (int e = threadIdx.x; e < kTokPerBlock * row_chunks; e += kThreads) {
    const long long tok = tok0 + e / row_chunks;
    if (tok >= n_tok) break;
    const int c = e % row_chunks;
    const int b = (int)(tok / g.S);
    const int p = (int)(tok - (long long)b * g.S);
    const int h = head_elems ? (c * chunk_elems) / head_elems : 0;
    // destination position p takes the token at position src_p of the source order
    const int src_p = source_position(g, hl.lay[h], p, inverse);
    dst[tok * row_chunks + c] = src[((long long)b * g.S + src_p) * row_chunks + c];
  }
}

}  // namespace

hipError_t launch_reorder(const void* src, void* dst, int32_t elem_bytes, int32_t B, int32_t H, int32_t D,
                          const Geom& g, const HeadLayouts& hl, int32_t inverse, hipStream_t stream) {
  const long long row_bytes = (long long)H * D * elem_bytes;
  if (row_bytes % 16 || H > VSA_MAX_HEADS) return hipErrorInvalidValue;
  bool uniform = true;
  for (int h = 1; h < H; ++h) uniform = uniform && hl.lay[h] == hl.lay[0];
  // a 16-byte chunk must not straddle two heads that move differently
  if (!uniform && ((long long)D * elem_bytes) % 16) return hipErrorInvalidValue;
  const int row_chunks = (int)(row_bytes / 16);
  const long long n_tok = (long long)B * g.S;
  const long long blocks = (n_tok + kTokPerBlock - 1) / kTokPerBlock;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(reorder_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, (const u32x4*)src,
                     (u32x4*)dst, g, hl, B, row_chunks, 16 / elem_bytes, uniform ? 0 : D, inverse);
  return hipGetLastError();
}

}  // namespace vsa
