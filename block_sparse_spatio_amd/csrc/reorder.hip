// Tile-major token reorder (and its inverse) of [B, S, H, D] tensors.
//
// Sliding-tile attention needs the tokens of each 3D tile contiguous in the sequence
// (Sliding Tile Attention explainer, method section 3; video-DiT attention blog,
// section 7.2: a token permutation is one gather before attention and one after).
// A token's H*D channels are contiguous, so the permutation moves whole rows: each
// workgroup copies a few destination tokens with 16-byte coalesced loads/stores.
// Pure data movement, bound by HBM bandwidth (read + write of every byte once).
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

__global__ __launch_bounds__(kThreads) void reorder_kernel(const u32x4* __restrict__ src,
                                                           u32x4* __restrict__ dst, Geom g, int B,
                                                           int row_chunks, int inverse) {
  const long long tok0 = (long long)blockIdx.x * kTokPerBlock;
  const long long n_tok = (long long)B * g.S;
  for (int e = threadIdx.x; e < kTokPerBlock * row_chunks; e += kThreads) {
    const long long tok = tok0 + e / row_chunks;
    if (tok >= n_tok) break;
    const int c = e % row_chunks;
    const int b = (int)(tok / g.S);
    const int p = (int)(tok - (long long)b * g.S);
    // destination position p takes the token at position src_p of the source order
    const int src_p = inverse ? frame_to_tile(g, p) : tile_to_frame(g, p);
    dst[tok * row_chunks + c] = src[((long long)b * g.S + src_p) * row_chunks + c];
  }
}

}  // namespace

hipError_t launch_reorder(const void* src, void* dst, int32_t elem_bytes, int32_t B, int32_t H,
                          int32_t D, const Geom& g, int32_t inverse, hipStream_t stream) {
  const long long row_bytes = (long long)H * D * elem_bytes;
  if (row_bytes % 16) return hipErrorInvalidValue;
  const int row_chunks = (int)(row_bytes / 16);
  const long long n_tok = (long long)B * g.S;
  const long long blocks = (n_tok + kTokPerBlock - 1) / kTokPerBlock;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(reorder_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     (const u32x4*)src, (u32x4*)dst, g, B, row_chunks, inverse);
  return hipGetLastError();
}

}  // namespace vsa
