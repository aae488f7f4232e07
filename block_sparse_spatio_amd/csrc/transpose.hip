// V -> blocked V^T: [B][S][H][D] bf16 -> [B][H][S_pad/64][D][64] bf16, keys past S
// zero-filled.
//
// The attention kernel reads its PV operand as V^T fragments (8 consecutive keys of one
// channel per lane).  Transposing V once per call lets those fragments be plain 16-byte
// LDS reads instead of transposing LDS reads, which run at half the LDS bandwidth; the
// transpose itself is one HBM read and one HBM write of V.  Each 64-key block of one
// head is stored as one contiguous D x 64 tile, so the attention kernel fetches a key
// tile's V^T as a single contiguous 2*64*D-byte block.
//
// One workgroup per (b, h, 64-key block): the 64 x D block is read with 16-byte
// coalesced loads (one 2*D-byte row per key), staged in LDS, and written as D rows of
// 64 keys (128 contiguous bytes each).  With gather set, V is the caller's frame-major
// tensor and key p of head h (in that head's executed order) is read from its
// frame-major row, so the V^T of a reordering call needs no reordered copy of V.
// Padding keys of a padded grid read as zeros in both cases.
#include "vsa_geom.h"

namespace vsa {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kKeys = 64;
constexpr int kThreads = 256;

template <int D>
__global__ __launch_bounds__(kThreads) void transpose_v_kernel(const uint16_t* __restrict__ v,
                                                               uint16_t* __restrict__ vt, int S, int H,
                                                               int s_pad, Geom g, HeadLayouts hl, int gather,
                                                               int S_src) {
  __shared__ uint16_t tile[kKeys][D + 2];  // +2: odd word stride keeps the column reads spread
  __shared__ int src_row[kKeys];
  const int kb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int k0 = kb * kKeys;
  constexpr int CH = D / 8;  // 16-byte chunks per key row
  if (threadIdx.x < kKeys) {
    const int key = k0 + threadIdx.x;
    int sr = key < S ? key : -1;
    if ((gather || g.padded) && sr >= 0) {
      // gather: the frame-major row of the key; a padded grid in place: the key itself,
      // unless it is padding.  Padding keys become zeros either way: they are never
      // kept, and whatever the caller's padding rows hold (uninitialised memory, NaN)
      // must not reach the PV product, where 0 * NaN would be NaN.
      Geom gh = g;
      gh.layout = hl.lay[h];
      const int fi = frame_index(gh, key);
      sr = gather ? fi : (fi >= 0 ? key : -1);
    }
    src_row[threadIdx.x] = sr;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < kKeys * CH; e += kThreads) {
    const int r = e / CH, c = e % CH;
    const int sr = src_row[r];
    u32x4 x = {0u, 0u, 0u, 0u};
    if (sr >= 0) x = *(const u32x4*)(v + (((size_t)b * S_src + sr) * H + h) * D + c * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      tile[r][c * 8 + 2 * j] = (uint16_t)(x[j] & 0xffffu);
      tile[r][c * 8 + 2 * j + 1] = (uint16_t)(x[j] >> 16);
    }
  }
  __syncthreads();
  // D rows x 8 chunks of 8 keys
  for (int e = threadIdx.x; e < D * (kKeys / 8); e += kThreads) {
    const int d = e / (kKeys / 8), c = e % (kKeys / 8);
    u32x4 y;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      y[j] = (uint32_t)tile[c * 8 + 2 * j][d] | ((uint32_t)tile[c * 8 + 2 * j + 1][d] << 16);
    *(u32x4*)(vt + ((((size_t)b * H + h) * (s_pad / kKeys) + kb) * D + d) * kKeys + c * 8) = y;
  }
}

}  // namespace

hipError_t launch_transpose_v(const void* v, void* vt, int32_t B, int32_t S, int32_t H, int32_t D,
                              int32_t s_pad, const Geom& g, const HeadLayouts& lay, int32_t gather, int32_t S_src,
                              hipStream_t stream) {
  dim3 grid(s_pad / kKeys, H, B);
  const int src_len = gather ? S_src : S;
  if (D == 128)
    hipLaunchKernelGGL(transpose_v_kernel<128>, grid, dim3(kThreads), 0, stream, (const uint16_t*)v,
                       (uint16_t*)vt, S, H, s_pad, g, lay, gather, src_len);
  else if (D == 64)
    hipLaunchKernelGGL(transpose_v_kernel<64>, grid, dim3(kThreads), 0, stream, (const uint16_t*)v,
                       (uint16_t*)vt, S, H, s_pad, g, lay, gather, src_len);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace vsa
