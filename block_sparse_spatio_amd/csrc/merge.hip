// Merge of partial attention results over disjoint key subsets (DSA study guide,
// section 18): each part carries its normalised output o_i and log-sum-exp lse_i; with
// m' = max_i lse_i the parts weigh w_i = exp(lse_i - m'), the merged row is
// o = sum_i w_i o_i / sum_i w_i and lse = m' + ln(sum_i w_i).  A part with lse_i = -inf
// (no kept key) weighs 0; a row with no kept key in any part stays o = 0, lse = -inf.
//
// HBM-bound: every part's output row is read once and the merged row written once.
// Lanes cover a row 8 channels at a time (16-byte bf16 or 2 x 16-byte fp32 loads), so
// the D/8 lanes of a row sit in one wave; each lane reads the row's n_parts lse values
// before any lane of the row writes, which makes in-place merges (o = o_parts[i],
// lse = lse_parts[i]) safe.
#include "vsa_internal.h"

namespace vsa {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

template <int D, bool BF16>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  constexpr int LPR = D / 8;  // lanes per row
  const long long rows = (long long)a.B * a.S * a.H;
  const long long row = (long long)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  if (row >= rows) return;
  const int c0 = (threadIdx.x % LPR) * 8;
  const int h = (int)(row % a.H);
  const long long bs = row / a.H;  // b*S + s
  const int s = (int)(bs % a.S);
  const int b = (int)(bs / a.S);
  const size_t li = ((size_t)b * a.H + h) * a.S + s;
  const size_t oi = (size_t)row * D + c0;

  float lv[16];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    lv[i] = i < a.n ? a.lse[i][li] : -INFINITY;
    mx = fmaxf(mx, lv[i]);
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (mx != -INFINITY) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i >= a.n || lv[i] == -INFINITY) continue;
      const float w = expf(lv[i] - mx);
      wsum += w;
      if (BF16) {
        const u32x4 x = *(const u32x4*)((const uint16_t*)a.o[i] + oi);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += w * bf16_lo(x[e]);
          acc[2 * e + 1] += w * bf16_hi(x[e]);
        }
      } else {
        const f32x4 x0 = *(const f32x4*)((const float*)a.o[i] + oi);
        const f32x4 x1 = *(const f32x4*)((const float*)a.o[i] + oi + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[e] += w * x0[e];
          acc[4 + e] += w * x1[e];
        }
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  if (BF16) {
    u32x4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = pack2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
    *(u32x4*)((uint16_t*)a.out + oi) = y;
  } else {
    *(f32x4*)((float*)a.out + oi) = f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    *(f32x4*)((float*)a.out + oi + 4) = f32x4{acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
  }
  if (a.lse_out && c0 == 0) a.lse_out[li] = wsum > 0.f ? mx + logf(wsum) : -INFINITY;
}

template <int D, bool BF16>
hipError_t launch_t(const MergeArgs& a, hipStream_t st) {
  constexpr int RPB = 256 / (D / 8);  // rows per block
  const long long rows = (long long)a.B * a.S * a.H;
  const long long blocks = (rows + RPB - 1) / RPB;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((merge_kernel<D, BF16>), dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  if (a.D == 128) return a.is_bf16 ? launch_t<128, true>(a, stream) : launch_t<128, false>(a, stream);
  if (a.D == 64) return a.is_bf16 ? launch_t<64, true>(a, stream) : launch_t<64, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace vsa
