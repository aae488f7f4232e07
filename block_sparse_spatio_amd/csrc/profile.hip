// Sampled-query head profiler (Sparse VideoGen on TPU, "how to accelerate attention"):
// for each head, a few sampled queries are attended under the reference mask (full
// attention) and under each candidate sparse mask; the deviation of each candidate's
// output from the reference is reduced to one number per (head, candidate) and the
// head is routed to the candidate with the smallest deviation ("supporting dynamic
// routing with fixed tensor shapes": one flag per head, no variable-size head groups).
//
// Pass 1 (profile_kernel): grid = (key chunk, head, batch).  A workgroup holds the
// sampled query rows of one (b, h) in registers (32 per wave), streams its chunk of key
// tiles through LDS once, and keeps one online-softmax state per candidate: the score
// tile S^T = K Q^T is computed once (bf16 MFMA) and masked per candidate.  Each
// candidate's partial (max, sum, unnormalised output) is written to the workspace.
// Pass 2 (profile_reduce_kernel): one workgroup per head merges the chunk partials with
// their softmax statistics, forms sum over (b, sample, channel) of (o_c - o_0)^2, and
// writes err[h][c] = sqrt(.) and route[h] = argmin over c >= 1 (lowest c on ties).
// Reads K and V once per head, so the first pass is bound by HBM bandwidth.
#include "mfma_tile.h"

namespace vsa {

namespace {

using namespace mfma;

template <int D, int NW, int NC>
__global__ __launch_bounds__(NW * 64) void profile_kernel(ProfArgs a, MaskTable cands) {
  constexpr int NT = NW * 64;
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;
  __shared__ TileSmem<D> sm;

  const Geom& g = a.g;
  const int S = a.S, H = a.H, n = a.n;
  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int nK = (S + BK - 1) / BK;
  const int kt0 = chunk * a.chunk_tiles;
  const int kt1 = imin(nK, kt0 + a.chunk_tiles);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g2 = lane >> 5, l32 = lane & 31;
  const int si = wave * 32 + l32;  // sample slot of this lane's query
  const int qrow = imin(imax(a.sample_idx[(size_t)h * n + imin(si, n - 1)], 0), S - 1);

  const uint16_t* qp = (const uint16_t*)a.q;
  const uint16_t* kp = (const uint16_t*)a.k;
  const uint16_t* vp = (const uint16_t*)a.v;
  const size_t tok_stride = (size_t)H * D;
  const size_t base_bh = ((size_t)b * S) * tok_stride + (size_t)h * D;

  bf16x8 qf[KSTEPS];
  {
    const uint16_t* src = qp + base_bh + (size_t)qrow * tok_stride + g2 * 8;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[s] = __builtin_bit_cast(bf16x8, *(const u32x4*)(src + s * 16));
  }
  QueryPos qpos[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) qpos[c] = make_query(g, cands.m[c], qrow);

  f32x16 acc[NC][DB];
  float m_run[NC], l_run[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    m_run[c] = -INFINITY;
    l_run[c] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[c][db] = f32x16{};
  }
  const float c_log2 = a.scale * 1.4426950408889634f;

  Stager<D, NT> stg;
  if (kt0 < kt1) stg.load(kp, vp, base_bh, tok_stride, kt0 * BK, S, tid);
  for (int kt = kt0; kt < kt1; ++kt) {
    __syncthreads();
    stg.store(sm, tid);
    __syncthreads();
    if (kt + 1 < kt1) stg.load(kp, vp, base_bh, tok_stride, (kt + 1) * BK, S, tid);
    f32x16 st[2];
    qk_tile<D>(sm, qf, l32, g2, st);
    const bool tail = (kt + 1) * BK > S;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const DevMask& mc = cands.m[c];
      f32x16 sc[2] = {st[0], st[1]};
      if (mc.kind != VSA_MASK_ALL || tail) apply_mask(sc, tile_row_mask(g, mc, qpos[c], kt * BK, BK), g2);
      uint32_t pk[2][8];
      const float alpha = softmax_step(sc, c_log2, m_run[c], l_run[c], pk);
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[c][db] *= alpha;
      pv_tile<D>(sm, pk, l32, g2, acc[c]);
    }
  }

  float l_tot[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) l_tot[c] = l_run[c] + __shfl_xor(l_run[c], 32);
  if (si < n) {
    const int stride = D + 2;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float* dst = a.ws + ((((size_t)(b * H + h) * a.n_chunks + chunk) * NC + c) * n + si) * stride;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) dst[db * 32 + (i >> 2) * 8 + g2 * 4 + (i & 3)] = acc[c][db][i];
      if (g2 == 0) {
        dst[D] = m_run[c];
        dst[D + 1] = l_tot[c];
      }
    }
  }
}

template <int D, int NC>
__global__ __launch_bounds__(256) void profile_reduce_kernel(ProfArgs a) {
  const int h = blockIdx.x;
  const int n = a.n, B = a.B, H = a.H;
  const int stride = D + 2;
  const float c_log2 = a.scale * 1.4426950408889634f;
  float part[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) part[c] = 0.f;
  for (int e = threadIdx.x; e < B * n; e += blockDim.x) {
    const int b = e / n, si = e % n;
    float mstar[NC], linv[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float mx = -INFINITY;
      for (int ch = 0; ch < a.n_chunks; ++ch) {
        const float* src = a.ws + ((((size_t)(b * H + h) * a.n_chunks + ch) * NC + c) * n + si) * stride;
        mx = fmaxf(mx, src[D]);
      }
      const float mu = mx == -INFINITY ? 0.f : mx;
      float l = 0.f;
      for (int ch = 0; ch < a.n_chunks; ++ch) {
        const float* src = a.ws + ((((size_t)(b * H + h) * a.n_chunks + ch) * NC + c) * n + si) * stride;
        l += src[D + 1] * __builtin_amdgcn_exp2f((src[D] - mu) * c_log2);
      }
      mstar[c] = mu;
      linv[c] = l > 0.f ? 1.f / l : 0.f;
    }
    for (int d = 0; d < D; ++d) {
      float o[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        float x = 0.f;
        for (int ch = 0; ch < a.n_chunks; ++ch) {
          const float* src = a.ws + ((((size_t)(b * H + h) * a.n_chunks + ch) * NC + c) * n + si) * stride;
          x += src[d] * __builtin_amdgcn_exp2f((src[D] - mstar[c]) * c_log2);
        }
        o[c] = x * linv[c];
      }
#pragma unroll
      for (int c = 1; c < NC; ++c) part[c] += (o[c] - o[0]) * (o[c] - o[0]);
    }
  }
  __shared__ float red[NC][256];
#pragma unroll
  for (int c = 0; c < NC; ++c) red[c][threadIdx.x] = part[c];
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) {
#pragma unroll
      for (int c = 0; c < NC; ++c) red[c][threadIdx.x] += red[c][threadIdx.x + s];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    int best = 1;
    float best_e = sqrtf(red[1][0]);
    a.err[(size_t)h * NC + 0] = 0.f;
#pragma unroll
    for (int c = 1; c < NC; ++c) {
      const float e = sqrtf(red[c][0]);
      a.err[(size_t)h * NC + c] = e;
      if (e < best_e) { best_e = e; best = c; }
    }
    a.route[h] = best;
  }
}

template <int D, int NW, int NC>
hipError_t launch_t(const ProfArgs& a, const MaskTable& cands, hipStream_t st) {
  hipLaunchKernelGGL((profile_kernel<D, NW, NC>), dim3(a.n_chunks, a.H, a.B), dim3(NW * 64), 0, st, a,
                     cands);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((profile_reduce_kernel<D, NC>), dim3(a.H), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int D, int NC>
hipError_t launch_nw(const ProfArgs& a, const MaskTable& cands, hipStream_t st) {
  const int nw = (a.n + 31) / 32;
  switch (nw) {
    case 1: return launch_t<D, 1, NC>(a, cands, st);
    case 2: return launch_t<D, 2, NC>(a, cands, st);
    case 3:
    case 4: return launch_t<D, 4, NC>(a, cands, st);
    default: return launch_t<D, 8, NC>(a, cands, st);
  }
}

template <int D>
hipError_t launch_nc(const ProfArgs& a, const MaskTable& cands, hipStream_t st) {
  switch (a.n_cand) {
    case 2: return launch_nw<D, 2>(a, cands, st);
    case 3: return launch_nw<D, 3>(a, cands, st);
    case 4: return launch_nw<D, 4>(a, cands, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int32_t profile_chunks(int32_t B, int32_t S, int32_t H) {
  const int nK = (S + mfma::BK - 1) / mfma::BK;
  const long long bh = (long long)B * H;
  int chunks = (int)((1024 + bh - 1) / bh);
  if (chunks < 1) chunks = 1;
  if (chunks > nK) chunks = nK;
  return chunks;
}

size_t profile_ws_floats(int32_t B, int32_t H, int32_t D, int32_t n, int32_t n_cand,
                         int32_t n_chunks) {
  return (size_t)B * H * n_chunks * n_cand * n * (D + 2);
}

hipError_t launch_profile(const ProfArgs& a, const MaskTable& cands, hipStream_t stream) {
  if (!a.is_bf16) return hipErrorInvalidValue;
  if (a.D == 128) return launch_nc<128>(a, cands, stream);
  if (a.D == 64) return launch_nc<64>(a, cands, stream);
  return hipErrorInvalidValue;
}

}  // namespace vsa
