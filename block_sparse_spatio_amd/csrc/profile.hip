// Sampled-query head profiler (Sparse VideoGen on TPU, "how to accelerate attention"):
// for each head, a few sampled queries are attended under the reference mask (full
// attention) and under each candidate sparse mask; the deviation of each candidate's
// output from the reference is reduced to one number per (head, candidate) and the
// head is routed to the candidate with the smallest deviation ("supporting dynamic
// routing with fixed tensor shapes": one flag per head, no variable-size head groups).
//
// Pass 1 (profile_part_kernel): one workgroup per (sample group, key chunk, b, h), with
// one group of waves per candidate.  Each wave holds 32 sampled query rows of (b, h) in
// registers and runs the attention pipeline of the bf16 forward kernel over the chunk's
// key tiles: K and V tiles reach LDS by DMA (issued by the first 2, 4 or 8 waves),
// double-buffered and shared by every candidate, S^T = K Q^T on the matrix cores
// overlaps the softmax of the previous tile, and the wave's candidate mask applies to
// every tile (the all-keep reference only at the sequence tail).  V stays row-major and
// is read with transposing LDS reads.  The chunk's unnormalised output, running max and
// row sum go to the workspace.  At most 8 waves per workgroup (two per SIMD); the
// sample groups of one (chunk, b, h) are adjacent on one XCD.
// Pass 2 (profile_merge_kernel, profile_route_kernel): groups of 16 samples merge their
// chunk partials with the softmax statistics (lanes over channels) into sums of
// (o_c - o_0)^2; per head these are added in a fixed order, err[h][c] = sqrt(.) and
// route[h] = argmin over c >= 1 (lowest c on ties).
#include "lds_pipe.h"

namespace vsa {

namespace {

using namespace pipe;

// one partial row of the workspace: D unnormalised outputs, the running max (raw score
// units) and the row sum, padded to a multiple of 16 bytes
template <int D>
constexpr int kProfRow = D + 4;

// waves that issue a workgroup's K/V DMAs: the largest power of two up to its waves
constexpr int dma_waves(int nw) { return nw >= 8 ? 8 : (nw >= 4 ? 4 : 2); }

template <int D, int NWS, int NC>
__global__ __launch_bounds__(NWS * NC * 64) __attribute__((amdgpu_waves_per_eu(2)))
void profile_part_kernel(ProfArgs a, MaskTable cands) {
  constexpr int NWT = NWS * NC;  // NWS waves of 32 samples per candidate
  constexpr int SG = NWS * 32;   // samples per workgroup
  constexpr int NWD = dma_waves(NWT);
  using C = Cfg<D, NWD>;
  constexpr int KSTEPS = C::KSTEPS;
  constexpr int DB = C::DB;
  constexpr int NI = C::NI;
  __shared__ __attribute__((aligned(1024))) char kbuf0[C::TILE_B];
  __shared__ __attribute__((aligned(1024))) char kbuf1[C::TILE_B];
  __shared__ __attribute__((aligned(1024))) char vbuf0[C::TILE_B];
  __shared__ __attribute__((aligned(1024))) char vbuf1[C::TILE_B];

  const Geom& g = a.g;
  const int S = a.S, H = a.H, n = a.n;
  const int n_sg = (n + SG - 1) / SG;
  // workgroup -> (sample group, chunk, b, h): XCD x = blockIdx & 7 takes units u = j*8 + x
  // of (chunk, b*H + h), each as n_sg consecutive workgroups
  const int xcd = blockIdx.x & 7;
  const int local = blockIdx.x >> 3;
  const int sg = local % n_sg;
  const int u = (local / n_sg) * 8 + xcd;
  if (u >= a.n_chunks * a.B * H) return;
  const int chunk = u % a.n_chunks;
  const int bh = u / a.n_chunks;
  const int h = bh % H, b = bh / H;
  const int nK = (S + BK - 1) / BK;
  const int kt_begin = chunk * a.chunk_tiles;
  const int n_tiles = imax(imin(nK, kt_begin + a.chunk_tiles) - kt_begin, 0);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = wv / NWS;                    // this wave's candidate
  const bool dma_wave = wv < dma_waves(NWT);
  const int wave = dma_wave ? wv : 0;        // DMA slot (unused by the other waves)
  const DevMask m = cands.m[c];
  const int g2 = lane >> 5;
  const int l32 = lane & 31;
  const int si = sg * SG + (wv % NWS) * 32 + l32;  // sample slot of this lane's query row
  const int qrow = imin(imax(a.sample_idx[(size_t)h * n + imin(si, n - 1)], 0), S - 1);

  const uint16_t* qp = (const uint16_t*)a.q;
  const uint16_t* kp = (const uint16_t*)a.k;
  const uint16_t* vp = (const uint16_t*)a.v;
  const int tok_stride = H * D;
  const size_t base_bh = ((size_t)b * S) * tok_stride + (size_t)h * D;

  bf16x8 qf[KSTEPS];
  {
    const uint16_t* src = qp + base_bh + (size_t)qrow * tok_stride + g2 * 8;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[s] = __builtin_bit_cast(bf16x8, *(const u32x4*)(src + s * 16));
  }
  const QueryPos qpos = make_query(g, m, qrow);

  // DMA: K row R of LDS holds key swap_bits23(R) (chunks swizzled by ksw), V row R holds
  // key R (chunks swizzled by vsw for the transposing reads)
  auto dma_off = [&](int i, bool is_v, int lim) __attribute__((always_inline)) -> int {  // element offset, rows clamped to lim
    const int R = (wave * NI + i) * C::ROWS_PER_DMA + lane / C::CH;
    const int p = lane % C::CH;
    return is_v ? imin(R, lim) * tok_stride + (p ^ vsw<D>(R)) * 8
                : imin(swap_bits23(R), lim) * tok_stride + (p ^ ksw<D, NWD>(R)) * 8;
  };
  // Whole-tile DMA offsets, split into a wave-uniform part (added to the scalar base)
  // and a per-lane part, which the DMA takes as an unsigned 32-bit offset and so must
  // not be negative.  The uniform part of DMA j = wave*NI + i is the key row of its
  // lane 0; the per-lane part (row difference and swizzled chunk, both >= 0) depends on
  // j only through j mod TK (the K swizzle repeats every TK DMAs, V's does not vary),
  // so a table of TK lane offsets serves every DMA when NI is a multiple of TK.
  constexpr int TK = D == 128 ? 4 : 2;
  constexpr bool PER = NI % TK == 0;
  constexpr int NKT = PER ? TK : NI;
  auto k_uniform = [&](int j) __attribute__((always_inline)) -> int {  // elements
    return swap_bits23(j * C::ROWS_PER_DMA) * tok_stride;
  };
  int ktab[NKT];  // bytes
#pragma unroll
  for (int t = 0; t < NKT; ++t) {
    const int i = PER ? t - wave * NI : t;  // DMA index whose table entry this is
    ktab[t] = 2 * (dma_off(i, false, BK) - (PER ? k_uniform(t) : 0));
  }
  const int vtab = 2 * dma_off(-wave * NI, true, BK);  // DMA j = 0; V's lane part is the same for all j
  int kofs[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) kofs[s] = l32 * C::ROWB + (((2 * s + g2) ^ ksw<D, NWD>(l32)) * 16);
  // transposing V reads: within 16 lanes, lane i gets element i%4 of rows 4e + i/4
  int vofs[DB];
  {
    const int r4 = (lane & 15) >> 2;
    const int gq = (lane >> 4) & 1;
    const int c4 = lane & 3;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int ch = 4 * db + 2 * gq + (c4 >> 1);
      vofs[db] = (8 * g2 + r4) * C::ROWB + ((ch ^ vsw<D>(r4)) * 16) + (c4 & 1) * 8;
    }
  }

  // DMA of the K (or V) rows of key tile kt; rows past S read row S-1 (masked keys)
  auto issue = [&](int kt, char* buf, bool is_v) __attribute__((always_inline)) {
    if (!dma_wave) return;
    const int c0 = kt * BK;
    const uint16_t* src = (is_v ? vp : kp) + base_bh + (size_t)c0 * tok_stride;
    const uint32_t lds0 = lds_addr(buf + wave * NI * 1024);
    if (c0 + BK <= S) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int j = wave * NI + i;
        if (is_v)
          dma16(src + (size_t)j * C::ROWS_PER_DMA * tok_stride, vtab, lds0 + i * 1024);
        else
          dma16(PER ? src + k_uniform(j) : src, ktab[PER ? i % TK : i], lds0 + i * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) dma16(src, 2 * dma_off(i, is_v, S - 1 - c0), lds0 + i * 1024);
    }
  };
  auto qk = [&](const char* kb_, f32x16* s) __attribute__((always_inline)) {
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 kf = *(const u32x4*)(kb_ + kb * 32 * C::ROWB + kofs[ks]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf), qf[ks], s[kb], 0, 0, 0);
      }
  };
  // register (kb, i) of S^T holds key kb*32 + (i>>3)*16 + 8*g2 + (i&7) of the tile
  auto mask_word = [&](int kt) __attribute__((always_inline)) -> uint32_t {
    const uint64_t bits = tile_row_mask(g, m, qpos, kt * BK, BK);
    const uint32_t lo = (uint32_t)bits, hi = (uint32_t)(bits >> 32);
    return ((lo >> (8 * g2)) & 0xffu) | (((lo >> (16 + 8 * g2)) & 0xffu) << 8) |
           (((hi >> (8 * g2)) & 0xffu) << 16) | (((hi >> (16 + 8 * g2)) & 0xffu) << 24);
  };
  auto masked = [](float x, uint32_t w, int v) __attribute__((always_inline)) {
    const uint32_t f = (uint32_t)((int32_t)(w << (31 - v)) >> 31);
    return __uint_as_float((__float_as_uint(x) & f) | (0xff800000u & ~f));
  };

  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f, mt_cur = -INFINITY;
  const float c_log2 = a.scale * 1.4426950408889634f;
  const float lazy = kLazyLog2 / c_log2;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  f32x16 s_cur[2];
  int kt0 = 0, kt1 = 0, kt2 = 0;

  // the all-keep reference needs the element mask only on the tile that holds the
  // sequence tail
  const bool need_mask = m.kind != VSA_MASK_ALL || (kt_begin + n_tiles) * BK > S;

  // One step per key tile (as in the forward kernel): entering step it, S(it) is
  // masked in registers with its row max, K(it+1) and V(it) are in LDS.
  auto run = [&](auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(mask_tag)::value;
    auto step = [&](auto par_tag, int it) __attribute__((always_inline)) {
      constexpr int P = decltype(par_tag)::value;
      char* k_use = P == 0 ? kbuf1 : kbuf0;
      char* k_fill = P == 0 ? kbuf0 : kbuf1;
      char* v_use = P == 0 ? vbuf0 : vbuf1;
      char* v_fill = P == 0 ? vbuf1 : vbuf0;
      wait_vmcnt<0>();
      barrier_lds();
      if (it + 2 < n_tiles) issue(kt2, k_fill, false);
      if (it + 1 < n_tiles) issue(kt1, v_fill, true);
      uint32_t w_next = ~0u;
      if (MASKED && it + 1 < n_tiles) w_next = mask_word(kt1);

      const bool grow = mt_cur > m_run + lazy;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float m_new = grow ? mt_cur : m_run;
        const float alpha = grow ? __builtin_amdgcn_exp2f((m_run - m_new) * c_log2) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] *= alpha;
        m_run = m_new;
      }
      const float mc = (m_run == -INFINITY) ? 0.f : m_run * c_log2;

      // S(it+1) on the matrix cores with the probabilities of S(it) (the product on the
      // last tile reads a stale buffer and is discarded)
      f32x16 s_next[2];
      qk(k_use, s_next);
      bf16x2 pk[16];
#pragma unroll
      for (int v = 0; v < 32; v += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s_cur[v >> 4][v & 15], c_log2, -mc));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s_cur[v >> 4][(v & 15) + 1], c_log2, -mc));
        pk[v >> 1] = pack_bf16x2(p0, p1);
        l_run = __builtin_amdgcn_fdot2_f32_bf16(pk[v >> 1], ones, l_run, false);
      }
      // O^T += V(it)^T P(it)^T
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 pf = __builtin_bit_cast(
            bf16x8, u32x4{__builtin_bit_cast(uint32_t, pk[4 * j + 0]), __builtin_bit_cast(uint32_t, pk[4 * j + 1]),
                          __builtin_bit_cast(uint32_t, pk[4 * j + 2]), __builtin_bit_cast(uint32_t, pk[4 * j + 3])});
        i16x4 v0[DB], v1[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const char* base = v_use + vofs[db] + j * 16 * C::ROWB;
          v0[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base));
          v1[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 4 * C::ROWB));
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const i16x8 vv = __builtin_shufflevector(v0[db], v1[db], 0, 1, 2, 3, 4, 5, 6, 7);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pf, acc[db], 0, 0, 0);
        }
      }
      // mask and row max of S(it+1)
      float mx = -INFINITY;
#pragma unroll
      for (int v = 0; v < 32; ++v) {
        float x = s_next[v >> 4][v & 15];
        if constexpr (MASKED) {
          x = masked(x, w_next, v);
          s_next[v >> 4][v & 15] = x;
        }
        mx = __builtin_elementwise_maximum(mx, x);
      }
      mt_cur = pair_max(mx);
      s_cur[0] = s_next[0];
      s_cur[1] = s_next[1];
      kt0 = kt1;
      kt1 = kt2;
      kt2 = it + 3 < n_tiles ? kt_begin + it + 3 : 0;
    };

    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    wait_vmcnt<0>();  // query fragments before the first DMA
    if (n_tiles > 0) {
      kt0 = kt_begin;
      kt1 = n_tiles > 1 ? kt_begin + 1 : 0;
      kt2 = n_tiles > 2 ? kt_begin + 2 : 0;
      issue(kt0, kbuf0, false);
      wait_vmcnt<0>();
      barrier_lds();
      if (n_tiles > 1) issue(kt1, kbuf1, false);
      issue(kt0, vbuf0, true);
      qk(kbuf0, s_cur);
      const uint32_t w = MASKED ? mask_word(kt0) : ~0u;
      float mx = -INFINITY;
#pragma unroll
      for (int v = 0; v < 32; ++v) {
        float x = s_cur[v >> 4][v & 15];
        if constexpr (MASKED) {
          x = masked(x, w, v);
          s_cur[v >> 4][v & 15] = x;
        }
        mx = __builtin_elementwise_maximum(mx, x);
      }
      mt_cur = pair_max(mx);
    }
    int it = 0;
    for (; it + 1 < n_tiles; it += 2) {
      step(P0{}, it);
      step(P1{}, it + 1);
    }
    if (it < n_tiles) step(P0{}, it);
    wait_vmcnt<0>();
  };
  if (need_mask)
    run(std::integral_constant<bool, true>{});
  else
    run(std::integral_constant<bool, false>{});

  const float l_tot = pair_sum(l_run);
  if (si < n) {
    float* dst = a.ws + ((((size_t)bh * a.n_chunks + chunk) * NC + c) * n + si) * kProfRow<D>;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = db * 32 + r4 * 8 + g2 * 4;
        *(float4*)(dst + d) = float4{acc[db][r4 * 4 + 0], acc[db][r4 * 4 + 1], acc[db][r4 * 4 + 2],
                                     acc[db][r4 * 4 + 3]};
      }
    if (g2 == 0) {
      dst[D] = m_run;
      dst[D + 1] = l_tot;
    }
  }
}

// Samples per merge workgroup (4 waves, 4 samples each)
constexpr int kMergeSamples = 16;

__host__ __device__ inline size_t part_floats(const ProfArgs& a) {
  return (size_t)a.B * a.H * a.n_chunks * a.n_cand * a.n * (a.D + 4);
}

// Pass 2a: workgroup (h, b, g) merges the chunk partials of samples g*16 .. g*16+15 of
// (b, h) (wave w: samples g*16 + 4w + k; lane l: channels l + 64 t) with a single-pass
// online max, and writes sum over its samples and channels of (o_c - o_0)^2.
template <int D, int NC>
__global__ __launch_bounds__(256) void profile_merge_kernel(ProfArgs a) {
  constexpr int DT = D / 64;
  const int h = blockIdx.x, b = blockIdx.y, grp = blockIdx.z;
  const int n = a.n, H = a.H;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float c_log2 = a.scale * 1.4426950408889634f;
  const size_t row = kProfRow<D>;
  const size_t ch_stride = (size_t)NC * n * row;
  float part[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) part[c] = 0.f;
  for (int k = 0; k < kMergeSamples / 4; ++k) {
    const int si = grp * kMergeSamples + wave * (kMergeSamples / 4) + k;
    if (si >= n) break;
    const float* base = a.ws + ((size_t)(b * H + h) * a.n_chunks) * ch_stride + (size_t)si * row;
    float o[NC][DT];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const float* pc = base + (size_t)c * n * row;
      float mu = -INFINITY, l = 0.f, x[DT];
#pragma unroll
      for (int t = 0; t < DT; ++t) x[t] = 0.f;
      for (int ch = 0; ch < a.n_chunks; ++ch) {
        const float* p = pc + ch * ch_stride;
        const float m = p[D];
        if (m == -INFINITY) continue;  // chunk without a kept key (uniform)
        const float nmu = fmaxf(mu, m);
        const float so = mu == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mu - nmu) * c_log2);
        const float w = __builtin_amdgcn_exp2f((m - nmu) * c_log2);
        l = l * so + p[D + 1] * w;
#pragma unroll
        for (int t = 0; t < DT; ++t) x[t] = x[t] * so + p[lane + 64 * t] * w;
        mu = nmu;
      }
      const float linv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
      for (int t = 0; t < DT; ++t) o[c][t] = x[t] * linv;
    }
#pragma unroll
    for (int c = 1; c < NC; ++c)
#pragma unroll
      for (int t = 0; t < DT; ++t) part[c] += (o[c][t] - o[0][t]) * (o[c][t] - o[0][t]);
  }
  __shared__ float red[NC][4];
#pragma unroll
  for (int c = 1; c < NC; ++c) {
    float v = part[c];
#pragma unroll
    for (int s = 32; s > 0; s >>= 1) v += __shfl_xor(v, s);
    if (lane == 0) red[c][wave] = v;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int G = gridDim.z;
    float* dst = a.ws + part_floats(a) + (((size_t)h * a.B + b) * G + grp) * NC;
    dst[0] = 0.f;
#pragma unroll
    for (int c = 1; c < NC; ++c) dst[c] = ((red[c][0] + red[c][1]) + red[c][2]) + red[c][3];
  }
}

// Pass 2b: per head, the merge sums in a fixed order, err = sqrt(.), route = argmin
// over c >= 1 (lowest c on ties).
template <int NC>
__global__ __launch_bounds__(64) void profile_route_kernel(ProfArgs a, int G) {
  const int h = blockIdx.x * 64 + threadIdx.x;
  if (h >= a.H) return;
  const float* src = a.ws + part_floats(a) + (size_t)h * a.B * G * NC;
  float tot[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) tot[c] = 0.f;
  for (int e = 0; e < a.B * G; ++e)
#pragma unroll
    for (int c = 1; c < NC; ++c) tot[c] += src[(size_t)e * NC + c];
  int best = 1;
  float best_e = 0.f;
  a.err[(size_t)h * NC + 0] = 0.f;
#pragma unroll
  for (int c = 1; c < NC; ++c) {
    const float e = sqrtf(tot[c]);
    a.err[(size_t)h * NC + c] = e;
    if (c == 1 || e < best_e) {
      best_e = e;
      best = c;
    }
  }
  a.route[h] = best;
}

template <int D, int NWS, int NC>
hipError_t launch_t(const ProfArgs& a, const MaskTable& cands, hipStream_t st) {
  const long long units = (long long)a.n_chunks * a.B * a.H;
  const int n_sg = (a.n + NWS * 32 - 1) / (NWS * 32);
  const long long blocks = ((units + 7) / 8) * 8 * n_sg;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((profile_part_kernel<D, NWS, NC>), dim3((unsigned)blocks), dim3(NWS * NC * 64), 0, st, a,
                     cands);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int G = (a.n + kMergeSamples - 1) / kMergeSamples;
  hipLaunchKernelGGL((profile_merge_kernel<D, NC>), dim3(a.H, a.B, G), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((profile_route_kernel<NC>), dim3((a.H + 63) / 64), dim3(64), 0, st, a, G);
  return hipGetLastError();
}

template <int D, int NC>
hipError_t launch_nw(const ProfArgs& a, const MaskTable& cands, hipStream_t st) {
  switch (profile_sample_waves(a.n, NC)) {
    case 1: return launch_t<D, 1, NC>(a, cands, st);
    case 2: return launch_t<D, 2, NC>(a, cands, st);
    default:
      if constexpr (NC == 2) return launch_t<D, 4, NC>(a, cands, st);
      return hipErrorInvalidValue;
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

int32_t profile_sample_waves(int32_t n, int32_t n_cand) {
  const int cap = n_cand <= 2 ? 4 : 2;  // at most 8 waves per workgroup
  const int need = (n + 31) / 32;
  return need <= 1 ? 1 : (need <= 2 || cap == 2 ? 2 : 4);
}

// Key chunks per (b, h): the count that minimises rounds of resident workgroups times
// key tiles per chunk (fewest chunks on ties), with 256 compute units holding one
// workgroup of more than 4 waves or two smaller ones (LDS and registers), and at most
// 8192 workgroups.
int32_t profile_chunks(int32_t B, int32_t S, int32_t H, int32_t n, int32_t n_cand) {
  const int nK = (S + pipe::BK - 1) / pipe::BK;
  const int nws = profile_sample_waves(n, n_cand);
  const long long per_chunk = (long long)B * H * ((n + nws * 32 - 1) / (nws * 32));
  const long long slots = 256LL * (nws * n_cand > 4 ? 1 : 2);
  const long long lim = 8192 / (per_chunk > 0 ? per_chunk : 1);
  const long long c_max = lim < 1 ? 1 : (lim < nK ? lim : nK);
  int best = 1;
  long long best_cost = -1;
  for (long long c = 1; c <= c_max; ++c) {
    const long long cost = ((c * per_chunk + slots - 1) / slots) * ((nK + c - 1) / c);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = (int)c;
    }
  }
  return best;
}

size_t profile_ws_floats(int32_t B, int32_t H, int32_t D, int32_t n, int32_t n_cand,
                         int32_t n_chunks) {
  const size_t groups = (size_t)(n + kMergeSamples - 1) / kMergeSamples;
  return (size_t)B * H * n_chunks * n_cand * n * (D + 4) + (size_t)H * B * groups * n_cand;
}

hipError_t launch_profile(const ProfArgs& a, const MaskTable& cands, hipStream_t stream) {
  if (!a.is_bf16) return hipErrorInvalidValue;
  if (a.D == 128) return launch_nc<128>(a, cands, stream);
  if (a.D == 64) return launch_nc<64>(a, cands, stream);
  return hipErrorInvalidValue;
}

}  // namespace vsa
