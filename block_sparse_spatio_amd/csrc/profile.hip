// Sampled-query head profiler (Sparse VideoGen on TPU, "how to accelerate attention"):
// for each head, a few sampled queries are attended under the reference mask (full
// attention) and under each candidate sparse mask; the deviation of each candidate's
// output from the reference is reduced to one number per (head, candidate) and the
// head is routed to the candidate with the smallest deviation ("supporting dynamic
// routing with fixed tensor shapes": one flag per head, no variable-size head groups).
//
// Pass 0 (profile_words_kernel): the element masks of the sampled rows under every
// candidate that keeps a strict subset of the keys, one 32-bit word per (row, key tile,
// half-wave) in the bit order of the score registers, shared by all batch items.
// Pass 1 (profile_part_kernel): a unit is (b, h, sample group); the key tiles of all
// units, unit after unit, form one sequence that is cut into as many equal contiguous
// ranges as workgroups can be resident at once, one range per workgroup.  A workgroup
// runs the segments of its range (the part of each unit it covers, at most two or three)
// one after the other.  Its score waves hold 32 sampled query rows each and compute
// S^T = K Q^T for every key tile once, into LDS; one softmax wave per (candidate, 32
// rows) takes those scores under its candidate's mask (the all-keep reference only at
// the sequence tail) through the online softmax and O^T += V^T P^T on the matrix cores,
// so the scores are not recomputed per candidate and every SIMD carries the same matrix
// work per tile.  K and V tiles (and the tile's mask words) reach LDS by DMA through a
// ring of stages shared by all waves; V stays row-major and is read with transposing LDS
// reads.  Each segment's unnormalised output, running max and row sum go to the
// workspace as the unit's partial slot (its index among the workgroups that cover the
// unit).  The ranges keep every workgroup equally busy with few partial rows: writes
// mixed into the K/V read stream slow it far more than their bytes.
// Pass 2 (profile_merge_kernel, profile_route_kernel): each sampled row merges its
// unit's partial slots with the softmax statistics (lanes over channels) into sums of
// (o_c - o_0)^2; per head these are added in a fixed order, err[h][c] = sqrt(.) and
// route[h] = argmin over c >= 1 (lowest c on ties).
#include "lds_pipe.h"

namespace vsa {

namespace {

using namespace pipe;

// LDS-typed pointers: arithmetic on them stays in 32-bit LDS addresses, so a read at a
// run-time stage is one base register plus the instruction's immediate offset
typedef __attribute__((address_space(3))) char lchar;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) f32x4 l_f32x4;
typedef __attribute__((address_space(3))) u32x4 l_u32x4;
typedef __attribute__((address_space(3))) uint32_t l_u32;

// one partial row of the workspace: D unnormalised outputs, the running max (raw score
// units) and the row sum, padded to a multiple of 16 bytes
template <int D>
constexpr int kProfRow = D + 4;

// waves that issue a workgroup's K/V DMAs: the largest power of two up to its waves
constexpr int dma_waves(int nw) { return nw >= 8 ? 8 : (nw >= 4 ? 4 : 2); }

// LDS of a pass-1 workgroup with NS ring stages: the K and V rings, NS stages of mask
// words (1 KB DMAs) and three 64 x 32 fp32 score blocks per sample wave.
constexpr int prof_word_dmas(int nws, int nc) { return (nc * nws * 32 * 8 + 1023) / 1024; }
constexpr int prof_lds(int d, int nws, int nc, int ns) {
  return 2 * ns * pipe::BK * d * 2 + ns * prof_word_dmas(nws, nc) * 1024 + 3 * nws * 8192;
}
// Ring depth in key tiles: the deepest of 4, 3, 2 stages whose LDS fits in 160 KB.
constexpr int prof_stages(int d, int nws, int nc) {
  return prof_lds(d, nws, nc, 4) <= 160 * 1024 ? 4 : (prof_lds(d, nws, nc, 3) <= 160 * 1024 ? 3 : 2);
}

// The tile sequence of all units cut into a.n_wg ranges: workgroup w takes tiles
// [range_start(w), range_start(w + 1)); tile x lies in the range of workgroup range_of(x).
__host__ __device__ inline int64_t range_start(const ProfArgs& a, int64_t w) { return w * a.total / a.n_wg; }
__host__ __device__ inline int64_t range_of(const ProfArgs& a, int64_t x) {
  return ((x + 1) * a.n_wg + a.total - 1) / a.total - 1;
}

// Score register (kb, i) of S^T holds key kb*32 + (i>>3)*16 + 8*g2 + (i&7) of the tile
// for the lanes of half-wave g2: the 32 bits of a 64-key row mask that half-wave g2
// needs, with bit kb*16 + i for register (kb, i).
__device__ __forceinline__ uint32_t reg_order_word(uint64_t bits, int g2) {
  const uint32_t lo = (uint32_t)bits, hi = (uint32_t)(bits >> 32);
  return ((lo >> (8 * g2)) & 0xffu) | (((lo >> (16 + 8 * g2)) & 0xffu) << 8) | (((hi >> (8 * g2)) & 0xffu) << 16) |
         (((hi >> (16 + 8 * g2)) & 0xffu) << 24);
}

// Pass 0: one wave per (kWordTiles key tiles, h, table index); lane l takes sample slots
// l, l + 64, ... and writes the two half-wave words of each slot's mask over every tile of
// the group (the key tile is the same for the whole wave, so the walk over its runs is
// scalar work).  Slots past the samples repeat the last sample.
constexpr int kWordTiles = 8;

__global__ __launch_bounds__(64) void profile_words_kernel(ProfArgs a, MaskTable cands) {
  const int nK = (a.S + BK - 1) / BK;
  const int cmi = blockIdx.y % a.n_masked;
  const int h = blockIdx.y / a.n_masked;
  const int kt0 = blockIdx.x * kWordTiles;
  const int kt1 = imin(kt0 + kWordTiles, nK);
  const DevMask m = cands.m[a.cand_of[cmi]];
  for (int si = threadIdx.x; si < a.n_pad; si += 64) {
    const int qrow = imin(imax(a.sample_idx[(size_t)h * a.n + imin(si, a.n - 1)], 0), a.S - 1);
    const QueryPos qp = make_query(a.g, m, qrow);
    for (int kt = kt0; kt < kt1; ++kt) {
      const uint64_t bits = tile_row_mask(a.g, m, qp, kt * BK, BK);
      const size_t t = (((size_t)h * nK + kt) * a.n_masked + cmi) * a.n_pad + si;
      *(u32x2*)(a.words + 2 * t) = u32x2{reg_order_word(bits, 0), reg_order_word(bits, 1)};
    }
  }
}

template <int D, int NWS, int NC>
__global__ __launch_bounds__(NWS * (NC + 1) * 64) __attribute__((amdgpu_waves_per_eu(2)))
void profile_part_kernel(ProfArgs a, MaskTable cands) {
  constexpr int NWT = NWS * (NC + 1);  // NWS score waves, then NWS waves per candidate
  constexpr int SG = NWS * 32;         // samples per workgroup
  constexpr int NWD = dma_waves(NWT);
  using C = Cfg<D, NWD>;
  constexpr int KSTEPS = C::KSTEPS;
  constexpr int DB = C::DB;
  constexpr int NI = C::NI;
  constexpr int NS = prof_stages(D, NWS, NC);
  constexpr int ND = prof_word_dmas(NWS, NC);  // 1 KB DMAs for one tile's mask words
  constexpr int SB = 32 * 64 * 4;                  // one 64 x 32 score block, fp32
  __shared__ __attribute__((aligned(1024))) char kring[NS * C::TILE_B];
  __shared__ __attribute__((aligned(1024))) char vring[NS * C::TILE_B];
  __shared__ __attribute__((aligned(1024))) char wring[NS * ND * 1024];
  __shared__ __attribute__((aligned(1024))) char sring[3 * NWS * SB];
  lchar* const KL = (lchar*)kring;
  lchar* const VL = (lchar*)vring;
  lchar* const WL = (lchar*)wring;
  lchar* const SL = (lchar*)sring;

  const Geom& g = a.g;
  const int S = a.S, H = a.H, n = a.n;
  const int nK = (S + BK - 1) / BK;
  const int64_t lo = range_start(a, blockIdx.x), hi = range_start(a, blockIdx.x + 1);
  if (lo >= hi) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool scorer = wv < NWS;
  const int sw = scorer ? wv : (wv - NWS) % NWS;  // sample wave: 32 of the group's rows
  const int c = scorer ? 0 : (wv - NWS) / NWS;    // candidate of a softmax wave
  const bool dma_wave = wv < NWD;
  const int wave = dma_wave ? wv : 0;  // DMA slot (unused by the other waves)
  const DevMask m = cands.m[c];
  const int g2 = lane >> 5;
  const int l32 = lane & 31;

  const uint16_t* qp = (const uint16_t*)a.q;
  const uint16_t* kp = (const uint16_t*)a.k;
  const uint16_t* vp = (const uint16_t*)a.v;
  const int tok_stride = H * D;
  const int cm = scorer ? -1 : a.cm[c];  // the candidate's rows in the word table, -1 for keep-all
  // wave 0 DMAs each tile's mask words: the workgroup's block is [table index][SG][2]
  // u32; 16 bytes per lane, lanes past the table read its first word (unused)
  const bool wdma = wv == 0 && a.n_masked > 0;
  const size_t wtile = (size_t)a.n_masked * a.n_pad * 8;  // bytes of one tile's words

  // the current segment: unit (b, h, sample group sg), its key tiles
  // [kt_begin, kt_begin + n_tiles) and this lane's sampled row
  int b = 0, h = 0, sg = 0, kt_begin = 0, n_tiles = 0, si = 0;
  size_t base_bh = 0;
  const char* wsrc = nullptr;
  uint32_t woff[ND];
  bf16x8 qf[KSTEPS];

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
  // score wave: S^T = K Q^T of the tile in K stage st for its 32 rows, stored to score
  // buffer sb as 8 float4 per lane (float4 q of lane l at (q*64 + l)*16: conflict-free)
  auto score = [&](int st, int sb) __attribute__((always_inline)) {
    const lchar* kb_ = KL + st * C::TILE_B;
    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 kf = *(const l_u32x4*)(kb_ + kb * 32 * C::ROWB + kofs[ks]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf), qf[ks], s[kb], 0, 0, 0);
      }
    lchar* dst = SL + (sb * NWS + sw) * SB + lane * 16;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      *(l_f32x4*)(dst + q * 1024) = f32x4{s[q >> 2][(q & 3) * 4 + 0], s[q >> 2][(q & 3) * 4 + 1],
                                          s[q >> 2][(q & 3) * 4 + 2], s[q >> 2][(q & 3) * 4 + 3]};
  };
  // register (kb, i) of S^T holds key kb*32 + (i>>3)*16 + 8*g2 + (i&7) of the tile
  auto masked = [](float x, uint32_t w, int v) __attribute__((always_inline)) {
    const uint32_t f = (uint32_t)((int32_t)(w << (31 - v)) >> 31);
    return __uint_as_float((__float_as_uint(x) & f) | (0xff800000u & ~f));
  };
  // this lane's mask word of the chunk tile in word stage st (table candidates)
  auto lds_word = [&](int st) __attribute__((always_inline)) -> uint32_t {
    return *(const l_u32*)(WL + st * ND * 1024 + ((cm * SG + sw * 32 + l32) * 2 + g2) * 4);
  };
  // keep-all candidates: only the keys past the sequence end are masked
  auto tail_word = [&](int kt) __attribute__((always_inline)) -> uint32_t {
    const int valid = S - kt * BK;
    if (valid >= BK) return ~0u;
    return reg_order_word(valid <= 0 ? 0ull : (1ull << valid) - 1, g2);
  };
  auto word = [&](int it) __attribute__((always_inline)) -> uint32_t {
    return cm >= 0 ? lds_word(it % NS) : tail_word(kt_begin + it);
  };

  f32x16 acc[DB];
  float m_run = -INFINITY, l_run = 0.f;
  const float c_log2 = a.scale * 1.4426950408889634f;
  const float lazy = kLazyLog2 / c_log2;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // DMA batch j (j = 0, 1, ...) loads K of segment tile j into K stage j % NS, the mask
  // words of tile j-1 into word stage (j-1) % NS and V of tile j-2 into V stage
  // (j-2) % NS: all three are first needed in step j-2.  The prologue issues batches
  // 0 .. NS (batch NS after S(0)) and step it issues batch it + NS + 1.  In step it the score waves turn K(it+2)
  // into S(it+2) (score buffer (it+2) % 3) while the softmax waves exponentiate S(it)
  // (masked, in registers since the step before), multiply it with V(it), and mask and
  // max-reduce S(it+1) (written in the step before) with the words of tile it+1.  The
  // stages a batch overwrites were last read in the step before it is issued, and a score
  // buffer is rewritten three steps after it was filled, both past a barrier.
  auto issue_batch = [&](int j) __attribute__((always_inline)) {
    if (j < n_tiles) issue(kt_begin + j, kring + (j % NS) * C::TILE_B, false);
    if (wdma && j >= 1 && j - 1 < n_tiles) {
      const char* src = wsrc + (size_t)(kt_begin + j - 1) * wtile;
      const uint32_t dst = lds_addr(wring + ((j - 1) % NS) * ND * 1024);
#pragma unroll
      for (int d = 0; d < ND; ++d) dma16(src, woff[d], dst + d * 1024);
    }
    if (j >= 2 && j - 2 < n_tiles) issue(kt_begin + j - 2, vring + ((j - 2) % NS) * C::TILE_B, true);
  };
  // wait until batch j has landed: while every batch after it up to j + later is whole
  // (2 NI DMAs per DMA wave, and ND more for wave 0's mask words), the later batches
  // may stay in flight (vector-memory loads count down vmcnt in the order they were
  // issued), else wait for all
  auto wait_batch = [&](int j, auto later_tag) __attribute__((always_inline)) {
    constexpr int L = decltype(later_tag)::value;
    if (j + L >= n_tiles)
      wait_vmcnt<0>();
    else if (wdma)
      wait_vmcnt<L * (2 * NI + ND)>();
    else
      wait_vmcnt<L * 2 * NI>();
  };

  // softmax wave: S(t) from score buffer t % 3, under this lane's mask word of tile t
  auto read_scores = [&](int t, f32x16* s) __attribute__((always_inline)) {
    const lchar* src = SL + ((t % 3) * NWS + sw) * SB + lane * 16;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const f32x4 x = *(const l_f32x4*)(src + q * 1024);
      s[q >> 2][(q & 3) * 4 + 0] = x.x;
      s[q >> 2][(q & 3) * 4 + 1] = x.y;
      s[q >> 2][(q & 3) * 4 + 2] = x.z;
      s[q >> 2][(q & 3) * 4 + 3] = x.w;
    }
  };
  f32x16 s_cur[2];
  float mt_cur = -INFINITY;

  // softmax wave, step it: the online softmax of S(it) and O^T += V(it)^T P(it)^T, with
  // the mask and row max of S(it+1) between the products
  auto softmax_pv = [&](auto mask_tag, int it) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(mask_tag)::value;
    // S(it+1) and its words; after the last tile a stale buffer and stage (nothing
    // writes them any more), read only to keep the step straight-line code
    f32x16 s_next[2];
    read_scores(it + 1, s_next);
    const uint32_t w_next = MASKED ? word(it + 1) : ~0u;
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
    bf16x2 pk[16];
#pragma unroll
    for (int v = 0; v < 32; v += 2) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s_cur[v >> 4][v & 15], c_log2, -mc));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s_cur[v >> 4][(v & 15) + 1], c_log2, -mc));
      pk[v >> 1] = pack_bf16x2(p0, p1);
      l_run = __builtin_amdgcn_fdot2_f32_bf16(pk[v >> 1], ones, l_run, false);
    }
    // the stage's byte offset as one scalar, so that each read is its lane's base plus
    // an immediate offset (the compiler otherwise spreads the ring index arithmetic
    // over one register per read)
    const lchar* v_use = VL + __builtin_amdgcn_readfirstlane((it % NS) * C::TILE_B);
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 pf = __builtin_bit_cast(
          bf16x8, u32x4{__builtin_bit_cast(uint32_t, pk[4 * j + 0]), __builtin_bit_cast(uint32_t, pk[4 * j + 1]),
                        __builtin_bit_cast(uint32_t, pk[4 * j + 2]), __builtin_bit_cast(uint32_t, pk[4 * j + 3])});
      i16x4 v0[DB], v1[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const lchar* base = v_use + vofs[db] + j * 16 * C::ROWB;
        v0[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base));
        v1[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 4 * C::ROWB));
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const i16x8 vv = __builtin_shufflevector(v0[db], v1[db], 0, 1, 2, 3, 4, 5, 6, 7);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pf, acc[db], 0, 0, 0);
      }
      // a quarter of S(it+1): mask and row max (discarded after the last tile)
#pragma unroll
      for (int v = 8 * j; v < 8 * j + 8; ++v) {
        float x = s_next[v >> 4][v & 15];
        if constexpr (MASKED) {
          x = masked(x, w_next, v);
          s_next[v >> 4][v & 15] = x;
        }
        mx = __builtin_elementwise_maximum(mx, x);
      }
    }
    mt_cur = pair_max(mx);
    s_cur[0] = s_next[0];
    s_cur[1] = s_next[1];
  };

  // Every wave passes the same barriers: two in the prologue, one per step.  The two
  // roles run their own loops so that the score waves' query fragments and the softmax
  // waves' accumulators are never live together.
  auto steps = [&](auto&& body) __attribute__((always_inline)) {
    for (int it = 0; it < n_tiles; ++it) {
      wait_batch(it + 2, std::integral_constant<int, NS - 2>{});
      barrier_lds();
      issue_batch(it + NS + 1);
      body(it);
    }
  };
  auto softmax_steps = [&](auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(mask_tag)::value;
    // S(0), written in the prologue
    read_scores(0, s_cur);
    const uint32_t w = MASKED ? word(0) : ~0u;
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
    steps([&](int it) __attribute__((always_inline)) { softmax_pv(mask_tag, it); });
  };

  for (int64_t pos = lo; pos < hi;) {
    // ---- segment: the part of unit U in this workgroup's range ----
    const int U = (int)(pos / nK);
    const int64_t seg_end = hi < (int64_t)(U + 1) * nK ? hi : (int64_t)(U + 1) * nK;
    const int slot = (int)(blockIdx.x - range_of(a, (int64_t)U * nK));  // index among the unit's ranges
    kt_begin = (int)(pos - (int64_t)U * nK);
    n_tiles = (int)(seg_end - pos);
    sg = U % a.n_sg;
    const int bh = U / a.n_sg;
    h = bh % H;
    b = bh / H;
    si = sg * SG + sw * 32 + l32;
    base_bh = ((size_t)b * S) * tok_stride + (size_t)h * D;
    if (scorer) {
      const int qrow = imin(imax(a.sample_idx[(size_t)h * n + imin(si, n - 1)], 0), S - 1);
      const uint16_t* src = qp + base_bh + (size_t)qrow * tok_stride + g2 * 8;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) qf[s] = __builtin_bit_cast(bf16x8, *(const u32x4*)(src + s * 16));
    }
    wsrc = (const char*)a.words + (size_t)h * nK * wtile;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      const int byte = d * 1024 + lane * 16;
      const int t = byte / (SG * 8);
      woff[d] = t < a.n_masked ? (uint32_t)(t * a.n_pad * 8 + sg * SG * 8 + byte % (SG * 8)) : 0u;
    }
#pragma unroll
    for (int i = 0; i < DB; ++i) acc[i] = f32x16{};
    m_run = -INFINITY;
    l_run = 0.f;
    // the all-keep reference needs the element mask only on the tile that holds the
    // sequence tail
    const bool need_mask = !scorer && (m.kind != VSA_MASK_ALL || (kt_begin + n_tiles) * BK > S);

    wait_vmcnt<0>();  // query fragments before the first DMA
    if (n_tiles > 0) {
      // prologue: K(0), K(1) and the words of tile 0 (batches 0 and 1), S(0) and S(1);
      // batch NS puts K(NS) into K(0)'s stage, so it goes out once S(0) is done
#pragma unroll
      for (int j = 0; j < NS; ++j) issue_batch(j);
      wait_batch(1, std::integral_constant<int, NS - 2>{});
      barrier_lds();
      if (scorer) {
        score(0, 0);
        if (n_tiles > 1) score(1, 1);
      }
      barrier_lds();
      issue_batch(NS);
      if (scorer) {
        steps([&](int it) __attribute__((always_inline)) {
          if (it + 2 < n_tiles) score((it + 2) % NS, (it + 2) % 3);
        });
      } else if (need_mask) {
        softmax_steps(std::integral_constant<bool, true>{});
      } else {
        softmax_steps(std::integral_constant<bool, false>{});
      }
    }
    wait_vmcnt<0>();  // no DMA may still be writing the rings
    if (!scorer) {
      const float l_tot = pair_sum(l_run);
      if (si < n) {
        float* dst = a.ws + ((((size_t)U * a.n_slots + slot) * NC + c) * SG + sw * 32 + l32) * kProfRow<D>;
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
    barrier_lds();  // every wave is done with the rings before the next segment's DMAs
    pos = seg_end;
  }
}

__host__ __device__ inline size_t part_floats(const ProfArgs& a) {
  return (size_t)a.B * a.H * a.n_slots * a.n_cand * a.n_pad * (a.D + 4);
}

// Pass 2a: one wave per (b, h, sample) merges that row's partial slots of every
// candidate with the softmax statistics: lane ch reads slot ch's max and row sum (64
// slots per round), the wave takes the largest max, and each slot's output row (lanes
// over channels, D/64 adjacent channels per lane) is added with weight exp of its max
// against that one.  Writes sum over channels of (o_c - o_0)^2 for c >= 1 to
// sums[h][b][sample][c].
template <int D, int NC>
__global__ __launch_bounds__(256) void profile_merge_kernel(ProfArgs a) {
  constexpr int DL = D / 64;
  typedef float fvec __attribute__((ext_vector_type(DL)));
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int n = a.n, H = a.H;
  if (row >= (long long)a.B * H * n) return;
  const int si = (int)(row % n);
  const int bh = (int)(row / n);
  const int h = bh % H, b = bh / H;
  const float c_log2 = a.scale * 1.4426950408889634f;
  constexpr size_t RW = kProfRow<D>;
  // the row's unit and the workgroup ranges that cover the unit's key tiles
  const int sgr = a.n_pad / a.n_sg;  // rows per sample group
  const int U = bh * a.n_sg + si / sgr;
  const int64_t nK = (a.S + BK - 1) / BK;
  const int64_t w0 = range_of(a, U * nK);
  const int nch = (int)(range_of(a, (U + 1) * nK - 1) - w0 + 1);
  const size_t ch_stride = (size_t)NC * sgr * RW;  // between partial slots
  const float* base = a.ws + ((size_t)U * a.n_slots * NC * sgr + si % sgr) * RW;
  fvec o[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const float* pc = base + (size_t)c * sgr * RW;
    float mu = -INFINITY;
    for (int c0 = 0; c0 < nch; c0 += 64)
      if (c0 + lane < nch) mu = fmaxf(mu, pc[(c0 + lane) * ch_stride + D]);
#pragma unroll
    for (int s = 32; s > 0; s >>= 1) mu = fmaxf(mu, __shfl_xor(mu, s));
    float l = 0.f;
    fvec x = {};
    if (mu != -INFINITY) {  // uniform: some chunk kept a key
      for (int c0 = 0; c0 < nch; c0 += 64) {
        const int ch = c0 + lane;
        const float m = ch < nch ? pc[ch * ch_stride + D] : -INFINITY;
        const float w = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m - mu) * c_log2);
        if (ch < nch) l = fmaf(pc[ch * ch_stride + D + 1], w, l);
        const int cnt = imin(64, nch - c0);
#pragma unroll 8
        for (int j = 0; j < cnt; ++j) {
          const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j));
          x += *(const fvec*)(pc + (c0 + j) * ch_stride + lane * DL) * wj;
        }
      }
#pragma unroll
      for (int s = 32; s > 0; s >>= 1) l += __shfl_xor(l, s);
    }
    o[c] = x * (l > 0.f ? 1.f / l : 0.f);
  }
  float* dst = a.ws + part_floats(a) + (((size_t)h * a.B + b) * n + si) * NC;
#pragma unroll
  for (int c = 1; c < NC; ++c) {
    const fvec e = o[c] - o[0];
    float v = 0.f;
#pragma unroll
    for (int t = 0; t < DL; ++t) v = fmaf(e[t], e[t], v);
#pragma unroll
    for (int s = 32; s > 0; s >>= 1) v += __shfl_xor(v, s);
    if (lane == 0) dst[c] = v;
  }
  if (lane == 0) dst[0] = 0.f;
}

// Pass 2b: one workgroup per head adds its B * n row sums in a fixed order (thread t
// takes rows t, t + 256, ..., then a fixed pairwise tree), err = sqrt(.), route =
// argmin over c >= 1 (lowest c on ties).
template <int NC>
__global__ __launch_bounds__(256) void profile_route_kernel(ProfArgs a) {
  const int h = blockIdx.x;
  const int t = threadIdx.x;
  const long long rows = (long long)a.B * a.n;
  const float* src = a.ws + part_floats(a) + (size_t)h * rows * NC;
  __shared__ float red[NC][256];
#pragma unroll
  for (int c = 1; c < NC; ++c) {
    float v = 0.f;
    for (long long r = t; r < rows; r += 256) v += src[r * NC + c];
    red[c][t] = v;
  }
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w)
#pragma unroll
      for (int c = 1; c < NC; ++c) red[c][t] += red[c][t + w];
    __syncthreads();
  }
  if (t == 0) {
    int best = 1;
    float best_e = 0.f;
    a.err[(size_t)h * NC + 0] = 0.f;
#pragma unroll
    for (int c = 1; c < NC; ++c) {
      const float e = sqrtf(red[c][0]);
      a.err[(size_t)h * NC + c] = e;
      if (c == 1 || e < best_e) {
        best_e = e;
        best = c;
      }
    }
    a.route[h] = best;
  }
}

template <int D, int NWS, int NC>
hipError_t launch_t(const ProfArgs& a, const MaskTable& cands, hipStream_t st) {
  if (a.n_pad != a.n_sg * NWS * 32 || a.n_wg <= 0) return hipErrorInvalidValue;
  hipError_t e;
  if (a.n_masked > 0) {
    const int wblocks = ((a.S + BK - 1) / BK + kWordTiles - 1) / kWordTiles;
    if ((long long)a.H * a.n_masked > 65535) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(profile_words_kernel, dim3(wblocks, a.H * a.n_masked), dim3(64), 0, st, a, cands);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL((profile_part_kernel<D, NWS, NC>), dim3((unsigned)a.n_wg), dim3(NWS * (NC + 1) * 64), 0, st, a,
                     cands);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const long long mrows = (long long)a.B * a.H * a.n;
  if ((mrows + 3) / 4 > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((profile_merge_kernel<D, NC>), dim3((unsigned)((mrows + 3) / 4)), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((profile_route_kernel<NC>), dim3(a.H), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int D, int NC>
hipError_t launch_nw(const ProfArgs& a, const MaskTable& cands, hipStream_t st) {
  switch (profile_sample_waves(a.n, NC)) {
    case 1: return launch_t<D, 1, NC>(a, cands, st);
    case 2:
      if constexpr (NC <= 3) return launch_t<D, 2, NC>(a, cands, st);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
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
  const int cap = n_cand <= 3 ? 2 : 1;  // (n_cand + 1) * waves <= 8 per workgroup
  return n <= 32 ? 1 : cap;
}

// The launch plan: units (b, h, sample group), the workgroups that can be resident at
// once (each of the 256 compute units holding as many as its LDS, 160 KB, and its waves,
// two per SIMD, allow), one contiguous range of the units' key tiles per workgroup, and
// the partial slots a unit needs (a range has at least total / n_wg tiles, so at most
// (nK - 1) / that + 2 ranges meet one unit).  Workspace: the partial rows, the per-row
// squared-deviation sums, then (at a 256-byte boundary) the mask-word table, sized for
// every candidate having one.
ProfPlan profile_plan(int32_t B, int32_t S, int32_t H, int32_t D, int32_t n, int32_t n_cand) {
  ProfPlan p;
  const int nws = profile_sample_waves(n, n_cand);
  const int sg = 32 * nws;
  p.n_sg = (n + sg - 1) / sg;
  p.n_pad = p.n_sg * sg;
  const int64_t nK = ((int64_t)S + pipe::BK - 1) / pipe::BK;
  p.total = (int64_t)B * H * p.n_sg * nK;
  const int lds = prof_lds(D, nws, n_cand, prof_stages(D, nws, n_cand));
  const int per_cu = imax(1, imin((160 * 1024) / lds, 8 / (nws * (n_cand + 1))));
  p.n_wg = (int32_t)(p.total < 256LL * per_cu ? p.total : 256LL * per_cu);
  const int64_t per_min = p.total / (p.n_wg > 0 ? p.n_wg : 1);
  p.n_slots = (int32_t)((nK - 1) / (per_min > 0 ? per_min : 1) + 2);
  const size_t part = (size_t)B * H * p.n_slots * n_cand * p.n_pad * (D + 4);
  const size_t sums = (size_t)H * B * n * n_cand;
  p.words_off = (part + sums + 63) / 64 * 64;
  p.ws_floats = p.words_off + (size_t)H * nK * n_cand * p.n_pad * 2;
  return p;
}

hipError_t launch_profile(const ProfArgs& a, const MaskTable& cands, hipStream_t stream) {
  if (!a.is_bf16) return hipErrorInvalidValue;
  if (a.D == 128) return launch_nc<128>(a, cands, stream);
  if (a.D == 64) return launch_nc<64>(a, cands, stream);
  return hipErrorInvalidValue;
}

}  // namespace vsa
