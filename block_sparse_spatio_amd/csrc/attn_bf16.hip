// Block-sparse masked attention forward, bf16 inputs, CDNA4 (gfx950) MFMA.
//
// What it computes (Sliding Tile Attention explainer, method section 2, eq. (1)):
// O = softmax(Q K^T * scale + M) V for every (b, h), visiting only the key tiles the
// classifier listed for each query tile.  FULL tiles run with no in-tile mask and
// BOUNDARY tiles apply the exact element mask (Sparse VideoGen on TPU, "avoid in-tile
// masking when nothing needs masking"); both feed one online softmax per query row, the
// running max/sum merge of the DSA study guide, section 18.
//
// CDNA4 mapping.
//  * One workgroup = one (b, h, query tile of Bq = 32*NW rows); NW waves of 64 lanes,
//    each wave owns 32 query rows.  The kernel forms the transposed products
//        S^T = K Q^T     (v_mfma_f32_32x32x16_bf16: A = K rows from LDS, B = Q in VGPRs)
//        O^T += V^T P^T  (A = V^T rows from LDS, B = P^T from the S^T registers)
//    so each lane's accumulator column is one query row: the softmax row max and row sum
//    are in-register reductions plus one v_permlane32_swap with the lane 32 apart, and
//    P never leaves registers.
//  * K and V tiles (64 keys) move HBM -> LDS with global_load_lds_dwordx4 (no VGPR
//    staging), double-buffered: the loads of tile i+1 are in flight while tile i computes.
//    K rows are stored with bits 2 and 3 of the row index swapped, so that the S^T output
//    layout hands every lane 8 consecutive keys per register half: exactly the 8
//    consecutive k-slots of the P^T operand.  V arrives pre-transposed (V^T, written by
//    transpose.hip once per call), so both operands are plain 16-byte LDS reads at full
//    LDS bandwidth.  16-byte chunks are XOR-swizzled per row so that the operand reads
//    spread over all LDS banks (the DMA writes are contiguous anyway).
//  * A boundary tile's element mask is one 32-bit word per lane (bit i: score register i
//    kept).  It comes from a word table computed beforehand (words.hip), DMA'd into LDS
//    beside the tile's K rows, or, for list entries the table does not hold, is derived
//    in the loop from the mask descriptor (vsa_geom.h).  Workgroups whose whole boundary
//    list is in the table run an instance with no mask arithmetic at all.
//  * With the caller's frame-major q and o (the reordering call), each lane gathers its
//    query row and scatters its output row through the head's order; k arrives in the
//    head's order and V^T was gathered by the transpose.
//  * The running max is refreshed lazily: the accumulator is rescaled only when a row's
//    tile max exceeds the reference by more than 2^8 in exp2 units (any lane of the
//    wave), which keeps every probability <= 256 and the result exact up to rounding.
//  * 2 waves per SIMD (register budget 256), so the MFMA work of one wave overlaps the
//    softmax VALU work of another.
#include <type_traits>

#include "lds_pipe.h"

namespace vsa {

namespace {

using namespace pipe;

constexpr int kAllWords = -2;  // kind tag: every boundary mask of the workgroup comes from the word table
constexpr int kOperandLead = 4;  // MFMAs between an LDS operand read and the MFMA that uses it

// WORDS: the instance for query tiles whose whole boundary list is in the word table
// (no mask arithmetic at all); the other instance serves every other query tile.  Two
// kernels rather than one, so that the registers of the mask-deriving bodies do not
// constrain the allocation of the table-driven one.
template <int D, int NW, bool WORDS>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void attn_fwd_bf16_kernel(FwdArgs a, const int32_t* __restrict__ n_full_p, const int32_t* __restrict__ n_bnd_p,
                          const int32_t* __restrict__ full_idx_p, const int32_t* __restrict__ bnd_idx_p,
                          MaskTable masks, HeadMap hm) {
  using C = Cfg<D, NW>;
  constexpr int KSTEPS = C::KSTEPS;
  constexpr int DB = C::DB;
  // K and V rings of two tiles each, as separate objects so that the compiler can tell
  // a DMA into one buffer from the operand reads of another
  __shared__ __attribute__((aligned(1024))) char kbuf0[C::TILE_B];
  __shared__ __attribute__((aligned(1024))) char kbuf1[C::TILE_B];
  __shared__ __attribute__((aligned(1024))) char vbuf0[C::TILE_B];
  __shared__ __attribute__((aligned(1024))) char vbuf1[C::TILE_B];
  // precomputed mask words of the boundary tile whose K is in kbuf0 / kbuf1 (one
  // 32-bit word per lane and wave), moved by the same DMA path as K
  __shared__ __attribute__((aligned(256))) char mbuf0[NW * 256];
  __shared__ __attribute__((aligned(256))) char mbuf1[NW * 256];

  const int S = a.S, H = a.H;
  const int Bq = 32 * NW;

  // ---- workgroup -> (b, h, query tile).  Workgroups are dealt to the 8 XCDs
  // round-robin; XCD x runs, head after head (heaviest first), one contiguous range of
  // each head's query tiles, the ranges of equal listed cost (the per-call schedule), so
  // that every XCD gets the same share of work and its resident workgroups share K/V in
  // its L2.  Workgroups past the end of their range exit at once. ----
  const int cq = a.cq;
  const int xcd = blockIdx.x & 7;
  const int kk = blockIdx.x >> 3;
  const int rank = kk / cq;  // (head rank, batch item)
  if (rank >= a.B * H) return;
  const int h = imin(imax(a.sched[VSA_MAX_UNIQUE_MASKS * 9 + rank / a.B], 0), H - 1);
  const int b = rank % a.B;
  const int slot = hm.slot[h];
  const int q_lo = a.sched[slot * 9 + xcd], q_hi = imin(a.sched[slot * 9 + xcd + 1], a.nQ);
  const int qv = q_lo + (kk - rank * cq);  // position in the mask's visiting order
  if (qv >= q_hi || qv < 0) return;

  const DevMask m_head = masks.m[slot];
  const int qt = qtile_visit(qv, qtile_bands(a.g, m_head, Bq), a.nQ);
  // The body is instantiated for the common (order, mask kind) pairs with both fixed at
  // compile time, so that the per-tile mask arithmetic of a boundary tile carries no
  // other case and stays in straight-line code, plus one generic instance.
  auto run = [&](auto order_tag, auto kind_tag) __attribute__((always_inline)) {
  constexpr int ORDER = decltype(order_tag)::value;  // token order fixed at compile time, or -1
  constexpr int KIND = decltype(kind_tag)::value;    // mask kind fixed at compile time, or -1
  // every boundary tile's mask comes from the word table (no mask arithmetic at all)
  constexpr bool ALL_WORDS = KIND == kAllWords;
  DevMask m = m_head;
  if constexpr (KIND >= 0) m.kind = KIND;
  Geom g = head_geom(a.g, m);
  if constexpr (ORDER >= 0) g.layout = ORDER;
  if constexpr (ORDER == VSA_LAYOUT_FRAME_MAJOR || ORDER == VSA_LAYOUT_POSITION_MAJOR) g.padded = 0;
  const size_t lrow = (size_t)slot * a.nQ + qt;
  // List lengths and entries are clamped to the list row, so malformed lists cannot
  // send a load outside the tensors.  The lists come in as read-only, non-aliased
  // arguments so that these uniform loads are scalar loads that never wait on the
  // vector-memory counter.
  const int nf = imin(imax(n_full_p[lrow], 0), a.nK);
  int nb = imin(imax(n_bnd_p[lrow], 0), a.nK);
  // the table-driven instance runs a list row only when the table holds all of it; a
  // row that the table would cut short (inconsistent lists) is cut to the table
  if constexpr (ALL_WORDS) nb = imin(nb, a.words_cap < 0 ? row_entries(a.bnd_offs, lrow, a.nK) : a.words_cap);
  const int32_t* full_list = full_idx_p + lrow * a.nK;
  const int32_t* bnd_list = bnd_idx_p + lrow * a.nK;
  const int n_tiles = nf + nb;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g2 = lane >> 5;
  const int l32 = lane & 31;

  const uint16_t* qp = (const uint16_t*)a.q;
  const uint16_t* kp = (const uint16_t*)a.k;
  const int tok_stride = H * D;  // elements between consecutive tokens
  const size_t base_bh = ((size_t)b * S) * tok_stride + (size_t)h * D;
  // q and o: the executed order, or the caller's frame-major rows (gathered / scattered)
  const size_t base_io = a.gather_io ? ((size_t)b * a.lse_S) * tok_stride + (size_t)h * D : base_bh;

  // ---- this lane's query row: B operand of S^T = K Q^T, pre-multiplied by
  // c = scale * log2(e) (one more bf16 rounding of q), so that the products are scores
  // in base-2 exponent units and the softmax needs no multiply per score ----
  const int qrow = qt * Bq + wave * 32 + l32;
  const int qrow_c = qrow < S ? qrow : S - 1;
  const float c_log2 = a.scale * 1.4426950408889634f;
  bf16x8 qf[KSTEPS];
  {
    // a padding row of a padded grid reads row 0 (finite data; its output is dropped)
    const int qsrc = a.gather_io ? imax(frame_index(g, qrow_c), 0) : qrow_c;
    const uint16_t* src = qp + base_io + (size_t)qsrc * tok_stride + g2 * 8;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const bf16x8 raw = __builtin_bit_cast(bf16x8, *(const u32x4*)(src + s * 16));
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[s][e] = (__bf16)((float)raw[e] * c_log2);
    }
  }
  const QueryPos qpos = make_query(g, m, qrow_c);

  // ---- per-lane DMA sources (element offsets inside a tile) and LDS read offsets ----
  // K tile: row R of LDS holds key swap_bits23(R), 16-byte chunks swizzled by ksw(R).
  // V^T tile (one contiguous D x 64 block in global memory): row d of LDS holds channel d
  // (64 keys, 128 bytes), chunks swizzled by vtsw(d).
  int dma_k[C::NI], dma_v[C::NI];
#pragma unroll
  for (int i = 0; i < C::NI; ++i) {
    const int R = (wave * C::NI + i) * C::ROWS_PER_DMA + lane / C::CH;
    const int p = lane % C::CH;
    dma_k[i] = 2 * (swap_bits23(R) * tok_stride + (p ^ ksw<D, NW>(R)) * 8);  // bytes
    const int d = (wave * C::NI + i) * 8 + lane / 8;                // 8 V^T rows per DMA
    dma_v[i] = 2 * (d * BK + (((lane % 8) ^ vtsw(d)) * 8));
  }
  int kofs[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) kofs[s] = l32 * C::ROWB + (((2 * s + g2) ^ ksw<D, NW>(l32)) * 16);
  int vofs[4];  // PV operand of 16-key step j: channel row l32 (+32*db), keys 16j + 8*g2 ..
#pragma unroll
  for (int j = 0; j < 4; ++j) vofs[j] = l32 * (BK * 2) + (((2 * j + g2) ^ vtsw(l32)) * 16);

  // list entry it of a boundary tile with precomputed words (uniform); its words
  // (a compact table, words_cap < 0, holds entries [bnd_offs[lrow], bnd_offs[lrow + 1])
  // of each list row)
  const uint32_t* words_row =
      a.words ? a.words + (a.words_cap < 0 ? a.bnd_offs[lrow] : (int64_t)lrow * a.words_cap) * (NW * 64) : nullptr;
  const int words_n = !a.words ? 0 : a.words_cap < 0 ? row_entries(a.bnd_offs, lrow, a.nK) : a.words_cap;
  auto has_words = [&](int it) -> bool {
    if constexpr (ALL_WORDS) return it >= nf && it < n_tiles;
    return words_row != nullptr && !a.pad_only && it >= nf && it < n_tiles && it - nf < words_n;
  };
  auto issue_words = [&](int it, char* mb) __attribute__((always_inline)) {
    dma4(words_row + (size_t)(it - nf) * (NW * 64) + wave * 64, 4u * (uint32_t)lane, lds_addr(mb + wave * 256));
  };
  auto tile_of = [&](int it) -> int {
    return imin(imax(it < nf ? full_list[it] : bnd_list[it - nf], 0), a.nK - 1);
  };

  // DMA of the K rows (or V^T rows) of key tile kt into one ring buffer
  const uint16_t* vtp = (const uint16_t*)a.vt + ((size_t)b * H + h) * D * a.s_pad;  // [s_pad/64][D][64]
  auto issue = [&](int kt, char* buf, bool is_v) {
    const int c0 = kt * BK;
    const uint32_t lds0 = lds_addr(buf + wave * C::NI * 1024);
    if (is_v) {  // V^T is padded to a multiple of 64 keys with zeros: no tail case
      const uint16_t* src = vtp + (size_t)c0 * D;
#pragma unroll
      for (int i = 0; i < C::NI; ++i) dma16(src, dma_v[i], lds0 + i * 1024);
      return;
    }
    const uint16_t* src = kp + base_bh + (size_t)c0 * tok_stride;
    if (c0 + BK <= S) {
#pragma unroll
      for (int i = 0; i < C::NI; ++i) dma16(src, dma_k[i], lds0 + i * 1024);
    } else {  // tail tile: rows past S read row S-1 (those keys are masked, data finite)
#pragma unroll
      for (int i = 0; i < C::NI; ++i) {
        const int R = (wave * C::NI + i) * C::ROWS_PER_DMA + lane / C::CH;
        const int p = lane % C::CH;
        const int off = imin(swap_bits23(R), S - 1 - c0) * tok_stride + ((p ^ ksw<D, NW>(R)) * 8);
        dma16(src, 2 * off, lds0 + i * 1024);
      }
    }
  };

  // Running softmax reference of this lane's row, in base-2 units of c*s: R (-inf until
  // a kept score is seen).  Products start from the accumulator 'bias' = -R (0 while
  // R = -inf) through the MFMA's C operand, so the scores come out already relative to
  // R and a probability is one exp2: no per-score subtraction.
  f32x16 bias = f32x16{};
  float R = -INFINITY;
  float lim = -INFINITY;  // rescale when the tile max exceeds this (kLazyLog2 once R is set)

  // S^T (64 keys x this wave's 32 queries) = K Q^T - R from one K buffer.  The two
  // 32-key halves alternate, so consecutive MFMAs never depend on each other.
  auto qk = [&](const char* kb_, f32x16* s) {
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 kf = *(const u32x4*)(kb_ + kb * 32 * C::ROWB + kofs[ks]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf), qf[ks],
                                                        ks == 0 ? bias : s[kb], 0, 0, 0);
      }
  };
  // Register (kb, i) of S^T holds key kb*32 + (i>>3)*16 + 8*g2 + (i&7) of the tile: gather
  // those 32 bits of the tile's 64-bit row mask (one word per lane).
  auto mask_word = [&](int kt) -> uint32_t {
    const uint64_t bits = a.pad_only ? real_key_mask(g, kt * BK, BK) : tile_row_mask(g, m, qpos, kt * BK, BK);
    const uint32_t lo = (uint32_t)bits, hi = (uint32_t)(bits >> 32);
    return ((lo >> (8 * g2)) & 0xffu) | (((lo >> (16 + 8 * g2)) & 0xffu) << 8) |
           (((hi >> (8 * g2)) & 0xffu) << 16) | (((hi >> (16 + 8 * g2)) & 0xffu) << 24);
  };
  auto apply_mask = [&](f32x16* s, uint32_t w) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int bit = kb * 16 + i;
        const uint32_t f = (uint32_t)((int32_t)(w << (31 - bit)) >> 31);  // all ones if kept
        s[kb][i] = __uint_as_float((__float_as_uint(s[kb][i]) & f) | (0xff800000u & ~f));
      }
  };
  auto row_max = [&](const f32x16* s) -> float {
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 32; ++i) mt = __builtin_elementwise_maximum(mt, s[i >> 4][i & 15]);
    return pair_max(mt);
  };

  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16{};
  float l_run = 0.f;        // this lane's share of the row sum
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // ---- software pipeline over the listed key tiles.  Entering step i, S(i) is in
  // registers (masked) with its row max, K(i+1) and V(i) are in LDS.  The step
  // prefetches K(i+2) and V(i+1), then runs two stages and a tail:
  //   A: S(i+1) = K(i+1) Q^T   with, in its second half,   P(i) = exp2(S(i) - max)
  //   B: O^T += V(i)^T P(i)^T  (the compiler places the vector work of B in the tail)
  //   tail: the element mask and row max of S(i+1), the row sums of P(i)
  // One barrier per step: after it, every wave has finished the previous step (so its
  // buffers may be refilled) and every DMA of this step's inputs has landed.
  f32x16 s_cur[2];
  float mt_cur = -INFINITY;
  // key tiles it, it+1, it+2 (uniform); the index of it+3 is loaded one step ahead
  int kt0 = 0, kt1 = 0, kt2 = 0;
  constexpr int NQK = 2 * KSTEPS;  // MFMAs of stage A
  constexpr int NPV = 4 * DB;      // MFMAs of stage B
  static_assert(NQK % C::NI == 0 && NPV % C::NI == 0, "DMA spread");
  constexpr int EA = 32 / NQK;     // scores per lane per stage-A MFMA on average (2*EA in its second half)
  constexpr int EB = 32 / NPV;     // scores per lane max-reduced per stage-B MFMA
  static_assert(EA % 2 == 0 && EB % 2 == 0, "score pairs");
  // LDS operand of stage-A MFMA i (key half i&1, k-step i>>1) and of stage-B MFMA i
  // (16-key step i/DB, channel block i%DB)
  auto kread = [&](const char* kb_, int i) -> u32x4 {
    return *(const u32x4*)(kb_ + (i & 1) * 32 * C::ROWB + kofs[i >> 1]);
  };
  auto vread = [&](const char* vb_, int i) -> u32x4 {
    return *(const u32x4*)(vb_ + (i % DB) * 32 * (BK * 2) + vofs[i / DB]);
  };
  auto step = [&](auto par_tag, auto nbnd_tag, int it) {
    constexpr int P = decltype(par_tag)::value;      // it & 1
    constexpr bool NEXT_BND = decltype(nbnd_tag)::value;  // tile it+1 needs the element mask
    char* k_use = P == 0 ? kbuf1 : kbuf0;   // K(it+1)
    char* k_fill = P == 0 ? kbuf0 : kbuf1;  // <- K(it+2)
    char* v_use = P == 0 ? vbuf0 : vbuf1;   // V(it)
    char* v_fill = P == 0 ? vbuf1 : vbuf0;  // <- V(it+1)
    const int kt3 = it + 3 < n_tiles ? tile_of(it + 3) : 0;
    wait_vmcnt<0>();
    barrier_lds();
    // The prefetch of K(it+2) and V(it+1) is spread over the MFMA chunks below, one
    // DMA every few MFMAs, instead of issued as one burst: a burst fills the
    // vector-memory queue and stalls the issuing wave.  When no tile is left to
    // prefetch, a listed tile is fetched again into the free buffer (never read).
    const int ktf = it + 2 < n_tiles ? kt2 : kt0;
    const int vtf = it + 1 < n_tiles ? kt1 : kt0;
    const uint16_t* ksrc = kp + base_bh + (size_t)(ktf * BK) * tok_stride;
    const uint16_t* vsrc = vtp + (size_t)(vtf * BK) * D;
    const uint32_t kl0 = lds_addr(k_fill + wave * C::NI * 1024);
    const uint32_t vl0 = lds_addr(v_fill + wave * C::NI * 1024);
    int koff[C::NI];  // tail tile: rows past S read row S-1 (masked keys, finite data)
#pragma unroll
    for (int i = 0; i < C::NI; ++i) koff[i] = dma_k[i];
    if (__builtin_expect(ktf * BK + BK > S, 0)) {
      // a real branch (the empty asm cannot be executed speculatively), so that the
      // other steps do not pay for the clamped offsets of the one tail tile
      asm volatile("");
      const int lim = S - 1 - ktf * BK;
#pragma unroll
      for (int i = 0; i < C::NI; ++i) {
        const int R = (wave * C::NI + i) * C::ROWS_PER_DMA + lane / C::CH;
        koff[i] = 2 * (imin(swap_bits23(R), lim) * tok_stride + ((lane % C::CH) ^ ksw<D, NW>(R)) * 8);
      }
    }
    uint32_t w_next = ~0u;
    if constexpr (NEXT_BND) {
      // the words landed with K(it+1) before this step's barrier; when the table holds the
      // whole boundary list, a boundary successor always has them
      const uint32_t* w_lds = (const uint32_t*)((P == 0 ? mbuf1 : mbuf0) + wave * 256 + 4 * lane);
      if (ALL_WORDS || has_words(it + 1))
        w_next = *w_lds;
      else
        w_next = mask_word(kt1);
    }

    // lazy rescaling: the reference moves only when a row's tile max (relative to R)
    // exceeds kLazyLog2, or when the row sees its first kept score
    const bool grow = mt_cur > lim;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      // lanes that do not grow keep their reference and scale by exactly 1 (their
      // reference may still be -inf, which must not meet a -inf - -inf); the scores of
      // S(it) already in registers move to the new reference
      const float sh = grow ? mt_cur : 0.f;
      const float R_new = grow ? mt_cur - bias[0] : R;
      const float alpha = grow ? __builtin_amdgcn_exp2f(R - R_new) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
#pragma unroll
      for (int i = 0; i < 32; ++i) s_cur[i >> 4][i & 15] -= sh;
      R = R_new;
      lim = R == -INFINITY ? -INFINITY : kLazyLog2;
      const float bv = R == -INFINITY ? 0.f : -R;
#pragma unroll
      for (int i = 0; i < 16; ++i) bias[i] = bv;
    }
    __builtin_amdgcn_sched_barrier(0);

    // stage A.  On the last tile the product runs on the stale buffer and is discarded:
    // keeping it unconditional keeps the stage straight-line code.  Chunk i issues the
    // operand read of MFMA i + kOperandLead, MFMA i, and (second half) the exponentials of 2*EA scores;
    // scheduling fences between chunks keep that order, so every LDS read has
    // kOperandLead MFMAs to land.
    f32x16 s_next[2] = {f32x16{}, f32x16{}};
    bf16x2 pk[16];  // P(it): pk[v/2] holds scores v, v+1 (v = kb*16 + register)
    // Issue priority: the other wave on this SIMD is usually in the opposite stage, and
    // letting stage A (exponentials between its MFMAs) issue first keeps both the
    // vector unit and the matrix core fed while stage B streams MFMAs.
    // One ring of LDS operands runs through both stages: MFMA n (stage A: n < NQK, stage
    // B: n - NQK) finds its operand read kOperandLead MFMAs earlier, so the first
    // operands of stage B are read during the last MFMAs of stage A.
    constexpr int LEAD = kOperandLead;
    constexpr int NOP = NQK + NPV;
    u32x4 ring[LEAD + 1];
    auto opread = [&](int n) __attribute__((always_inline)) -> u32x4 {
      return n < NQK ? kread(k_use, n) : vread(v_use, n - NQK);
    };
#pragma unroll
    for (int n = 0; n < LEAD; ++n) ring[n] = opread(n);
    __builtin_amdgcn_s_setprio(1);
    {
#pragma unroll
      for (int i = 0; i < NQK; ++i) {
        if (i + LEAD < NOP) ring[(i + LEAD) % (LEAD + 1)] = opread(i + LEAD);
        s_next[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ring[i % (LEAD + 1)]),
                                                                qf[i >> 1], i < 2 ? bias : s_next[i & 1], 0, 0, 0);
        if (i % (NQK / C::NI) == 0) {
          const int d = i / (NQK / C::NI);
          dma16(ksrc, koff[d], kl0 + d * 1024);
          if (d == 0 && has_words(it + 2)) issue_words(it + 2, P == 0 ? mbuf0 : mbuf1);
        }
        // The exponentials ride on the second half of the stage only (2*EA per chunk), so
        // that the stage opens with back-to-back MFMAs: measured on one box, bit-identical
        // output, mixed layer 1.0-1.8 %, single mask 0.6 %, sliding tiles 0.6-1.1 % faster
        // than EA per chunk throughout; front-loading them was slower.
        if (i >= NQK / 2) {
#pragma unroll
          for (int e = 0; e < 2 * EA; e += 2) {
            const int v = (i - NQK / 2) * 2 * EA + e;
            const float p0 = __builtin_amdgcn_exp2f(s_cur[v >> 4][v & 15]);
            const float p1 = __builtin_amdgcn_exp2f(s_cur[v >> 4][(v & 15) + 1]);
            pk[v >> 1] = pack_bf16x2(p0, p1);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // stage B: O^T += V(it)^T P(it)^T in four 16-key steps of DB MFMAs; chunk i also
    // masks (boundary successor) and max-reduces EB scores of S(it+1)
    __builtin_amdgcn_s_setprio(0);
    {
      float mx = -INFINITY;
      const uint32_t w = w_next;
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        const int n = NQK + i;
        if (n + LEAD < NOP) ring[(n + LEAD) % (LEAD + 1)] = opread(n + LEAD);
        const int j = i / DB, db = i % DB;
        const bf16x8 pf = __builtin_bit_cast(
            bf16x8, u32x4{__builtin_bit_cast(uint32_t, pk[4 * j + 0]), __builtin_bit_cast(uint32_t, pk[4 * j + 1]),
                          __builtin_bit_cast(uint32_t, pk[4 * j + 2]), __builtin_bit_cast(uint32_t, pk[4 * j + 3])});
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ring[n % (LEAD + 1)]), pf,
                                                          acc[db], 0, 0, 0);
        if (i % (NPV / C::NI) == 0) {
          const int d = i / (NPV / C::NI);
          dma16(vsrc, dma_v[d], vl0 + d * 1024);
        }
#pragma unroll
        for (int e = 0; e < EB; e += 2) {
          const int v = i * EB + e;
          float x0 = s_next[v >> 4][v & 15], x1 = s_next[v >> 4][(v & 15) + 1];
          if constexpr (NEXT_BND) {
            const uint32_t f0 = (uint32_t)((int32_t)(w << (31 - v)) >> 31);  // all ones if kept
            const uint32_t f1 = (uint32_t)((int32_t)(w << (30 - v)) >> 31);
            x0 = __uint_as_float((__float_as_uint(x0) & f0) | (0xff800000u & ~f0));
            x1 = __uint_as_float((__float_as_uint(x1) & f1) | (0xff800000u & ~f1));
            s_next[v >> 4][v & 15] = x0;
            s_next[v >> 4][(v & 15) + 1] = x1;
          }
          // NaN-propagating maximum: v_maximum3_f32, no operand canonicalisation
          mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx, x0), x1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      mt_cur = pair_max(mx);
      // The row sum adds exactly the rounded probabilities the PV product used.  It runs
      // here, in the stage's tail where this wave has no matrix work left, rather than
      // between the QK^T products of stage A: stage A's vector work is what the two waves
      // of a SIMD contend for (same box, bit-identical output: mixed layer 0.3 %, single
      // mask 1.7 %, sliding tiles 1.3 % faster).
#pragma unroll
      for (int v = 0; v < 16; ++v) l_run = __builtin_amdgcn_fdot2_f32_bf16(pk[v], ones, l_run, false);
    }
    s_cur[0] = s_next[0];
    s_cur[1] = s_next[1];
    kt0 = kt1;
    kt1 = kt2;
    kt2 = kt3;
  };

  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using NextFull = std::integral_constant<bool, false>;
  using NextBnd = std::integral_constant<bool, true>;
  // full tiles (listed first) take no element mask, unless every tile is forced through
  // the masked path
  const int n_full_path = a.force_mask ? 0 : nf;
  // The query fragments must have landed before the first DMA is issued: the compiler
  // counts only its own loads, so a later wait for them would also wait for the DMAs.
  wait_vmcnt<0>();
  if (n_tiles > 0) {
    // prologue: S(0) from K(0) in kbuf0; K(1) -> kbuf1 and V(0) -> vbuf0, which is
    // where step 0 expects them
    kt0 = tile_of(0);
    kt1 = n_tiles > 1 ? tile_of(1) : 0;
    kt2 = n_tiles > 2 ? tile_of(2) : 0;
    issue(kt0, kbuf0, false);
    if (has_words(0)) issue_words(0, mbuf0);
    wait_vmcnt<0>();
    barrier_lds();
    if (n_tiles > 1) issue(kt1, kbuf1, false);
    if (has_words(1)) issue_words(1, mbuf1);
    issue(kt0, vbuf0, true);
    qk(kbuf0, s_cur);
    if (n_full_path == 0)  // tile 0 is a boundary tile (with words when the table holds the list)
      apply_mask(s_cur, (ALL_WORDS || has_words(0)) ? *(const uint32_t*)(mbuf0 + wave * 256 + 4 * lane)
                                                    : mask_word(kt0));
    mt_cur = row_max(s_cur);
  }
  // steps [0, n_full_path - 1) are followed by a full tile, steps up to n_tiles - 2 by
  // a boundary tile; the last step's successor is never used.  Parity alternates.
  const int last = n_tiles - 1;
  const int end_full = imin(imax(n_full_path - 1, 0), imax(last, 0));
  int it = 0;
  for (; it + 1 < end_full; it += 2) {
    step(P0{}, NextFull{}, it);
    step(P1{}, NextFull{}, it + 1);
  }
  if (it < end_full) {
    step(P0{}, NextFull{}, it);
    ++it;
  }
  if ((it & 1) && it < last) {
    step(P1{}, NextBnd{}, it);
    ++it;
  }
  for (; it + 1 < last; it += 2) {
    step(P0{}, NextBnd{}, it);
    step(P1{}, NextBnd{}, it + 1);
  }
  if (it < last) {
    step(P0{}, NextBnd{}, it);
    ++it;
  }
  if (it == last) {
    if (it & 1)
      step(P1{}, NextFull{}, it);
    else
      step(P0{}, NextFull{}, it);
  }

  wait_vmcnt<0>();  // no DMA may still be writing this workgroup's LDS when it ends

  // ---- epilogue: O = acc / l, lse = scale*m + ln(l) ----
  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int orow = qrow >= S ? -1 : a.gather_io ? frame_index(g, qrow) : qrow;  // -1: no output row
  if (orow >= 0) {
    uint16_t* op = (uint16_t*)a.o + base_io + (size_t)orow * tok_stride;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = db * 32 + r4 * 8 + g2 * 4;
        const uint32_t w0 = __builtin_bit_cast(uint32_t, pack_bf16x2(acc[db][r4 * 4 + 0] * inv, acc[db][r4 * 4 + 1] * inv));
        const uint32_t w1 = __builtin_bit_cast(uint32_t, pack_bf16x2(acc[db][r4 * 4 + 2] * inv, acc[db][r4 * 4 + 3] * inv));
        *(u32x2*)(op + d) = u32x2{w0, w1};
      }
    if (a.write_lse && g2 == 0) {
      const int lpos = a.lse_frame_major ? (a.gather_io ? orow : frame_index(g, qrow)) : qrow;  // -1: padding
      if (lpos >= 0)
        a.lse[((size_t)b * H + h) * a.lse_S + lpos] = l_tot > 0.f ? R * 0.69314718055994531f + logf(l_tot) : -INFINITY;
    }
  }
  };
  using Any = std::integral_constant<int, -1>;
  using Box = std::integral_constant<int, VSA_MASK_BOX>;
  using Stripe = std::integral_constant<int, VSA_MASK_STRIPE>;
  using Frame = std::integral_constant<int, VSA_LAYOUT_FRAME_MAJOR>;
  using Position = std::integral_constant<int, VSA_LAYOUT_POSITION_MAJOR>;
  using AnyOrder = std::integral_constant<int, -1>;
  using AllWords = std::integral_constant<int, kAllWords>;
  // a word table that holds this query tile's whole boundary list serves every order and
  // kind (the per-workgroup choice is uniform)
  const size_t row = (size_t)slot * a.nQ + qt;
  const int nb_row = imin(imax(n_bnd_p[row], 0), a.nK);
  const bool table_row = a.words && !a.pad_only && !a.force_mask &&
                         (a.words_cap < 0 || nb_row <= a.words_cap);
  if constexpr (WORDS) {
    if (table_row) run(AnyOrder{}, AllWords{});
  } else {
    if (table_row)
      return;
    else if (m_head.layout == VSA_LAYOUT_FRAME_MAJOR && m_head.kind == VSA_MASK_BOX)
      run(Frame{}, Box{});
    else if (m_head.layout == VSA_LAYOUT_FRAME_MAJOR && m_head.kind == VSA_MASK_STRIPE)
      run(Frame{}, Stripe{});
    else if (m_head.layout == VSA_LAYOUT_POSITION_MAJOR && m_head.kind == VSA_MASK_BOX)
      run(Position{}, Box{});
    else if (m_head.layout == VSA_LAYOUT_POSITION_MAJOR && m_head.kind == VSA_MASK_STRIPE)
      run(Position{}, Stripe{});
    else
      run(AnyOrder{}, Any{});
  }
}

template <int D, int NW>
hipError_t launch_t(const FwdArgs& a, const MaskTable& masks, const HeadMap& hm, hipStream_t st) {
  const long long n_blocks = 8LL * a.cq * a.B * a.H;
  if (n_blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  // query tiles whose boundary list is in the word table run the table-driven kernel;
  // with a compact table (cap < 0) or cap >= nK that is every query tile
  const bool use_table = a.words && !a.pad_only && !a.force_mask;
  const bool all_in_table = use_table && (a.words_cap < 0 || a.words_cap >= a.nK);
  if (use_table) {
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, NW, true>), dim3((unsigned)n_blocks), dim3(NW * 64), 0, st, a,
                       a.n_full, a.n_bnd, a.full_idx, a.bnd_idx, masks, hm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!all_in_table)
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, NW, false>), dim3((unsigned)n_blocks), dim3(NW * 64), 0, st, a,
                       a.n_full, a.n_bnd, a.full_idx, a.bnd_idx, masks, hm);
  return hipGetLastError();
}

// Per-call schedule, one workgroup.  Cost of a query tile = 5 per full and 6 per
// boundary key tile (a boundary tile is about 1.2 full tiles) plus 10 for the per-tile
// prologue and epilogue.  For every distinct mask u: the prefix sum P of the costs over
// its query tiles in the mask's visiting order (qtile_visit), raw splits
// s_x = min{k : P(k) >= x*P(nQ)/8}, then the ranges clamped to at most cq tiles each
// (sched_cq), so that the grid covers every tile.  Then the heads in descending order of
// their mask's total cost (ties by head index).
constexpr int kSchedThreads = 1024;

__global__ __launch_bounds__(kSchedThreads) void fwd_schedule_kernel(const int32_t* __restrict__ n_full,
                                                                     const int32_t* __restrict__ n_bnd, int U,
                                                                     int nQ, int nK, int H, int cq, HeadMap hm,
                                                                     Geom g, MaskTable masks, int Bq,
                                                                     int32_t* __restrict__ sched) {
  __shared__ long long seg[kSchedThreads];
  __shared__ long long tot[VSA_MAX_UNIQUE_MASKS];
  __shared__ int raw[8];
  const int t = threadIdx.x;
  const int per = (nQ + kSchedThreads - 1) / kSchedThreads;
  const int i0 = imin(t * per, nQ), i1 = imin(i0 + per, nQ);
  auto cost = [&](size_t r) -> long long {
    return 10 + 5LL * imin(imax(n_full[r], 0), nK) + 6LL * imin(imax(n_bnd[r], 0), nK);
  };
  for (int u = 0; u < U; ++u) {
    const size_t row0 = (size_t)u * nQ;
    const int W = qtile_bands(g, masks.m[u], Bq);
    long long sum = 0;
    for (int i = i0; i < i1; ++i) sum += cost(row0 + qtile_visit(i, W, nQ));
    seg[t] = sum;
    __syncthreads();
    for (int d = 1; d < kSchedThreads; d <<= 1) {
      const long long v = t >= d ? seg[t - d] : 0;
      __syncthreads();
      seg[t] += v;
      __syncthreads();
    }
    const long long total = seg[kSchedThreads - 1];
    // P(i0) = seg[t] - sum; raw split x (1..7): the first k with P(k) >= x*total/8
    long long p = seg[t] - sum;
    for (int i = i0; i < i1; ++i) {
      const long long pn = p + cost(row0 + qtile_visit(i, W, nQ));
      for (int x = 1; x < 8; ++x) {
        const long long tgt = (total * x + 7) / 8;  // P(k) >= x*total/8 <=> 8*P(k) >= x*total
        if (p < tgt && pn >= tgt) raw[x] = i + 1;
      }
      p = pn;
    }
    if (t == 0) {
      tot[u] = total;
      for (int x = 1; x < 8; ++x)
        if (total <= 0) raw[x] = 0;
    }
    __syncthreads();
    if (t == 0) {
      int sp = 0;
      sched[u * 9] = 0;
      for (int x = 0; x < 8; ++x) {
        const int tgt = x < 7 ? raw[x + 1] : nQ;
        int nx = imin(sp + cq, imax(tgt, nQ - (7 - x) * cq));
        nx = imax(imin(nx, nQ), sp);
        sched[u * 9 + x + 1] = nx;
        sp = nx;
      }
    }
    __syncthreads();
  }
  if (t < H) {
    const long long c = tot[hm.slot[t]];
    int rank = 0;
    for (int j = 0; j < H; ++j) {
      const long long cj = tot[hm.slot[j]];
      rank += (cj > c) || (cj == c && j < t);
    }
    sched[VSA_MAX_UNIQUE_MASKS * 9 + rank] = t;
  }
}

}  // namespace

// Query tiles per XCD and head the grid provides: half again the even share, so that a
// range of equal cost may hold up to 1.5x the average count (the schedule clamps to it).
int32_t sched_cq(int32_t nQ) { return (int32_t)((3LL * nQ + 15) / 16); }

size_t sched_ints(int32_t U, int32_t H) { return (size_t)VSA_MAX_UNIQUE_MASKS * 9 + VSA_MAX_HEADS; }

hipError_t launch_fwd_schedule(const FwdArgs& a, int32_t U, const HeadMap& hm, const MaskTable& masks, int32_t* sched,
                               hipStream_t stream) {
  if (U < 1 || U > VSA_MAX_UNIQUE_MASKS || a.H > VSA_MAX_HEADS) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fwd_schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, a.n_full, a.n_bnd, U, a.nQ, a.nK,
                     a.H, a.cq, hm, a.g, masks, a.Bq, sched);
  return hipGetLastError();
}

hipError_t launch_attn_bf16(const FwdArgs& a, const MaskTable& masks, const HeadMap& hm, hipStream_t stream) {
  // element offsets inside one (b, h) slab use 32-bit arithmetic
  if ((long long)a.S * a.H * a.D >= (1LL << 31)) return hipErrorInvalidValue;
  const int nw = a.Bq / 32;
  if (a.D == 128) {
    if (nw == 2) return launch_t<128, 2>(a, masks, hm, stream);
    if (nw == 4) return launch_t<128, 4>(a, masks, hm, stream);
    if (nw == 8) return launch_t<128, 8>(a, masks, hm, stream);
  } else if (a.D == 64) {
    if (nw == 2) return launch_t<64, 2>(a, masks, hm, stream);
    if (nw == 4) return launch_t<64, 4>(a, masks, hm, stream);
    if (nw == 8) return launch_t<64, 8>(a, masks, hm, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace vsa
