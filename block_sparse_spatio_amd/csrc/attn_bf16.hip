// Block-sparse masked attention forward, bf16 inputs, CDNA4 (gfx950) MFMA.
//
// What it computes (Sliding Tile Attention explainer, method section 2, eq. (1)):
// O = softmax(Q K^T * scale + M) V for every (b, h), visiting only the key tiles the
// classifier listed for each query tile.  FULL tiles run with no in-tile mask and
// BOUNDARY tiles apply the exact element mask (Sparse VideoGen on TPU, "avoid in-tile
// masking when nothing needs masking"); both feed one online softmax per query row, the
// running max/sum merge of the DSA study guide, section 18.
//
// CDNA4 mapping.  One workgroup = one (b, h, query tile) of Bq = 32*NW rows, NW waves of
// 64 lanes, each wave owning 32 query rows.  The kernel computes the transposed products
//     S^T = K Q^T      (v_mfma_f32_32x32x16_bf16, A = K rows from LDS, B = Q in VGPRs)
//     O^T += V^T P^T   (A = V^T rows from LDS, B = P^T straight from the S^T registers)
// so that a lane's accumulator column is one query row: the row max and row sum of the
// online softmax are in-register reductions plus one exchange with the lane 32 apart,
// and P never leaves registers.  K rows are stored in LDS in the order the S^T output
// layout wants (bits 2 and 3 of the row index swapped), so the 16 S^T values a lane holds
// per 32-key block are keys 8g..8g+7 and 16+8g..16+8g+7 (g = lane/32): exactly the
// 8 consecutive k-slots the P^T operand of the next MFMA needs.  V is transposed once
// per tile while it is staged into LDS.  Both LDS tiles use XOR swizzles so that the
// 16-byte operand reads and the staging writes spread over all banks.
// K/V tiles are prefetched into registers one tile ahead while the current tile computes.
#include "mfma_tile.h"

namespace vsa {

namespace {

using namespace mfma;

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attn_fwd_bf16_kernel(FwdArgs a, MaskTable masks,
                                                                HeadMap hm) {
  constexpr int NT = NW * 64;
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;

  __shared__ TileSmem<D> sm;

  const Geom& g = a.g;
  const int S = a.S, H = a.H;
  const int Bq = 32 * NW;

  // ---- workgroup -> (b, h, query tile).  Workgroups are dealt to the 8 XCDs
  // round-robin; XCD x takes query tiles [x*cq, (x+1)*cq) of every head, so the work
  // of each XCD has the same head mix and its resident workgroups share K/V in L2. ----
  const int cq = (a.nQ + 7) / 8;
  const int xcd = blockIdx.x & 7;
  const int kk = blockIdx.x >> 3;
  const int bh = kk / cq;
  const int qt = xcd * cq + (kk - bh * cq);
  if (qt >= a.nQ || bh >= a.B * H) return;
  const int h = bh % H;
  const int b = bh / H;

  const int slot = hm.slot[h];
  const DevMask m = masks.m[slot];
  const size_t lrow = (size_t)slot * a.nQ + qt;
  // list lengths and entries are clamped to the list row, so malformed lists cannot
  // send a load outside the tensors
  const int nf = imin(imax(a.n_full[lrow], 0), a.nK);
  const int nb = imin(imax(a.n_bnd[lrow], 0), a.nK);
  const int32_t* full_list = a.full_idx + lrow * a.nK;
  const int32_t* bnd_list = a.bnd_idx + lrow * a.nK;
  const int n_tiles = nf + nb;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g2 = lane >> 5;
  const int l32 = lane & 31;

  const uint16_t* qp = (const uint16_t*)a.q;
  const uint16_t* kp = (const uint16_t*)a.k;
  const uint16_t* vp = (const uint16_t*)a.v;
  const size_t tok_stride = (size_t)H * D;
  const size_t base_bh = ((size_t)b * S) * tok_stride + (size_t)h * D;

  // ---- this lane's query row: B operand of S^T = K Q^T ----
  const int qrow = qt * Bq + wave * 32 + l32;
  const int qrow_c = qrow < S ? qrow : S - 1;
  bf16x8 qf[KSTEPS];
  {
    const uint16_t* src = qp + base_bh + (size_t)qrow_c * tok_stride + g2 * 8;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[s] = __builtin_bit_cast(bf16x8, *(const u32x4*)(src + s * 16));
  }
  const QueryPos qpos = make_query(g, m, qrow_c);

  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float c_log2 = a.scale * 1.4426950408889634f;

  Stager<D, NT> stg;
  auto tile_of = [&](int it) -> int {
    return imin(imax(it < nf ? full_list[it] : bnd_list[it - nf], 0), a.nK - 1);
  };

  if (n_tiles > 0) stg.load(kp, vp, base_bh, tok_stride, tile_of(0) * BK, S, tid);

  for (int it = 0; it < n_tiles; ++it) {
    const int kt = tile_of(it);
    const bool boundary = (it >= nf) || a.force_mask;
    __syncthreads();
    stg.store(sm, tid);
    __syncthreads();
    if (it + 1 < n_tiles) stg.load(kp, vp, base_bh, tok_stride, tile_of(it + 1) * BK, S, tid);

    f32x16 st[2];
    qk_tile<D>(sm, qf, l32, g2, st);
    if (boundary) apply_mask(st, tile_row_mask(g, m, qpos, kt * BK, BK), g2);
    uint32_t pk[2][8];
    const float alpha = softmax_step(st, c_log2, m_run, l_run, pk);
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] *= alpha;
    pv_tile<D>(sm, pk, l32, g2, acc);
  }

  // ---- epilogue: O = acc / l, lse = scale*m + ln(l) ----
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < S) {
    uint16_t* op = (uint16_t*)a.o + base_bh + (size_t)qrow * tok_stride;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = db * 32 + r4 * 8 + g2 * 4;
        const uint32_t w0 = pack_bf16x2(acc[db][r4 * 4 + 0] * inv, acc[db][r4 * 4 + 1] * inv);
        const uint32_t w1 = pack_bf16x2(acc[db][r4 * 4 + 2] * inv, acc[db][r4 * 4 + 3] * inv);
        *(u32x2*)(op + d) = u32x2{w0, w1};
      }
    if (a.write_lse && g2 == 0) {
      const int lpos = a.lse_frame_major ? frame_index(g, qrow) : qrow;
      a.lse[((size_t)b * H + h) * S + lpos] =
          l_tot > 0.f ? m_run * a.scale + logf(l_tot) : -INFINITY;
    }
  }
}

template <int D, int NW>
hipError_t launch_t(const FwdArgs& a, const MaskTable& masks, const HeadMap& hm, hipStream_t st) {
  const int cq = (a.nQ + 7) / 8;
  const long long n_blocks = 8LL * cq * a.B * a.H;
  if (n_blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, NW>), dim3((unsigned)n_blocks), dim3(NW * 64), 0, st,
                     a, masks, hm);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const FwdArgs& a, const MaskTable& masks, const HeadMap& hm,
                            hipStream_t stream) {
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
