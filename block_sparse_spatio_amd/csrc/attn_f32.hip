// Block-sparse masked attention forward for fp32 inputs (fp32 FMA throughout).
//
// Same listing, masking and online-softmax contract as the bf16 MFMA kernel
// (Sliding Tile Attention explainer, eq. (1); Sparse VideoGen on TPU, full/boundary
// tile paths; DSA study guide, section 18, online softmax), written for accuracy:
// every product and sum is fp32, exp is expf.  One workgroup per (b, h, query tile);
// one thread per query row; the key tile (Bk rows of K and V) is staged in
// LDS and read as broadcasts.  Bq (threads per workgroup) is 32, 64 or 128.
#include "vsa_geom.h"

namespace vsa {

namespace {

template <int D, int BKT>
__global__ __launch_bounds__(128) void attn_fwd_f32_kernel(FwdArgs a, MaskTable masks, HeadMap hm) {
  __shared__ float ks[BKT][D];
  __shared__ float vs[BKT][D];
  __shared__ int key_real[BKT];
  const int S = a.S, H = a.H;
  const int qt = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int slot = hm.slot[h];
  const DevMask m = masks.m[slot];
  const Geom g = head_geom(a.g, m);
  const size_t lrow = (size_t)slot * a.nQ + qt;
  const int nf = imin(imax(a.n_full[lrow], 0), a.nK);
  const int nb = imin(imax(a.n_bnd[lrow], 0), a.nK);
  const int32_t* full_list = a.full_idx + lrow * a.nK;
  const int32_t* bnd_list = a.bnd_idx + lrow * a.nK;

  const float* qp = (const float*)a.q;
  const float* kp = (const float*)a.k;
  const float* vp = (const float*)a.v;
  const size_t tok = (size_t)H * D;
  const size_t base = (size_t)b * S * tok + (size_t)h * D;

  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int qrow = qt * nthr + tid;
  const int qrow_c = qrow < S ? qrow : S - 1;
  float q[D];
#pragma unroll
  for (int d = 0; d < D; ++d) q[d] = qp[base + (size_t)qrow_c * tok + d];
  const QueryPos qpos = make_query(g, m, qrow_c);

  float acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  for (int it = 0; it < nf + nb; ++it) {
    const int kt = imin(imax(it < nf ? full_list[it] : bnd_list[it - nf], 0), a.nK - 1);
    const bool boundary = it >= nf || a.force_mask;
    const int c0 = kt * BKT;
    __syncthreads();
    // padding keys of a padded grid (never kept) stage zero values, so that whatever
    // the caller's padding rows hold cannot turn 0 * v into NaN
    for (int r = tid; r < BKT; r += nthr) key_real[r] = !g.padded || frame_index(g, imin(c0 + r, S - 1)) >= 0;
    __syncthreads();
    for (int e = tid; e < BKT * D; e += nthr) {
      const int r = e / D, d = e % D;
      const int key = imin(c0 + r, S - 1);
      ks[r][d] = kp[base + (size_t)key * tok + d];
      vs[r][d] = key_real[r] ? vp[base + (size_t)key * tok + d] : 0.f;
    }
    __syncthreads();
    uint64_t bits = ~0ull;
    if (boundary) bits = a.pad_only ? real_key_mask(g, c0, BKT) : tile_row_mask(g, m, qpos, c0, BKT);
    float s[BKT];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < BKT; ++j) {
      float x = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) x = fmaf(q[d], ks[j][d], x);
      x *= a.scale;
      if (!((bits >> j) & 1ull)) x = -INFINITY;
      s[j] = x;
      mt = fmaxf(mt, x);
    }
    const float m_new = fmaxf(m_run, mt);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = expf(m_run - m_use);
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] *= alpha;
    float lsum = 0.f;
#pragma unroll
    for (int j = 0; j < BKT; ++j) {
      const float p = expf(s[j] - m_use);
      lsum += p;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(p, vs[j][d], acc[d]);
    }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
  }
  if (qrow < S) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float* op = (float*)a.o + base + (size_t)qrow * tok;
#pragma unroll
    for (int d = 0; d < D; ++d) op[d] = acc[d] * inv;
    if (a.write_lse) {
      const int lpos = a.lse_frame_major ? frame_index(g, qrow) : qrow;  // -1: padding row
      if (lpos >= 0) a.lse[((size_t)b * H + h) * a.lse_S + lpos] = l_run > 0.f ? m_run + logf(l_run) : -INFINITY;
    }
  }
}

template <int D, int BKT>
hipError_t launch_t(const FwdArgs& a, const MaskTable& masks, const HeadMap& hm, hipStream_t st) {
  dim3 grid(a.nQ, a.H, a.B);
  hipLaunchKernelGGL((attn_fwd_f32_kernel<D, BKT>), grid, dim3(a.Bq), 0, st, a, masks, hm);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(const FwdArgs& a, const MaskTable& masks, const HeadMap& hm,
                           hipStream_t stream) {
  if (a.Bq != 32 && a.Bq != 64 && a.Bq != 128) return hipErrorInvalidValue;
  if (a.D == 64 && a.Bk == 32) return launch_t<64, 32>(a, masks, hm, stream);
  if (a.D == 64 && a.Bk == 64) return launch_t<64, 64>(a, masks, hm, stream);
  if (a.D == 128 && a.Bk == 32) return launch_t<128, 32>(a, masks, hm, stream);
  if (a.D == 128 && a.Bk == 64) return launch_t<128, 64>(a, masks, hm, stream);
  return hipErrorInvalidValue;
}

}  // namespace vsa
