// Tile classification kernel: for every distinct mask and query tile, the class of
// every key tile (full / boundary / empty) and the ascending compact lists of full
// and boundary key tiles (Sparse VideoGen on TPU, "logical sparsity is not physical
// sparsity"; video-DiT attention blog, section 7.3: the per-Q-block K-block table).
//
// With tile-aligned rounding (Sparse VideoGen on TPU, "aligning the sparse mask with
// execution", B3) a boundary tile becomes full (or, if it reaches past S, a boundary
// tile masked only at the padding) when at least half of its real pairs are kept,
// and empty otherwise.
//
// One workgroup per (query tile, mask).  The query range's boxes are computed once, into
// LDS; each thread classifies key tiles with interval arithmetic (vsa_classify_geom.h), visiting
// the key tile's boxes one at a time so that nothing is held in private memory, and a
// workgroup-wide prefix count keeps the lists in ascending key-tile order.
// HBM-bound on the class map and list writes; integer-exact.
#include "vsa_classify_geom.h"

namespace vsa {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__global__ __launch_bounds__(kThreads) void classify_kernel(Geom g_call, MaskTable masks, int Bq, int Bk,
                                                            int round_tiles, int nQ, int nK, uint8_t* __restrict__ cls,
                                                            int32_t* __restrict__ n_full,
                                                            int32_t* __restrict__ n_bnd,
                                                            int32_t* __restrict__ full_idx,
                                                            int32_t* __restrict__ bnd_idx) {
  const int qt = blockIdx.x;
  const int u = blockIdx.y;
  const DevMask m = masks.m[u];
  const Geom g = head_geom(g_call, m);
  const int r0 = qt * Bq;
  const int r1 = imin(r0 + Bq, g.S);
  const PairDivs dv = pair_divs(g, m);

  // boxes of the query tile's real tokens (padding of a padded grid is never kept), the
  // same for every thread: built once into LDS
  __shared__ Box s_R[11];
  __shared__ int s_nr, s_qpad;
  if (threadIdx.x == 0) {
    int nr = 0;
    bool qp = (r0 + Bq) > g.S;
    for_each_box(g, r0, r1, [&](Box b) {
      if (!g.padded || clip_box(g, b, qp)) s_R[nr++] = b;
    });
    s_nr = nr;
    s_qpad = qp;
  }
  __syncthreads();
  const int nr = s_nr;
  const bool q_padded = s_qpad;
  const Box* R = s_R;
  const Box qb = nr > 0 ? bounding_box(R, nr) : Box{0, 0, 0, 0, 0, 0};
  long long q_real = 0;
  for (int i = 0; i < nr; ++i) q_real += box_volume(R[i]);

  __shared__ int s_cnt[2][kWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const size_t row = (size_t)u * nQ + qt;
  uint8_t* cls_row = cls ? cls + row * nK : nullptr;
  int32_t* full_row = full_idx + row * nK;
  int32_t* bnd_row = bnd_idx + row * nK;

  int base_full = 0, base_bnd = 0;
  for (int k0 = 0; k0 < nK; k0 += kThreads) {
    const int kt = k0 + threadIdx.x;
    int c = VSA_TILE_EMPTY;
    if (kt < nK) {
      const int c0 = kt * Bk;
      const int c1 = imin(c0 + Bk, g.S);
      bool padded = q_padded || (c0 + Bk) > g.S;
      c = tile_class_range(g, m, dv, R, nr, qb, c0, c1, padded);
      if (round_tiles && c == VSA_TILE_BOUNDARY) {
        // tile-aligned rounding: keep the tile's real pairs iff at least half are kept
        // kept pairs: summed over box pairs where the predicate is a product over the
        // axes, else per-row popcounts of the exact row masks (Bk <= 64)
        long long kept = 0, k_real = 0;
        const bool by_boxes = m.kind != VSA_MASK_STRIPE;
        tile_counts(g, m, R, nr, c0, c1, by_boxes, kept, k_real, padded);
        if (!by_boxes) {
          for (int r = r0; r < r1; ++r) {
            if (g.padded) {  // padding query rows hold no pair
              int t, y, x;
              pos_coords(g, r, t, y, x);
              if (t >= g.T || y >= g.Hg || x >= g.Wg) continue;
            }
            kept += __popcll(tile_row_mask(g, m, make_query(g, m, r), c0, c1 - c0));
          }
        }
        const long long real = q_real * k_real;
        c = 2 * kept >= real ? (padded ? VSA_TILE_BOUNDARY : VSA_TILE_FULL) : VSA_TILE_EMPTY;
      }
      if (cls_row) cls_row[kt] = (uint8_t)c;
    }
    const uint64_t bf = __ballot(c == VSA_TILE_FULL);
    const uint64_t bb = __ballot(c == VSA_TILE_BOUNDARY);
    if (lane == 0) {
      s_cnt[0][wave] = __popcll(bf);
      s_cnt[1][wave] = __popcll(bb);
    }
    __syncthreads();
    int off_f = base_full, off_b = base_bnd, tot_f = 0, tot_b = 0;
    for (int w = 0; w < kWaves; ++w) {
      if (w < wave) { off_f += s_cnt[0][w]; off_b += s_cnt[1][w]; }
      tot_f += s_cnt[0][w];
      tot_b += s_cnt[1][w];
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    if (c == VSA_TILE_FULL) full_row[off_f + __popcll(bf & below)] = kt;
    if (c == VSA_TILE_BOUNDARY) bnd_row[off_b + __popcll(bb & below)] = kt;
    base_full += tot_f;
    base_bnd += tot_b;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    n_full[row] = base_full;
    n_bnd[row] = base_bnd;
  }
}

// Exclusive prefix sum of the boundary-list lengths over the n = U*nQ list rows:
// offs[r] = sum of n_bnd[0 .. r-1] (each clamped to [0, nK], as the lists are read),
// offs[n] = the total.  It indexes the compact boundary-word table.  One workgroup: each
// thread sums a contiguous segment, the segment sums are scanned in LDS, then every
// thread writes its segment's running sums.
constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void bnd_offsets_kernel(const int32_t* __restrict__ n_bnd, int64_t n,
                                                                   int nK, int64_t* __restrict__ offs) {
  __shared__ int64_t s[kScanThreads];
  const int t = threadIdx.x;
  const int64_t per = (n + kScanThreads - 1) / kScanThreads;
  const int64_t i0 = t * per < n ? t * per : n;
  const int64_t i1 = i0 + per < n ? i0 + per : n;
  int64_t sum = 0;
  for (int64_t i = i0; i < i1; ++i) sum += imin(imax(n_bnd[i], 0), nK);
  s[t] = sum;
  __syncthreads();
  for (int d = 1; d < kScanThreads; d <<= 1) {  // inclusive scan of the segment sums
    const int64_t v = t >= d ? s[t - d] : 0;
    __syncthreads();
    s[t] += v;
    __syncthreads();
  }
  int64_t run = s[t] - sum;
  for (int64_t i = i0; i < i1; ++i) {
    offs[i] = run;
    run += imin(imax(n_bnd[i], 0), nK);
  }
  if (t == kScanThreads - 1) offs[n] = s[t];
}

}  // namespace

hipError_t launch_classify(const Geom& g, const MaskTable& masks, int32_t U, int32_t Bq,
                           int32_t Bk, int32_t round_tiles, int32_t nQ, int32_t nK,
                           const vsa_tile_lists& out, hipStream_t stream) {
  dim3 grid(nQ, U);
  hipLaunchKernelGGL(classify_kernel, grid, dim3(kThreads), 0, stream, g, masks, Bq, Bk, round_tiles, nQ, nK,
                     out.cls, out.n_full, out.n_bnd, out.full_idx, out.bnd_idx);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !out.bnd_offs) return e;
  hipLaunchKernelGGL(bnd_offsets_kernel, dim3(1), dim3(kScanThreads), 0, stream, out.n_bnd, (int64_t)U * nQ, nK,
                     out.bnd_offs);
  return hipGetLastError();
}

}  // namespace vsa
