// Element masks of the listed boundary tiles, computed ahead of the forward.
//
// A boundary tile needs the exact mask of each query row over its 64 keys (Sparse
// VideoGen on TPU, "avoid in-tile masking ...": only partially kept tiles pay for
// element masking).  The forward can derive it in the loop, where it competes for the
// vector unit with the softmax; this kernel derives the same bits beforehand, in the
// register layout the bf16 forward consumes, so that the forward reads one 32-bit word
// per lane from the lists' side table instead.
//
// Layout of the output: [U][nQ][cap][Bq/32][64] words, or with cap < 0 the compact
// [N][Bq/32][64] whose list row r starts at entry bnd_offs[r] (the exclusive prefix sum
// of the list lengths, N their total).  Word (w, lane) of boundary entry j of query tile
// qt belongs to query row qt*Bq + w*32 + (lane & 31) and holds keys 8*(lane >> 5) +
// {0..7}, + {16..23}, + {32..39}, + {48..55} of the key tile, in that order from bit 0
// (the keys of that lane's score registers).  Rows past S take row S-1, as in the
// forward.  Entries j >= min(n_bnd, cap) are not written.
//
// One thread per query row computes its 64-bit row mask (vsa_geom.h) and writes both
// lanes' words; gridDim.z strides over the entries.  The list row is staged in LDS with
// coalesced loads, so the entry loop does not wait on a global load per entry.
// Integer-exact.
#include "vsa_geom.h"

namespace vsa {

namespace {

constexpr int kStride = 4;  // entries of a row split over this many workgroups
constexpr int kStage = 1024;  // list entries staged in LDS at a time (a multiple of kStride)

__global__ __launch_bounds__(256) void boundary_words_kernel(Geom g_call, MaskTable masks, int Bq, int nQ, int nK,
                                                             const int32_t* __restrict__ n_bnd,
                                                             const int32_t* __restrict__ bnd_idx,
                                                             const int64_t* __restrict__ bnd_offs,
                                                             uint32_t* __restrict__ words, int cap) {
  const int qt = blockIdx.x, u = blockIdx.y;
  const DevMask m = masks.m[u];
  const Geom g = head_geom(g_call, m);
  // stripe periods as multiply-high divisors, prepared once
  const bool stripe = m.kind == VSA_MASK_STRIPE;
  const Divisor dss = make_divisor(stripe ? m.Ss : 1), dts = make_divisor(stripe ? m.Ts : 1);
  const size_t row = (size_t)u * nQ + qt;
  const int nb_list = imin(imax(n_bnd[row], 0), nK);
  // compact table: the row owns entries [bnd_offs[row], bnd_offs[row + 1])
  const int nb = imin(nb_list, cap < 0 ? row_entries(bnd_offs, row, nK) : cap);
  const int r = threadIdx.x;  // query row inside the tile
  const int qrow = qt * Bq + r;
  const QueryPos qpos = make_query(g, m, qrow < g.S ? qrow : g.S - 1);
  const int nw = Bq / 32;
  const int32_t* list = bnd_idx + row * nK;
  const size_t entry0 = cap < 0 ? (size_t)bnd_offs[row] : row * (size_t)cap;  // first entry of the row
  uint32_t* out = words + entry0 * (size_t)(nw * 64) + (r >> 5) * 64 + (r & 31);
  __shared__ int s_kt[kStage];
  for (int base = 0; base < nb; base += kStage) {
    const int cnt = imin(kStage, nb - base);
    __syncthreads();  // the previous chunk's entries are read
    for (int i = threadIdx.x; i < cnt; i += blockDim.x) s_kt[i] = imin(imax(list[base + i], 0), nK - 1);
    __syncthreads();
    for (int jj = blockIdx.z; jj < cnt; jj += kStride) {  // base is a multiple of kStride
      const int kt = s_kt[jj];
      const uint64_t bits = tile_row_mask(g, m, qpos, kt * 64, 64, dss, dts);
      const uint32_t lo = (uint32_t)bits, hi = (uint32_t)(bits >> 32);
#pragma unroll
      for (int g2 = 0; g2 < 2; ++g2) {
        const uint32_t w = ((lo >> (8 * g2)) & 0xffu) | (((lo >> (16 + 8 * g2)) & 0xffu) << 8) |
                           (((hi >> (8 * g2)) & 0xffu) << 16) | (((hi >> (16 + 8 * g2)) & 0xffu) << 24);
        out[(size_t)(base + jj) * (nw * 64) + 32 * g2] = w;
      }
    }
  }
}

}  // namespace

hipError_t launch_boundary_words(const Geom& g, const MaskTable& masks, int32_t U, int32_t Bq, int32_t nQ,
                                 int32_t nK, const int32_t* n_bnd, const int32_t* bnd_idx, const int64_t* bnd_offs,
                                 uint32_t* words, int32_t cap, hipStream_t stream) {
  if (Bq % 32 || Bq > 256 || Bq <= 0) return hipErrorInvalidValue;
  if (nQ == 0 || U == 0 || cap == 0) return hipSuccess;
  hipLaunchKernelGGL(boundary_words_kernel, dim3(nQ, U, kStride), dim3(Bq), 0, stream, g, masks, Bq, nQ, nK, n_bnd,
                     bnd_idx, bnd_offs, words, cap);
  return hipGetLastError();
}

}  // namespace vsa
