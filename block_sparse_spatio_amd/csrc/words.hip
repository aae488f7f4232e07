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
//
// Stripe masks in frame-major order take a shortcut.  There the spatial test depends on
// the key and the query only through s_k - s_q = (k - q) - HW (t_k - t_q) and the
// temporal test only through t_k - t_q (PSA notes, key design 1: both are periodic in
// the coordinate difference), so for a fixed frame difference dt the keep bit is one
// function of the position difference k - q.  A wave's 64 consecutive rows see at most
// two query frames and a 64-key tile at most two key frames (when a frame holds at least
// 64 tokens), so dt takes at most three values; for each the wave evaluates that
// function once over the 127 position differences its rows meet (one difference per
// lane and word, gathered by ballot), and each row's 64-bit mask is a shifted window of
// those bits per key frame.  Integer-exact either way.
#include "vsa_geom.h"

namespace vsa {

namespace {

constexpr int kStride = 4;  // entries of a row split over this many workgroups
constexpr int kStage = 1024;  // list entries staged in LDS at a time (a multiple of kStride)

// the frame-major stripe shortcut applies: whole 64-row waves, frames of at least 64
// tokens
__host__ __device__ inline bool fm_stripe_words(const Geom& g_call, const DevMask& m, int Bq) {
  return m.kind == VSA_MASK_STRIPE && m.layout == VSA_LAYOUT_FRAME_MAJOR && !g_call.padded && g_call.HW >= 64 &&
         Bq % 64 == 0;
}

// FM: the instance for the masks that take the frame-major stripe shortcut (the other
// instance takes the rest); each returns at once on the other's masks, so that neither
// carries the other's registers
template <bool FM>
__global__ __launch_bounds__(256) void boundary_words_kernel(Geom g_call, MaskTable masks, int Bq, int nQ, int nK,
                                                             const int32_t* __restrict__ n_bnd,
                                                             const int32_t* __restrict__ bnd_idx,
                                                             const int64_t* __restrict__ bnd_offs,
                                                             uint32_t* __restrict__ words, int cap) {
  const int qt = blockIdx.x, u = blockIdx.y;
  const DevMask m = masks.m[u];
  if (fm_stripe_words(g_call, m, Bq) != FM) return;
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
  const int lane = threadIdx.x & 63;
  // rows of this wave (all real tiles have q0 <= S - 1): q_lo .. q_hi, clamped to S - 1,
  // in frames tq_lo .. tq_hi; this lane's row qr in frame tq
  Divisor dhw{};
  int q_hi = 0, qr = 0, tq_lo = 0, tq_hi = 0, tq = 0;
  if constexpr (FM) {
    dhw = make_divisor(g.HW);
    q_hi = imin(qt * Bq + (r | 63), g.S - 1);
    qr = imin(qrow, g.S - 1);
    tq_lo = (int)udiv(dhw, (uint32_t)imin(qt * Bq + (r & ~63), g.S - 1));
    tq_hi = (int)udiv(dhw, (uint32_t)q_hi);
    tq = (int)udiv(dhw, (uint32_t)qr);
  }
  const size_t entry0 = cap < 0 ? (size_t)bnd_offs[row] : row * (size_t)cap;  // first entry of the row
  uint32_t* out = words + entry0 * (size_t)(nw * 64) + (r >> 5) * 64 + (r & 31);
  __shared__ int s_kt[kStage];
  // the entry loop, with the row-mask derivation fixed per instance
  auto entries = [&](auto&& row_bits) __attribute__((always_inline)) {
    for (int base = 0; base < nb; base += kStage) {
      const int cnt = imin(kStage, nb - base);
      __syncthreads();  // the previous chunk's entries are read
      for (int i = threadIdx.x; i < cnt; i += blockDim.x) s_kt[i] = imin(imax(list[base + i], 0), nK - 1);
      __syncthreads();
      for (int jj = blockIdx.z; jj < cnt; jj += kStride) {  // base is a multiple of kStride
        const uint64_t bits = row_bits(s_kt[jj]);
        const uint32_t lo = (uint32_t)bits, hi = (uint32_t)(bits >> 32);
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) {
          const uint32_t w = ((lo >> (8 * g2)) & 0xffu) | (((lo >> (16 + 8 * g2)) & 0xffu) << 8) |
                             (((hi >> (8 * g2)) & 0xffu) << 16) | (((hi >> (16 + 8 * g2)) & 0xffu) << 24);
          out[(size_t)(base + jj) * (nw * 64) + 32 * g2] = w;
        }
      }
    }
  };
  if constexpr (!FM) {
    entries([&](int kt) __attribute__((always_inline)) { return tile_row_mask(g, m, qpos, kt * 64, 64, dss, dts); });
  } else {
  entries([&](int kt) __attribute__((always_inline)) {
    const int c0 = kt * 64;
    const int c_last = imin(c0 + 63, g.S - 1);
    const int tk0 = (int)udiv(dhw, (uint32_t)c0), tk1 = (int)udiv(dhw, (uint32_t)c_last);
    // G[e]: bit j of word b <-> position difference d = c0 - q_hi + 64 b + j, under frame
    // difference dt = tk0 - tq_hi + e: the spatial stripe test of s_k - s_q = d - HW dt,
    // and-ed with the temporal test of dt (wave-uniform; usually only e = 0 is in range,
    // as neither the wave's rows nor the key tile cross a frame)
    const int dlo = c0 - q_hi;
    const int dt0 = tk0 - tq_hi;
    uint64_t G[3][2];
#pragma unroll
    for (int e = 0; e < 3; ++e) {
      const int dt = dt0 + e;
      const int adt = iabs(dt - m.To);
      G[e][0] = G[e][1] = 0ull;
      if (dt <= tk1 - tq_lo && (int)((uint32_t)adt - udiv(dts, (uint32_t)adt) * (uint32_t)m.Ts) < m.Tw) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int au = iabs(dlo + 64 * b + lane - g.HW * dt - m.So);
          G[e][b] = __ballot((int)((uint32_t)au - udiv(dss, (uint32_t)au) * (uint32_t)m.Ss) < m.Sw);
        }
      }
    }
    // this row's window: bit i <-> key c0 + i <-> difference c0 + i - q, i.e. G bit
    // i + (q_hi - q), per key frame
    const int o = q_hi - qr;  // 0 .. 63
    const int split = imin((tk0 + 1) * g.HW - c0, 64);  // keys [0, split) in frame tk0
    uint64_t seg[2];
    seg[0] = split >= 64 ? ~0ull : ((1ull << split) - 1);
    seg[1] = ~seg[0];
    uint64_t bits = 0;
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int tk = tk0 + f;
      if (f == 1 && tk > tk1) break;
      if (tk < m.sink) {
        bits |= seg[f];
        continue;
      }
      const int e = tk - tq - dt0;  // 0 .. 2
      const uint64_t g0 = e == 0 ? G[0][0] : (e == 1 ? G[1][0] : G[2][0]);
      const uint64_t g1 = e == 0 ? G[0][1] : (e == 1 ? G[1][1] : G[2][1]);
      const uint64_t win = o == 0 ? g0 : ((g0 >> o) | (g1 << (64 - o)));
      bits |= win & seg[f];
    }
    if (c0 + 64 > g.S) bits &= g.S - c0 >= 64 ? ~0ull : ((1ull << (g.S - c0)) - 1);
    return bits;
  });
  }
}

}  // namespace

hipError_t launch_boundary_words(const Geom& g, const MaskTable& masks, int32_t U, int32_t Bq, int32_t nQ,
                                 int32_t nK, const int32_t* n_bnd, const int32_t* bnd_idx, const int64_t* bnd_offs,
                                 uint32_t* words, int32_t cap, hipStream_t stream) {
  if (Bq % 32 || Bq > 256 || Bq <= 0) return hipErrorInvalidValue;
  if (nQ == 0 || U == 0 || cap == 0) return hipSuccess;
  bool fm = false, other = false;
  for (int u = 0; u < U; ++u) (fm_stripe_words(g, masks.m[u], Bq) ? fm : other) = true;
  if (other) {
    hipLaunchKernelGGL(boundary_words_kernel<false>, dim3(nQ, U, kStride), dim3(Bq), 0, stream, g, masks, Bq, nQ, nK,
                       n_bnd, bnd_idx, bnd_offs, words, cap);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  if (fm) {
    hipLaunchKernelGGL(boundary_words_kernel<true>, dim3(nQ, U, kStride), dim3(Bq), 0, stream, g, masks, Bq, nQ, nK,
                       n_bnd, bnd_idx, bnd_offs, words, cap);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace vsa
