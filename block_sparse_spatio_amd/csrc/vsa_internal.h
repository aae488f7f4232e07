// Internal declarations shared by the host API and the kernels of libvsa.
// Not part of the public ABI (include/vsa.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/vsa.h"

namespace vsa {

// Mask descriptor as the kernels see it: 16-bit fields so that a table of
// VSA_MAX_UNIQUE_MASKS descriptors plus the head map fits in kernel arguments.
// The host normalises every descriptor first (periods and radii clamped to the grid,
// which leaves the predicate unchanged) and rejects values that do not fit.
struct DevMask {
  int16_t kind, sink;
  int16_t rt, rh, rw;
  int16_t Tw, To, Ts, Sw, So, Ss;
  int16_t wt, wh, ww;
  int16_t layout;  // executed token order of the heads using this descriptor (VSA_LAYOUT_*)
  int16_t pad1;
};
static_assert(sizeof(DevMask) == 32, "DevMask layout");

// Division of 0 <= n < 2^31 by a divisor d >= 1 fixed for a call, as a multiply-high, an
// add and a shift (Granlund and Montgomery, "Division by invariant integers using
// multiplication", PLDI 1994): with l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1,
// n / d = (mulhi(m, n) + n) >> l; mulhi(m, n) < n keeps the sum below 2^32.  Used where
// every element of a memory-bound kernel divides by a few call constants.
struct FastDiv {
  uint32_t m, l;
};

__host__ __device__ inline FastDiv fastdiv_make(int32_t d) {
  const uint32_t dd = d < 1 ? 1u : (uint32_t)d;
  uint32_t l = 0;
  while ((1ull << l) < dd) ++l;
  FastDiv f;
  f.m = (uint32_t)((((1ull << l) - dd) << 32) / dd + 1);
  f.l = l;
  return f;
}

__host__ __device__ inline int32_t fastdiv_q(int32_t n, FastDiv f) {
  const uint32_t hi = (uint32_t)(((uint64_t)f.m * (uint32_t)n) >> 32);
  return (int32_t)((hi + (uint32_t)n) >> f.l);
}

// Geometry of the token grid and the executed order.
struct Geom {
  int32_t T, Hg, Wg;     // the token grid
  int32_t bt, bh, bw;    // 3D tile (tile-major layout and STA masks), else 1
  int32_t nT, nH, nW;    // tile grid (of the padded grid: each axis rounded up to tiles)
  int32_t S, HW;         // executed length (T*Hg*Wg, or the padded grid's size), Hg*Wg
  int32_t layout;        // VSA_LAYOUT_FRAME/TILE/POSITION_MAJOR (kernels take it per head
                         // from DevMask::layout; the padded layout is TILE_MAJOR + padded)
  int32_t padded;        // tile-major over the padded grid: positions may be padding
};

// The geometry of one head: the grid with that head's executed order.
__host__ __device__ inline Geom head_geom(const Geom& g, const DevMask& m) {
  Geom r = g;
  r.layout = m.layout;
  return r;
}

struct MaskTable {
  DevMask m[VSA_MAX_UNIQUE_MASKS];
};

struct HeadMap {
  uint8_t slot[VSA_MAX_HEADS];
};

// Executed token order (VSA_LAYOUT_*) of every head, for the token reorder.
struct HeadLayouts {
  uint8_t lay[VSA_MAX_HEADS];
};

// ---- launch wrappers (defined next to their kernels) ----
hipError_t launch_classify(const Geom& g, const MaskTable& masks, int32_t U, int32_t Bq,
                           int32_t Bk, int32_t round_tiles, int32_t nQ, int32_t nK,
                           const vsa_tile_lists& out, hipStream_t stream);

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* vt;       // bf16 path: blocked V^T [B][H][s_pad/64][D][64] (launch_transpose_v)
  int32_t s_pad;        // S rounded up to a multiple of 64
  void* o;
  float* lse;
  const int32_t* n_full;
  const int32_t* n_bnd;
  const int32_t* full_idx;
  const int32_t* bnd_idx;
  int32_t B, S, H, D;
  int32_t nQ, nK;
  int32_t Bq, Bk;
  float scale;
  int32_t force_mask;
  int32_t pad_only;     // boundary tiles mask only keys past S (tile-aligned lists)
  int32_t write_lse;
  int32_t lse_frame_major;  // q/k/v/o were reordered: write lse in frame-major order
  int32_t lse_S;            // length of an lse row (the caller's sequence length)
  // bf16 with the reorder: q and o are the caller's frame-major tensors (lse_S rows per
  // batch item) and each query row is gathered / each output row scattered through its
  // head's order; only k is reordered (v is gathered by the transpose)
  int32_t gather_io;
  // bf16 path, optional: precomputed mask words of boundary list entries j < words_cap,
  // [U][nQ][words_cap][Bq/32 waves][64 lanes] (launch_boundary_words); words_cap < 0:
  // the compact table, entry j of list row r at bnd_offs[r] + j
  const uint32_t* words;
  int32_t words_cap;
  const int64_t* bnd_offs;
  // bf16 path: the per-call schedule (launch_fwd_schedule): for every distinct mask the
  // query tiles that XCD x runs, positions [sched[u*9 + x], sched[u*9 + x + 1]) of the
  // mask's visiting order (qtile_visit), and after the U*9 entries the heads in
  // descending order of cost; cq = query tiles per XCD and head that the grid provides
  // (sched_cq, at least every chunk's length)
  const int32_t* sched;
  int32_t cq;
  Geom g;
};

hipError_t launch_attn_bf16(const FwdArgs& a, const MaskTable& masks, const HeadMap& hm,
                            hipStream_t stream);
// The bf16 forward's grid serves 8 XCDs; each XCD runs one contiguous range of query
// tiles of every head (neighbouring tiles share key tiles in that XCD's L2).  The
// schedule splits each distinct mask's query tiles into 8 ranges of equal listed cost and
// orders the heads heaviest first; it is written by one small kernel per call.
int32_t sched_cq(int32_t nQ);
size_t sched_ints(int32_t U, int32_t H);
// The order in which a head's query tiles are dealt to the XCDs.  A box mask that is
// unbounded in time and bounded in space (a temporal head) keeps the keys of the query's
// in-frame neighbourhood in every frame, so in frame-major order the query tiles at the
// same place in different frames need the same key tiles.  Such heads visit the tiles
// band by band: the tiles form a grid of W = round(HW / Bq) columns (qt = r*W + c, so a
// column holds the tiles about one frame apart), read column after column; the
// workgroups an XCD runs at once then walk nearly the same key tiles in the same order,
// and those reach L2 once.  Every other head keeps the identity order (W = 1).
__host__ __device__ inline int32_t qtile_bands(const Geom& g, const DevMask& m, int32_t Bq) {
  if (m.layout != VSA_LAYOUT_FRAME_MAJOR || g.padded || m.kind != VSA_MASK_BOX || m.rt >= 0 ||
      (m.rh < 0 && m.rw < 0))
    return 1;
  const int32_t w = (g.HW + Bq / 2) / Bq;
  return w >= 2 ? w : 1;
}
// position j of the visiting order -> query tile (a bijection on [0, nQ)): column c of
// the W-column grid holds R = ceil(nQ / W) tiles for c < full = nQ - (R - 1) W, else R - 1
__host__ __device__ inline int32_t qtile_visit(int32_t j, int32_t W, int32_t nQ) {
  if (W <= 1) return j;
  const int32_t R = (nQ + W - 1) / W;
  const int32_t full = nQ - (R - 1) * W;
  int32_t c, r;
  if (j < full * R) {
    c = j / R;
    r = j - c * R;
  } else {
    const int32_t jj = j - full * R;
    c = full + jj / (R - 1);
    r = jj - (c - full) * (R - 1);
  }
  return r * W + c;
}

hipError_t launch_fwd_schedule(const FwdArgs& a, int32_t U, const HeadMap& hm, const MaskTable& masks, int32_t* sched,
                               hipStream_t stream);
hipError_t launch_attn_f32(const FwdArgs& a, const MaskTable& masks, const HeadMap& hm,
                           hipStream_t stream);
// cap < 0: the compact table indexed by bnd_offs
hipError_t launch_boundary_words(const Geom& g, const MaskTable& masks, int32_t U, int32_t Bq, int32_t nQ,
                                 int32_t nK, const int32_t* n_bnd, const int32_t* bnd_idx, const int64_t* bnd_offs,
                                 uint32_t* words, int32_t cap, hipStream_t stream);
// g, hl: the call's geometry and every head's executed order.  gather != 0: v is
// frame-major with S_src rows per batch item and key p of head h is its frame-major row
// under layout hl.lay[h]; else v is in the executed order.  Padding keys of a padded grid
// are written as zeros either way.
hipError_t launch_transpose_v(const void* v, void* vt, int32_t B, int32_t S, int32_t H, int32_t D,
                              int32_t s_pad, const Geom& g, const HeadLayouts& hl, int32_t gather, int32_t S_src,
                              hipStream_t stream);
hipError_t launch_reorder(const void* src, void* dst, int32_t elem_bytes, int32_t B,
                          int32_t H, int32_t D, const Geom& g, const HeadLayouts& hl,
                          int32_t inverse, hipStream_t stream);

struct ProfArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* sample_idx;
  float* err;
  int32_t* route;
  float* ws;
  int32_t B, S, H, D, n, n_cand;
  int32_t n_sg;     // sample groups per (b, h); a unit is (b, h, sample group)
  int32_t n_wg;     // workgroups of pass 1, each one contiguous range of the units' key tiles
  int32_t n_slots;  // partial slots per unit
  int64_t total;    // key tiles of all units
  float scale;
  int32_t is_bf16;
  Geom g;
  // element-mask words of the sampled rows under the candidates that keep a strict
  // subset of the keys (in the workspace): u32 [H][nK][n_masked][n_pad][2]
  uint32_t* words;
  int32_t n_masked;    // candidates with a word table
  int32_t n_pad;       // samples rounded up to whole sample groups
  int32_t cm[4];       // candidate -> its index in the table, -1 for keep-all candidates
  int32_t cand_of[4];  // table index -> candidate
};
struct MergeArgs {
  const void* o[16];
  const float* lse[16];
  void* out;
  float* lse_out;
  int32_t n, B, S, H, D, is_bf16;
};
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);

struct ProfPlan {
  int32_t n_sg, n_pad, n_wg, n_slots;
  int64_t total;
  size_t words_off;  // floats before the mask-word table
  size_t ws_floats;  // workspace size in floats
};
ProfPlan profile_plan(int32_t B, int32_t S, int32_t H, int32_t D, int32_t n, int32_t n_cand);
int32_t profile_sample_waves(int32_t n, int32_t n_cand);
hipError_t launch_profile(const ProfArgs& a, const MaskTable& cands, hipStream_t stream);

}  // namespace vsa
