// libvsa C ABI: argument validation, descriptor deduplication and normalisation,
// workspace sizing and kernel launches.  Every check runs before the first HIP call,
// so invalid arguments are rejected (with a message in vsa_last_error) on any machine.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "vsa_internal.h"

namespace {

thread_local std::string g_err;

vsa_status fail(vsa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

vsa_status ok() {
  g_err.clear();
  return VSA_OK;
}

vsa_status hip_fail(hipError_t e, const char* what) {
  return fail(VSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr long long kMaxS = 1LL << 30;
constexpr int kMaxDevices = 64;

long long ceil_to(long long a, long long b) { return (a + b - 1) / b * b; }

// Validate the grid for a call layout; *S = T*Hg*Wg (the frame-major sequence length).
vsa_status check_grid(const vsa_grid* g, vsa_layout layout, bool need_tile, long long* S) {
  if (!g) return fail(VSA_ERR_INVALID_ARG, "grid is NULL");
  if (g->T <= 0 || g->Hg <= 0 || g->Wg <= 0)
    return fail(VSA_ERR_INVALID_ARG, "grid T, Hg, Wg must be positive (got %d, %d, %d)", g->T, g->Hg,
                g->Wg);
  if (g->T > 32767 || g->Hg > 32767 || g->Wg > 32767)
    return fail(VSA_ERR_UNSUPPORTED, "grid dimensions above 32767 are not supported");
  const long long s = (long long)g->T * g->Hg * g->Wg;
  if (s > kMaxS) return fail(VSA_ERR_UNSUPPORTED, "sequence length %lld above 2^30", s);
  if (layout != VSA_LAYOUT_FRAME_MAJOR && layout != VSA_LAYOUT_TILE_MAJOR && layout != VSA_LAYOUT_POSITION_MAJOR &&
      layout != VSA_LAYOUT_TILE_PADDED)
    return fail(VSA_ERR_INVALID_ARG, "unknown layout %d", (int)layout);
  if (g->tile_t < 0 || g->tile_h < 0 || g->tile_w < 0)
    return fail(VSA_ERR_INVALID_ARG, "negative tile size");
  // the tile matters only to tile-major orders and sliding-tile masks; elsewhere it is
  // ignored
  if (layout == VSA_LAYOUT_TILE_MAJOR || layout == VSA_LAYOUT_TILE_PADDED || need_tile) {
    if (g->tile_t <= 0 || g->tile_h <= 0 || g->tile_w <= 0)
      return fail(VSA_ERR_INVALID_ARG, "tile-major layouts and sliding-tile masks need tile_t/h/w > 0");
    if (layout == VSA_LAYOUT_TILE_PADDED) {  // each axis is padded up to whole tiles
      const long long tp = ceil_to(g->T, g->tile_t), hp = ceil_to(g->Hg, g->tile_h), wp = ceil_to(g->Wg, g->tile_w);
      if (tp > 32767 || hp > 32767 || wp > 32767 || tp * hp * wp > kMaxS)
        return fail(VSA_ERR_UNSUPPORTED, "padded grid %lldx%lldx%lld too large", tp, hp, wp);
    } else if (g->T % g->tile_t || g->Hg % g->tile_h || g->Wg % g->tile_w) {
      return fail(VSA_ERR_INVALID_ARG, "tile %dx%dx%d does not divide grid %dx%dx%d (the padded layout pads it)",
                  g->tile_t, g->tile_h, g->tile_w, g->T, g->Hg, g->Wg);
    }
  }
  *S = s;
  return VSA_OK;
}

// Executed sequence length of the call layout: the padded grid's size for the padded
// layout, else T*Hg*Wg.  The grid must have passed check_grid.
long long exec_len(const vsa_grid* g, vsa_layout layout) {
  if (layout != VSA_LAYOUT_TILE_PADDED) return (long long)g->T * g->Hg * g->Wg;
  return ceil_to(g->T, g->tile_t) * ceil_to(g->Hg, g->tile_h) * ceil_to(g->Wg, g->tile_w);
}

vsa::Geom make_geom(const vsa_grid* g, vsa_layout layout) {
  vsa::Geom G;
  G.T = g->T; G.Hg = g->Hg; G.Wg = g->Wg;
  G.bt = g->tile_t > 0 ? g->tile_t : 1;
  G.bh = g->tile_h > 0 ? g->tile_h : 1;
  G.bw = g->tile_w > 0 ? g->tile_w : 1;
  // tile counts of the grid padded up to whole tiles (equal to the exact counts when
  // the tile divides the grid, which every layout but the padded one requires)
  G.nT = (G.T + G.bt - 1) / G.bt; G.nH = (G.Hg + G.bh - 1) / G.bh; G.nW = (G.Wg + G.bw - 1) / G.bw;
  G.HW = G.Hg * G.Wg;
  G.padded = layout == VSA_LAYOUT_TILE_PADDED ? 1 : 0;
  G.S = (int32_t)exec_len(g, layout);
  G.layout = (int32_t)(layout == VSA_LAYOUT_TILE_PADDED ? VSA_LAYOUT_TILE_MAJOR : layout);
  return G;
}

bool fits16(long long v) { return v >= -32768 && v <= 32767; }

// Validate one descriptor and convert it to the kernels' 16-bit form.  Periods, widths,
// radii and windows beyond what the grid can reach are clamped to an equivalent value.
// `layout` is the call's layout, which heads with head_layout = VSA_HEAD_LAYOUT_CALL use.
vsa_status normalise(const vsa_mask_desc& d, const vsa_grid* g, vsa_layout layout, int index, vsa::DevMask* out) {
  memset(out, 0, sizeof *out);
  if (d.sink_frames < 0) return fail(VSA_ERR_INVALID_ARG, "mask %d: sink_frames < 0", index);
  if (d.head_layout < VSA_HEAD_LAYOUT_CALL || d.head_layout > VSA_HEAD_LAYOUT_POSITION)
    return fail(VSA_ERR_INVALID_ARG, "mask %d: unknown head_layout %d", index, d.head_layout);
  if (layout == VSA_LAYOUT_TILE_PADDED && d.head_layout != VSA_HEAD_LAYOUT_CALL)
    return fail(VSA_ERR_INVALID_ARG, "mask %d: the padded layout applies to every head (head_layout must be 0)",
                index);
  if (layout == VSA_LAYOUT_TILE_PADDED)
    out->layout = VSA_LAYOUT_TILE_MAJOR;  // over the padded grid
  else
    out->layout = (int16_t)(d.head_layout == VSA_HEAD_LAYOUT_CALL ? (int)layout : d.head_layout - 1);
  out->kind = (int16_t)d.kind;
  out->sink = (int16_t)(d.sink_frames < g->T ? d.sink_frames : g->T);
  const bool box_unused = d.rt == 0 && d.rh == 0 && d.rw == 0;
  const bool stripe_unused = d.Tw == 0 && d.To == 0 && d.Ts == 0 && d.Sw == 0 && d.So == 0 && d.Ss == 0;
  const bool sta_unused = d.win_t == 0 && d.win_h == 0 && d.win_w == 0;
  auto clamp_r = [](int r, int n) -> int16_t { return (int16_t)(r < 0 ? -1 : (r < n ? r : n)); };
  switch (d.kind) {
    case VSA_MASK_ALL:
      if (!box_unused || !stripe_unused || !sta_unused)
        return fail(VSA_ERR_INVALID_ARG, "mask %d: ALL with non-zero parameters", index);
      break;
    case VSA_MASK_BOX:
      if (!stripe_unused || !sta_unused)
        return fail(VSA_ERR_INVALID_ARG, "mask %d: BOX with stripe/window fields set", index);
      out->rt = clamp_r(d.rt, g->T);
      out->rh = clamp_r(d.rh, g->Hg);
      out->rw = clamp_r(d.rw, g->Wg);
      break;
    case VSA_MASK_STRIPE: {
      if (!box_unused || !sta_unused)
        return fail(VSA_ERR_INVALID_ARG, "mask %d: STRIPE with box/window fields set", index);
      if (d.Ts < 1 || d.Ss < 1) return fail(VSA_ERR_INVALID_ARG, "mask %d: stripe periods must be >= 1", index);
      if (d.Tw < 0 || d.Sw < 0) return fail(VSA_ERR_INVALID_ARG, "mask %d: stripe widths must be >= 0", index);
      const long long HW = (long long)g->Hg * g->Wg;
      // |dt - To| < T + |To|: a period at least that large never wraps
      long long Ts = d.Ts, Ss = d.Ss;
      const long long tmax = (long long)g->T + llabs((long long)d.To);
      const long long smax = HW + llabs((long long)d.So);
      if (Ts > tmax) Ts = tmax;
      if (Ss > smax) Ss = smax;
      long long Tw = d.Tw < Ts ? d.Tw : Ts, Sw = d.Sw < Ss ? d.Sw : Ss;
      if (!fits16(d.To) || !fits16(d.So) || !fits16(Ts) || !fits16(Ss) || !fits16(tmax) || !fits16(smax))
        return fail(VSA_ERR_UNSUPPORTED, "mask %d: stripe parameters or frame size exceed 16 bits", index);
      out->Tw = (int16_t)Tw; out->To = (int16_t)d.To; out->Ts = (int16_t)Ts;
      out->Sw = (int16_t)Sw; out->So = (int16_t)d.So; out->Ss = (int16_t)Ss;
      break;
    }
    case VSA_MASK_STA: {
      if (!box_unused || !stripe_unused)
        return fail(VSA_ERR_INVALID_ARG, "mask %d: STA with box/stripe fields set", index);
      if (d.win_t < 1 || d.win_h < 1 || d.win_w < 1)
        return fail(VSA_ERR_INVALID_ARG, "mask %d: STA window must be >= 1 tile per axis", index);
      // tiles per axis of the grid padded up to whole tiles
      const int nT = (g->T + g->tile_t - 1) / g->tile_t, nH = (g->Hg + g->tile_h - 1) / g->tile_h,
                nW = (g->Wg + g->tile_w - 1) / g->tile_w;
      out->wt = (int16_t)(d.win_t < nT ? d.win_t : nT);
      out->wh = (int16_t)(d.win_h < nH ? d.win_h : nH);
      out->ww = (int16_t)(d.win_w < nW ? d.win_w : nW);
      break;
    }
    default:
      return fail(VSA_ERR_INVALID_ARG, "mask %d: unknown kind %d", index, d.kind);
  }
  return VSA_OK;
}

// Whether the grid's 3D tile must be set: some mask is sliding-tile, or some head runs
// in the tile-major order.
bool needs_tile(const vsa_mask_desc* m, int n) {
  for (int i = 0; i < n; ++i)
    if (m[i].kind == VSA_MASK_STA || m[i].head_layout == VSA_HEAD_LAYOUT_TILE) return true;
  return false;
}

// Dedupe + normalise H descriptors into a table.  head_map[h] = slot.
vsa_status build_table(const vsa_mask_desc* masks, int32_t H, const vsa_grid* g, vsa_layout layout,
                       vsa::MaskTable* table, vsa::HeadMap* hm, int32_t* U) {
  if (!masks) return fail(VSA_ERR_INVALID_ARG, "masks is NULL");
  if (H <= 0) return fail(VSA_ERR_INVALID_ARG, "H must be positive");
  if (H > VSA_MAX_HEADS) return fail(VSA_ERR_UNSUPPORTED, "H=%d above VSA_MAX_HEADS", H);
  int32_t first[VSA_MAX_UNIQUE_MASKS];
  int32_t u = 0;
  memset(table, 0, sizeof *table);
  memset(hm, 0, sizeof *hm);
  for (int h = 0; h < H; ++h) {
    int slot = -1;
    for (int j = 0; j < u; ++j)
      if (memcmp(&masks[first[j]], &masks[h], sizeof(vsa_mask_desc)) == 0) { slot = j; break; }
    if (slot < 0) {
      if (u == VSA_MAX_UNIQUE_MASKS)
        return fail(VSA_ERR_UNSUPPORTED, "more than %d distinct masks", VSA_MAX_UNIQUE_MASKS);
      vsa_status st = normalise(masks[h], g, layout, h, &table->m[u]);
      if (st != VSA_OK) return st;
      first[u] = h;
      slot = u++;
    }
    hm->slot[h] = (uint8_t)slot;
  }
  *U = u;
  return VSA_OK;
}

int elem_size(vsa_dtype dt) { return dt == VSA_BF16 ? 2 : 4; }

// Byte sizes of the arrays of vsa_tile_lists, each rounded up to 256 bytes, in struct
// order: cls, n_full, n_bnd, full_idx, bnd_idx, bnd_offs.
vsa_status tile_list_sizes(const vsa_grid* grid, vsa_layout layout, int32_t U, int32_t Bq, int32_t Bk,
                           size_t sz[6]) {
  long long S;
  vsa_status st = check_grid(grid, layout, false, &S);
  if (st != VSA_OK) return st;
  if (U < 1 || U > VSA_MAX_UNIQUE_MASKS) return fail(VSA_ERR_INVALID_ARG, "U=%d (1..%d)", U, VSA_MAX_UNIQUE_MASKS);
  if (Bq < 1 || Bk < 1 || Bq > 4096 || Bk > 4096) return fail(VSA_ERR_INVALID_ARG, "tile sizes must be in 1..4096");
  S = exec_len(grid, layout);
  const size_t nQ = (size_t)((S + Bq - 1) / Bq), nK = (size_t)((S + Bk - 1) / Bk), rows = (size_t)U * nQ;
  auto a256 = [](size_t x) { return (x + 255) / 256 * 256; };
  sz[0] = a256(rows * nK);
  sz[1] = a256(rows * 4);
  sz[2] = a256(rows * 4);
  sz[3] = a256(rows * nK * 4);
  sz[4] = a256(rows * nK * 4);
  sz[5] = a256((rows + 1) * 8);
  return VSA_OK;
}

}  // namespace

extern "C" {

const char* vsa_last_error(void) { return g_err.c_str(); }

vsa_status vsa_unique_masks(const vsa_mask_desc* masks, int32_t H, int32_t* head_map, int32_t* n_unique) {
  if (!masks || !n_unique) return fail(VSA_ERR_INVALID_ARG, "masks and n_unique must be non-NULL");
  if (H <= 0) return fail(VSA_ERR_INVALID_ARG, "H must be positive");
  if (H > VSA_MAX_HEADS) return fail(VSA_ERR_UNSUPPORTED, "H=%d above VSA_MAX_HEADS", H);
  int32_t first[VSA_MAX_HEADS];
  int32_t u = 0;
  for (int h = 0; h < H; ++h) {
    int slot = -1;
    for (int j = 0; j < u; ++j)
      if (memcmp(&masks[first[j]], &masks[h], sizeof(vsa_mask_desc)) == 0) { slot = j; break; }
    if (slot < 0) { first[u] = h; slot = u++; }
    if (head_map) head_map[h] = slot;
  }
  *n_unique = u;
  return ok();
}

vsa_status vsa_tile_counts(const vsa_grid* grid, int32_t Bq, int32_t Bk, int32_t* nQ, int32_t* nK) {
  long long S;
  vsa_status st = check_grid(grid, VSA_LAYOUT_FRAME_MAJOR, false, &S);
  if (st != VSA_OK) return st;
  if (Bq < 1 || Bk < 1 || Bq > 4096 || Bk > 4096) return fail(VSA_ERR_INVALID_ARG, "tile sizes must be in 1..4096");
  if (!nQ || !nK) return fail(VSA_ERR_INVALID_ARG, "nQ/nK must be non-NULL");
  *nQ = (int32_t)((S + Bq - 1) / Bq);
  *nK = (int32_t)((S + Bk - 1) / Bk);
  return ok();
}

vsa_status vsa_seq_len(const vsa_grid* grid, vsa_layout layout, int32_t* S) {
  long long s;
  vsa_status st = check_grid(grid, layout, false, &s);
  if (st != VSA_OK) return st;
  if (!S) return fail(VSA_ERR_INVALID_ARG, "S is NULL");
  *S = (int32_t)exec_len(grid, layout);
  return ok();
}

vsa_status vsa_tile_lists_bytes(const vsa_grid* grid, vsa_layout layout, int32_t U, int32_t Bq, int32_t Bk,
                                size_t* bytes) {
  if (!bytes) return fail(VSA_ERR_INVALID_ARG, "bytes is NULL");
  size_t sz[6];
  vsa_status st = tile_list_sizes(grid, layout, U, Bq, Bk, sz);
  if (st != VSA_OK) return st;
  *bytes = sz[0] + sz[1] + sz[2] + sz[3] + sz[4] + sz[5];
  return ok();
}

vsa_status vsa_tile_lists_carve(const vsa_grid* grid, vsa_layout layout, int32_t U, int32_t Bq, int32_t Bk,
                                void* base, vsa_tile_lists* out) {
  if (!base || !out) return fail(VSA_ERR_INVALID_ARG, "base and out must be non-NULL");
  if ((uintptr_t)base & 255) return fail(VSA_ERR_INVALID_ARG, "base must be 256-byte aligned");
  size_t sz[6];
  vsa_status st = tile_list_sizes(grid, layout, U, Bq, Bk, sz);
  if (st != VSA_OK) return st;
  char* p = (char*)base;
  out->cls = (uint8_t*)p;
  p += sz[0];
  out->n_full = (int32_t*)p;
  p += sz[1];
  out->n_bnd = (int32_t*)p;
  p += sz[2];
  out->full_idx = (int32_t*)p;
  p += sz[3];
  out->bnd_idx = (int32_t*)p;
  p += sz[4];
  out->bnd_offs = (int64_t*)p;
  return ok();
}

vsa_status vsa_classify_tiles(const vsa_grid* grid, vsa_layout layout, const vsa_mask_desc* masks, int32_t H,
                              int32_t Bq, int32_t Bk, const vsa_tile_lists* out, void* stream) {
  return vsa_classify_tiles_ex(grid, layout, masks, H, Bq, Bk, 0, out, stream);
}

vsa_status vsa_classify_tiles_ex(const vsa_grid* grid, vsa_layout layout, const vsa_mask_desc* masks, int32_t H,
                                 int32_t Bq, int32_t Bk, int32_t flags, const vsa_tile_lists* out, void* stream) {
  long long S;
  vsa_status st = check_grid(grid, layout, masks && H > 0 && H <= VSA_MAX_HEADS && needs_tile(masks, H), &S);
  if (st != VSA_OK) return st;
  if (Bq < 1 || Bk < 1 || Bq > 4096 || Bk > 4096) return fail(VSA_ERR_INVALID_ARG, "tile sizes must be in 1..4096");
  if (!out || !out->n_full || !out->n_bnd || !out->full_idx || !out->bnd_idx)
    return fail(VSA_ERR_INVALID_ARG, "tile list arrays must be non-NULL (cls may be NULL)");
  if (flags & ~VSA_CLASSIFY_ROUND_TILES) return fail(VSA_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
  const int32_t round_tiles = (flags & VSA_CLASSIFY_ROUND_TILES) ? 1 : 0;
  if (round_tiles && Bk > 64) return fail(VSA_ERR_UNSUPPORTED, "tile rounding needs Bk <= 64 (Bk=%d)", Bk);
  vsa::MaskTable table;
  vsa::HeadMap hm;
  int32_t U = 0;
  st = build_table(masks, H, grid, layout, &table, &hm, &U);
  if (st != VSA_OK) return st;
  S = exec_len(grid, layout);
  const int32_t nQ = (int32_t)((S + Bq - 1) / Bq), nK = (int32_t)((S + Bk - 1) / Bk);
  hipError_t e = vsa::launch_classify(make_geom(grid, layout), table, U, Bq, Bk, round_tiles, nQ, nK, *out,
                                      (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "classify launch");
  return ok();
}

vsa_status vsa_boundary_words(const vsa_grid* grid, vsa_layout layout, const vsa_mask_desc* masks, int32_t H,
                              int32_t Bq, int32_t Bk, const vsa_tile_lists* tiles, uint32_t* words, int32_t cap,
                              void* stream) {
  long long S;
  vsa_status st = check_grid(grid, layout, masks && H > 0 && H <= VSA_MAX_HEADS && needs_tile(masks, H), &S);
  if (st != VSA_OK) return st;
  if ((Bq != 64 && Bq != 128 && Bq != 256) || Bk != 64)
    return fail(VSA_ERR_UNSUPPORTED, "mask words for tiles Bq=%d Bk=%d (supported: Bq 64/128/256, Bk 64)", Bq, Bk);
  if (!tiles || !tiles->n_bnd || !tiles->bnd_idx)
    return fail(VSA_ERR_INVALID_ARG, "tile lists (n_bnd, bnd_idx) must be non-NULL");
  if (cap < 0 && cap != VSA_WORDS_COMPACT) return fail(VSA_ERR_INVALID_ARG, "cap=%d is negative", cap);
  if (cap == VSA_WORDS_COMPACT && !tiles->bnd_offs)
    return fail(VSA_ERR_INVALID_ARG, "the compact table (cap = VSA_WORDS_COMPACT) needs tiles->bnd_offs");
  if (cap != 0 && !words) return fail(VSA_ERR_INVALID_ARG, "words is NULL");
  if (((uintptr_t)words & 15)) return fail(VSA_ERR_INVALID_ARG, "words must be 16-byte aligned");
  vsa::MaskTable table;
  vsa::HeadMap hm;
  int32_t U = 0;
  st = build_table(masks, H, grid, layout, &table, &hm, &U);
  if (st != VSA_OK) return st;
  S = exec_len(grid, layout);
  const int32_t nQ = (int32_t)((S + Bq - 1) / Bq), nK = (int32_t)((S + Bk - 1) / Bk);
  if (cap > nK) return fail(VSA_ERR_INVALID_ARG, "cap=%d above the %d key tiles", cap, nK);
  hipError_t e = vsa::launch_boundary_words(make_geom(grid, layout), table, U, Bq, nQ, nK, tiles->n_bnd,
                                            tiles->bnd_idx, tiles->bnd_offs, words, cap, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "mask words launch");
  return ok();
}

// bf16: V^T [B][H][D][S rounded up to 64] (the PV operand, transposed once per call);
// with VSA_FWD_REORDER_IO, k in each head's executed order before it (q and v are
// gathered and o scattered by row); then the per-call schedule of the grid (a few KB).
// f32 with VSA_FWD_REORDER_IO: reordered copies of q, k and v.
static size_t vt_pad(int32_t S) { return ((size_t)S + 63) / 64 * 64; }
static size_t sched_bytes() {
  return (vsa::sched_ints(VSA_MAX_UNIQUE_MASKS, VSA_MAX_HEADS) * sizeof(int32_t) + 255) / 256 * 256;
}
static size_t fwd_ws_bytes(int32_t B, int32_t S, int32_t H, int32_t D, vsa_dtype dtype, int32_t flags) {
  const size_t eb = elem_size(dtype);
  const size_t copies = dtype == VSA_BF16 ? 1 : 3;
  size_t n = (flags & VSA_FWD_REORDER_IO) ? copies * B * S * H * D * eb : 0;
  if (dtype == VSA_BF16) n += (size_t)B * H * D * vt_pad(S) * eb + sched_bytes();
  return n;
}

vsa_status vsa_fwd_workspace_bytes(int32_t B, int32_t S, int32_t H, int32_t D, vsa_dtype dtype, int32_t flags,
                                   size_t* bytes) {
  if (!bytes) return fail(VSA_ERR_INVALID_ARG, "bytes is NULL");
  if (B <= 0 || S <= 0 || H <= 0 || D <= 0) return fail(VSA_ERR_INVALID_ARG, "B, S, H, D must be positive");
  if (dtype != VSA_BF16 && dtype != VSA_F32) return fail(VSA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  *bytes = fwd_ws_bytes(B, S, H, D, dtype, flags);
  return ok();
}

vsa_status vsa_sparse_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, vsa_dtype dtype,
                               int32_t B, int32_t S, int32_t H, int32_t D, const vsa_grid* grid, vsa_layout layout,
                               const vsa_mask_desc* masks, const vsa_tile_lists* tiles, int32_t Bq, int32_t Bk,
                               float scale, int32_t flags, void* workspace, size_t ws_bytes, void* stream) {
  return vsa_sparse_attn_fwd_ex(q, k, v, o, lse, dtype, B, S, H, D, grid, layout, masks, tiles, Bq, Bk, scale, flags,
                                nullptr, 0, workspace, ws_bytes, stream);
}

}  // extern "C"

// Scratch of vsa_sparse_attn_fwd_noalloc: a file-scope device array, one copy per GPU,
// which holds what the forward's workspace holds (V^T per 64-key block, the reordered k
// with VSA_FWD_REORDER_IO, the per-call schedule).  In host code `scratch` only names
// the symbol; its device address on each GPU comes from hipGetSymbolAddress, taken once
// per device with that device current, and only that address is ever passed on.
static __device__ __align__(256) char scratch[VSA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kScratchBytes = VSA_NOALLOC_SCRATCH_BYTES;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The calling thread's current device's copy of `scratch`.
vsa_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(VSA_ERR_UNSUPPORTED, "device %d above %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return VSA_OK;
}

// The forward behind vsa_sparse_attn_fwd(_ex) and vsa_sparse_attn_fwd_noalloc: every
// check first, then (use_scratch) the static scratch in place of a workspace argument.
vsa_status fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, vsa_dtype dtype, int32_t B,
                    int32_t S, int32_t H, int32_t D, const vsa_grid* grid, vsa_layout layout,
                    const vsa_mask_desc* masks, const vsa_tile_lists* tiles, int32_t Bq, int32_t Bk, float scale,
                    int32_t flags, const uint32_t* words, int32_t words_cap, void* workspace, size_t ws_bytes,
                    bool use_scratch, void* stream) {
  long long S_grid;
  vsa_status st = check_grid(grid, layout, masks && H > 0 && H <= VSA_MAX_HEADS && needs_tile(masks, H), &S_grid);
  if (st != VSA_OK) return st;
  if (!q || !k || !v || !o) return fail(VSA_ERR_INVALID_ARG, "q, k, v, o must be non-NULL");
  if (o == q || o == k || o == v) return fail(VSA_ERR_INVALID_ARG, "o must not alias q, k or v");
  if (B <= 0 || H <= 0) return fail(VSA_ERR_INVALID_ARG, "B and H must be positive");
  // q/k/v/o hold the executed order (the padded grid's length for the padded layout), or
  // the frame-major sequence when the call reorders them
  const long long S_exec = exec_len(grid, layout);
  const long long S_io = (flags & VSA_FWD_REORDER_IO) ? S_grid : S_exec;
  if (S != S_io)
    return fail(VSA_ERR_INVALID_ARG, "S=%d but the grid and layout give %lld positions%s", S, S_io,
                (flags & VSA_FWD_REORDER_IO) ? " (frame-major I/O)" : "");
  if (dtype != VSA_BF16 && dtype != VSA_F32) return fail(VSA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (D != 64 && D != 128) return fail(VSA_ERR_UNSUPPORTED, "head dim D=%d (supported: 64, 128)", D);
  if (flags & ~(VSA_FWD_FORCE_MASK | VSA_FWD_REORDER_IO | VSA_FWD_WRITE_LSE | VSA_FWD_TILE_ALIGNED))
    return fail(VSA_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
  if ((flags & VSA_FWD_WRITE_LSE) && !lse) return fail(VSA_ERR_INVALID_ARG, "VSA_FWD_WRITE_LSE needs lse");
  if (dtype == VSA_BF16) {
    if ((Bq != 64 && Bq != 128 && Bq != 256) || Bk != 64)
      return fail(VSA_ERR_UNSUPPORTED, "bf16 tiles Bq=%d Bk=%d (supported: Bq 64/128/256, Bk 64)", Bq, Bk);
  } else {
    if ((Bq != 32 && Bq != 64 && Bq != 128) || (Bk != 32 && Bk != 64))
      return fail(VSA_ERR_UNSUPPORTED, "f32 tiles Bq=%d Bk=%d (supported: Bq 32/64/128, Bk 32/64)", Bq, Bk);
  }
  if (!tiles || !tiles->n_full || !tiles->n_bnd || !tiles->full_idx || !tiles->bnd_idx)
    return fail(VSA_ERR_INVALID_ARG, "tile lists must be non-NULL");
  if (!isfinite(scale)) return fail(VSA_ERR_INVALID_ARG, "scale is not finite");
  if ((words_cap < 0 && words_cap != VSA_WORDS_COMPACT) || (words_cap != 0 && !words) || (words && words_cap == 0))
    return fail(VSA_ERR_INVALID_ARG, "words and words_cap must be both set or both unset (words_cap=%d)", words_cap);
  if (words_cap == VSA_WORDS_COMPACT && !tiles->bnd_offs)
    return fail(VSA_ERR_INVALID_ARG, "the compact word table (VSA_WORDS_COMPACT) needs tiles->bnd_offs");
  if (words && dtype != VSA_BF16) return fail(VSA_ERR_UNSUPPORTED, "precomputed mask words are for bf16 only");
  if (words && (flags & VSA_FWD_TILE_ALIGNED))
    return fail(VSA_ERR_INVALID_ARG, "precomputed mask words do not apply to VSA_FWD_TILE_ALIGNED lists");
  if (((uintptr_t)words & 15)) return fail(VSA_ERR_INVALID_ARG, "words must be 16-byte aligned");
  const bool reorder = (flags & VSA_FWD_REORDER_IO) != 0;
  const size_t eb = elem_size(dtype);
  const size_t nelem = (size_t)B * S_exec * H * D;  // one reordered tensor
  // every limit of the kernels is checked here, before anything is enqueued: offsets
  // inside one batch item are 32-bit, batch items are a grid dimension (<= 65535), and
  // the bf16 kernel's one-dimensional grid holds 8*ceil(nQ/8)*B*H workgroups
  if (S_exec * H * D >= (1LL << 31))
    return fail(VSA_ERR_UNSUPPORTED, "S*H*D = %lld elements per batch item (must be below 2^31)", S_exec * H * D);
  if (B > 65535) return fail(VSA_ERR_UNSUPPORTED, "B=%d above 65535", B);
  if (dtype == VSA_BF16 && 8LL * vsa::sched_cq((int32_t)((S_exec + Bq - 1) / Bq)) * B * H > 0x7fffffffLL)
    return fail(VSA_ERR_UNSUPPORTED, "B*H*ceil(S/Bq) = %lld query tiles: the grid would exceed 2^31 workgroups",
                (S_exec + Bq - 1) / Bq * B * H);
  vsa::MaskTable table;
  vsa::HeadMap hm;
  int32_t U = 0;
  st = build_table(masks, H, grid, layout, &table, &hm, &U);
  if (st != VSA_OK) return st;
  vsa::HeadLayouts hl;
  memset(&hl, 0, sizeof hl);
  bool any_permuted = false;
  for (int h = 0; h < H; ++h) {
    hl.lay[h] = (uint8_t)table.m[hm.slot[h]].layout;
    any_permuted = any_permuted || hl.lay[h] != VSA_LAYOUT_FRAME_MAJOR;
  }
  if (reorder && !any_permuted)
    return fail(VSA_ERR_INVALID_ARG, "VSA_FWD_REORDER_IO needs a head whose layout is not frame-major");
  const size_t need = fwd_ws_bytes(B, (int32_t)S_exec, H, D, dtype, flags);
  if (use_scratch) {
    if (need > kScratchBytes)
      return fail(VSA_ERR_WORKSPACE, "the call needs %zu bytes of scratch; the static scratch holds %zu", need,
                  kScratchBytes);
  } else {
    if (need && (!workspace || ws_bytes < need))
      return fail(VSA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, need);
    if (need && ((uintptr_t)workspace & 15))
      return fail(VSA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  }

  vsa::FwdArgs a;
  memset(&a, 0, sizeof a);
  a.g = make_geom(grid, layout);
  a.B = B; a.S = (int32_t)S_exec; a.H = H; a.D = D;
  a.Bq = Bq; a.Bk = Bk;
  a.nQ = (a.S + Bq - 1) / Bq;
  a.nK = (a.S + Bk - 1) / Bk;
  a.lse_S = S;
  a.scale = scale == 0.f ? 1.f / sqrtf((float)D) : scale;
  a.force_mask = (flags & VSA_FWD_FORCE_MASK) ? 1 : 0;
  a.pad_only = (flags & VSA_FWD_TILE_ALIGNED) ? 1 : 0;
  a.write_lse = (flags & VSA_FWD_WRITE_LSE) ? 1 : 0;
  a.lse_frame_major = reorder ? 1 : 0;
  a.gather_io = (reorder && dtype == VSA_BF16) ? 1 : 0;
  a.lse = lse;
  a.n_full = tiles->n_full; a.n_bnd = tiles->n_bnd;
  a.full_idx = tiles->full_idx; a.bnd_idx = tiles->bnd_idx;
  a.words = words;
  a.words_cap = words ? words_cap : 0;
  a.bnd_offs = tiles->bnd_offs;
  if (words_cap > a.nK) return fail(VSA_ERR_INVALID_ARG, "words_cap=%d above the %d key tiles", words_cap, a.nK);
  if (use_scratch && need) {  // every argument is valid: the first HIP call may be made
    st = scratch_of_current_device(&workspace);
    if (st != VSA_OK) return st;
  }
  hipStream_t hs = (hipStream_t)stream;
  const vsa::Geom& G = a.g;
  char* ws = (char*)workspace;
  hipError_t e;
  if (dtype == VSA_BF16) {
    // with the reorder only k is copied into each head's order: the kernel gathers its
    // query rows and scatters its output rows, and the V^T transpose gathers v
    a.q = q; a.k = k; a.v = v; a.o = o;
    if (reorder) {
      if ((e = vsa::launch_reorder(k, ws, (int)eb, B, H, D, G, hl, 0, hs)) != hipSuccess) return hip_fail(e, "reorder k");
      a.k = ws;
    }
    a.s_pad = (int32_t)vt_pad(a.S);
    void* vt = ws + (reorder ? nelem * eb : 0);
    int32_t* sched = (int32_t*)((char*)vt + (size_t)B * H * D * a.s_pad * eb);
    a.cq = vsa::sched_cq(a.nQ);
    a.sched = sched;
    if ((e = vsa::launch_fwd_schedule(a, U, hm, table, sched, hs)) != hipSuccess) return hip_fail(e, "schedule");
    if ((e = vsa::launch_transpose_v(v, vt, B, a.S, H, D, a.s_pad, G, hl, reorder ? 1 : 0, S, hs)) != hipSuccess)
      return hip_fail(e, "transpose v");
    a.vt = vt;
    e = vsa::launch_attn_bf16(a, table, hm, hs);
    if (e != hipSuccess) return hip_fail(e, "attention launch");
    return ok();
  }
  if (reorder) {
    void* wq = ws;
    void* wk = ws + nelem * eb;
    void* wv = ws + 2 * nelem * eb;
    if ((e = vsa::launch_reorder(q, wq, (int)eb, B, H, D, G, hl, 0, hs)) != hipSuccess) return hip_fail(e, "reorder q");
    if ((e = vsa::launch_reorder(k, wk, (int)eb, B, H, D, G, hl, 0, hs)) != hipSuccess) return hip_fail(e, "reorder k");
    if ((e = vsa::launch_reorder(v, wv, (int)eb, B, H, D, G, hl, 0, hs)) != hipSuccess) return hip_fail(e, "reorder v");
    // each workgroup reads its own query rows before writing the same output rows, so
    // the output may overwrite the reordered queries in place
    a.q = wq; a.k = wk; a.v = wv; a.o = wq;
  } else {
    a.q = q; a.k = k; a.v = v; a.o = o;
  }
  e = vsa::launch_attn_f32(a, table, hm, hs);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  if (reorder) {
    e = vsa::launch_reorder(ws, o, (int)eb, B, H, D, G, hl, 1, hs);
    if (e != hipSuccess) return hip_fail(e, "inverse reorder o");
  }
  return ok();
}

}  // namespace

extern "C" {

vsa_status vsa_sparse_attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, vsa_dtype dtype,
                                  int32_t B, int32_t S, int32_t H, int32_t D, const vsa_grid* grid, vsa_layout layout,
                                  const vsa_mask_desc* masks, const vsa_tile_lists* tiles, int32_t Bq, int32_t Bk,
                                  float scale, int32_t flags, const uint32_t* words, int32_t words_cap,
                                  void* workspace, size_t ws_bytes, void* stream) {
  return fwd_impl(q, k, v, o, lse, dtype, B, S, H, D, grid, layout, masks, tiles, Bq, Bk, scale, flags, words,
                  words_cap, workspace, ws_bytes, false, stream);
}

vsa_status vsa_sparse_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                       vsa_dtype dtype, int32_t B, int32_t S, int32_t H, int32_t D,
                                       const vsa_grid* grid, vsa_layout layout, const vsa_mask_desc* masks,
                                       const vsa_tile_lists* tiles, int32_t Bq, int32_t Bk, float scale,
                                       int32_t flags, const uint32_t* words, int32_t words_cap, void* stream) {
  return fwd_impl(q, k, v, o, lse, dtype, B, S, H, D, grid, layout, masks, tiles, Bq, Bk, scale, flags, words,
                  words_cap, nullptr, 0, true, stream);
}

vsa_status vsa_merge_partials(const void* const* o_parts, const float* const* lse_parts, int32_t n_parts, void* o,
                              float* lse, vsa_dtype dtype, int32_t B, int32_t S, int32_t H, int32_t D,
                              void* stream) {
  if (!o_parts || !lse_parts || !o) return fail(VSA_ERR_INVALID_ARG, "o_parts, lse_parts and o must be non-NULL");
  if (n_parts < 1 || n_parts > VSA_MAX_MERGE_PARTS)
    return fail(VSA_ERR_INVALID_ARG, "n_parts=%d (1..%d)", n_parts, VSA_MAX_MERGE_PARTS);
  if (B <= 0 || S <= 0 || H <= 0) return fail(VSA_ERR_INVALID_ARG, "B, S, H must be positive");
  if (dtype != VSA_BF16 && dtype != VSA_F32) return fail(VSA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (D != 64 && D != 128) return fail(VSA_ERR_UNSUPPORTED, "head dim D=%d (supported: 64, 128)", D);
  vsa::MergeArgs a;
  memset(&a, 0, sizeof a);
  for (int i = 0; i < n_parts; ++i) {
    if (!o_parts[i] || !lse_parts[i]) return fail(VSA_ERR_INVALID_ARG, "part %d has a NULL pointer", i);
    if (((uintptr_t)o_parts[i] & 15) || ((uintptr_t)lse_parts[i] & 3))
      return fail(VSA_ERR_INVALID_ARG, "part %d is not aligned (o 16 bytes, lse 4 bytes)", i);
    a.o[i] = o_parts[i];
    a.lse[i] = lse_parts[i];
  }
  if ((uintptr_t)o & 15) return fail(VSA_ERR_INVALID_ARG, "o is not 16-byte aligned");
  for (int i = n_parts; i < 16; ++i) {  // unused slots point at part 0 (never read)
    a.o[i] = o_parts[0];
    a.lse[i] = lse_parts[0];
  }
  a.out = o;
  a.lse_out = lse;
  a.n = n_parts;
  a.B = B; a.S = S; a.H = H; a.D = D;
  a.is_bf16 = dtype == VSA_BF16;
  hipError_t e = vsa::launch_merge(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return ok();
}

vsa_status vsa_reorder_heads(const void* src, void* dst, vsa_dtype dtype, int32_t B, int32_t H, int32_t D,
                             const vsa_grid* grid, const int32_t* layouts, int32_t inverse, void* stream) {
  if (!layouts) return fail(VSA_ERR_INVALID_ARG, "layouts is NULL");
  if (H <= 0 || H > VSA_MAX_HEADS) return fail(VSA_ERR_INVALID_ARG, "H must be in 1..%d", VSA_MAX_HEADS);
  vsa::HeadLayouts hl;
  memset(&hl, 0, sizeof hl);
  bool any_tile = false, any_padded = false, uniform = true;
  for (int h = 0; h < H; ++h) {
    if (layouts[h] != VSA_LAYOUT_FRAME_MAJOR && layouts[h] != VSA_LAYOUT_TILE_MAJOR &&
        layouts[h] != VSA_LAYOUT_POSITION_MAJOR && layouts[h] != VSA_LAYOUT_TILE_PADDED)
      return fail(VSA_ERR_INVALID_ARG, "head %d: unknown layout %d", h, layouts[h]);
    hl.lay[h] = (uint8_t)(layouts[h] == VSA_LAYOUT_TILE_PADDED ? VSA_LAYOUT_TILE_MAJOR : layouts[h]);
    any_tile = any_tile || layouts[h] == VSA_LAYOUT_TILE_MAJOR;
    any_padded = any_padded || layouts[h] == VSA_LAYOUT_TILE_PADDED;
    uniform = uniform && layouts[h] == layouts[0];
  }
  if (any_padded && !uniform)
    return fail(VSA_ERR_INVALID_ARG, "the padded layout applies to every head or none");
  const vsa_layout call = any_padded ? VSA_LAYOUT_TILE_PADDED : any_tile ? VSA_LAYOUT_TILE_MAJOR : VSA_LAYOUT_FRAME_MAJOR;
  long long S;
  vsa_status st = check_grid(grid, call, any_tile || any_padded, &S);
  if (st != VSA_OK) return st;
  if (!src || !dst) return fail(VSA_ERR_INVALID_ARG, "src and dst must be non-NULL");
  if (src == dst) return fail(VSA_ERR_INVALID_ARG, "src and dst must not alias");
  if (dtype != VSA_BF16 && dtype != VSA_F32) return fail(VSA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (B <= 0 || D <= 0) return fail(VSA_ERR_INVALID_ARG, "B, H, D must be positive");
  if (B > 65535) return fail(VSA_ERR_UNSUPPORTED, "B=%d above 65535", B);
  if (((long long)H * D * elem_size(dtype)) % 16)
    return fail(VSA_ERR_UNSUPPORTED, "token row of H*D elements must be a multiple of 16 bytes");
  if (!uniform && ((long long)D * elem_size(dtype)) % 16)
    return fail(VSA_ERR_UNSUPPORTED, "heads with different layouts need D*element size a multiple of 16 bytes");
  hipError_t e = vsa::launch_reorder(src, dst, elem_size(dtype), B, H, D, make_geom(grid, call), hl,
                                     inverse ? 1 : 0, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "reorder launch");
  return ok();
}

vsa_status vsa_reorder_tokens(const void* src, void* dst, vsa_dtype dtype, int32_t B, int32_t H, int32_t D,
                              const vsa_grid* grid, int32_t inverse, void* stream) {
  if (H <= 0 || H > VSA_MAX_HEADS) return fail(VSA_ERR_INVALID_ARG, "H must be in 1..%d", VSA_MAX_HEADS);
  int32_t layouts[VSA_MAX_HEADS];
  for (int h = 0; h < H; ++h) layouts[h] = VSA_LAYOUT_TILE_MAJOR;
  return vsa_reorder_heads(src, dst, dtype, B, H, D, grid, layouts, inverse, stream);
}

vsa_status vsa_profile_workspace_bytes(int32_t B, int32_t S, int32_t H, int32_t D, int32_t n_samples,
                                       int32_t n_cand, size_t* bytes) {
  if (!bytes) return fail(VSA_ERR_INVALID_ARG, "bytes is NULL");
  if (B <= 0 || S <= 0 || H <= 0 || D <= 0 || n_samples <= 0 || n_cand <= 0)
    return fail(VSA_ERR_INVALID_ARG, "sizes must be positive");
  *bytes = vsa::profile_plan(B, S, H, D, n_samples, n_cand).ws_floats * sizeof(float);
  return ok();
}

vsa_status vsa_profile_heads(const void* q, const void* k, const void* v, vsa_dtype dtype, int32_t B, int32_t S,
                             int32_t H, int32_t D, const vsa_grid* grid, vsa_layout layout,
                             const int32_t* sample_idx, int32_t n_samples, const vsa_mask_desc* cands,
                             int32_t n_cand, float* err, int32_t* route, float scale, void* workspace,
                             size_t ws_bytes, void* stream) {
  long long S_grid;
  vsa_status st = check_grid(grid, layout, cands && n_cand > 0 && n_cand <= 4 && needs_tile(cands, n_cand), &S_grid);
  if (st != VSA_OK) return st;
  if (!q || !k || !v || !sample_idx || !err || !route)
    return fail(VSA_ERR_INVALID_ARG, "q, k, v, sample_idx, err, route must be non-NULL");
  if (B <= 0 || H <= 0) return fail(VSA_ERR_INVALID_ARG, "B and H must be positive");
  if (layout == VSA_LAYOUT_TILE_PADDED)
    return fail(VSA_ERR_UNSUPPORTED, "the profiler samples real tokens; the padded layout is not supported");
  if (S != S_grid) return fail(VSA_ERR_INVALID_ARG, "S=%d but grid gives T*Hg*Wg=%lld", S, S_grid);
  if (dtype != VSA_BF16 && dtype != VSA_F32) return fail(VSA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (dtype != VSA_BF16) return fail(VSA_ERR_UNSUPPORTED, "the profiler takes bf16 inputs");
  if (D != 64 && D != 128) return fail(VSA_ERR_UNSUPPORTED, "head dim D=%d (supported: 64, 128)", D);
  if (n_samples < 1 || n_samples > 256) return fail(VSA_ERR_INVALID_ARG, "n_samples must be in 1..256");
  if (!cands || n_cand < 2 || n_cand > 4) return fail(VSA_ERR_INVALID_ARG, "n_cand must be in 2..4");
  if (!isfinite(scale)) return fail(VSA_ERR_INVALID_ARG, "scale is not finite");
  vsa::MaskTable table;
  memset(&table, 0, sizeof table);
  for (int c = 0; c < n_cand; ++c) {
    st = normalise(cands[c], grid, layout, c, &table.m[c]);
    if (st != VSA_OK) return st;
    if (table.m[c].layout != (int16_t)layout)
      return fail(VSA_ERR_UNSUPPORTED, "candidate %d: the profiler scores every candidate in the call's layout", c);
  }
  vsa::ProfArgs a;
  memset(&a, 0, sizeof a);
  const vsa::ProfPlan plan = vsa::profile_plan(B, S, H, D, n_samples, n_cand);
  const size_t need = plan.ws_floats * sizeof(float);
  if (!workspace || ws_bytes < need)
    return fail(VSA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, need);
  a.n_sg = plan.n_sg;
  a.n_wg = plan.n_wg;
  a.n_slots = plan.n_slots;
  a.total = plan.total;
  a.q = q; a.k = k; a.v = v;
  a.sample_idx = sample_idx;
  a.err = err; a.route = route;
  a.ws = (float*)workspace;
  a.B = B; a.S = S; a.H = H; a.D = D; a.n = n_samples; a.n_cand = n_cand;
  a.scale = scale == 0.f ? 1.f / sqrtf((float)D) : scale;
  a.is_bf16 = 1;
  a.g = make_geom(grid, layout);
  a.n_pad = plan.n_pad;
  a.words = (uint32_t*)(a.ws + plan.words_off);
  for (int c = 0; c < 4; ++c) a.cm[c] = a.cand_of[c] = -1;
  for (int c = 0; c < n_cand; ++c)
    if (table.m[c].kind != VSA_MASK_ALL) {
      a.cand_of[a.n_masked] = c;
      a.cm[c] = a.n_masked++;
    }
  hipError_t e = vsa::launch_profile(a, table, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "profiler launch");
  return ok();
}

}  // extern "C"
