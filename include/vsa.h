/*
 * vsa.h -- C ABI of libvsa: mask-driven block-sparse attention over 3D video
 * token sequences on AMD Instinct MI355X (gfx950).
 *
 * The problem, as the pages state it:
 *   - Q, K, V are [B, S, H, D] tensors of S video tokens (DSA study guide,
 *     sections 5-6: per-device shards [B, S/N, H, D]; this library works on one
 *     GPU's full sequence);
 *   - the tokens come from a latent grid of T frames x Hg rows x Wg columns;
 *   - every head has a mask (spatial, temporal, first-frame sink, sliding tile
 *     window, PSA stripe six-tuple);
 *   - attention is O = softmax(Q K^T * scale + M) V (Sliding Tile Attention
 *     explainer, method section 2, eq. (1));
 *   - the mask is reduced to a per-(query-tile, key-tile) class: full, boundary or
 *     empty (Sparse VideoGen on TPU, "logical sparsity is not physical sparsity");
 *     empty tiles are skipped, full tiles run without an in-tile mask, boundary
 *     tiles apply an exact element mask (same page, "avoid in-tile masking when
 *     nothing needs masking"), and every kept key contributes through online
 *     softmax (DSA study guide, section 18).
 *
 * Conventions for every entry point
 *   - Device pointers are caller-owned HIP device memory; the library never
 *     allocates or frees device memory and keeps no state between calls.
 *   - Host pointers (descriptors) are read only during the call.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the null
 *     stream).  The return status covers argument validation and launch errors;
 *     faults during execution surface at the caller's next synchronisation.
 *   - On error nothing is enqueued, the function returns a negative vsa_status and
 *     vsa_last_error() returns a message for the calling thread.  No C++
 *     exception crosses this boundary.
 *   - Argument validation happens before any HIP call, so invalid arguments are
 *     rejected on machines without a GPU as well.
 */
#ifndef VSA_H_
#define VSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VSA_OK = 0,
  VSA_ERR_INVALID_ARG = -1, /* malformed argument (null pointer, bad shape, ...) */
  VSA_ERR_UNSUPPORTED = -2, /* well-formed but not implemented (D, dtype, tile size) */
  VSA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  VSA_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed */
} vsa_status;

typedef enum { VSA_BF16 = 0, VSA_F32 = 1 } vsa_dtype;

/* Executed token order of a head: the order of the positions along the sequence axis
 * of Q/K/V/O (unless the call reorders them, VSA_FWD_REORDER_IO).
 *   FRAME_MAJOR:    position p = (t*Hg + y)*Wg + x, the natural order.
 *   TILE_MAJOR:     3D tiles of tile_t x tile_h x tile_w tokens contiguous, tiles and
 *                   in-tile tokens row-major (Sliding Tile Attention explainer, method
 *                   section 3; PSA notes, key design 2).  The tile must divide the grid.
 *   POSITION_MAJOR: frame 0 first in frame-major order, then for every spatial
 *                   position s = y*Wg + x (ascending) its frames 1 .. T-1: position
 *                   Hg*Wg + s*(T-1) + (t-1).  The temporal order of Sparse VideoGen on
 *                   TPU ("arranging tokens for temporal access": (F,H,W) -> (H,W,F)),
 *                   with the first frame kept as a leading block so that the
 *                   first-frame sink stays contiguous.
 *   TILE_PADDED:    TILE_MAJOR over the grid padded up to whole tiles on every axis
 *                   (PSA notes, key design 2, 3D padding: T' = ceil(T/tile_t)*tile_t,
 *                   likewise H', W').  The executed length is T'*H'*W' (vsa_seq_len);
 *                   positions outside the real grid are padding: never kept as keys,
 *                   and their query outputs are unspecified.  A call-level layout only:
 *                   it applies to every head (head_layout must be 0). */
typedef enum {
  VSA_LAYOUT_FRAME_MAJOR = 0,
  VSA_LAYOUT_TILE_MAJOR = 1,
  VSA_LAYOUT_POSITION_MAJOR = 2,
  VSA_LAYOUT_TILE_PADDED = 3
} vsa_layout;

/* Latent grid.  S = T*Hg*Wg.  tile_* is the 3D token tile used by the tile-major orders
 * and by STA masks (0 when unused; ignored by calls that use neither).  TILE_MAJOR and
 * STA masks in the other orders need it to divide T, Hg, Wg; TILE_PADDED does not. */
typedef struct {
  int32_t T, Hg, Wg;
  int32_t tile_t, tile_h, tile_w;
} vsa_grid;

typedef enum {
  VSA_MASK_ALL = 0,    /* every pair kept */
  VSA_MASK_BOX = 1,    /* |dt|<=rt && |dy|<=rh && |dx|<=rw, radius < 0 = unbounded */
  VSA_MASK_STRIPE = 2, /* PSA: (|t_k-t_q-To| mod Ts) <= Tw-1 && (|s_k-s_q-So| mod Ss) <= Sw-1 */
  VSA_MASK_STA = 3     /* sliding tile window of win_t x win_h x win_w tiles */
} vsa_mask_kind;

/* Per-head mask descriptor.  Every kind also keeps keys whose frame index is below
 * sink_frames (first-frame attention sink: Sparse VideoGen on TPU, "how to
 * accelerate attention", both masks keep frame F00; DSA study guide, section 3).
 *   BOX:    spatial head = {BOX, 1, rt=1, rh=-1, rw=-1}; temporal head =
 *           {BOX, 1, rt=-1, rh=r, rw=r} (Sparse VideoGen on TPU; DSA section 3).
 *   STRIPE: s = y*Wg + x; Ts >= 1 and Ss >= 1 (PSA notes, key design 1); the
 *           absolute value is taken before the modulus, so To/So != 0 is asymmetric.
 *   STA:    with a, b the query and key tile coordinates along an axis of n tiles,
 *           start = clamp(a - w/2, 0, n - w) and the pair is kept iff
 *           start <= b < start + w on all three axes; the window is shifted inward
 *           at the edges and keeps its size (Sliding Tile Attention explainer,
 *           method section 3).  Requires grid tile_* > 0 dividing T, Hg, Wg.
 * head_layout: executed token order of this head; VSA_HEAD_LAYOUT_CALL (0) takes the
 *           call's layout argument, VSA_HEAD_LAYOUT_(FRAME|TILE|POSITION) set it for
 *           this head alone (Sparse VideoGen on TPU, "dynamic routing with fixed tensor
 *           shapes": per-head flags choose the original or the permuted order).
 * Unused fields must be zero.  Descriptors that compare equal field by field share
 * one classification. */
#define VSA_HEAD_LAYOUT_CALL 0
#define VSA_HEAD_LAYOUT_FRAME 1
#define VSA_HEAD_LAYOUT_TILE 2
#define VSA_HEAD_LAYOUT_POSITION 3
typedef struct {
  int32_t kind;
  int32_t sink_frames;
  int32_t rt, rh, rw;
  int32_t Tw, To, Ts, Sw, So, Ss;
  int32_t win_t, win_h, win_w;
  int32_t head_layout;
} vsa_mask_desc;

/* Tile classes stored in vsa_tile_lists.cls. */
enum { VSA_TILE_EMPTY = 0, VSA_TILE_FULL = 1, VSA_TILE_BOUNDARY = 2 };

/* Output of the classifier, all caller-allocated device arrays.  With
 * nQ = ceil(S/Bq), nK = ceil(S/Bk) for the executed length S of the layout
 * (vsa_seq_len) and U = number of distinct descriptors:
 *   cls       uint8 [U][nQ][nK]  tile class (may be NULL: not written)
 *   n_full    int32 [U][nQ]      number of FULL key tiles of each query tile
 *   n_bnd     int32 [U][nQ]      number of BOUNDARY key tiles
 *   full_idx  int32 [U][nQ][nK]  ascending FULL key-tile indices in the first
 *                                n_full entries of each row; the rest is unspecified
 *   bnd_idx   int32 [U][nQ][nK]  same for BOUNDARY tiles
 *   bnd_offs  int64 [U*nQ + 1]   exclusive prefix sum of n_bnd over the list rows in
 *                                (u, qt) order, bnd_offs[U*nQ] = total boundary entries
 *                                (may be NULL: not written); it indexes the compact
 *                                boundary-word table (vsa_boundary_words, cap
 *                                VSA_WORDS_COMPACT)
 * A tile reaching past S is padded and never FULL (Sparse VideoGen on TPU,
 * "aligning the sparse mask with execution": padding contributes zero weight).
 * Unique descriptors are numbered in order of first appearance in masks[]; the
 * head -> descriptor map is vsa_unique_masks' head_map (a host array: the kernels take
 * it as a launch argument, so no device copy exists). */
typedef struct {
  uint8_t* cls;
  int32_t* n_full;
  int32_t* n_bnd;
  int32_t* full_idx;
  int32_t* bnd_idx;
  int64_t* bnd_offs;
} vsa_tile_lists;

/* Limits. */
#define VSA_MAX_HEADS 256
#define VSA_MAX_UNIQUE_MASKS 64

/* Host-only helpers ---------------------------------------------------------- */

/* Deduplicate per-head descriptors.  head_map (host, [H], may be NULL) receives
 * each head's unique-descriptor slot; *n_unique the number of distinct ones. */
vsa_status vsa_unique_masks(const vsa_mask_desc* masks, int32_t H, int32_t* head_map,
                            int32_t* n_unique);

/* nQ = ceil(S/Bq), nK = ceil(S/Bk) for S = T*Hg*Wg (every layout but TILE_PADDED). */
vsa_status vsa_tile_counts(const vsa_grid* grid, int32_t Bq, int32_t Bk, int32_t* nQ,
                           int32_t* nK);

/* Executed sequence length of a layout: T*Hg*Wg, or T'*H'*W' for VSA_LAYOUT_TILE_PADDED.
 * Tile lists of that layout have nQ = ceil(S/Bq), nK = ceil(S/Bk). */
vsa_status vsa_seq_len(const vsa_grid* grid, vsa_layout layout, int32_t* S);

/* Device bytes of one allocation that holds every array of vsa_tile_lists for U
 * distinct masks on this grid, layout and tile size (cls, n_full, n_bnd, full_idx,
 * bnd_idx, bnd_offs, each starting on a 256-byte boundary), and the carving of such an
 * allocation into the struct.  `base` is only offset, never dereferenced, so it may be
 * any caller-owned device pointer (256-byte aligned).  INVALID_ARG for a bad grid,
 * U outside 1..VSA_MAX_UNIQUE_MASKS or tiles outside 1..4096. */
vsa_status vsa_tile_lists_bytes(const vsa_grid* grid, vsa_layout layout, int32_t U, int32_t Bq,
                                int32_t Bk, size_t* bytes);
vsa_status vsa_tile_lists_carve(const vsa_grid* grid, vsa_layout layout, int32_t U, int32_t Bq,
                                int32_t Bk, void* base, vsa_tile_lists* out);

/* Tile classification -------------------------------------------------------- */

/* Classify every (query tile, key tile) of each distinct mask and write compact
 * ascending lists (Sparse VideoGen on TPU, "logical sparsity is not physical
 * sparsity"; video-DiT attention blog, section 7.3: a per-Q-block table of the K
 * blocks it computes).  The result is exact: it equals counting kept pairs of the
 * materialised mask in each tile.
 *   grid, layout:  token grid and sequence order of the positions (a descriptor's
 *                  head_layout overrides the order for the heads that use it)
 *   masks:         host [H] descriptors (deduplicated internally)
 *   Bq, Bk:        query / key tile sizes in positions, 1..4096
 *   out:           device arrays sized for U unique masks (see vsa_tile_lists)
 * Errors: INVALID_ARG for a null pointer, bad grid or descriptor; UNSUPPORTED when
 * H > VSA_MAX_HEADS or U > VSA_MAX_UNIQUE_MASKS. */
vsa_status vsa_classify_tiles(const vsa_grid* grid, vsa_layout layout,
                              const vsa_mask_desc* masks, int32_t H, int32_t Bq,
                              int32_t Bk, const vsa_tile_lists* out, void* stream);

/* Tile-aligned rounding (Sparse VideoGen on TPU, "aligning the sparse mask with
 * execution", configuration B3).  With VSA_CLASSIFY_ROUND_TILES each BOUNDARY tile is
 * rounded to all-or-nothing on its real pairs (both positions < S): kept when at least
 * half of them are kept by the mask, else dropped.  A kept tile is FULL, or BOUNDARY if
 * it reaches past S (then only the padding is masked).  FULL and EMPTY tiles are
 * unchanged.  The rounded lists define a slightly different mask; run the forward on
 * them with VSA_FWD_TILE_ALIGNED.  Needs Bk <= 64.  Otherwise as vsa_classify_tiles
 * (which is vsa_classify_tiles_ex with flags = 0). */
#define VSA_CLASSIFY_ROUND_TILES 1
vsa_status vsa_classify_tiles_ex(const vsa_grid* grid, vsa_layout layout,
                                 const vsa_mask_desc* masks, int32_t H, int32_t Bq,
                                 int32_t Bk, int32_t flags, const vsa_tile_lists* out,
                                 void* stream);

/* Attention forward ----------------------------------------------------------- */

#define VSA_FWD_FORCE_MASK 1  /* ablation: run every listed tile through the masked path */
#define VSA_FWD_REORDER_IO 2  /* q/k/v/o are frame-major; each head attends in its executed
                                 layout (the call's, or its descriptor's head_layout): bf16
                                 reorders k into the workspace and maps the rows of q, v and
                                 o through the layout, f32 reorders q, k, v into the
                                 workspace and o back (Sparse VideoGen on TPU, "layout
                                 transforms on local heads"); needs a head not frame-major */
#define VSA_FWD_WRITE_LSE 4   /* write lse (must then be non-NULL) */
#define VSA_FWD_TILE_ALIGNED 8  /* listed BOUNDARY tiles mask only keys past S: the
                                   forward of lists from VSA_CLASSIFY_ROUND_TILES */

/* Workspace bytes vsa_sparse_attn_fwd needs for these arguments, with S the executed
 * length (vsa_seq_len; T*Hg*Wg except for VSA_LAYOUT_TILE_PADDED): for bf16,
 * B*H*D*S64 elements (S64 = S rounded up to a multiple of 64) that hold V
 * transposed per 64-key block to [B][H][S64/64][D][64], and with VSA_FWD_REORDER_IO
 * B*S*H*D elements more (k in each head's executed order; q and v are gathered and o
 * scattered by row), plus 3,328 bytes for the per-call schedule that deals each head's
 * query tiles to the 8 XCDs in ranges of equal listed cost; f32 with VSA_FWD_REORDER_IO: 3*B*S*H*D elements (q, k, v in each head's executed
 * order), without it none. */
vsa_status vsa_fwd_workspace_bytes(int32_t B, int32_t S, int32_t H, int32_t D,
                                   vsa_dtype dtype, int32_t flags, size_t* bytes);

/* Block-sparse masked attention forward.
 *   q, k, v:  device [B][S][H][D], dtype, contiguous; position p of head h is that
 *             head's executed position (its layout) and S the executed length
 *             (vsa_seq_len), unless VSA_FWD_REORDER_IO: then they are frame-major and
 *             S = T*Hg*Wg
 *   o:        device [B][S][H][D], dtype (output; must not alias q/k/v); padding rows
 *             of the padded layout (without the reorder) are unspecified
 *   lse:      device float [B][H][S] = m + ln(l), natural log (written only with
 *             VSA_FWD_WRITE_LSE; -inf for a row with no kept key; padding rows as o)
 *   grid, layout, masks[H]: as given to vsa_classify_tiles for `tiles`
 *   tiles:    lists from vsa_classify_tiles with the same grid, layout, masks, Bq, Bk
 *   Bq, Bk:   bf16: Bq in {64, 128, 256}, Bk = 64; f32: Bq in {32, 64, 128}, Bk in {32, 64}
 *   scale:    softmax scale; 0 selects 1/sqrt(D)
 *   flags:    VSA_FWD_* bits
 *   workspace, ws_bytes: device scratch, 16-byte aligned, owned by the caller and
 *             free again once the stream has run the call; see
 *             vsa_fwd_workspace_bytes (may be NULL when 0 bytes are needed)
 * Output rows whose query has no kept key are 0.  D must be 64 or 128.  The kernels
 * index one batch item's [S][H][D] elements with 32-bit offsets, so S*H*D (S the
 * executed length) must be below 2^31: larger calls return UNSUPPORTED before anything
 * is enqueued.
 * The full tiles take an unmasked path and boundary tiles an element-masked path;
 * both feed one online softmax per query row, so the result does not depend on
 * the split (Sparse VideoGen on TPU, "avoid in-tile masking ..."). */
vsa_status vsa_sparse_attn_fwd(const void* q, const void* k, const void* v, void* o,
                               float* lse, vsa_dtype dtype, int32_t B, int32_t S,
                               int32_t H, int32_t D, const vsa_grid* grid,
                               vsa_layout layout, const vsa_mask_desc* masks,
                               const vsa_tile_lists* tiles, int32_t Bq, int32_t Bk,
                               float scale, int32_t flags, void* workspace,
                               size_t ws_bytes, void* stream);

/* Precomputed element masks of boundary tiles (bf16 forward) ------------------- */

/* The forward masks each listed BOUNDARY tile element by element (Sparse VideoGen on
 * TPU, "avoid in-tile masking ...": only partially kept tiles pay for it).  It can
 * derive those masks itself, or read them from a table that this call fills
 * beforehand, which frees the forward's vector unit for the softmax.  Like the tile
 * lists, the table depends only on the grid, the masks and the tile sizes, so one
 * table serves every forward with the same lists.
 *   grid, layout, masks[H], Bq, Bk, tiles: as given to vsa_classify_tiles (exact
 *          lists, not rounded ones); Bq in {64, 128, 256}, Bk = 64
 *   words: device uint32 [U][nQ][cap][Bq/32][64] (U unique masks, nQ = ceil(S/Bq) with
 *          S the executed length); entry j < min(n_bnd, cap) of a list row holds the
 *          masks of that row's j-th boundary tile; other entries are not written.
 *          Compact form (cap = VSA_WORDS_COMPACT): uint32 [N][Bq/32][64] with
 *          N = tiles->bnd_offs[U*nQ], the total of the boundary lists; entry j of list
 *          row r is entry bnd_offs[r] + j.  Needs tiles->bnd_offs from the classifier.
 *   cap:   entries per list row, 0..nK (a forward masks entries past cap itself), or
 *          VSA_WORDS_COMPACT
 * Word (w, l) of an entry belongs to query row w*32 + (l mod 32) of the query tile
 * (rows past S use row S-1) and holds, from bit 0, whether keys 8*(l div 32) + {0..7},
 * {16..23}, {32..39}, {48..55} of the key tile are kept.  16-byte aligned.  Asynchronous
 * on stream; integer-exact. */
#define VSA_WORDS_COMPACT (-1)
vsa_status vsa_boundary_words(const vsa_grid* grid, vsa_layout layout,
                              const vsa_mask_desc* masks, int32_t H, int32_t Bq,
                              int32_t Bk, const vsa_tile_lists* tiles, uint32_t* words,
                              int32_t cap, void* stream);

/* vsa_sparse_attn_fwd reading the boundary masks of list entries j < words_cap from
 * words (vsa_boundary_words with the same arguments and cap = words_cap); the output is
 * identical.  Query tiles whose boundary list fits in the table (n_bnd <= words_cap, so
 * every list with cap = nK or cap = the longest list, and every list of a compact table,
 * words_cap = VSA_WORDS_COMPACT, which reads tiles->bnd_offs) run with no mask
 * arithmetic at all; the others derive the masks of the entries past the cap.
 * words = NULL with words_cap = 0 is vsa_sparse_attn_fwd.  bf16 only, not with
 * VSA_FWD_TILE_ALIGNED. */
vsa_status vsa_sparse_attn_fwd_ex(const void* q, const void* k, const void* v, void* o,
                                  float* lse, vsa_dtype dtype, int32_t B, int32_t S,
                                  int32_t H, int32_t D, const vsa_grid* grid,
                                  vsa_layout layout, const vsa_mask_desc* masks,
                                  const vsa_tile_lists* tiles, int32_t Bq, int32_t Bk,
                                  float scale, int32_t flags, const uint32_t* words,
                                  int32_t words_cap, void* workspace, size_t ws_bytes,
                                  void* stream);

/* Allocation-free forward ------------------------------------------------------ */

/* For callers that cannot allocate device memory at call time: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same forward as
 * vsa_sparse_attn_fwd_ex (same arguments without the workspace, same kernels, same
 * output bit for bit), with its workspace taken from a scratch array that the library
 * holds on each GPU it runs on, VSA_NOALLOC_SCRATCH_BYTES bytes, from the first call on
 * that GPU (the calling thread's current device, which must own `stream`) until the
 * process ends.  The call allocates nothing: no hipMalloc, hipFree or allocating library
 * routine.  A call whose workspace (vsa_fwd_workspace_bytes) exceeds the scratch returns
 * VSA_ERR_WORKSPACE and enqueues nothing; for bf16 that is B*H*D*S64*2 bytes (plus the
 * reordered k with VSA_FWD_REORDER_IO), e.g. 10 heads of 75,600 tokens at D = 128.  Every
 * call on one GPU shares that GPU's scratch and overwrites it completely (nothing in it
 * needs to start at zero), so calls that overlap on one GPU, on concurrent streams or
 * threads, race: serialise them.  Errors as for vsa_sparse_attn_fwd_ex. */
#define VSA_NOALLOC_SCRATCH_BYTES (256u << 20)
vsa_status vsa_sparse_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o,
                                       float* lse, vsa_dtype dtype, int32_t B, int32_t S,
                                       int32_t H, int32_t D, const vsa_grid* grid,
                                       vsa_layout layout, const vsa_mask_desc* masks,
                                       const vsa_tile_lists* tiles, int32_t Bq, int32_t Bk,
                                       float scale, int32_t flags, const uint32_t* words,
                                       int32_t words_cap, void* stream);

/* Token reorder ---------------------------------------------------------------- */

/* Permute the sequence axis of src [B][S][H][D] into dst (no aliasing), each head h
 * into its own order layouts[h] (VSA_LAYOUT_*, host array [H]):
 * inverse = 0: frame-major -> layouts[h]; inverse != 0: layouts[h] -> frame-major.
 * Tile-major heads need grid tile_* dividing T, Hg, Wg (Sliding Tile Attention
 * explainer, method section 3: tokens of a tile are contiguous); TILE_PADDED (all heads
 * or none) reads src [B][T*Hg*Wg][H][D] and writes dst [B][T'*H'*W'][H][D] with zero
 * padding rows, and inverse reads the padded sequence and drops its padding (PSA notes,
 * key design 2); position-major heads
 * gather each spatial position's frames (Sparse VideoGen on TPU, "arranging tokens for
 * temporal access").  H*D*element size must be a multiple of 16 bytes, and D*element
 * size too when the layouts differ.  Asynchronous on stream; the caller owns both
 * buffers. */
vsa_status vsa_reorder_heads(const void* src, void* dst, vsa_dtype dtype, int32_t B,
                             int32_t H, int32_t D, const vsa_grid* grid,
                             const int32_t* layouts, int32_t inverse, void* stream);

/* vsa_reorder_heads with every head tile-major. */
vsa_status vsa_reorder_tokens(const void* src, void* dst, vsa_dtype dtype, int32_t B,
                              int32_t H, int32_t D, const vsa_grid* grid,
                              int32_t inverse, void* stream);

/* Merging partial results ------------------------------------------------------ */

#define VSA_MAX_MERGE_PARTS 16

/* Merge attention results computed over disjoint key subsets of the same queries
 * (DSA study guide, section 18: online-softmax partials combine by their softmax
 * statistics, in any order, into one softmax over the union).  Per row:
 *   m' = max_i lse_i,  w_i = exp(lse_i - m')  (0 for a part with lse_i = -inf),
 *   lse = m' + ln(sum_i w_i),  o = sum_i w_i o_i / sum_i w_i;
 * a row where every part has lse = -inf gets o = 0 and lse = -inf.
 *   o_parts:   host array [n_parts] of device pointers, each [B][S][H][D] of dtype
 *              (normalised partial outputs, as vsa_sparse_attn_fwd writes them)
 *   lse_parts: host array [n_parts] of device pointers, each float [B][H][S]
 *              (natural log, as written with VSA_FWD_WRITE_LSE)
 *   n_parts:   1 .. VSA_MAX_MERGE_PARTS
 *   o:         device [B][S][H][D] of dtype (output; may be one of o_parts)
 *   lse:       device float [B][H][S] (output, may be NULL; may be one of lse_parts)
 * D must be 64 or 128.  Accumulation is fp32; bf16 output is rounded to nearest even.
 * Asynchronous on stream; the caller owns every buffer. */
vsa_status vsa_merge_partials(const void* const* o_parts, const float* const* lse_parts,
                              int32_t n_parts, void* o, float* lse, vsa_dtype dtype,
                              int32_t B, int32_t S, int32_t H, int32_t D, void* stream);

/* Head profiler --------------------------------------------------------------- */

/* Workspace bytes vsa_profile_heads needs. */
vsa_status vsa_profile_workspace_bytes(int32_t B, int32_t S, int32_t H, int32_t D,
                                       int32_t n_samples, int32_t n_cand, size_t* bytes);

/* Sampled-query head profiler (Sparse VideoGen on TPU, "how to accelerate
 * attention": sample a few queries, compute their outputs under full attention and
 * each candidate mask, route the head to the mask with the smallest deviation;
 * "supporting dynamic routing with fixed tensor shapes": one flag per head).
 *   q, k, v:     device [B][S][H][D], dtype
 *   sample_idx:  device int32 [H][n_samples], positions in [0, S), shared across b
 *   cands:       host [n_cand] descriptors, cands[0] is the reference (normally ALL);
 *                2 <= n_cand <= 4; all are scored in the call's layout, so a
 *                head_layout naming another order is UNSUPPORTED (the routed
 *                result is the same in any order, since attention commutes with a
 *                permutation of the tokens applied to q, k, v and o alike)
 *   err:         device float [H][n_cand]: sqrt(sum over b, samples, channels of
 *                (o_c - o_0)^2); err[h][0] = 0
 *   route:       device int32 [H]: argmin over c >= 1 of err[h][c], lowest c on ties
 *   n_samples:   1..256
 * Errors as for the other entry points; WORKSPACE when ws_bytes is too small. */
vsa_status vsa_profile_heads(const void* q, const void* k, const void* v, vsa_dtype dtype,
                             int32_t B, int32_t S, int32_t H, int32_t D,
                             const vsa_grid* grid, vsa_layout layout,
                             const int32_t* sample_idx, int32_t n_samples,
                             const vsa_mask_desc* cands, int32_t n_cand, float* err,
                             int32_t* route, float scale, void* workspace,
                             size_t ws_bytes, void* stream);

/* Thread-local message of the last error on this thread ("" if none). */
const char* vsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* VSA_H_ */
