"""Block-sparse attention over 3D video token sequences for AMD Instinct MI355X.

The compute lives in libvsa.so (HIP kernels for gfx950 behind the C ABI of
include/vsa.h); this package is its ctypes binding.
"""
from ._lib import (  # noqa: F401
    VSA_BF16, VSA_F32, VSA_FWD_FORCE_MASK, VSA_FWD_REORDER_IO, VSA_FWD_WRITE_LSE, VSA_FWD_TILE_ALIGNED,
    VSA_CLASSIFY_ROUND_TILES, VSA_WORDS_COMPACT, vsa_tile_lists_bytes,
    VSA_LAYOUT_FRAME_MAJOR, VSA_LAYOUT_TILE_MAJOR, VSA_LAYOUT_POSITION_MAJOR, VSA_LAYOUT_TILE_PADDED, VSA_HEAD_LAYOUT_CALL,
    VSA_HEAD_LAYOUT_FRAME, VSA_HEAD_LAYOUT_TILE, VSA_HEAD_LAYOUT_POSITION, VSA_TILE_BOUNDARY, VSA_TILE_EMPTY, VSA_TILE_FULL,
    LIB_PATH, VsaError, alloc_tile_lists, default_scale, load, make_grid, make_masks,
    vsa_classify_tiles, vsa_fwd_workspace_bytes, vsa_last_error, vsa_profile_heads,
    vsa_profile_workspace_bytes, vsa_reorder_tokens, vsa_sparse_attn_fwd, vsa_tile_counts, vsa_boundary_words,
    vsa_merge_partials, vsa_reorder_heads, vsa_seq_len, vsa_unique_masks, vsa_sparse_attn_fwd_noalloc,
)
