"""Tile classification (oracle; test infrastructure).

The attention matrix of one head is cut into tiles of Bq query positions by Bk key
positions, in executed order.  Each tile is one of three classes (Sparse VideoGen on
TPU, "logical sparsity is not physical sparsity"; Sliding Tile Attention explainer,
method section 2 and its Table 1):

* FULL: every pair in the tile is kept, so no in-tile mask is needed;
* BOUNDARY: some pairs are kept and some are not, so scores need an element mask;
* EMPTY: no pair is kept, so the tile is skipped.

When S is not a multiple of the tile size, positions past S are padding.  Padding
must contribute exactly zero weight (Sparse VideoGen on TPU, "aligning the sparse
mask with execution"), so padding counts as "not kept": a tile that reaches past S
is never FULL.  The padding tokens of the padded layout (PSA notes, key design 2,
3D padding) are treated the same way, wherever they fall in the sequence.

The classification is computed from its definition: materialise the explicit
boolean mask of one query tile against all keys, count kept pairs per key tile, and
compare with the tile's area.  The per-query-tile lists of FULL and of BOUNDARY key
tiles are the ascending key-tile indices of each class: the "which K blocks each Q
block computes" index table of block-sparse attention (video-DiT attention blog,
section 7.3).

Tile-aligned rounding (Sparse VideoGen on TPU, "aligning the sparse mask with
execution", configuration B3): every boundary tile is rounded to all-or-nothing, so
that element masking is left only where the tile reaches past S (padding).  The page
leaves the rule open beyond balancing outward rounding (adding pairs) against inward
rounding (dropping pairs) to roughly keep the pair budget; the reading used here is
rounding each tile to the nearer of the two: a tile keeps all of its real pairs
(both positions < S) when at least half of them are kept by the mask, and none
otherwise.  Full and empty tiles are unchanged.  After rounding, a tile that keeps
its pairs is FULL unless it reaches past S, where it stays BOUNDARY (padding is the
only masked part).
"""
from __future__ import annotations

import numpy as np

from .coords import is_real, num_tiles, seq_len, token_coords
from .masks import keep_matrix

EMPTY, FULL, BOUNDARY = 0, 1, 2


def _real(grid, layout, pos):
    return is_real(grid, *token_coords(grid, layout, pos))


def _qtile_keep(grid, layout, desc, S, Bq, qt):
    """Keep rows of query tile qt against all keys; padding rows and keys are not kept."""
    rows = np.arange(qt * Bq, min(S, (qt + 1) * Bq))
    cols = np.arange(S)
    m = keep_matrix(desc, grid, token_coords(grid, layout, rows), token_coords(grid, layout, cols))
    return m & _real(grid, layout, rows)[:, None] & _real(grid, layout, cols)[None, :]


def _tile_counts(grid, layout, m, S, Bq, Bk, qt):
    """Kept pairs and real pairs (both positions real tokens) of every key tile of query
    tile qt whose keep rows are m [rows, S]."""
    nK = num_tiles(S, Bk)
    padded = np.zeros((Bq, nK * Bk), dtype=bool)
    padded[: m.shape[0], : m.shape[1]] = m
    kept = padded.reshape(Bq, nK, Bk).sum(axis=(0, 2))
    col_real = np.zeros(nK * Bk, dtype=np.int64)
    col_real[:S] = _real(grid, layout, np.arange(S))
    rows_real = int(_real(grid, layout, np.arange(qt * Bq, min(S, (qt + 1) * Bq))).sum())
    return kept, rows_real * col_real.reshape(nK, Bk).sum(axis=1)


def classify_qtile(grid, layout, desc, S, Bq, Bk, qt, round_tiles=False):
    """Class of every key tile for query tile ``qt``: uint8 array [nK]."""
    m = _qtile_keep(grid, layout, desc, S, Bq, qt)
    kept, real = _tile_counts(grid, layout, m, S, Bq, Bk, qt)
    cls = np.full(len(kept), BOUNDARY, dtype=np.uint8)
    cls[kept == 0] = EMPTY
    cls[kept == Bq * Bk] = FULL
    if round_tiles:
        padded = (real < Bq * Bk)
        keep_tile = (cls == FULL) | ((cls == BOUNDARY) & (2 * kept >= real))
        cls = np.where(keep_tile, np.where(padded, BOUNDARY, FULL), EMPTY).astype(np.uint8)
    return cls


def rounded_keep_rows(grid, layout, desc, Bq, Bk, rows):
    """Keep rows of the tile-aligned (B3) mask for executed query positions ``rows``:
    bool [len(rows), S], every (query tile, key tile) block all-kept or all-dropped on
    its real pairs."""
    S = seq_len(grid, layout)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), S), dtype=bool)
    col_real = _real(grid, layout, np.arange(S))
    for qt in np.unique(rows // Bq):
        m = _qtile_keep(grid, layout, desc, S, Bq, int(qt))
        kept, real = _tile_counts(grid, layout, m, S, Bq, Bk, int(qt))
        keep_tile = 2 * kept >= real
        keep_tile[kept == 0] = False
        cols = np.repeat(keep_tile, Bk)[:S] & col_real
        sel = np.flatnonzero(rows // Bq == qt)
        out[sel] = cols[None, :]
    return out & _real(grid, layout, rows)[:, None]


def classify(grid, layout, desc, Bq, Bk, q_tiles=None, round_tiles=False):
    """Classify tiles of one mask.

    Returns dict with
      cls      uint8 [len(q_tiles), nK]
      full     list of int32 arrays (ascending FULL key-tile indices per query tile)
      bnd      list of int32 arrays (ascending BOUNDARY key-tile indices per query tile)
      q_tiles  the query tiles classified (default: all).
    round_tiles: classes of the tile-aligned (B3) mask instead of the exact one."""
    S = seq_len(grid, layout)
    nQ = num_tiles(S, Bq)
    if q_tiles is None:
        q_tiles = np.arange(nQ)
    q_tiles = np.asarray(q_tiles, dtype=np.int64)
    cls = np.stack([classify_qtile(grid, layout, desc, S, Bq, Bk, int(qt), round_tiles) for qt in q_tiles])
    full = [np.flatnonzero(row == FULL).astype(np.int32) for row in cls]
    bnd = [np.flatnonzero(row == BOUNDARY).astype(np.int32) for row in cls]
    return {"cls": cls, "full": full, "bnd": bnd, "q_tiles": q_tiles}
