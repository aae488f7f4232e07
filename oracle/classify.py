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
is never FULL.

The classification is computed from its definition: materialise the explicit
boolean mask of one query tile against all keys, count kept pairs per key tile, and
compare with the tile's area.  The per-query-tile lists of FULL and of BOUNDARY key
tiles are the ascending key-tile indices of each class: the "which K blocks each Q
block computes" index table of block-sparse attention (video-DiT attention blog,
section 7.3).
"""
from __future__ import annotations

import numpy as np

from .coords import num_tiles, token_coords
from .masks import keep_matrix

EMPTY, FULL, BOUNDARY = 0, 1, 2


def classify_qtile(grid, layout, desc, S, Bq, Bk, qt):
    """Class of every key tile for query tile ``qt``: uint8 array [nK]."""
    nK = num_tiles(S, Bk)
    rows = np.arange(qt * Bq, min(S, (qt + 1) * Bq))
    cols = np.arange(S)
    m = keep_matrix(desc, grid, token_coords(grid, layout, rows), token_coords(grid, layout, cols))
    padded = np.zeros((Bq, nK * Bk), dtype=bool)
    padded[: m.shape[0], : m.shape[1]] = m
    kept = padded.reshape(Bq, nK, Bk).sum(axis=(0, 2))
    cls = np.full(nK, BOUNDARY, dtype=np.uint8)
    cls[kept == 0] = EMPTY
    cls[kept == Bq * Bk] = FULL
    return cls


def classify(grid, layout, desc, Bq, Bk, q_tiles=None):
    """Classify tiles of one mask.

    Returns dict with
      cls      uint8 [len(q_tiles), nK]
      full     list of int32 arrays (ascending FULL key-tile indices per query tile)
      bnd      list of int32 arrays (ascending BOUNDARY key-tile indices per query tile)
      q_tiles  the query tiles classified (default: all)."""
    S = grid["T"] * grid["Hg"] * grid["Wg"]
    nQ = num_tiles(S, Bq)
    if q_tiles is None:
        q_tiles = np.arange(nQ)
    q_tiles = np.asarray(q_tiles, dtype=np.int64)
    cls = np.stack([classify_qtile(grid, layout, desc, S, Bq, Bk, int(qt)) for qt in q_tiles])
    full = [np.flatnonzero(row == FULL).astype(np.int32) for row in cls]
    bnd = [np.flatnonzero(row == BOUNDARY).astype(np.int32) for row in cls]
    return {"cls": cls, "full": full, "bnd": bnd, "q_tiles": q_tiles}
