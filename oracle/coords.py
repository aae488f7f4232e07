"""Token coordinates of an executed sequence position (oracle; test infrastructure).

A video latent of T frames x Hg rows x Wg columns is flattened to S = T*Hg*Wg
tokens.  Two orders are used:

* frame-major: (t, y, x) flattened row-major, the natural order in which the
  tokens of one frame are contiguous (video-DiT attention blog, section 7.2
  "layout transforms").
* tile-major: the grid is cut into non-overlapping tiles of bt x bh x bw tokens,
  and every tile's tokens are contiguous (Sliding Tile Attention explainer,
  method section 3: tokens inside one tile get consecutive sequence numbers;
  PSA notes, key design 2: the (T', H', W', b_t, b_h, b_w) layout).  Tiles are
  ordered row-major over the tile grid, and tokens row-major inside a tile.
  The pages fix only that tiles are contiguous; the row-major orders are the
  plain reading.
"""
from __future__ import annotations

import numpy as np


def _check_tile(grid):
    bt, bh, bw = grid["tile_t"], grid["tile_h"], grid["tile_w"]
    if min(bt, bh, bw) <= 0:
        raise ValueError("tile-major layout needs a positive tile size")
    if grid["T"] % bt or grid["Hg"] % bh or grid["Wg"] % bw:
        raise ValueError("grid must be a whole number of tiles in tile-major layout")
    return bt, bh, bw


def token_coords(grid, layout, pos):
    """Return (t, y, x) int64 arrays for executed positions ``pos`` (any int array).

    layout is "frame" or "tile"."""
    pos = np.asarray(pos, dtype=np.int64)
    T, Hg, Wg = grid["T"], grid["Hg"], grid["Wg"]
    if layout == "frame":
        t = pos // (Hg * Wg)
        y = (pos // Wg) % Hg
        x = pos % Wg
        return t, y, x
    if layout == "tile":
        bt, bh, bw = _check_tile(grid)
        nH, nW = Hg // bh, Wg // bw
        vol = bt * bh * bw
        tau, iota = pos // vol, pos % vol
        tau_t, tau_h, tau_w = tau // (nH * nW), (tau // nW) % nH, tau % nW
        i_t, i_h, i_w = iota // (bh * bw), (iota // bw) % bh, iota % bw
        return tau_t * bt + i_t, tau_h * bh + i_h, tau_w * bw + i_w
    raise ValueError(f"unknown layout {layout!r}")


def num_tiles(S, B):
    """Number of length-B tiles covering S positions (the last one may be padded)."""
    return (S + B - 1) // B
