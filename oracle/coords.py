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
* position-major: the temporal order of Sparse VideoGen on TPU ("arranging tokens
  for temporal access"): tokens are permuted from (frame, row, column) to (row,
  column, frame), so that one spatial position's tokens across frames are
  contiguous and a temporal head's diagonal stripes become contiguous bands
  (video-DiT attention blog, section 7.2, the (h, w, t) reorder).  Frame 0 is kept
  as a leading block in frame-major order, so that the first-frame sink keys stay
  contiguous: positions [0, Hg*Wg) are frame 0 row-major, and position
  Hg*Wg + s*(T-1) + (t-1) holds frame t >= 1 at spatial index s = y*Wg + x.  The
  leading sink block is this implementation's reading; the page permutes all frames.
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

    layout is "frame", "tile" or "position"."""
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
    if layout == "position":
        HW = Hg * Wg
        head = pos < HW
        q = np.where(head, 0, pos - HW)
        T1 = max(T - 1, 1)
        s = np.where(head, pos, q // T1)
        t = np.where(head, 0, 1 + q % T1)
        return t, s // Wg, s % Wg
    raise ValueError(f"unknown layout {layout!r}")


def num_tiles(S, B):
    """Number of length-B tiles covering S positions (the last one may be padded)."""
    return (S + B - 1) // B
