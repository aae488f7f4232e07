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
* padded (tile-major with 3D padding, PSA notes, key design 2): each axis is padded up
  to the smallest multiple of the tile (T' = ceil(T / bt) * bt, likewise H' and W'),
  and the padded grid is laid out tile-major as above.  Positions whose coordinates
  fall outside the real grid are padding tokens: they are never kept as keys, and a
  padding query's output is not part of the result.  The executed length is
  T' * H' * W' (``seq_len``).  With tiles that divide the grid it is the tile-major
  order.
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


def padded_dims(grid):
    """(T', H', W'): every axis rounded up to a multiple of the grid's tile."""
    bt, bh, bw = grid["tile_t"], grid["tile_h"], grid["tile_w"]
    if min(bt, bh, bw) <= 0:
        raise ValueError("the padded layout needs a positive tile size")
    return (-(-grid["T"] // bt) * bt, -(-grid["Hg"] // bh) * bh, -(-grid["Wg"] // bw) * bw)


def seq_len(grid, layout):
    """Executed sequence length: T*Hg*Wg, or T'*H'*W' for the padded layout."""
    if layout == "padded":
        Tp, Hp, Wp = padded_dims(grid)
        return Tp * Hp * Wp
    return grid["T"] * grid["Hg"] * grid["Wg"]


def is_real(grid, t, y, x):
    """True where (t, y, x) is a token of the grid (not padding)."""
    return (np.asarray(t) < grid["T"]) & (np.asarray(y) < grid["Hg"]) & (np.asarray(x) < grid["Wg"])


def token_coords(grid, layout, pos):
    """Return (t, y, x) int64 arrays for executed positions ``pos`` (any int array).

    layout is "frame", "tile", "position" or "padded" (coordinates of padding
    positions lie outside the grid)."""
    pos = np.asarray(pos, dtype=np.int64)
    T, Hg, Wg = grid["T"], grid["Hg"], grid["Wg"]
    if layout == "frame":
        t = pos // (Hg * Wg)
        y = (pos // Wg) % Hg
        x = pos % Wg
        return t, y, x
    if layout in ("tile", "padded"):
        if layout == "tile":
            _check_tile(grid)
        bt, bh, bw = grid["tile_t"], grid["tile_h"], grid["tile_w"]
        Tp, Hp, Wp = padded_dims(grid)
        nH, nW = Hp // bh, Wp // bw
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
