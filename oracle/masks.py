"""Keep-predicates of the mask kinds (oracle; test infrastructure).

``keep_matrix`` returns the explicit boolean matrix M[i, j] = "query i may attend
to key j" for given query and key coordinates.  It is the mask M of the masked
softmax in the Sliding Tile Attention explainer, eq. (1), with "keep" meaning
M = 0 and "drop" meaning M = -inf.

Kinds (descriptor dicts as produced by ``workloads``):

* ``all``: every pair kept (dense attention).
* ``box``: |t_k - t_q| <= rt and |y_k - y_q| <= rh and |x_k - x_q| <= rw, where a
  negative radius means "unbounded".  Spatial heads attend within the same or
  adjacent frames, temporal heads to a small spatial neighbourhood across frames
  (Sparse VideoGen on TPU, "how to accelerate attention"; DSA guide section 3).
  Spatial = box(1, -, -); temporal = box(-, r, r).
* ``stripe``: the PSA six-tuple (PSA notes, key design 1):
  inter: (|t_k - t_q - T_o| mod T_s) <= T_w - 1, intra: (|s_k - s_q - S_o| mod S_s) <= S_w - 1,
  kept iff both, with s = y*Wg + x the in-frame index.  The absolute value is taken
  first, then the modulus of a non-negative number, as the formula is printed.
* ``sta``: tile-granular sliding window (Sliding Tile Attention explainer, method
  section 3): with tile coordinates a (query) and b (key) along an axis of n tiles
  and a window of w tiles, the window starts at clamp(a - floor(w/2), 0, n - w) and
  the pair is kept iff start <= b < start + w on all three axes.  n counts the tiles
  of the axis padded up to a whole number of tiles (PSA notes, key design 2), which is
  the plain tile count when the tile divides the grid.  The window keeps
  its size and is shifted inward at the grid edges; that reading reproduces the
  sparsities the explainer prints (91.00%, 58.33%, 75.00%), a truncated window
  would not.

For every kind, keys whose frame index is below ``sink_frames`` are kept for every
query: the first-frame attention sink (Sparse VideoGen on TPU: both masks keep full
attention to frame F00; DSA guide section 3, attention sink).  The sink is a
property of the key only.
"""
from __future__ import annotations

import numpy as np


def _axis_band(d, r):
    """|d| <= r, with r < 0 meaning unbounded."""
    if r < 0:
        return np.ones(d.shape, dtype=bool)
    return np.abs(d) <= r


def _sta_start(a, w, n):
    """First tile of the window of w tiles around tile a on an axis of n tiles,
    shifted inward so it stays inside [0, n) (a window wider than the axis starts at 0)."""
    return np.minimum(np.maximum(a - w // 2, 0), max(n - w, 0))


def keep_matrix(desc, grid, cq, ck):
    """Boolean matrix [len(q), len(k)] for query coords cq=(t,y,x) and key coords ck."""
    tq, yq, xq = (np.asarray(c, dtype=np.int64)[:, None] for c in cq)
    tk, yk, xk = (np.asarray(c, dtype=np.int64)[None, :] for c in ck)
    kind = desc["kind"]
    if kind == "all":
        m = np.ones((tq.shape[0], tk.shape[1]), dtype=bool)
    elif kind == "box":
        m = _axis_band(tk - tq, desc["rt"]) & _axis_band(yk - yq, desc["rh"]) \
            & _axis_band(xk - xq, desc["rw"])
    elif kind == "stripe":
        Tw, To, Ts = desc["Tw"], desc["To"], desc["Ts"]
        Sw, So, Ss = desc["Sw"], desc["So"], desc["Ss"]
        if Ts < 1 or Ss < 1:
            raise ValueError("stripe periods must be >= 1")
        sq = yq * grid["Wg"] + xq
        sk = yk * grid["Wg"] + xk
        inter = (np.abs(tk - tq - To) % Ts) <= Tw - 1
        intra = (np.abs(sk - sq - So) % Ss) <= Sw - 1
        m = inter & intra
    elif kind == "sta":
        bt, bh, bw = grid["tile_t"], grid["tile_h"], grid["tile_w"]
        if min(bt, bh, bw) <= 0:
            raise ValueError("sta mask needs the grid's tile size")
        m = np.ones((tq.shape[0], tk.shape[1]), dtype=bool)
        for cq_ax, ck_ax, b, n, w in ((tq, tk, bt, -(-grid["T"] // bt), desc["win_t"]),
                                      (yq, yk, bh, -(-grid["Hg"] // bh), desc["win_h"]),
                                      (xq, xk, bw, -(-grid["Wg"] // bw), desc["win_w"])):
            if w < 1:
                raise ValueError("sta window must be >= 1 tile")
            start = _sta_start(cq_ax // b, w, n)
            kb = ck_ax // b
            m = m & (kb >= start) & (kb < start + w)
    else:
        raise ValueError(f"unknown mask kind {kind!r}")
    sink = desc.get("sink_frames", 0)
    if sink > 0:
        m = m | (tk < sink)
    return m
