"""Token permutations between frame-major order and an executed layout (oracle;
test infrastructure).

Sliding-tile attention needs the tokens of each 3D tile to be contiguous in the
sequence (Sliding Tile Attention explainer, method section 3; video-DiT attention
blog, section 7.2).  The permutation is defined by coordinates: tile-major position
p' holds the token whose (t, y, x) coordinates ``token_coords(grid, "tile", p')``
names, i.e. the frame-major token (t*Hg + y)*Wg + x.  The position-major order of
temporal heads (oracle.coords) is permuted the same way, per head.
"""
from __future__ import annotations

import numpy as np

from .coords import is_real, seq_len, token_coords


def layout_permutation(grid, layout):
    """perm[p'] = frame-major index of the token at executed position p' of layout, or -1
    where p' is a padding position (padded layout)."""
    S = seq_len(grid, layout)
    t, y, x = token_coords(grid, layout, np.arange(S))
    frame = (t * grid["Hg"] + y) * grid["Wg"] + x
    return np.where(is_real(grid, t, y, x), frame, -1)


def tile_major_permutation(grid):
    """perm[p'] = frame-major index of the token at tile-major position p'."""
    return layout_permutation(grid, "tile")


def reorder_tokens(x, grid, inverse=False, layout="tile"):
    """Permute axis 1 of x [B, S, ...]: frame-major -> layout (padding positions zero),
    or back when inverse (padding positions dropped)."""
    perm = layout_permutation(grid, layout)
    x = np.asarray(x)
    real = perm >= 0
    if not inverse:
        out = np.zeros((x.shape[0], len(perm)) + x.shape[2:], dtype=x.dtype)
        out[:, real] = x[:, perm[real]]
        return out
    S = grid["T"] * grid["Hg"] * grid["Wg"]
    out = np.empty((x.shape[0], S) + x.shape[2:], dtype=x.dtype)
    out[:, perm[real]] = x[:, real]
    return out
