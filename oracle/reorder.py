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

from .coords import token_coords


def layout_permutation(grid, layout):
    """perm[p'] = frame-major index of the token at executed position p' of layout."""
    S = grid["T"] * grid["Hg"] * grid["Wg"]
    t, y, x = token_coords(grid, layout, np.arange(S))
    return (t * grid["Hg"] + y) * grid["Wg"] + x


def tile_major_permutation(grid):
    """perm[p'] = frame-major index of the token at tile-major position p'."""
    return layout_permutation(grid, "tile")


def reorder_tokens(x, grid, inverse=False, layout="tile"):
    """Permute axis 1 of x [B, S, ...]: frame-major -> layout, or back when inverse."""
    perm = layout_permutation(grid, layout)
    x = np.asarray(x)
    if not inverse:
        return x[:, perm]
    out = np.empty_like(x)
    out[:, perm] = x
    return out
