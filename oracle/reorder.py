"""Tile-major token permutation (oracle; test infrastructure).

Sliding-tile attention needs the tokens of each 3D tile to be contiguous in the
sequence (Sliding Tile Attention explainer, method section 3; video-DiT attention
blog, section 7.2).  The permutation is defined by coordinates: tile-major position
p' holds the token whose (t, y, x) coordinates ``token_coords(grid, "tile", p')``
names, i.e. the frame-major token (t*Hg + y)*Wg + x.
"""
from __future__ import annotations

import numpy as np

from .coords import token_coords


def tile_major_permutation(grid):
    """perm[p'] = frame-major index of the token at tile-major position p'."""
    S = grid["T"] * grid["Hg"] * grid["Wg"]
    t, y, x = token_coords(grid, "tile", np.arange(S))
    return (t * grid["Hg"] + y) * grid["Wg"] + x


def reorder_tokens(x, grid, inverse=False):
    """Permute axis 1 of x [B, S, ...]: frame-major -> tile-major, or back when inverse."""
    perm = tile_major_permutation(grid)
    x = np.asarray(x)
    if not inverse:
        return x[:, perm]
    out = np.empty_like(x)
    out[:, perm] = x
    return out
