"""Per-head token orders chosen by tile cost (a host-side policy over the classify ABI).

Sparse VideoGen on TPU ("dynamic routing with fixed tensor shapes"; "layout transforms
on local heads") gives each head a flag that selects the original or a permuted token
order, and measures that a permutation which makes a head's kept keys contiguous beats
in-kernel indexing ("arranging tokens for temporal access").  Which order pays off is a
property of the mask and the tile size, so this helper asks the library's own
classifier: it classifies every head in each candidate order and keeps, per head, the
order whose lists cost least.  The decision is made once per shape, outside any timed
step; it needs no data, only the grid, the masks and the tile sizes.
"""
from __future__ import annotations

from . import _lib


def choose_head_layouts(grid, masks, Bq, Bk, device, bnd_cost=1.2, widths=(1, 2, 4, 8, 16)):
    """Per-head token order with the lowest tile cost among frame-major, position-major
    and tile-major over one grid tile (1, Hg, w) for w in `widths` dividing Wg (a frame
    read w columns at a time, which makes column-band stripes contiguous).  A full tile
    costs 1 and a boundary tile `bnd_cost` (its element masks come from the word table).
    All heads that run tile-major share one grid tile: the w with the lowest total is
    kept.  Returns (grid, masks): the grid with the chosen tile (unchanged when no head
    runs tile-major) and the masks with their head_layout set (frame-major heads keep
    their descriptor as given)."""
    def per_head(g, order):
        om = [dict(m, head_layout=order) for m in masks]
        t = _lib.vsa_classify_tiles(g, "frame", om, Bq, Bk, device=device, with_cls=False)
        hm, _ = _lib.vsa_unique_masks(om)
        nt = (t["n_full"].double() + bnd_cost * t["n_bnd"].double()).sum(dim=1).cpu().tolist()
        return [nt[hm[h]] for h in range(len(masks))]

    base = {"frame": per_head(grid, "frame"), "position": per_head(grid, "position")}
    best_total, best = None, None
    tiles = [None] + [(1, grid["Hg"], w) for w in widths if grid["Wg"] % w == 0]
    for tile in tiles:
        cand = dict(base)
        g = grid
        if tile is not None:
            g = dict(grid, tile_t=tile[0], tile_h=tile[1], tile_w=tile[2])
            cand["tile"] = per_head(g, "tile")
        picks = [min(cand, key=lambda o: cand[o][h]) for h in range(len(masks))]
        total = sum(cand[o][h] for h, o in enumerate(picks))
        if best_total is None or total < best_total:
            best_total, best = total, (g if "tile" in picks else grid, picks)
    g, picks = best
    return g, [dict(m, head_layout=o) if o != "frame" else m for m, o in zip(masks, picks)]
