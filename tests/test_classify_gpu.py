"""Tile classification on the GPU: bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import check_lists_against, dev, say

pytestmark = pytest.mark.gpu


def _random_desc(rng, layout):
    kinds = ["all", "box", "stripe"] + (["sta"] if layout == "tile" else [])
    kind = kinds[rng.integers(len(kinds))]
    sink = int(rng.integers(0, 3))
    if kind == "all":
        return W.mask_all()
    if kind == "box":
        r = lambda: int(rng.integers(-1, 4))  # noqa: E731
        return W.mask_box(r(), r(), r(), sink_frames=sink)
    if kind == "stripe":
        return W.mask_stripe(int(rng.integers(0, 4)), int(rng.integers(-2, 3)), int(rng.integers(1, 6)),
                             int(rng.integers(0, 5)), int(rng.integers(-3, 4)), int(rng.integers(1, 40)),
                             sink_frames=sink)
    return W.mask_sta(int(rng.integers(1, 4)), int(rng.integers(1, 4)), int(rng.integers(1, 4)),
                      sink_frames=sink)


@pytest.mark.parametrize("seed", range(48))
def test_classify_random_small(gpu_lib, seed):
    rng = np.random.default_rng(seed)
    layout = "tile" if seed % 3 == 2 else "frame"
    if layout == "tile":
        tile = tuple(int(x) for x in rng.integers(1, 4, 3))
        g = W.grid(tile[0] * int(rng.integers(1, 4)), tile[1] * int(rng.integers(1, 4)),
                   tile[2] * int(rng.integers(1, 5)), tile)
    else:
        g = W.grid(int(rng.integers(1, 7)), int(rng.integers(1, 9)), int(rng.integers(1, 12)))
    H = int(rng.integers(1, 5))
    masks = [_random_desc(rng, layout) for _ in range(H)]
    Bq = int(rng.choice([1, 3, 8, 16, 32, 64, 128]))
    Bk = int(rng.choice([1, 5, 16, 32, 64]))
    say(f"classify seed={seed} grid={g} layout={layout} Bq={Bq} Bk={Bk} masks={masks}")
    tiles = gpu_lib.vsa_classify_tiles(g, layout, masks, Bq, Bk, device=dev())
    torch.cuda.synchronize()
    hm, U = gpu_lib.vsa_unique_masks(masks)
    for h, desc in enumerate(masks):
        ref = oracle.classify(g, layout, desc, Bq, Bk)
        check_lists_against(tiles, hm[h], ref["q_tiles"], ref["cls"])


def test_classify_null_cls(gpu_lib):
    g = W.grid(5, 6, 7)
    masks = [W.mask_temporal(2)]
    t = gpu_lib.vsa_classify_tiles(g, "frame", masks, 32, 16, device=dev(), with_cls=False)
    torch.cuda.synchronize()
    ref = oracle.classify(g, "frame", masks[0], 32, 16)
    t["cls"] = None
    check_lists_against(t, 0, ref["q_tiles"], ref["cls"])


@pytest.mark.parametrize("seed", range(24))
def test_classify_rounded_random_small(gpu_lib, seed):
    """Tile-aligned rounding (B3) on the GPU equals the oracle's rounded classes."""
    rng = np.random.default_rng(1000 + seed)
    layout = "tile" if seed % 3 == 2 else "frame"
    if layout == "tile":
        tile = tuple(int(x) for x in rng.integers(1, 4, 3))
        g = W.grid(tile[0] * int(rng.integers(1, 4)), tile[1] * int(rng.integers(1, 4)),
                   tile[2] * int(rng.integers(1, 5)), tile)
    else:
        g = W.grid(int(rng.integers(1, 7)), int(rng.integers(1, 9)), int(rng.integers(1, 12)))
    H = int(rng.integers(1, 4))
    masks = [_random_desc(rng, layout) for _ in range(H)]
    Bq = int(rng.choice([1, 8, 16, 32, 64, 128]))
    Bk = int(rng.choice([1, 5, 16, 32, 64]))
    say(f"classify rounded seed={seed} grid={g} layout={layout} Bq={Bq} Bk={Bk} masks={masks}")
    tiles = gpu_lib.vsa_classify_tiles(g, layout, masks, Bq, Bk, device=dev(), round_tiles=True)
    torch.cuda.synchronize()
    hm, U = gpu_lib.vsa_unique_masks(masks)
    for h, desc in enumerate(masks):
        ref = oracle.classify(g, layout, desc, Bq, Bk, round_tiles=True)
        check_lists_against(tiles, hm[h], ref["q_tiles"], ref["cls"])


@pytest.mark.parametrize("seed", range(36))
def test_classify_random_head_layouts(gpu_lib, seed):
    """Heads in their own token orders (frame-, tile- or position-major): every head's
    classes equal the oracle's in that head's order, exact and rounded."""
    rng = np.random.default_rng(2000 + seed)
    tiled = seed % 2 == 1
    if tiled:
        tile = tuple(int(x) for x in rng.integers(1, 4, 3))
        g = W.grid(tile[0] * int(rng.integers(1, 4)), tile[1] * int(rng.integers(1, 4)),
                   tile[2] * int(rng.integers(1, 5)), tile)
    else:
        g = W.grid(int(rng.integers(1, 9)), int(rng.integers(1, 9)), int(rng.integers(1, 12)))
    orders = ["frame", "position"] + (["tile"] if tiled else [])
    layout = orders[rng.integers(len(orders))]
    H = int(rng.integers(1, 6))
    masks = []
    for _ in range(H):
        m = _random_desc(rng, "tile" if tiled else "frame")
        pick = int(rng.integers(len(orders) + 1))
        masks.append(m if pick == len(orders) else W.with_head_layout(m, orders[pick]))
    Bq = int(rng.choice([1, 3, 8, 16, 32, 64, 128]))
    Bk = int(rng.choice([1, 5, 16, 32, 64]))
    round_tiles = seed % 3 == 0
    say(f"classify head layouts seed={seed} grid={g} layout={layout} Bq={Bq} Bk={Bk} round={round_tiles} "
        f"masks={masks}")
    tiles = gpu_lib.vsa_classify_tiles(g, layout, masks, Bq, Bk, device=dev(), round_tiles=round_tiles)
    torch.cuda.synchronize()
    hm, U = gpu_lib.vsa_unique_masks(masks)
    for h, (desc, lay) in enumerate(zip(masks, W.head_layouts(masks, layout))):
        ref = oracle.classify(g, lay, desc, Bq, Bk, round_tiles=round_tiles)
        check_lists_against(tiles, hm[h], ref["q_tiles"], ref["cls"])


@pytest.mark.parametrize("seed", range(30))
def test_classify_random_padded(gpu_lib, seed):
    """Tile-major order over a grid padded up to whole tiles: classes bit-exact against
    the oracle (padding pairs are never kept), exact and rounded."""
    rng = np.random.default_rng(3000 + seed)
    tile = tuple(int(x) for x in rng.integers(1, 5, 3))
    g = W.grid(int(rng.integers(1, 8)), int(rng.integers(1, 9)), int(rng.integers(1, 12)), tile)
    H = int(rng.integers(1, 5))
    masks = [_random_desc(rng, "tile") for _ in range(H)]
    Bq = int(rng.choice([1, 3, 8, 16, 32, 64, 128]))
    Bk = int(rng.choice([1, 5, 16, 32, 64]))
    round_tiles = seed % 3 == 1
    say(f"classify padded seed={seed} grid={g} Bq={Bq} Bk={Bk} round={round_tiles} masks={masks}")
    tiles = gpu_lib.vsa_classify_tiles(g, "padded", masks, Bq, Bk, device=dev(), round_tiles=round_tiles)
    torch.cuda.synchronize()
    hm, U = gpu_lib.vsa_unique_masks(masks)
    for h, desc in enumerate(masks):
        ref = oracle.classify(g, "padded", desc, Bq, Bk, round_tiles=round_tiles)
        check_lists_against(tiles, hm[h], ref["q_tiles"], ref["cls"])
