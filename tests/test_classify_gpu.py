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


def _sampled_q_tiles(nQ, rng, n=6):
    return np.unique(np.concatenate([[0, nQ - 1, nQ // 2], rng.choice(nQ, n, replace=False)]))


@pytest.mark.parametrize("name,Bq", [("wan_mixed", 128), ("wan_single", 64), ("wan_single", 128),
                                     ("wan_single", 256), ("sta_hunyuan", 128), ("stripe_route", 128)])
def test_classify_full_configs(gpu_lib, name, Bq):
    cfg = W.config(name)
    g, layout, masks = cfg["grid"], cfg["layout"], cfg["masks"]
    say(f"classify full config {name} Bq={Bq}")
    tiles = gpu_lib.vsa_classify_tiles(g, layout, masks, Bq, cfg["Bk"], device=dev())
    torch.cuda.synchronize()
    hm, U = gpu_lib.vsa_unique_masks(masks)
    rng = np.random.default_rng(7)
    nQ = tiles["nQ"]
    seen = set()
    for h, desc in enumerate(masks):
        u = hm[h]
        if u in seen:
            continue
        seen.add(u)
        qts = _sampled_q_tiles(nQ, rng, 3 if U > 8 else 6)
        ref = oracle.classify(g, layout, desc, Bq, cfg["Bk"], q_tiles=qts)
        check_lists_against(tiles, u, qts, ref["cls"])
    # whole-map properties: the lists agree with the class map everywhere
    cls = tiles["cls"].cpu()
    assert torch.equal((cls == 1).sum(-1).int(), tiles["n_full"].cpu())
    assert torch.equal((cls == 2).sum(-1).int(), tiles["n_bnd"].cpu())
    if name == "sta_hunyuan":
        # sliding tiles: every tile pair is full or empty; 3x3x3 tiles of 384 tokens
        # = 27 * 6 key tiles of 64 per query tile
        assert int(tiles["n_bnd"].sum()) == 0
        assert torch.all(tiles["n_full"].cpu() == 27 * 6)
    if name == "wan_single" and Bq == 128:
        # |dt| <= 3 plus sink keeps 152 of 441 frame pairs; the kept-pair count
        # equals the sum over FULL tiles plus the kept pairs inside BOUNDARY tiles,
        # so the FULL tiles alone stay below it
        full_pairs = int(tiles["n_full"].sum()) * 128 * 64
        assert full_pairs <= 152 * 3600 * 3600


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


@pytest.mark.parametrize("name,Bq", [("wan_single", 128), ("wan_mixed", 128)])
def test_classify_rounded_full_configs(gpu_lib, name, Bq):
    cfg = W.config(name)
    g, layout, masks = cfg["grid"], cfg["layout"], cfg["masks"]
    say(f"classify rounded full config {name} Bq={Bq}")
    tiles = gpu_lib.vsa_classify_tiles(g, layout, masks, Bq, cfg["Bk"], device=dev(), round_tiles=True)
    exact = gpu_lib.vsa_classify_tiles(g, layout, masks, Bq, cfg["Bk"], device=dev())
    torch.cuda.synchronize()
    hm, U = gpu_lib.vsa_unique_masks(masks)
    rng = np.random.default_rng(8)
    seen = set()
    for h, desc in enumerate(masks):
        u = hm[h]
        if u in seen:
            continue
        seen.add(u)
        qts = _sampled_q_tiles(tiles["nQ"], rng, 3)
        ref = oracle.classify(g, layout, desc, Bq, cfg["Bk"], q_tiles=qts, round_tiles=True)
        check_lists_against(tiles, u, qts, ref["cls"])
    # rounding touches only boundary tiles, and boundary tiles remain only at the tail
    ce, cr = exact["cls"].cpu(), tiles["cls"].cpu()
    assert torch.equal(ce[ce != 2], cr[ce != 2])
    S = W.seq_len(g)
    nK = cr.shape[-1]
    if S % cfg["Bk"] == 0 and S % Bq:
        assert torch.all(cr[:, :-1] != 2)


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


def test_classify_position_major_full_config(gpu_lib):
    """Wan 2.1 720p mixed heads with the temporal heads position-major: sampled query
    tiles bit-exact, and far fewer executed tiles than the same heads frame-major."""
    cfg = W.config("wan_mixed")
    g, Bq, Bk = cfg["grid"], cfg["Bq"], cfg["Bk"]
    masks = cfg["position_masks"]
    say("classify position-major full config wan_mixed")
    tiles = gpu_lib.vsa_classify_tiles(g, "frame", masks, Bq, Bk, device=dev())
    frame = gpu_lib.vsa_classify_tiles(g, "frame", cfg["masks"], Bq, Bk, device=dev(), with_cls=False)
    torch.cuda.synchronize()
    hm, U = gpu_lib.vsa_unique_masks(masks)
    assert U == 2
    rng = np.random.default_rng(9)
    for u, h in ((hm[0], 0), (hm[-1], len(masks) - 1)):
        qts = _sampled_q_tiles(tiles["nQ"], rng, 6)
        lay = W.head_layouts(masks, "frame")[h]
        ref = oracle.classify(g, lay, masks[h], Bq, Bk, q_tiles=qts)
        check_lists_against(tiles, u, qts, ref["cls"])
    cls = tiles["cls"].cpu()
    assert torch.equal((cls == 1).sum(-1).int(), tiles["n_full"].cpu())
    assert torch.equal((cls == 2).sum(-1).int(), tiles["n_bnd"].cpu())
    n_pos = int(tiles["n_full"][hm[-1]].sum() + tiles["n_bnd"][hm[-1]].sum())
    hmf, _ = gpu_lib.vsa_unique_masks(cfg["masks"])
    n_frame = int(frame["n_full"][hmf[-1]].sum() + frame["n_bnd"][hmf[-1]].sum())
    say(f"temporal head executed tiles: position-major {n_pos}, frame-major {n_frame}")
    assert n_pos < n_frame / 2


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


def test_classify_padded_full_config(gpu_lib):
    """Sliding tiles on the padded Wan 2.1 720p latent (21 x 48 x 80 for 3 x 8 x 16
    tiles): sampled query tiles bit-exact."""
    cfg = W.config("wan_sta_padded")
    g, Bq, Bk = cfg["grid"], cfg["Bq"], cfg["Bk"]
    say("classify padded full config wan_sta_padded")
    tiles = gpu_lib.vsa_classify_tiles(g, "padded", cfg["masks"], Bq, Bk, device=dev())
    torch.cuda.synchronize()
    assert tiles["nQ"] == -(-80640 // Bq)
    rng = np.random.default_rng(11)
    qts = _sampled_q_tiles(tiles["nQ"], rng, 6)
    ref = oracle.classify(g, "padded", cfg["masks"][0], Bq, Bk, q_tiles=qts)
    check_lists_against(tiles, 0, qts, ref["cls"])


def test_classify_stripes_column_and_position_full_config(gpu_lib):
    """The routed stripe layer in the orders its heads run in: stripes whose period is
    the row width tile-major over one-column tiles (1x45x1, each frame read column by
    column), the others position-major.  Sampled query tiles of several heads of each
    order bit-exact against the oracle, and the lists agree with the class map."""
    cfg = W.config("stripe_route")
    g = W.grid(21, 45, 80, (1, 45, 1))
    Bq, Bk = cfg["Bq"], cfg["Bk"]
    masks = [W.with_head_layout(m, "tile" if m["Ss"] == 80 else "position") for m in cfg["masks"]]
    say("classify stripe layer, column and position orders, full size")
    tiles = gpu_lib.vsa_classify_tiles(g, "frame", masks, Bq, Bk, device=dev())
    torch.cuda.synchronize()
    hm, U = gpu_lib.vsa_unique_masks(masks)
    lays = W.head_layouts(masks, "frame")
    rng = np.random.default_rng(11)
    picked = [h for h in range(len(masks)) if lays[h] == "tile"][:4] + \
        [h for h in range(len(masks)) if lays[h] == "position"][:4]
    assert len(picked) == 8
    for h in picked:
        qts = _sampled_q_tiles(tiles["nQ"], rng, 3)
        ref = oracle.classify(g, lays[h], masks[h], Bq, Bk, q_tiles=qts)
        check_lists_against(tiles, hm[h], qts, ref["cls"])
    cls = tiles["cls"].cpu()
    assert torch.equal((cls == 1).sum(-1).int(), tiles["n_full"].cpu())
    assert torch.equal((cls == 2).sum(-1).int(), tiles["n_bnd"].cpu())
