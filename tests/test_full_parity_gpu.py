"""Full-size parity of the five workloads on the GPU, in the launch configuration the
benchmark times.

Tile classes: the whole class map of every distinct mask of every workload, in every
order its heads run in, bit for bit against the oracle (Sparse VideoGen on TPU,
"logical sparsity is not physical sparsity").  The oracle's maps take about half an
hour of CPU time, so tests/golden/make_class_goldens.py (which calls only the oracle)
stores each map's SHA-256 and its per-query-tile list lengths; the lists are checked
against the GPU's own map everywhere.

Attention: every executed query tile of every workload, on its first and last row and
one random row of each 32-row wave of the workgroup, for at least two heads of every
distinct mask (the only head where a mask has one), against the oracle on the same
bf16 inputs: max-abs <= 2e-2 and mean-abs <= 1e-3 on o, 5e-3 on lse.  The oracle runs
on a process pool (tests/oracle_pool.py).
"""
import hashlib
import json
import os
import zlib

import numpy as np
import pytest
import torch

import block_sparse_spatio_amd as vsa
import oracle
import workloads as W
from block_sparse_spatio_amd.layouts import choose_head_layouts
from tests import oracle_pool
from tests.conftest import ROOT
from tests.gpu_helpers import assert_close, dev, say

pytestmark = pytest.mark.gpu

with open(os.path.join(ROOT, "tests", "golden", "class_maps_full.json")) as _f:
    GOLDEN = {c["case"]: c for c in json.load(_f)["cases"]}


def _unrle(text):
    out = []
    for tok in text.split():
        v, _, n = tok.partition("*")
        out += [int(v)] * (int(n) if n else 1)
    return np.array(out, dtype=np.int64)


def _case_masks(case):
    """The per-head mask list of a golden case (heads of the call's order carry no
    head_layout)."""
    H = 1 + max(h for e in case["masks"] for h in e["heads"])
    masks = [None] * H
    for e in case["masks"]:
        d = dict(e["desc"])
        if d["head_layout"] == case["layout"] or case["layout"] == "padded":
            del d["head_layout"]
        for h in e["heads"]:
            masks[h] = d
    return masks


def _check_lists_follow_map(tiles):
    """On the whole map: the FULL (BOUNDARY) list of every row is exactly the ascending
    positions of its FULL (BOUNDARY) classes."""
    cls = tiles["cls"]
    nK = cls.shape[-1]
    for c, n_key, idx_key in ((1, "n_full", "full_idx"), (2, "n_bnd", "bnd_idx")):
        hit = cls == c
        assert torch.equal(hit.sum(-1).int(), tiles[n_key]), n_key
        # positions of class c first, ascending (stable sort of "not c")
        order = torch.sort((~hit).to(torch.uint8), dim=-1, stable=True).indices.int()
        used = torch.arange(nK, device=cls.device)[None, None, :] < tiles[n_key][..., None]
        assert torch.equal(torch.where(used, order, 0), torch.where(used, tiles[idx_key], 0)), idx_key


@pytest.mark.parametrize("name", list(GOLDEN))
def test_class_map_full_size(gpu_lib, name):
    case = GOLDEN[name]
    g, layout, Bq, Bk = case["grid"], case["layout"], case["Bq"], case["Bk"]
    masks = _case_masks(case)
    say(f"class map {name}: {len(case['masks'])} distinct masks, Bq={Bq} Bk={Bk}")
    tiles = vsa.vsa_classify_tiles(g, layout, masks, Bq, Bk, device=dev(), round_tiles=case["round_tiles"])
    torch.cuda.synchronize()
    hm, U = vsa.vsa_unique_masks(masks)
    assert U == len(case["masks"])
    _check_lists_follow_map(tiles)
    offs = tiles["bnd_offs"].cpu().numpy()
    assert offs[0] == 0 and np.array_equal(np.diff(offs), tiles["n_bnd"].cpu().numpy().reshape(-1))
    for e in case["masks"]:
        u = hm[e["heads"][0]]
        assert all(hm[h] == u for h in e["heads"])
        cls = tiles["cls"][u].cpu().numpy()
        assert cls.shape == (e["nQ"], e["nK"])
        nf, nb = tiles["n_full"][u].cpu().numpy(), tiles["n_bnd"][u].cpu().numpy()
        want_f, want_b = _unrle(e["n_full"]), _unrle(e["n_bnd"])
        bad = np.flatnonzero((nf != want_f) | (nb != want_b))
        assert bad.size == 0, (f"{name} mask {e['desc']}: list lengths differ first at query tile {bad[0]} "
                               f"(full {nf[bad[0]]} vs {want_f[bad[0]]}, boundary {nb[bad[0]]} vs {want_b[bad[0]]})")
        assert hashlib.sha256(np.ascontiguousarray(cls).tobytes()).hexdigest() == e["sha256"], \
            f"{name} mask {e['desc']}: class map differs from the oracle's"
    if name == "sta_hunyuan":
        # sliding tiles: only full tiles, 3x3x3 tiles of 384 tokens = 27 * 6 key tiles
        assert int(tiles["n_bnd"].sum()) == 0 and torch.all(tiles["n_full"] == 27 * 6)


# ---------------------------------------------------------------------------
# attention on every query tile
# ---------------------------------------------------------------------------
def rows_per_tile(S, Bq, seed):
    """Executed positions: per query tile its first and last row and one random row in
    each 32-row wave (rows past S dropped), sorted."""
    rng = np.random.default_rng(seed)
    rows = []
    for t in range(-(-S // Bq)):
        lo, hi = t * Bq, min(S, (t + 1) * Bq)
        rows += [lo, hi - 1]
        for w0 in range(lo, hi, 32):
            rows.append(int(rng.integers(w0, min(hi, w0 + 32))))
    return np.unique(np.array(rows, dtype=np.int64))


def heads_per_mask(masks, n=2):
    """The first n heads of every distinct descriptor."""
    seen = {}
    for h, m in enumerate(masks):
        seen.setdefault(json.dumps(m, sort_keys=True), []).append(h)
    return sorted(h for hs in seen.values() for h in hs[:n])


def _variant(name):
    """(workload, grid, call layout, masks, Bq, reorder) as the benchmark runs it."""
    base, _, var = name.partition("/")
    cfg = W.config(base)
    g, layout, masks, Bq = cfg["grid"], cfg["layout"], cfg["masks"], cfg["Bq"]
    if var == "position":
        masks = cfg["position_masks"]
    elif var.startswith("bq"):
        Bq = int(var[2:])
    elif var == "all":
        masks = cfg["extra_masks"]
    elif var == "chosen":
        g, masks = choose_head_layouts(g, masks, Bq, cfg["Bk"], dev())
    reorder = layout in ("tile", "padded") or any(m.get("head_layout", layout) != layout for m in masks)
    return cfg, g, layout, masks, Bq, reorder


FULL_VARIANTS = ["wan_mixed", "wan_mixed/position", "wan_single/bq64", "wan_single/bq128", "wan_single/bq256",
                 "wan_single/all", "sta_hunyuan", "wan_sta_padded", "stripe_route", "stripe_route/chosen"]


@pytest.mark.parametrize("name", FULL_VARIANTS)
def test_attention_full_size_every_query_tile(gpu_lib, name):
    cfg, g, layout, masks, Bq, reorder = _variant(name)
    B, H, D, Bk = cfg["B"], cfg["H"], cfg["D"], cfg["Bk"]
    S = W.seq_len(g)
    d = dev()
    say(f"full-size attention {name}: B={B} S={S} H={H} Bq={Bq} layout={layout} reorder={reorder}")
    q, k, v = W.qkv(B, S, H, D, cfg["dtype"], seed=cfg["seed"])
    tiles = vsa.vsa_classify_tiles(g, layout, masks, Bq, Bk, device=d, with_cls=False)
    words = vsa.vsa_boundary_words(g, layout, masks, tiles)  # the compact table, as benchmarked
    flags = vsa.VSA_FWD_WRITE_LSE | (vsa.VSA_FWD_REORDER_IO if reorder else 0)
    o, lse = vsa.vsa_sparse_attn_fwd(q.to(d), k.to(d), v.to(d), g, layout, masks, tiles, words=words, flags=flags)
    torch.cuda.synchronize()
    del words, tiles
    o, lse = o.cpu(), lse.cpu().numpy()
    assert torch.isfinite(o).all()
    heads = heads_per_mask(masks)
    lays = W.head_layouts(masks, layout)
    # rows per head: every query tile of the order the head runs in, mapped to frame-major
    groups = {}
    for i, h in enumerate(heads):
        groups.setdefault(lays[h], []).append((i % B, h))
    n_rows = 0
    for lay, pairs in groups.items():
        S_exec = oracle.seq_len(g, lay)
        ex = rows_per_tile(S_exec, Bq, seed=zlib.crc32(name.encode()))
        if reorder:
            perm = oracle.layout_permutation(g, lay)  # executed position -> frame-major row (-1: padding)
            rows = np.unique(perm[ex][perm[ex] >= 0])
            ref_layout = "frame"
        else:
            rows, ref_layout = ex, lay
        ref = oracle_pool.attention_rows(q, k, v, g, ref_layout, masks, rows, pairs)
        for (b, h), (ro, rl) in ref.items():
            assert_close(o[b, rows, h], ro, "bf16", f"{name} head {h} ({lay}) batch {b}")
            lerr = np.abs(lse[b, h, rows] - rl).max()
            assert lerr <= 5e-3, f"{name} head {h}: lse error {lerr:.3e}"
        n_rows += len(rows) * len(pairs)
    say(f"{name}: {n_rows} (row, head) pairs compared on heads {heads}")
