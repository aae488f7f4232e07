"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: every expected value is a number
the pages print (tests/golden), a closed form counted a different way, a special
case that reduces to another mask or to a library routine, or a brute-force loop
on tiny inputs.  CPU only.
"""
import itertools
import math

import numpy as np
import pytest

import oracle
import workloads as W
from oracle.coords import token_coords
from oracle.masks import keep_matrix
from tests.conftest import golden


def full_keep(desc, g, layout="frame"):
    S = W.seq_len(g)
    c = token_coords(g, layout, np.arange(S))
    return keep_matrix(desc, g, c, c)


# ---------------------------------------------------------------------------
# sliding-tile masks: printed sparsities and block fractions
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("row", golden("sta_sparsity.txt"))
def test_sta_sparsity_printed(row):
    """STA windows on the 30x48x80 grid with 6x8x8 tiles: the printed sparsity."""
    wt, wh, ww, pct = int(row[0]), int(row[1]), int(row[2]), float(row[3])
    # the STA mask depends on tile coordinates only: a grid of unit tiles over the
    # 5 x 6 x 10 tile grid has the same kept fraction as the token grid
    g1 = W.grid(5, 6, 10, (1, 1, 1))
    m = full_keep(W.mask_sta(wt // 6, wh // 8, ww // 8), g1, "tile")
    sparsity = 100.0 * (1.0 - m.sum() / m.size)
    assert round(sparsity, 2) == pct
    # every token query keeps exactly its window's tiles on the real token grid
    g = W.grid(30, 48, 80, (6, 8, 8))
    S = W.seq_len(g)
    rng = np.random.default_rng(0)
    rows = np.concatenate([[0, S - 1, 384 * 37 + 5], rng.integers(0, S, 5)])
    keep = keep_matrix(W.mask_sta(wt // 6, wh // 8, ww // 8), g,
                       token_coords(g, "tile", rows), token_coords(g, "tile", np.arange(S)))
    assert np.all(keep.sum(axis=1) == (wt // 6) * (wh // 8) * (ww // 8) * 384)


@pytest.mark.parametrize("row", [r for r in golden("block_fractions_table1.txt") if r[0] == "sta"])
def test_table1_sta_fractions(row):
    """Table 1: STA dense-block fraction (W/L)^3 and no mixed blocks, L=48, T=4."""
    win, dense_pct, mixed_pct = int(row[1]), float(row[2]), float(row[3])
    w_tiles = win // 4
    # tile-level count on the 12^3 tile grid
    g1 = W.grid(12, 12, 12, (1, 1, 1))
    m = full_keep(W.mask_sta(w_tiles, w_tiles, w_tiles), g1, "tile")
    assert round(100.0 * m.sum() / m.size, 2) == dense_pct
    # token level: 64-token blocks (4^3 tiles, tile-major) are only FULL or EMPTY
    g = W.grid(48, 48, 48, (4, 4, 4))
    qts = [0, 1727, 13 + 12 * 7, 6 * 144 + 6 * 12 + 6]
    res = oracle.classify(g, "tile", W.mask_sta(w_tiles, w_tiles, w_tiles), 64, 64, q_tiles=qts)
    for row_cls in res["cls"]:
        assert np.count_nonzero(row_cls == oracle.BOUNDARY) == 0
        assert np.count_nonzero(row_cls == oracle.FULL) == w_tiles ** 3
    assert mixed_pct == 0.0


@pytest.mark.parametrize("row", golden("natten_eq23.txt"))
def test_natten_eq2_eq3_interior(row):
    """Tiled NATTEN eq. (2)/(3): a centred token window classified on T^3 tiles."""
    Wn, T, dense, mixed = (int(x) for x in row)
    r = (Wn - 1) // 2
    L = 8 * T  # 8 tiles per axis; the query tile (3,3,3) is interior for r <= 2T
    g = W.grid(L, L, L, (T, T, T))
    qt = 3 * 64 + 3 * 8 + 3
    res = oracle.classify(g, "tile", W.mask_box(r, r, r), T ** 3, T ** 3, q_tiles=[qt])
    cls = res["cls"][0]
    assert np.count_nonzero(cls == oracle.FULL) == dense
    assert np.count_nonzero(cls == oracle.BOUNDARY) == mixed


def test_table1_natten_percentages():
    """Table 1's Tiled NATTEN (11,11,11) row: per-query-tile counts over 1728 tiles."""
    (row,) = [r for r in golden("block_fractions_table1.txt") if r[0] == "tiled_natten"]
    g = W.grid(32, 32, 32, (4, 4, 4))
    qt = 3 * 64 + 3 * 8 + 3
    cls = oracle.classify(g, "tile", W.mask_box(5, 5, 5), 64, 64, q_tiles=[qt])["cls"][0]
    dense = 100.0 * np.count_nonzero(cls == oracle.FULL) / 1728
    mixed = 100.0 * np.count_nonzero(cls == oracle.BOUNDARY) / 1728
    assert round(dense, 2) == float(row[2])
    assert math.floor(mixed * 100) / 100 == float(row[3])


# ---------------------------------------------------------------------------
# box masks: kept-pair closed forms (counted per axis / per frame pair)
# ---------------------------------------------------------------------------
def _axis_pairs(n, r):
    """#(a, b) in [0,n)^2 with |a-b| <= r (r<0: all), counted by offsets."""
    if r < 0:
        return n * n
    return sum(n - abs(d) for d in range(-min(r, n - 1), min(r, n - 1) + 1))


def _box_count(T, Hg, Wg, rt, rh, rw, sink):
    HW = Hg * Wg
    within = _axis_pairs(Hg, rh) * _axis_pairs(Wg, rw)
    total = 0
    for tq in range(T):
        for tk in range(T):
            if tk < sink:
                total += HW * HW
            elif rt < 0 or abs(tk - tq) <= rt:
                total += within
    return total


@pytest.mark.parametrize("T,Hg,Wg,rt,rh,rw,sink", [
    (4, 8, 8, 1, -1, -1, 1), (4, 8, 8, -1, 1, 1, 1), (6, 5, 7, 2, 1, 3, 0),
    (5, 4, 9, -1, 2, 2, 2), (3, 6, 6, 0, 0, 0, 0), (7, 3, 4, 3, -1, 1, 1)])
def test_box_kept_count_closed_form(T, Hg, Wg, rt, rh, rw, sink):
    g = W.grid(T, Hg, Wg)
    m = full_keep(W.mask_box(rt, rh, rw, sink), g)
    assert m.sum() == _box_count(T, Hg, Wg, rt, rh, rw, sink)


def test_workload_kept_fractions():
    """Kept fractions of the workloads' masks from the closed form (derived values):
    spatial |dt|<=1 + sink 80/441, |dt|<=3 + sink 152/441; tiny temporal 22,192 pairs."""
    assert _box_count(21, 1, 1, 1, -1, -1, 1) == 80
    assert _box_count(21, 1, 1, 3, -1, -1, 1) == 152
    assert _box_count(4, 8, 8, -1, 1, 1, 1) == 22192
    # the oracle agrees on a grid whose frames are smaller than the workloads'
    g = W.grid(21, 2, 3)
    assert full_keep(W.mask_spatial(1), g).sum() == 80 * 36
    assert full_keep(W.mask_spatial(3), g).sum() == 152 * 36


# ---------------------------------------------------------------------------
# stripe masks: special cases that reduce to other masks
# ---------------------------------------------------------------------------
def test_stripe_reduces_to_spatial():
    """T_s beyond any frame distance and S_w = S_s (every s): |dt| <= T_w - 1."""
    g = W.grid(6, 3, 5)
    a = full_keep(W.mask_stripe(2, 0, 50, 15, 0, 15, sink_frames=1), g)
    b = full_keep(W.mask_spatial(1, sink_frames=1), g)
    assert np.array_equal(a, b)


def test_stripe_period_wg_is_same_column():
    """S_s = Wg, S_w = 1: |dy*Wg + dx| divisible by Wg iff dx = 0 (|dx| < Wg)."""
    g = W.grid(3, 4, 6)
    a = full_keep(W.mask_stripe(3, 0, 3, 1, 0, 6, sink_frames=0), g)
    b = full_keep(W.mask_box(-1, -1, 0), g)
    assert np.array_equal(a, b)


def test_stripe_offset_is_key_minus_query():
    """T_o = 1, T_w = 1, large T_s: only keys one frame after the query."""
    g = W.grid(5, 2, 2)
    m = full_keep(W.mask_stripe(1, 1, 99, 4, 0, 4, sink_frames=0), g)
    t = token_coords(g, "frame", np.arange(20))[0]
    for i in range(20):
        for j in range(20):
            assert m[i, j] == (t[j] == t[i] + 1)


def test_stripe_periodic_frames():
    """T_s = 3, T_w = 1: frames at distance 0, 3, 6 ...; with S_w = S_s all s kept."""
    g = W.grid(8, 1, 2)
    m = full_keep(W.mask_stripe(1, 0, 3, 2, 0, 2, sink_frames=0), g)
    t = token_coords(g, "frame", np.arange(16))[0]
    assert np.array_equal(m, (np.abs(t[None, :] - t[:, None]) % 3) == 0)


# ---------------------------------------------------------------------------
# coordinates and the tile-major permutation
# ---------------------------------------------------------------------------
def test_frame_major_roundtrip():
    g = W.grid(3, 4, 5)
    t, y, x = token_coords(g, "frame", np.arange(60))
    assert np.array_equal((t * 4 + y) * 5 + x, np.arange(60))


def test_tile_major_tiles_are_contiguous():
    g = W.grid(4, 6, 8, (2, 3, 4))
    S = 192
    perm = oracle.tile_major_permutation(g)
    assert np.array_equal(np.sort(perm), np.arange(S))
    t, y, x = token_coords(g, "tile", np.arange(S))
    vol = 24
    nT, nH, nW = 2, 2, 2
    for tau in range(S // vol):
        sl = slice(tau * vol, (tau + 1) * vol)
        a = (tau // (nH * nW), (tau // nW) % nH, tau % nW)
        assert set(t[sl] // 2) == {a[0]} and set(y[sl] // 3) == {a[1]} and set(x[sl] // 4) == {a[2]}
        # inside the tile: row-major (t, y, x)
        inner = ((t[sl] % 2) * 3 + y[sl] % 3) * 4 + x[sl] % 4
        assert np.array_equal(inner, np.arange(vol))
    xx = np.random.default_rng(1).standard_normal((2, S, 3))
    assert np.array_equal(oracle.reorder_tokens(oracle.reorder_tokens(xx, g), g, inverse=True), xx)


# ---------------------------------------------------------------------------
# classification against brute force on tiny grids
# ---------------------------------------------------------------------------
def _brute_classes(desc, g, layout, Bq, Bk):
    S = W.seq_len(g)
    c = token_coords(g, layout, np.arange(S))
    keep = keep_matrix(desc, g, c, c)
    nQ, nK = -(-S // Bq), -(-S // Bk)
    out = np.zeros((nQ, nK), dtype=np.uint8)
    for qt in range(nQ):
        for kt in range(nK):
            kept = total = 0
            for i in range(qt * Bq, (qt + 1) * Bq):
                for j in range(kt * Bk, (kt + 1) * Bk):
                    total += 1
                    if i < S and j < S and keep[i, j]:
                        kept += 1
            out[qt, kt] = 0 if kept == 0 else (1 if kept == total else 2)
    return out


def _tiny_descs():
    return [W.mask_all(), W.mask_spatial(1), W.mask_temporal(1), W.mask_box(0, 1, 2, 0),
            W.mask_stripe(1, 1, 3, 2, 1, 5, 1), W.mask_stripe(2, 0, 2, 1, 0, 4, 0),
            W.mask_sta(1, 2, 1, 0), W.mask_sta(3, 1, 2, 1)]


@pytest.mark.parametrize("di", range(8))
@pytest.mark.parametrize("Bq,Bk", [(8, 8), (16, 4), (7, 12)])
def test_classify_matches_bruteforce(di, Bq, Bk):
    desc = _tiny_descs()[di]
    g = W.grid(4, 4, 6, (2, 2, 3))
    layout = "tile" if desc["kind"] == "sta" else "frame"
    res = oracle.classify(g, layout, desc, Bq, Bk)
    assert np.array_equal(res["cls"], _brute_classes(desc, g, layout, Bq, Bk))
    for row, f, b in zip(res["cls"], res["full"], res["bnd"]):
        assert list(f) == [j for j in range(len(row)) if row[j] == 1]
        assert list(b) == [j for j in range(len(row)) if row[j] == 2]


def test_classify_tiny_workload_counts():
    """4x8x8 grid, 32x32 tiles: spatial 48 full / 0 boundary / 16 empty, temporal
    16 / 48 / 0, all-keep 64 / 0 / 0 (derived by frame-pair counting: frame 0 keys
    are full for every query; spatial keeps 2+3+3+2 key frames plus the sink)."""
    cfg = W.config("tiny")
    expect = [(48, 0, 16), (16, 48, 0), (64, 0, 0)]
    for desc, (nf, nb, ne) in zip(cfg["masks"] + [W.mask_all()], expect):
        cls = oracle.classify(cfg["grid"], "frame", desc, 32, 32)["cls"]
        assert (np.count_nonzero(cls == 1), np.count_nonzero(cls == 2),
                np.count_nonzero(cls == 0)) == (nf, nb, ne)


def test_classify_padding_never_full():
    g = W.grid(3, 3, 3)  # S = 27
    cls = oracle.classify(g, "frame", W.mask_all(), 8, 8)["cls"]
    assert cls.shape == (4, 4)
    assert np.all(cls[:3, :3] == oracle.FULL)
    assert np.all(cls[3, :] == oracle.BOUNDARY) and np.all(cls[:, 3] == oracle.BOUNDARY)


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------
def _py_attention(q, k, v, keep, scale):
    """Pure-Python masked softmax attention (math.exp, explicit loops)."""
    n, D = q.shape
    S = k.shape[0]
    out = []
    for i in range(n):
        s = [sum(q[i, d] * k[j, d] for d in range(D)) * scale for j in range(S)]
        kept = [j for j in range(S) if keep[i, j]]
        if not kept:
            out.append([0.0] * D)
            continue
        m = max(s[j] for j in kept)
        w = {j: math.exp(s[j] - m) for j in kept}
        z = sum(w.values())
        out.append([sum(w[j] * v[j, d] for j in kept) / z for d in range(D)])
    return np.array(out)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_all_keep_equals_python_loop():
    g = W.grid(2, 2, 3)
    q, k, v = (_rand((1, 12, 1, 4), s) for s in (1, 2, 3))
    o, _ = oracle.attention(q, k, v, g, "frame", [W.mask_all()])
    ref = _py_attention(q[0, :, 0], k[0, :, 0], v[0, :, 0], np.ones((12, 12), bool), 0.5)
    assert np.allclose(o[0, :, 0], ref, atol=1e-13, rtol=0)


def test_all_keep_equals_torch_sdpa():
    import torch
    g = W.grid(4, 8, 8)
    q, k, v = (_rand((1, 256, 2, 64), s) for s in (4, 5, 6))
    o, _ = oracle.attention(q, k, v, g, "frame", [W.mask_all()] * 2)
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1, 3))) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).numpy().transpose(0, 2, 1, 3)
    assert np.abs(o - ref).max() < 1e-12


@pytest.mark.parametrize("di", range(8))
def test_masked_equals_python_loop(di):
    desc = _tiny_descs()[di]
    g = W.grid(4, 2, 3, (2, 1, 3))
    layout = "tile" if desc["kind"] == "sta" else "frame"
    S = 24
    q, k, v = (_rand((1, S, 1, 3), 10 + s) for s in range(3))
    o, _ = oracle.attention(q, k, v, g, layout, [desc], scale=0.7)
    c = token_coords(g, layout, np.arange(S))
    keep = keep_matrix(desc, g, c, c)
    ref = _py_attention(q[0, :, 0], k[0, :, 0], v[0, :, 0], keep, 0.7)
    assert np.allclose(o[0, :, 0], ref, atol=1e-13, rtol=0)


def test_rows_sum_to_one():
    """V = 1 gives O = sum of the softmax row = 1 for every row with a kept key."""
    g = W.grid(5, 4, 4)
    q, k = _rand((1, 80, 2, 8), 7), _rand((1, 80, 2, 8), 8)
    v = np.ones((1, 80, 2, 8))
    o, _ = oracle.attention(q, k, v, g, "frame", [W.mask_temporal(1), W.mask_stripe(2, 1, 3, 2, 0, 5)])
    assert np.abs(o - 1.0).max() < 1e-12


def test_zero_query_gives_mean_of_kept_values():
    g = W.grid(4, 3, 3)
    S = 36
    q = np.zeros((1, S, 1, 4))
    k, v = _rand((1, S, 1, 4), 9), _rand((1, S, 1, 4), 10)
    desc = W.mask_box(1, 1, 0, sink_frames=1)
    o, lse = oracle.attention(q, k, v, g, "frame", [desc])
    c = token_coords(g, "frame", np.arange(S))
    keep = keep_matrix(desc, g, c, c)
    for i in range(S):
        assert np.allclose(o[0, i, 0], v[0, keep[i], 0].mean(axis=0), atol=1e-14)
        assert abs(lse[0, 0, i] - math.log(keep[i].sum())) < 1e-13


def test_self_only_stripe_is_identity():
    g = W.grid(3, 4, 5)
    S = 60
    q, k, v = (_rand((2, S, 1, 6), 20 + s) for s in range(3))
    desc = W.mask_stripe(1, 0, 10, 1, 0, 100, sink_frames=0)
    o, lse = oracle.attention(q, k, v, g, "frame", [desc], scale=0.3)
    assert np.array_equal(o[:, :, 0], v[:, :, 0])
    assert np.allclose(lse[:, 0], 0.3 * np.einsum("bsd,bsd->bs", q[:, :, 0], k[:, :, 0]), atol=1e-14)


def test_empty_rows_are_zero():
    g = W.grid(3, 2, 2)
    q, k, v = (_rand((1, 12, 1, 4), 30 + s) for s in range(3))
    desc = W.mask_stripe(1, 5, 99, 4, 0, 4, sink_frames=0)  # dt = 5 never happens
    o, lse = oracle.attention(q, k, v, g, "frame", [desc])
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_partial_results_merge_by_lse():
    """Attention over two disjoint key sets, merged with their log-sum-exp, equals
    attention over the union (DSA guide, section 18)."""
    g = W.grid(6, 3, 4)
    S = 72
    q, k, v = (_rand((1, S, 1, 8), 40 + s) for s in range(3))
    even = W.mask_stripe(1, 0, 2, 12, 0, 12, sink_frames=0)  # key frames with even dt
    odd = W.mask_stripe(1, 1, 2, 12, 0, 12, sink_frames=0)   # |dt - 1| even: odd dt
    oa, la = oracle.attention(q, k, v, g, "frame", [even])
    ob, lb = oracle.attention(q, k, v, g, "frame", [odd])
    o, l = oracle.attention(q, k, v, g, "frame", [W.mask_all()])
    lm = np.logaddexp(la, lb)
    merged = (np.exp(la - lm)[0, 0, :, None] * oa[0, :, 0] + np.exp(lb - lm)[0, 0, :, None] * ob[0, :, 0])
    assert np.abs(merged - o[0, :, 0]).max() < 1e-13
    assert np.abs(lm - l).max() < 1e-13


def _dt_classes(g, parts):
    """Stripe masks keeping key frames with dt = r (mod parts), r = 0..parts-1, no sink."""
    return [W.mask_stripe(1, r, parts, 1, 0, 1, sink_frames=0) for r in range(parts)]


def test_merge_partials_equals_attention_over_union():
    """oracle.merge_partials over a partition of the keys (dt mod 3) equals attention
    over all keys (DSA guide, section 18), for every row and head."""
    g = W.grid(7, 3, 4)
    S = W.seq_len(g)
    q, k, v = (_rand((2, S, 2, 8), 50 + s) for s in range(3))
    classes = _dt_classes(g, 3)
    c = token_coords(g, "frame", np.arange(S))
    keeps = [keep_matrix(m, g, c, c) for m in classes]
    assert np.all(sum(kp.astype(int) for kp in keeps) == 1)  # a partition of all pairs
    parts = [oracle.attention(q, k, v, g, "frame", [m, m]) for m in classes]
    o, l = oracle.merge_partials([p[0] for p in parts], [p[1] for p in parts])
    ref_o, ref_l = oracle.attention(q, k, v, g, "frame", [W.mask_all(), W.mask_all()])
    assert np.abs(o - ref_o).max() < 1e-13 and np.abs(l - ref_l).max() < 1e-13
    # any order of arrival gives the same result
    o2, l2 = oracle.merge_partials([parts[i][0] for i in (2, 0, 1)], [parts[i][1] for i in (2, 0, 1)])
    assert np.abs(o2 - o).max() < 1e-14 and np.abs(l2 - l).max() < 1e-14


def test_merge_partials_special_cases():
    rng = np.random.default_rng(7)
    B, S, H, D = 1, 6, 2, 4
    o1 = rng.standard_normal((B, S, H, D))
    l1 = rng.standard_normal((B, H, S))
    # one part: identity
    o, l = oracle.merge_partials([o1], [l1])
    assert np.array_equal(o, o1) and np.array_equal(l, l1)
    # a part merged with itself: same output, lse + ln 2
    o, l = oracle.merge_partials([o1, o1], [l1, l1])
    assert np.abs(o - o1).max() < 1e-15 and np.abs(l - (l1 + math.log(2))).max() < 1e-15
    # an empty part (lse = -inf) adds nothing, whatever its output holds
    junk = np.full_like(o1, np.nan)
    o, l = oracle.merge_partials([o1, junk], [l1, np.full_like(l1, -np.inf)])
    assert np.array_equal(o, o1) and np.array_equal(l, l1)
    # all parts empty: o = 0, lse = -inf
    o, l = oracle.merge_partials([junk, junk], [np.full_like(l1, -np.inf)] * 2)
    assert np.all(o == 0) and np.all(np.isneginf(l))
    # two parts with known weights: lse 0 and ln 3 weigh 1 : 3
    o2 = rng.standard_normal((B, S, H, D))
    o, l = oracle.merge_partials([o1, o2], [np.zeros((B, H, S)), np.full((B, H, S), math.log(3))])
    assert np.abs(o - (0.25 * o1 + 0.75 * o2)).max() < 1e-15
    assert np.abs(l - math.log(4)).max() < 1e-15


def _brute_fraction(keep, S, Bq, Bk, qt, kt):
    r = range(qt * Bq, min(S, (qt + 1) * Bq))
    c = range(kt * Bk, min(S, (kt + 1) * Bk))
    kept = sum(int(keep[i, j]) for i in r for j in c)
    return kept, len(r) * len(c)


@pytest.mark.parametrize("gi", range(3))
def test_rounded_classes_follow_the_half_rule(gi):
    """Tile-aligned rounding (B3): full and empty tiles stay; a boundary tile keeps all
    of its real pairs iff at least half of them are kept; tiles reaching past S stay
    boundary when kept.  Checked pair by pair on small grids."""
    g, desc, Bq, Bk = [(W.grid(3, 5, 7), W.mask_box(1, 1, 2, sink_frames=1), 16, 16),
                       (W.grid(4, 6, 5), W.mask_stripe(1, 0, 2, 2, 1, 6, sink_frames=0), 32, 16),
                       (W.grid(2, 9, 9), W.mask_box(-1, 2, 2), 16, 32)][gi]
    S = W.seq_len(g)
    c = token_coords(g, "frame", np.arange(S))
    keep = keep_matrix(desc, g, c, c)
    exact = oracle.classify(g, "frame", desc, Bq, Bk)["cls"]
    rnd = oracle.classify(g, "frame", desc, Bq, Bk, round_tiles=True)["cls"]
    rk = oracle.rounded_keep_rows(g, "frame", desc, Bq, Bk, np.arange(S))
    for qt in range(rnd.shape[0]):
        for kt in range(rnd.shape[1]):
            kept, real = _brute_fraction(keep, S, Bq, Bk, qt, kt)
            padded = (qt + 1) * Bq > S or (kt + 1) * Bk > S
            on = kept > 0 and 2 * kept >= real
            want = (oracle.BOUNDARY if padded else oracle.FULL) if on else oracle.EMPTY
            assert rnd[qt, kt] == want
            if exact[qt, kt] != oracle.BOUNDARY:
                assert rnd[qt, kt] == exact[qt, kt] or (padded and exact[qt, kt] == oracle.FULL)
            block = rk[qt * Bq:min(S, (qt + 1) * Bq), kt * Bk:min(S, (kt + 1) * Bk)]
            assert np.all(block == on)


def test_rounding_threshold_is_one_half():
    """On a 1-D grid the stripe |dx| mod 2 == 0 keeps exactly half of every 4 x 4 tile
    (kept: rounds up); |dx| mod 3 == 0 keeps at most 6 of 16 (dropped)."""
    g = W.grid(1, 1, 16)
    half = W.mask_stripe(1, 0, 1, 1, 0, 2, sink_frames=0)
    third = W.mask_stripe(1, 0, 1, 1, 0, 3, sink_frames=0)
    c = token_coords(g, "frame", np.arange(16))
    kh = keep_matrix(half, g, c, c)
    assert all(kh[i * 4:(i + 1) * 4, j * 4:(j + 1) * 4].sum() == 8 for i in range(4) for j in range(4))
    assert np.all(oracle.classify(g, "frame", half, 4, 4, round_tiles=True)["cls"] == oracle.FULL)
    r3 = oracle.classify(g, "frame", third, 4, 4, round_tiles=True)["cls"]
    k3 = keep_matrix(third, g, c, c)
    for i in range(4):
        for j in range(4):
            n = k3[i * 4:(i + 1) * 4, j * 4:(j + 1) * 4].sum()
            assert r3[i, j] == (oracle.FULL if 2 * n >= 16 else oracle.EMPTY)
    assert np.all(r3 == oracle.EMPTY)  # no 4 x 4 tile keeps more than 6 of its 16 pairs


def test_rounding_leaves_tile_aligned_masks_unchanged():
    """A sliding-tile mask whose tiles coincide with the kernel tiles has no boundary
    tile, so rounding changes neither classes nor the attention output."""
    g = W.grid(4, 8, 8, (2, 4, 4))  # 32-token tiles, kernel tiles 32 x 32
    desc = W.mask_sta(1, 1, 1)
    ex = oracle.classify(g, "tile", desc, 32, 32)["cls"]
    assert not np.any(ex == oracle.BOUNDARY)
    assert np.array_equal(oracle.classify(g, "tile", desc, 32, 32, round_tiles=True)["cls"], ex)
    S = W.seq_len(g)
    q, k, v = (_rand((1, S, 1, 8), 60 + s) for s in range(3))
    o1, l1 = oracle.attention(q, k, v, g, "tile", [desc])
    o2, l2 = oracle.attention(q, k, v, g, "tile", [desc], round_tiles=(32, 32))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_position_major_order_by_hand():
    """Position-major order on a 3 x 2 x 2 grid: frame 0 first (row-major), then for
    each spatial position its frames 1 and 2 (written out from the definition)."""
    g = W.grid(3, 2, 2)
    perm = oracle.layout_permutation(g, "position")
    assert list(perm) == [0, 1, 2, 3, 4, 8, 5, 9, 6, 10, 7, 11]


@pytest.mark.parametrize("T,Hg,Wg", [(1, 3, 5), (2, 4, 3), (5, 3, 7), (21, 2, 3)])
def test_position_major_is_a_permutation(T, Hg, Wg):
    g = W.grid(T, Hg, Wg)
    S = T * Hg * Wg
    perm = oracle.layout_permutation(g, "position")
    assert np.array_equal(np.sort(perm), np.arange(S))
    if T <= 2:  # the frame-0 block followed by one frame in spatial order is frame-major
        assert np.array_equal(perm, np.arange(S))
    t, y, x = oracle.token_coords(g, "position", np.arange(S))
    assert np.all(t[: Hg * Wg] == 0)
    if T > 1:  # after the leading block, consecutive positions step through frames
        tt = t[Hg * Wg:].reshape(Hg * Wg, T - 1)
        assert np.all(tt == np.arange(1, T)[None, :])


def test_position_major_attention_matches_frame_major():
    """Attention depends on coordinates only: permuting inputs into position-major
    order and attending there gives the permuted frame-major result."""
    g = W.grid(4, 3, 3)
    S = W.seq_len(g)
    q, k, v = (_rand((1, S, 2, 8), 70 + s) for s in range(3))
    masks = [W.mask_temporal(1), W.mask_stripe(1, 0, 2, 2, 1, 4)]
    ref, ref_l = oracle.attention(q, k, v, g, "frame", masks)
    perm = oracle.layout_permutation(g, "position")
    o, l = oracle.attention(q[:, perm], k[:, perm], v[:, perm], g, "position", masks)
    assert np.abs(o - ref[:, perm]).max() < 1e-13
    assert np.abs(l - ref_l[:, :, perm]).max() < 1e-13


def test_position_major_turns_temporal_stripes_into_full_tiles():
    """A temporal head (same position across frames, plus the frame-0 sink) has a
    boundary tile per frame in every query tile in frame-major order, and none outside
    the sink block's query tiles in position-major order (Sparse VideoGen on TPU,
    arranging tokens for temporal access)."""
    g = W.grid(9, 4, 8)  # 32 positions x 8 frames after the sink block
    desc = W.mask_box(-1, 0, 0, sink_frames=1)
    fr = oracle.classify(g, "frame", desc, 8, 8)["cls"]
    po = oracle.classify(g, "position", desc, 8, 8)["cls"]
    assert np.all((fr == oracle.BOUNDARY).sum(axis=1) == 8)  # 8 frames, one partial tile each
    # in position-major order every query tile (8 frames of one position) keeps the
    # sink block (4 full tiles) and its own 8-frame tile: full tiles only
    assert not np.any(po[4:] == oracle.BOUNDARY)
    assert np.all((po[4:] == oracle.FULL).sum(axis=1) == 5)


def test_tile_major_equals_frame_major_after_inverse():
    g = W.grid(4, 4, 6, (2, 2, 3))
    S = 96
    q, k, v = (_rand((1, S, 2, 4), 50 + s) for s in range(3))
    masks = [W.mask_sta(1, 1, 1), W.mask_temporal(1)]
    o_f, _ = oracle.attention(q, k, v, g, "frame", masks)
    qt, kt, vt = (oracle.reorder_tokens(x, g) for x in (q, k, v))
    o_t, _ = oracle.attention(qt, kt, vt, g, "tile", masks)
    assert np.abs(oracle.reorder_tokens(o_t, g, inverse=True) - o_f).max() < 1e-13


# ---------------------------------------------------------------------------
# profiler: inputs with a known answer
# ---------------------------------------------------------------------------
def _coded_inputs(g, H, D, by, alpha, seed):
    """K = Q = alpha * code, with one random unit code per spatial position (shared
    across frames) or per frame; V random."""
    rng = np.random.default_rng(seed)
    S = W.seq_len(g)
    t, y, x = token_coords(g, "frame", np.arange(S))
    key = (y * g["Wg"] + x) if by == "position" else t
    n_codes = key.max() + 1
    codes = rng.standard_normal((n_codes, H, D))
    codes /= np.linalg.norm(codes, axis=-1, keepdims=True)
    qk = alpha * codes[key][None]
    return qk, qk.copy(), rng.standard_normal((1, S, H, D))


@pytest.mark.parametrize("by,winner", [("position", 2), ("frame", 1)])
def test_profiler_known_winner(by, winner):
    g = W.grid(8, 12, 12)
    q, k, v = _coded_inputs(g, 2, 32, by, 8.0, 3)
    S = W.seq_len(g)
    idx = W.sample_rows(S, 24, 2, 5)
    cands = [W.mask_all(), W.mask_spatial(1), W.mask_temporal(4)]
    err, route = oracle.profile_heads(q, k, v, g, "frame", idx, cands)
    assert np.all(route == winner)
    assert np.all(err[:, 0] == 0)


def test_profiler_iid_inputs_prefer_spatial_and_ties():
    g = W.grid(6, 12, 12)
    q, k, v = (_rand((1, 864, 1, 8), 60 + s) for s in range(3))
    idx = W.sample_rows(864, 16, 1, 0)
    _, route = oracle.profile_heads(q, k, v, g, "frame", idx,
                                    [W.mask_all(), W.mask_spatial(1), W.mask_temporal(2)])
    assert route[0] == 1
    _, route = oracle.profile_heads(q, k, v, g, "frame", idx,
                                    [W.mask_all(), W.mask_temporal(2), W.mask_temporal(2)])
    assert route[0] == 1


# ---------------------------------------------------------------------------
# 3D padding (PSA notes, key design 2 and the worked example)
# ---------------------------------------------------------------------------
def test_padded_dims_of_the_psa_example():
    """The worked example pads Wan 2.1's 21 x 45 x 80 latent to 21 x 48 x 80 for a
    3 x 8 x 16 block (only H changes: 45 -> 48)."""
    g = W.grid(21, 45, 80, (3, 8, 16))
    assert oracle.padded_dims(g) == (21, 48, 80)
    assert oracle.seq_len(g, "padded") == 21 * 48 * 80
    assert oracle.seq_len(g, "frame") == 75600


def test_padded_order_by_hand():
    """1 x 3 x 3 grid, 1 x 2 x 2 tiles: padded to 1 x 4 x 4 and cut into 2 x 2 tiles,
    tiles row-major, tokens row-major inside a tile; -1 marks padding (written out
    from the definition)."""
    g = W.grid(1, 3, 3, (1, 2, 2))
    perm = oracle.layout_permutation(g, "padded")
    assert list(perm) == [0, 1, 3, 4, 2, -1, 5, -1, 6, 7, -1, -1, 8, -1, -1, -1]


@pytest.mark.parametrize("T,Hg,Wg,tile", [(3, 5, 7, (2, 2, 4)), (4, 4, 6, (2, 2, 3)), (1, 3, 3, (1, 2, 2)),
                                          (5, 9, 2, (3, 4, 1))])
def test_padded_order_is_an_injection(T, Hg, Wg, tile):
    g = W.grid(T, Hg, Wg, tile)
    perm = oracle.layout_permutation(g, "padded")
    S = T * Hg * Wg
    real = perm[perm >= 0]
    assert np.array_equal(np.sort(real), np.arange(S))
    assert len(perm) - len(real) == oracle.seq_len(g, "padded") - S
    if T % tile[0] == 0 and Hg % tile[1] == 0 and Wg % tile[2] == 0:
        assert np.array_equal(perm, oracle.layout_permutation(g, "tile"))
    # round trip through the padded order, padding rows zero
    x = _rand((2, S, 3), 90)
    y = oracle.reorder_tokens(x, g, layout="padded")
    assert np.all(y[:, perm < 0] == 0)
    assert np.array_equal(oracle.reorder_tokens(y, g, inverse=True, layout="padded"), x)


def _padded_order_brute(g):
    """(t, y, x) of the padded order by nested loops: tiles row-major over the padded
    tile grid, tokens row-major inside a tile."""
    bt, bh, bw = g["tile_t"], g["tile_h"], g["tile_w"]
    nT, nH, nW = (-(-g["T"] // bt), -(-g["Hg"] // bh), -(-g["Wg"] // bw))
    out = []
    for a, b, c in itertools.product(range(nT), range(nH), range(nW)):
        for i, j, l in itertools.product(range(bt), range(bh), range(bw)):
            out.append((a * bt + i, b * bh + j, c * bw + l))
    return out


@pytest.mark.parametrize("desc", [W.mask_box(1, 1, 2, sink_frames=1), W.mask_all(), W.mask_sta(1, 2, 1),
                                  W.mask_stripe(1, 0, 2, 2, 1, 5)])
def test_padded_classes_by_brute_force(desc):
    """Classes over the padded order from pair-by-pair loops: padding pairs are never
    kept, so a tile holding padding is never FULL."""
    g = W.grid(3, 5, 7, (2, 2, 4))
    pos = _padded_order_brute(g)
    S = len(pos)
    assert S == oracle.seq_len(g, "padded") == 4 * 6 * 8
    real = [t < 3 and y < 5 and x < 7 for t, y, x in pos]
    Bq, Bk = 16, 12
    nQ, nK = -(-S // Bq), -(-S // Bk)

    def kept(i, j):
        if not (real[i] and real[j]):
            return False
        (tq, yq, xq), (tk, yk, xk) = pos[i], pos[j]
        return bool(keep_matrix(desc, g, ([tq], [yq], [xq]), ([tk], [yk], [xk]))[0, 0])

    got = oracle.classify(g, "padded", desc, Bq, Bk)["cls"]
    for qt in range(nQ):
        for kt in range(nK):
            n = sum(kept(i, j) for i in range(qt * Bq, min(S, qt * Bq + Bq))
                    for j in range(kt * Bk, min(S, kt * Bk + Bk)))
            ref = oracle.EMPTY if n == 0 else (oracle.FULL if n == Bq * Bk else oracle.BOUNDARY)
            assert got[qt, kt] == ref, (qt, kt, n)


def test_padded_sliding_tiles_are_full_or_empty_away_from_padding():
    """Sliding tiles with kernel tiles equal to the 3D tiles: a tile pair of real tokens
    only is full or empty, and a pair holding padding is never full."""
    g = W.grid(5, 6, 10, (2, 4, 4))  # padded to 6 x 8 x 12: 3 x 2 x 3 tiles of 32
    desc = W.mask_sta(3, 1, 3)
    cls = oracle.classify(g, "padded", desc, 32, 32)["cls"]
    perm = oracle.layout_permutation(g, "padded")
    tile_real = (perm.reshape(-1, 32) >= 0).all(axis=1)
    both = tile_real[:, None] & tile_real[None, :]
    assert not np.any(cls[both] == oracle.BOUNDARY)
    assert not np.any(cls[~both] == oracle.FULL)


def test_padded_attention_matches_frame_major():
    """Attention in the padded order with zero padding rows equals frame-major
    attention on the real rows: padding keys carry no weight."""
    g = W.grid(3, 5, 7, (2, 2, 4))
    S = 105
    q, k, v = (_rand((1, S, 2, 8), 95 + s) for s in range(3))
    masks = [W.mask_box(1, 2, 2, sink_frames=1), W.mask_sta(1, 1, 1)]
    ref, ref_l = oracle.attention(q, k, v, g, "frame", masks)
    qp, kp, vp = (oracle.reorder_tokens(x, g, layout="padded") for x in (q, k, v))
    o, l = oracle.attention(qp, kp, vp, g, "padded", masks)
    perm = oracle.layout_permutation(g, "padded")
    real = perm >= 0
    assert np.abs(oracle.reorder_tokens(o, g, inverse=True, layout="padded") - ref).max() < 1e-13
    assert np.abs(l[:, :, real] - ref_l[:, :, perm[real]]).max() < 1e-13


def test_padded_rounding_counts_real_pairs_only():
    """B3 rounding on the padded order: a tile keeps its real pairs iff at least half of
    its real pairs are kept (padding inside the tile is not counted)."""
    g = W.grid(3, 5, 7, (2, 2, 4))
    desc = W.mask_box(0, 1, 1)
    Bq, Bk = 16, 16
    pos = _padded_order_brute(g)
    S = len(pos)
    real = np.array([t < 3 and y < 5 and x < 7 for t, y, x in pos])
    t, y, x = (np.array(c) for c in zip(*pos))
    keep = keep_matrix(desc, g, (t, y, x), (t, y, x)) & real[:, None] & real[None, :]
    ex = oracle.classify(g, "padded", desc, Bq, Bk)["cls"]
    rd = oracle.classify(g, "padded", desc, Bq, Bk, round_tiles=True)["cls"]
    for qt in range(S // Bq):
        for kt in range(S // Bk):
            blk = keep[qt * Bq:(qt + 1) * Bq, kt * Bk:(kt + 1) * Bk]
            n_real = real[qt * Bq:(qt + 1) * Bq].sum() * real[kt * Bk:(kt + 1) * Bk].sum()
            has_pad = n_real < Bq * Bk
            if ex[qt, kt] != oracle.BOUNDARY:
                assert rd[qt, kt] == ex[qt, kt]
            elif 2 * blk.sum() >= n_real:
                assert rd[qt, kt] == (oracle.BOUNDARY if has_pad else oracle.FULL)
            else:
                assert rd[qt, kt] == oracle.EMPTY
    rows = np.arange(S)
    rk = oracle.rounded_keep_rows(g, "padded", desc, Bq, Bk, rows)
    assert not rk[~real].any() and not rk[:, ~real].any()


def test_padded_sta_window_of_one_tile_is_block_diagonal():
    """A 1 x 1 x 1 sliding window keeps exactly the pairs inside one 3D tile, also for
    the partial tiles at the padded edges (the window counts the padded tiles)."""
    g = W.grid(5, 3, 7, (2, 2, 4))  # partial tiles on every axis
    S = W.seq_len(g)
    t, y, x = token_coords(g, "frame", np.arange(S))
    keep = keep_matrix(W.mask_sta(1, 1, 1), g, (t, y, x), (t, y, x))
    tile = (t // 2) * 100 + (y // 2) * 10 + (x // 4)
    assert np.array_equal(keep, tile[:, None] == tile[None, :])
