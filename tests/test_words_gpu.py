"""Precomputed element masks of boundary tiles on the GPU: the words are bit-exact
against the oracle's keep predicate, entries past the lists are left alone, and the
bf16 forward that reads them gives exactly the output of the forward that derives the
masks itself (tables holding every list, tables cut short, and the forced-mask ablation)."""
import numpy as np
import pytest
import torch

import block_sparse_spatio_amd as vsa
import oracle
import workloads as W
from tests.gpu_helpers import dev, say

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A5A5A5A

# bit b of lane half g2's word <-> key of the 64-key tile (the forward's score registers)
_KEY_OF_BIT = np.array([[(b >> 4) * 32 + ((b >> 3) & 1) * 16 + 8 * g2 + (b & 7) for b in range(32)]
                        for g2 in range(2)])


def _random_mask(rng, tiled):
    kinds = ["all", "box", "box", "stripe", "stripe"] + (["sta", "sta"] if tiled else [])
    kind = kinds[rng.integers(len(kinds))]
    sink = int(rng.integers(0, 3))
    if kind == "all":
        return W.mask_all()
    if kind == "box":
        r = lambda: int(rng.integers(-1, 5))  # noqa: E731
        return W.mask_box(r(), r(), r(), sink_frames=sink)
    if kind == "stripe":
        return W.mask_stripe(int(rng.integers(1, 4)), int(rng.integers(-2, 3)), int(rng.integers(1, 6)),
                             int(rng.integers(1, 6)), int(rng.integers(-3, 4)), int(rng.integers(1, 60)),
                             sink_frames=sink)
    return W.mask_sta(int(rng.integers(1, 4)), int(rng.integers(1, 4)), int(rng.integers(1, 4)), sink_frames=sink)


def _case(seed):
    """Grids of several query tiles with ragged tails; every mask kind; per-head orders
    or the padded grid."""
    rng = np.random.default_rng(9100 + seed)
    tiled = rng.random() < 0.5
    tile = tuple(int(x) for x in rng.integers(1, 5, 3)) if tiled else (0, 0, 0)
    dims = [int(rng.integers(2, 8)), int(rng.integers(3, 17)), int(rng.integers(3, 29))]
    if tiled and rng.random() < 0.5:
        dims = [max(1, d // b) * b for d, b in zip(dims, tile)]
    g = W.grid(*dims, tile)
    divides = tiled and all(d % b == 0 for d, b in zip(dims, tile))
    padded = tiled and not divides
    H = int(rng.integers(1, 5))
    masks = [_random_mask(rng, divides or padded) for _ in range(H)]
    if padded:
        layout = "padded"
    else:
        layout = "tile" if divides and rng.random() < 0.5 else "frame"
        orders = ["frame", "position"] + (["tile"] if divides else [])
        masks = [m if rng.random() < 0.4 else W.with_head_layout(m, orders[rng.integers(len(orders))])
                 for m in masks]
    Bq = int(rng.choice([64, 128, 256]))
    D = int(rng.choice([64, 128]))
    return g, layout, masks, Bq, D


def _words(g, layout, masks, tiles, cap):
    """A word table pre-filled with a sentinel; cap="compact" for the compact table."""
    if cap == "compact":
        n = max(1, int(tiles["bnd_offs"][-1]))
        out = torch.full((n, tiles["Bq"] // 32, 64), SENTINEL, dtype=torch.int32, device=dev())
    else:
        out = torch.full((tiles["n_unique"], tiles["nQ"], cap, tiles["Bq"] // 32, 64), SENTINEL, dtype=torch.int32,
                         device=dev())
    return vsa.vsa_boundary_words(g, layout, masks, tiles, cap=cap, out=out)


def _check_words(g, layout, masks, tiles, words):
    """Every written word against the oracle's keep predicate; the rest untouched."""
    hm, U = vsa.vsa_unique_masks(masks)
    lays = W.head_layouts(masks, layout)
    S = oracle.seq_len(g, layout)
    Bq, nQ, nK, cap = tiles["Bq"], tiles["nQ"], tiles["nK"], words["cap"]
    n_bnd = tiles["n_bnd"].cpu().numpy()
    bnd_idx = tiles["bnd_idx"].cpu().numpy()
    compact = cap == vsa.VSA_WORDS_COMPACT
    if compact:
        # list row r owns entries [offs[r], offs[r] + n_bnd[r]) of the table
        offs = tiles["bnd_offs"].cpu().numpy()
        assert offs[0] == 0 and np.array_equal(np.diff(offs), n_bnd.reshape(-1)), "bnd_offs is not the prefix sum"
        flat = words["words"].cpu().numpy().view(np.uint32)
        assert flat.shape[0] == max(1, int(offs[-1]))
        if offs[-1] == 0:
            assert np.all(flat == SENTINEL)
        w_all = None
    else:
        w_all = words["words"].cpu().numpy().view(np.uint32)
    cols = np.arange(S)
    checked = 0
    for u in range(U):
        h = hm.index(u)
        lay, desc = lays[h], masks[h]
        ck = oracle.token_coords(g, lay, cols)
        col_real = oracle.is_real(g, *ck)
        for qt in range(nQ):
            rows = np.arange(qt * Bq, min(S, (qt + 1) * Bq))
            cq = oracle.token_coords(g, lay, rows)
            keep = np.zeros((len(rows), nK * 64), dtype=bool)
            keep[:, :S] = oracle.keep_matrix(desc, g, cq, ck) & col_real[None, :]
            real_rows = oracle.is_real(g, *cq)
            nb = int(n_bnd[u, qt]) if compact else min(int(n_bnd[u, qt]), cap)
            for j in range(nb):
                kt = int(bnd_idx[u, qt, j])
                bits = keep[:, kt * 64:(kt + 1) * 64][:, _KEY_OF_BIT]  # [rows, 2, 32]
                want = (bits.astype(np.uint64) << np.arange(32, dtype=np.uint64)).sum(-1).astype(np.uint32)
                r = np.arange(len(rows))
                ent = flat[offs[u * nQ + qt] + j] if compact else w_all[u, qt, j]
                got = np.stack([ent[r // 32, g2 * 32 + r % 32] for g2 in range(2)], axis=1)
                bad = np.nonzero((got != want).any(axis=1) & real_rows)[0]
                assert bad.size == 0, (f"mask {u} query tile {qt} entry {j} (key tile {kt}): row "
                                       f"{rows[bad[0]]} words {got[bad[0]]} expected {want[bad[0]]}")
                checked += 1
            if not compact:
                assert np.all(w_all[u, qt, nb:] == SENTINEL), f"mask {u} query tile {qt}: entries past {nb} written"
    return checked


@pytest.mark.parametrize("seed", range(16))
def test_words_match_oracle(gpu_lib, seed):
    g, layout, masks, Bq, D = _case(seed)
    say(f"words seed={seed} grid={g} layout={layout} Bq={Bq} masks={masks}")
    tiles = vsa.vsa_classify_tiles(g, layout, masks, Bq, 64, device=dev(), with_cls=False)
    cap = max(1, int(tiles["n_bnd"].max()))
    words = _words(g, layout, masks, tiles, cap)
    torch.cuda.synchronize()
    _check_words(g, layout, masks, tiles, words)
    # a table cut short writes only its first entries
    short = _words(g, layout, masks, tiles, max(1, cap // 2))
    torch.cuda.synchronize()
    _check_words(g, layout, masks, tiles, short)
    # the compact table: exactly one entry per listed boundary tile, every one written
    compact = _words(g, layout, masks, tiles, "compact")
    torch.cuda.synchronize()
    assert compact["cap"] == vsa.VSA_WORDS_COMPACT
    _check_words(g, layout, masks, tiles, compact)


@pytest.mark.parametrize("seed", range(8))
def test_words_frame_major_stripes(gpu_lib, seed):
    """Stripe heads in frame-major order on frames of at least 64 tokens (the kernel's
    shortcut through the position difference, frame crossings inside query and key
    tiles, sink frames, ragged tails): every word against the oracle."""
    rng = np.random.default_rng(9200 + seed)
    while True:
        dims = [int(rng.integers(1, 7)), int(rng.integers(2, 20)), int(rng.integers(2, 30))]
        if dims[1] * dims[2] >= 64:
            break
    g = W.grid(*dims)
    masks = [W.mask_stripe(int(rng.integers(1, 4)), int(rng.integers(-2, 3)), int(rng.integers(1, 6)),
                           int(rng.integers(1, 6)), int(rng.integers(-3, 4)), int(rng.integers(1, 120)),
                           sink_frames=int(rng.integers(0, 3))) for _ in range(int(rng.integers(1, 5)))]
    Bq = int(rng.choice([64, 128, 256]))
    say(f"frame-major stripe words seed={seed} grid={g} Bq={Bq} masks={masks}")
    tiles = vsa.vsa_classify_tiles(g, "frame", masks, Bq, 64, device=dev(), with_cls=False)
    words = _words(g, "frame", masks, tiles, "compact")
    torch.cuda.synchronize()
    assert _check_words(g, "frame", masks, tiles, words) == int(tiles["bnd_offs"][-1])


@pytest.mark.parametrize("seed", range(16))
def test_forward_with_words_is_identical(gpu_lib, seed):
    g, layout, masks, Bq, D = _case(seed)
    lays = W.head_layouts(masks, layout)
    reorder = any(x != "frame" for x in lays) and seed % 2 == 0
    force = seed % 4 == 3
    flags = (vsa.VSA_FWD_REORDER_IO if reorder else 0) | (vsa.VSA_FWD_FORCE_MASK if force else 0) \
        | vsa.VSA_FWD_WRITE_LSE
    H = len(masks)
    S_io = W.seq_len(g) if reorder else vsa.vsa_seq_len(g, layout)
    say(f"words forward seed={seed} grid={g} layout={layout} heads={lays} Bq={Bq} D={D} force={force} "
        f"reorder={reorder} masks={masks}")
    q, k, v = (x.to(dev()) for x in W.qkv(1, S_io, H, D, "bf16", seed=9300 + seed))
    tiles = vsa.vsa_classify_tiles(g, layout, masks, Bq, 64, device=dev(), with_cls=False)
    o0, l0 = vsa.vsa_sparse_attn_fwd(q, k, v, g, layout, masks, tiles, flags=flags)
    cap = max(1, int(tiles["n_bnd"].max()))
    # nK and the longest list: every workgroup's list fits (the instance without any mask
    # arithmetic); shorter tables mix it with workgroups that derive the masks past the cap
    for c in sorted({tiles["nK"], cap, max(1, cap // 2), 1}) + ["compact"]:
        words = _words(g, layout, masks, tiles, c)
        o1, l1 = vsa.vsa_sparse_attn_fwd(q, k, v, g, layout, masks, tiles, flags=flags, words=words)
        torch.cuda.synchronize()
        if layout == "padded" and not reorder:  # padding rows are unspecified
            real = torch.from_numpy(oracle.is_real(g, *oracle.token_coords(g, "padded",
                                                                          np.arange(S_io)))).to(dev())
            o0r, o1r = o0[:, real], o1[:, real]
            l0r, l1r = l0[:, :, real], l1[:, :, real]
        else:
            o0r, o1r, l0r, l1r = o0, o1, l0, l1
        assert torch.equal(o0r.view(torch.int16), o1r.view(torch.int16)), f"cap={c}: outputs differ"
        assert torch.equal(l0r.view(torch.int32), l1r.view(torch.int32)), f"cap={c}: lse differ"


@pytest.mark.parametrize("name", ["wan_mixed", "stripe_route", "wan_sta_padded"])
def test_forward_with_words_full_config(gpu_lib, name):
    """Full-size workloads: the forward reading the table equals the one deriving the masks."""
    cfg = W.config(name)
    g, layout, masks = cfg["grid"], cfg["layout"], cfg["masks"]
    B, H, D, Bq = cfg["B"], cfg["H"], cfg["D"], cfg["Bq"]
    S = vsa.vsa_seq_len(g, layout)
    say(f"words full config {name}: B={B} S={S} H={H} D={D} Bq={Bq}")
    q, k, v = (x.to(dev()) for x in W.qkv(B, S, H, D, "bf16", seed=cfg["seed"]))
    tiles = vsa.vsa_classify_tiles(g, layout, masks, Bq, cfg["Bk"], device=dev(), with_cls=False)
    o0, _ = vsa.vsa_sparse_attn_fwd(q, k, v, g, layout, masks, tiles)
    cap = max(1, int(tiles["n_bnd"].max()))
    words = vsa.vsa_boundary_words(g, layout, masks, tiles, cap=cap)
    o1, _ = vsa.vsa_sparse_attn_fwd(q, k, v, g, layout, masks, tiles, words=words)
    del words
    # the compact table (one entry per listed boundary tile), as the benchmark runs it
    full = vsa.vsa_boundary_words(g, layout, masks, tiles)
    say(f"compact table: {full['words'].numel() * 4 / 2**20:.1f} MiB for {int(tiles['bnd_offs'][-1])} entries")
    o2, _ = vsa.vsa_sparse_attn_fwd(q, k, v, g, layout, masks, tiles, words=full)
    torch.cuda.synchronize()
    if layout == "padded":
        real = torch.from_numpy(oracle.is_real(g, *oracle.token_coords(g, "padded", np.arange(S)))).to(dev())
        o0, o1, o2 = o0[:, real], o1[:, real], o2[:, real]
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(o0.view(torch.int16), o2.view(torch.int16))
