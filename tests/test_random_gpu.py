"""Seeded random combinations of the forward path on the GPU against the CPU oracle:
grid shapes with ragged tails, every mask kind, per-head token orders (frame-,
tile-, position-major) or the padded grid, both dtypes, tile sizes, batch and head
counts, the forced-mask ablation and tile-aligned (B3) lists.  Inputs and outputs are
frame-major (the call reorders), and the oracle runs each head in its own order."""
import numpy as np
import pytest
import torch

import block_sparse_spatio_amd as vsa
import oracle
import workloads as W
from tests.gpu_helpers import assert_close, dev, say

pytestmark = pytest.mark.gpu


def _random_mask(rng, tiled):
    kinds = ["all", "box", "stripe"] + (["sta"] if tiled else [])
    kind = kinds[rng.integers(len(kinds))]
    sink = int(rng.integers(0, 3))
    if kind == "all":
        return W.mask_all()
    if kind == "box":
        r = lambda: int(rng.integers(-1, 4))  # noqa: E731
        return W.mask_box(r(), r(), r(), sink_frames=sink)
    if kind == "stripe":
        return W.mask_stripe(int(rng.integers(1, 4)), int(rng.integers(-2, 3)), int(rng.integers(1, 6)),
                             int(rng.integers(1, 5)), int(rng.integers(-3, 4)), int(rng.integers(1, 40)),
                             sink_frames=sink)
    return W.mask_sta(int(rng.integers(1, 4)), int(rng.integers(1, 4)), int(rng.integers(1, 4)), sink_frames=sink)


def _case(seed):
    rng = np.random.default_rng(5000 + seed)
    tiled = rng.random() < 0.6
    tile = tuple(int(x) for x in rng.integers(1, 4, 3)) if tiled else (0, 0, 0)
    dims = [int(rng.integers(1, 7)), int(rng.integers(1, 10)), int(rng.integers(1, 13))]
    if tiled and rng.random() < 0.5:  # a grid of whole tiles
        dims = [max(1, d // b) * b for d, b in zip(dims, tile)]
    g = W.grid(*dims, tile)
    divides = tiled and g["T"] % tile[0] == 0 and g["Hg"] % tile[1] == 0 and g["Wg"] % tile[2] == 0
    H = int(rng.integers(1, 5))
    padded = tiled and rng.random() < 0.4
    # sliding-tile masks need whole tiles, or the padded grid
    masks = [_random_mask(rng, divides or padded) for _ in range(H)]
    if padded:
        layout = "padded"
    else:
        layout = "tile" if divides and rng.random() < 0.5 else "frame"
        orders = ["frame", "position"] + (["tile"] if divides else [])
        masks = [m if rng.random() < 0.4 else W.with_head_layout(m, orders[rng.integers(len(orders))])
                 for m in masks]
    dtype = "bf16" if rng.random() < 0.7 else "f32"
    if dtype == "bf16":
        Bq, Bk = int(rng.choice([64, 128, 256])), 64
    else:
        Bq, Bk = int(rng.choice([32, 64, 128])), int(rng.choice([32, 64]))
    D = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 3))
    force = rng.random() < 0.2
    rounded = (not force) and rng.random() < 0.3
    return g, layout, masks, dtype, Bq, Bk, D, B, force, rounded


def _oracle_head(q, k, v, g, lay, desc, h, round_tiles):
    """Oracle attention of head h in its own order, returned in frame-major order."""
    perm = oracle.layout_permutation(g, lay)
    real = perm >= 0
    qh, kh, vh = (oracle.reorder_tokens(x[:, :, h:h + 1].float().numpy(), g, layout=lay) for x in (q, k, v))
    o, lse = oracle.attention(qh, kh, vh, g, lay, [desc], round_tiles=round_tiles)
    S = W.seq_len(g)
    of = np.zeros((q.shape[0], S, q.shape[-1]))
    lf = np.zeros((q.shape[0], S))
    of[:, perm[real]] = o[:, real, 0]
    lf[:, perm[real]] = lse[:, 0, real]
    return of, lf


@pytest.mark.parametrize("seed", range(40))
def test_random_forward(gpu_lib, seed):
    g, layout, masks, dtype, Bq, Bk, D, B, force, rounded = _case(seed)
    S, H = W.seq_len(g), len(masks)
    lays = W.head_layouts(masks, layout)
    reorder = any(x != "frame" for x in lays)
    say(f"random forward seed={seed} grid={g} layout={layout} heads={lays} {dtype} Bq={Bq} Bk={Bk} D={D} B={B} "
        f"force={force} rounded={rounded} masks={masks}")
    q, k, v = W.qkv(B, S, H, D, dtype, seed=700 + seed)
    d = dev()
    tiles = vsa.vsa_classify_tiles(g, layout, masks, Bq, Bk, device=d, round_tiles=rounded)
    flags = vsa.VSA_FWD_WRITE_LSE | (vsa.VSA_FWD_REORDER_IO if reorder else 0) \
        | (vsa.VSA_FWD_FORCE_MASK if force else 0) | (vsa.VSA_FWD_TILE_ALIGNED if rounded else 0)
    o, lse = vsa.vsa_sparse_attn_fwd(q.to(d), k.to(d), v.to(d), g, layout, masks, tiles, flags=flags)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu().numpy()
    for h, (desc, lay) in enumerate(zip(masks, lays)):
        ref_o, ref_l = _oracle_head(q, k, v, g, lay, desc, h, (Bq, Bk) if rounded else None)
        assert_close(o[:, :, h], ref_o, dtype, f"head {h} ({lay}, {desc['kind']})")
        tol = 5e-3 if dtype == "bf16" else 1e-5
        fin = np.isfinite(ref_l)
        assert np.array_equal(np.isfinite(lse[:, h]), fin), f"head {h}: empty rows differ"
        assert np.abs(lse[:, h][fin] - ref_l[fin]).max(initial=0.0) <= tol, f"head {h} lse"
