"""Attention forward on the GPU against the CPU oracle (parity tolerances:
fp32 max-abs <= 1e-5; bf16 max-abs <= 2e-2 and mean-abs <= 1e-3, the oracle run on
the same bf16-rounded inputs)."""
import numpy as np
import pytest
import torch

import block_sparse_spatio_amd as vsa
import oracle
import workloads as W
from tests.gpu_helpers import assert_close, dev, run_attention, say

pytestmark = pytest.mark.gpu


def test_tiny_config_fp32(gpu_lib):
    cfg = W.config("tiny")
    q, k, v = W.qkv(cfg["B"], 256, cfg["H"], cfg["D"], "f32", seed=cfg["seed"])
    for masks in (cfg["masks"], cfg["extra_masks"]):
        say(f"tiny fp32 masks={masks}")
        o, lse, _ = run_attention(q, k, v, cfg["grid"], "frame", masks, 32, 32, flags=vsa.VSA_FWD_WRITE_LSE)
        ref_o, ref_lse = oracle.attention(q, k, v, cfg["grid"], "frame", masks)
        assert_close(o, ref_o, "f32", "tiny fp32")
        assert np.abs(lse.cpu().numpy() - ref_lse).max() <= 1e-5
    # the all-keep mask is dense attention: compare with a library routine too
    o, _, _ = run_attention(q, k, v, cfg["grid"], "frame", cfg["extra_masks"], 32, 32)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(x.double().permute(0, 2, 1, 3) for x in (q, k, v))).permute(0, 2, 1, 3)
    assert (o.double().cpu() - ref).abs().max() <= 1e-5


@pytest.mark.parametrize("Bq,Bk", [(32, 64), (64, 32), (128, 64)])
def test_fp32_tile_shapes(gpu_lib, Bq, Bk):
    g = W.grid(3, 7, 9)  # S = 189: ragged tails on both sides
    masks = [W.mask_spatial(1), W.mask_temporal(2), W.mask_stripe(2, 0, 3, 3, 1, 10)]
    q, k, v = W.qkv(2, 189, 3, 128, "f32", seed=11)
    o, _, _ = run_attention(q, k, v, g, "frame", masks, Bq, Bk)
    ref, _ = oracle.attention(q, k, v, g, "frame", masks)
    assert_close(o, ref, "f32", f"fp32 Bq={Bq} Bk={Bk}")


SMALL_CASES = [
    # (grid, layout, masks, D, B)
    (W.grid(5, 6, 7), "frame", [W.mask_spatial(1), W.mask_temporal(2), W.mask_all()], 128, 1),
    (W.grid(4, 9, 10), "frame", [W.mask_box(0, 2, 3, 0), W.mask_box(2, -1, 1, 2)], 128, 2),
    (W.grid(6, 5, 16), "frame", [W.mask_stripe(1, 0, 3, 1, 0, 16), W.mask_stripe(2, 1, 2, 4, 0, 80),
                                 W.mask_stripe(3, 0, 7, 2, 3, 5)], 128, 1),
    (W.grid(4, 8, 8, (2, 4, 4)), "tile", [W.mask_sta(1, 1, 1), W.mask_sta(2, 2, 1, sink_frames=1)], 128, 1),
    (W.grid(4, 8, 8, (2, 4, 4)), "tile", [W.mask_temporal(2), W.mask_stripe(1, 0, 2, 3, 0, 9)], 64, 1),
    (W.grid(3, 11, 13), "frame", [W.mask_spatial(0, sink_frames=0), W.mask_temporal(1)], 64, 1),
]


@pytest.mark.parametrize("case", range(len(SMALL_CASES)))
@pytest.mark.parametrize("Bq", [64, 128, 256])
def test_small_bf16(gpu_lib, case, Bq):
    g, layout, masks, D, B = SMALL_CASES[case]
    S = W.seq_len(g)
    q, k, v = W.qkv(B, S, len(masks), D, "bf16", seed=100 + case)
    say(f"small bf16 case={case} Bq={Bq} S={S} D={D} layout={layout}")
    o, lse, _ = run_attention(q, k, v, g, layout, masks, Bq, 64, flags=vsa.VSA_FWD_WRITE_LSE)
    ref_o, ref_lse = oracle.attention(q, k, v, g, layout, masks)
    assert_close(o, ref_o, "bf16", f"case {case} Bq {Bq}")
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= 5e-3


def test_force_mask_matches_specialised_path(gpu_lib):
    """The B1 ablation (every tile through the masked path) equals the full/boundary
    split bit for bit: on a full tile the element mask keeps everything."""
    g = W.grid(6, 8, 16)
    masks = [W.mask_spatial(1), W.mask_temporal(3), W.mask_all()]
    q, k, v = W.qkv(1, W.seq_len(g), 3, 128, "bf16", seed=5)
    o1, _, _ = run_attention(q, k, v, g, "frame", masks, 128, 64)
    o2, _, _ = run_attention(q, k, v, g, "frame", masks, 128, 64, flags=vsa.VSA_FWD_FORCE_MASK)
    assert torch.equal(o1, o2)


def test_deterministic(gpu_lib):
    g = W.grid(5, 10, 16)
    masks = [W.mask_temporal(2), W.mask_stripe(2, 0, 3, 2, 0, 16)]
    q, k, v = W.qkv(1, W.seq_len(g), 2, 128, "bf16", seed=6)
    o1, _, _ = run_attention(q, k, v, g, "frame", masks, 128, 64)
    o2, _, _ = run_attention(q, k, v, g, "frame", masks, 128, 64)
    assert torch.equal(o1, o2)


def test_zero_query_is_mean_of_kept_values(gpu_lib):
    g = W.grid(4, 6, 10)
    S = W.seq_len(g)
    masks = [W.mask_box(1, 1, 2, sink_frames=1)]
    _, k, v = W.qkv(1, S, 1, 128, "bf16", seed=8)
    q = torch.zeros_like(k)
    o, _, _ = run_attention(q, k, v, g, "frame", masks, 64, 64)
    c = oracle.token_coords(g, "frame", np.arange(S))
    keep = oracle.keep_matrix(masks[0], g, c, c)
    vv = v[0, :, 0].double().numpy()
    ref = np.stack([vv[keep[i]].mean(axis=0) for i in range(S)])
    assert_close(o[0, :, 0], ref, "bf16", "zero query")


def test_self_only_stripe_is_identity(gpu_lib):
    g = W.grid(3, 5, 20)
    masks = [W.mask_stripe(1, 0, 10, 1, 0, 500, sink_frames=0)]
    q, k, v = W.qkv(1, W.seq_len(g), 1, 128, "bf16", seed=9)
    o, _, _ = run_attention(q, k, v, g, "frame", masks, 128, 64)
    assert torch.equal(o.cpu(), v)


def test_empty_rows_are_zero(gpu_lib):
    g = W.grid(3, 4, 8)
    masks = [W.mask_stripe(1, 5, 99, 4, 0, 4, sink_frames=0)]
    q, k, v = W.qkv(1, W.seq_len(g), 1, 64, "bf16", seed=10)
    o, lse, tiles = run_attention(q, k, v, g, "frame", masks, 64, 64, flags=vsa.VSA_FWD_WRITE_LSE)
    assert int(tiles["n_full"].sum() + tiles["n_bnd"].sum()) == 0
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_sta_reorder_io_matches_frame_major(gpu_lib):
    """Tile-major attention with the reorder inside the call equals frame-major attention
    with the same coordinate mask, and the oracle."""
    g = W.grid(6, 16, 32, (2, 8, 8))  # 128-token tiles: query and key tiles nest inside them
    S = W.seq_len(g)
    masks = [W.mask_sta(1, 1, 3), W.mask_sta(2, 1, 3, sink_frames=1)]
    q, k, v = W.qkv(1, S, 2, 128, "bf16", seed=12)
    o_t, lse_t, tiles = run_attention(q, k, v, g, "tile", masks, 128, 64, reorder_io=True,
                                      flags=vsa.VSA_FWD_WRITE_LSE)
    o_f, lse_f, _ = run_attention(q, k, v, g, "frame", masks, 128, 64, flags=vsa.VSA_FWD_WRITE_LSE)
    ref, ref_lse = oracle.attention(q, k, v, g, "frame", masks)
    assert_close(o_t, ref, "bf16", "sta tile-major")
    assert_close(o_f, ref, "bf16", "sta frame-major")
    assert np.abs(lse_t.cpu().numpy() - ref_lse).max() <= 5e-3
    assert int(tiles["n_bnd"][0].sum()) == 0  # sliding tiles: full or empty only
    # tiles that straddle two sliding tiles are boundary tiles and still exact
    g2 = W.grid(6, 16, 16, (3, 4, 4))
    q2, k2, v2 = W.qkv(1, W.seq_len(g2), 2, 128, "bf16", seed=13)
    masks2 = [W.mask_sta(1, 3, 3), W.mask_sta(2, 1, 3, sink_frames=1)]
    o2, _, tiles2 = run_attention(q2, k2, v2, g2, "tile", masks2, 128, 64, reorder_io=True)
    assert int(tiles2["n_bnd"].sum()) > 0
    assert_close(o2, oracle.attention(q2, k2, v2, g2, "frame", masks2)[0], "bf16", "sta straddling")


@pytest.mark.parametrize("case", [0, 1, 2, 5])
def test_tile_aligned_forward(gpu_lib, case):
    """Rounded lists (B3) with VSA_FWD_TILE_ALIGNED equal the oracle's attention under
    the rounded mask (padding masked only), bf16 and fp32."""
    g, layout, masks, D, B = SMALL_CASES[case]
    S = W.seq_len(g)
    for dtype, Bq, Bk in (("bf16", 128, 64), ("f32", 64, 32)):
        q, k, v = W.qkv(B, S, len(masks), D, dtype, seed=200 + case)
        say(f"tile-aligned case={case} {dtype} Bq={Bq} Bk={Bk}")
        d = dev()
        tiles = vsa.vsa_classify_tiles(g, layout, masks, Bq, Bk, device=d, round_tiles=True)
        o, lse = vsa.vsa_sparse_attn_fwd(q.to(d), k.to(d), v.to(d), g, layout, masks, tiles,
                                         flags=vsa.VSA_FWD_TILE_ALIGNED | vsa.VSA_FWD_WRITE_LSE)
        torch.cuda.synchronize()
        ref_o, ref_lse = oracle.attention(q, k, v, g, layout, masks, round_tiles=(Bq, Bk))
        assert_close(o, ref_o, dtype, f"tile-aligned case {case} {dtype}")
        fin = np.isfinite(ref_lse)
        got = lse.cpu().numpy()
        assert np.array_equal(np.isneginf(got), ~fin)
        assert np.abs(got[fin] - ref_lse[fin]).max() <= (5e-3 if dtype == "bf16" else 1e-5)


def _head_layout_case(dtype):
    """Grid, masks and inputs with heads in frame-, position- and tile-major order."""
    g = W.grid(6, 16, 16, (2, 8, 8))
    masks = [W.mask_spatial(1),
             W.with_head_layout(W.mask_temporal(2), "position"),
             W.with_head_layout(W.mask_sta(2, 1, 1, sink_frames=1), "tile"),
             W.with_head_layout(W.mask_stripe(1, 0, 2, 3, 0, 16), "position"),
             W.mask_temporal(1)]
    q, k, v = W.qkv(2, W.seq_len(g), len(masks), 64 if dtype == "f32" else 128, dtype, seed=21)
    return g, masks, q, k, v


@pytest.mark.parametrize("dtype,Bq,Bk", [("bf16", 64, 64), ("bf16", 128, 64), ("bf16", 256, 64),
                                         ("f32", 64, 32)])
def test_head_layouts_reorder_io(gpu_lib, dtype, Bq, Bk):
    """Frame-major I/O with every head attended in its own order (the reorder inside the
    call) equals frame-major attention with the same coordinate masks: o and lse."""
    g, masks, q, k, v = _head_layout_case(dtype)
    say(f"head layouts reorder io {dtype} Bq={Bq} Bk={Bk}")
    o, lse, _ = run_attention(q, k, v, g, "frame", masks, Bq, Bk, reorder_io=True, flags=vsa.VSA_FWD_WRITE_LSE)
    ref_o, ref_lse = oracle.attention(q, k, v, g, "frame", masks)
    assert_close(o, ref_o, dtype, "per-head layouts, reorder inside")
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= (5e-3 if dtype == "bf16" else 1e-5)


def test_head_layouts_in_place(gpu_lib):
    """Without the reorder flag each head's q, k, v and o are in that head's order: inputs
    gathered per head by the oracle's permutation give the permuted frame-major result."""
    g, masks, q, k, v = _head_layout_case("bf16")
    lays = W.head_layouts(masks, "frame")
    perms = [torch.from_numpy(oracle.layout_permutation(g, lay)) for lay in lays]
    qp, kp, vp = (torch.stack([x[:, perms[h], h] for h in range(len(lays))], dim=2) for x in (q, k, v))
    say(f"head layouts in place {lays}")
    o, lse, _ = run_attention(qp, kp, vp, g, "frame", masks, 128, 64, flags=vsa.VSA_FWD_WRITE_LSE)
    ref_o, ref_lse = oracle.attention(q, k, v, g, "frame", masks)
    o, lse = o.cpu(), lse.cpu().numpy()
    for h, p in enumerate(perms):
        assert_close(o[:, :, h], ref_o[:, p.numpy(), h], "bf16", f"head {h} ({lays[h]})")
        assert np.abs(lse[:, h] - ref_lse[:, h][:, p.numpy()]).max() <= 5e-3


def _padded_case(dtype):
    g = W.grid(5, 6, 10, (2, 4, 4))  # padded to 6 x 8 x 12
    masks = [W.mask_sta(3, 1, 3), W.mask_box(1, 2, 3, sink_frames=1), W.mask_stripe(1, 0, 2, 2, 1, 7)]
    q, k, v = W.qkv(2, W.seq_len(g), len(masks), 64 if dtype == "f32" else 128, dtype, seed=31)
    return g, masks, q, k, v


@pytest.mark.parametrize("dtype,Bq,Bk", [("bf16", 64, 64), ("bf16", 128, 64), ("bf16", 256, 64),
                                         ("f32", 32, 32), ("f32", 64, 64)])
def test_padded_reorder_io(gpu_lib, dtype, Bq, Bk):
    """Frame-major I/O attended tile-major over the padded grid (reorder inside the
    call) equals frame-major attention: o and lse."""
    g, masks, q, k, v = _padded_case(dtype)
    say(f"padded reorder io {dtype} Bq={Bq} Bk={Bk}")
    o, lse, tiles = run_attention(q, k, v, g, "padded", masks, Bq, Bk, reorder_io=True, flags=vsa.VSA_FWD_WRITE_LSE)
    ref_o, ref_lse = oracle.attention(q, k, v, g, "frame", masks)
    assert_close(o, ref_o, dtype, "padded, reorder inside")
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= (5e-3 if dtype == "bf16" else 1e-5)


def test_padded_in_place(gpu_lib):
    """Without the reorder flag q, k, v are already in the padded order (zero padding
    rows from the oracle's permutation): the real rows equal the frame-major result."""
    g, masks, q, k, v = _padded_case("bf16")
    qp, kp, vp = (torch.from_numpy(oracle.reorder_tokens(x.float().numpy(), g, layout="padded")).to(x.dtype)
                  for x in (q, k, v))
    say("padded in place")
    o, lse, _ = run_attention(qp, kp, vp, g, "padded", masks, 128, 64, flags=vsa.VSA_FWD_WRITE_LSE)
    perm = oracle.layout_permutation(g, "padded")
    real = perm >= 0
    ref_o, ref_lse = oracle.attention(q, k, v, g, "frame", masks)
    o = o.cpu()[:, torch.from_numpy(np.flatnonzero(real))]
    assert_close(o, ref_o[:, perm[real]], "bf16", "padded in place")
    assert np.abs(lse.cpu().numpy()[:, :, real] - ref_lse[:, :, perm[real]]).max() <= 5e-3


@pytest.mark.parametrize("dtype,Bq,Bk", [("bf16", 128, 64), ("bf16", 64, 64), ("f32", 64, 32)])
def test_padded_in_place_nan_padding(gpu_lib, dtype, Bq, Bk):
    """Padding rows of q, k and v in the padded order may hold anything, here NaN: they
    are never kept, and the real rows' o and lse equal those with zero padding bit for
    bit (a padding value must not reach the PV product, where 0 * NaN is NaN)."""
    g, masks, q, k, v = _padded_case(dtype)
    pad = torch.from_numpy(oracle.layout_permutation(g, "padded") < 0)
    zero = [torch.from_numpy(oracle.reorder_tokens(x.float().numpy(), g, layout="padded")).to(x.dtype)
            for x in (q, k, v)]
    nan = [x.clone() for x in zero]
    for x in nan:
        x[:, pad] = float("nan")
    say(f"padded in place, NaN padding, {dtype} Bq={Bq} Bk={Bk}")
    o0, l0, _ = run_attention(*zero, g, "padded", masks, Bq, Bk, flags=vsa.VSA_FWD_WRITE_LSE)
    o1, l1, _ = run_attention(*nan, g, "padded", masks, Bq, Bk, flags=vsa.VSA_FWD_WRITE_LSE)
    real = (~pad).to(o0.device)
    assert torch.isfinite(o1[:, real]).all()
    assert torch.equal(o0[:, real], o1[:, real])
    assert torch.equal(l0[:, :, real], l1[:, :, real])


def test_padded_tile_aligned_forward(gpu_lib):
    """B3 rounding on the padded order, forward with VSA_FWD_TILE_ALIGNED: equals the
    oracle's attention under the rounded mask (padding keys masked, interior too)."""
    g, masks, q, k, v = _padded_case("bf16")
    Bq, Bk = 128, 64
    d = dev()
    qp, kp, vp = (torch.from_numpy(oracle.reorder_tokens(x.float().numpy(), g, layout="padded")).to(x.dtype)
                  for x in (q, k, v))
    say("padded tile-aligned forward")
    tiles = vsa.vsa_classify_tiles(g, "padded", masks, Bq, Bk, device=d, round_tiles=True)
    o, _ = vsa.vsa_sparse_attn_fwd(qp.to(d), kp.to(d), vp.to(d), g, "padded", masks, tiles,
                                   flags=vsa.VSA_FWD_TILE_ALIGNED)
    torch.cuda.synchronize()
    real = np.flatnonzero(oracle.layout_permutation(g, "padded") >= 0)
    ref_o, _ = oracle.attention(qp, kp, vp, g, "padded", masks, rows=real, round_tiles=(Bq, Bk))
    assert_close(o.cpu()[:, torch.from_numpy(real)], ref_o, "bf16", "padded B3")


@pytest.mark.parametrize("tile", [(1, 9, 1), (1, 9, 2), (2, 3, 4)])
def test_column_strip_tiles_reorder_io(gpu_lib, tile):
    """Stripe heads attended tile-major over narrow grid tiles (a frame read a few
    columns at a time, which makes column-band stripes contiguous), beside position- and
    frame-major heads, with the reorder inside the call: o and lse against the oracle in
    frame-major coordinates, with and without the mask-word table."""
    g = W.grid(4, 9, 16, tile)
    masks = [W.with_head_layout(W.mask_stripe(1, 0, 3, 2, 0, 16), "tile"),
             W.with_head_layout(W.mask_stripe(2, 1, 7, 3, 0, 16), "tile"),
             W.with_head_layout(W.mask_stripe(1, 1, 3, 2, 0, 144), "position"),
             W.mask_stripe(1, 0, 2, 4, 0, 16)]
    q, k, v = W.qkv(2, W.seq_len(g), len(masks), 128, "bf16", seed=33)
    say(f"column strip tiles {tile}")
    d = dev()
    tiles = vsa.vsa_classify_tiles(g, "frame", masks, 128, 64, device=d, with_cls=False)
    flags = vsa.VSA_FWD_WRITE_LSE | vsa.VSA_FWD_REORDER_IO
    ref_o, ref_lse = oracle.attention(q, k, v, g, "frame", masks)
    for words in (None, vsa.vsa_boundary_words(g, "frame", masks, tiles)):
        o, lse = vsa.vsa_sparse_attn_fwd(q.to(d), k.to(d), v.to(d), g, "frame", masks, tiles, flags=flags,
                                         words=words)
        torch.cuda.synchronize()
        assert_close(o, ref_o, "bf16", f"column strips {tile}, words={words is not None}")
        assert np.abs(lse.cpu().numpy() - ref_lse).max() <= 5e-3
