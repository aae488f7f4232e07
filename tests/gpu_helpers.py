"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI and
compare it with the CPU oracle."""
import numpy as np
import torch

import block_sparse_spatio_amd as vsa
import oracle
import workloads as W

# parity tolerances (oracle run on the same bf16-rounded / fp32 inputs)
BF16_MAX_ABS, BF16_MEAN_ABS = 2e-2, 1e-3
F32_MAX_ABS = 1e-5


def dev():
    return torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)


def run_attention(q, k, v, g, layout, masks, Bq, Bk, flags=0, scale=0.0, reorder_io=False):
    """Classify + forward on the GPU; returns (o, lse) device tensors and the tile lists.
    With reorder_io the inputs are frame-major and the call reorders around the kernel."""
    d = dev()
    tiles = vsa.vsa_classify_tiles(g, layout, masks, Bq, Bk, device=d)
    f = flags | (vsa.VSA_FWD_REORDER_IO if reorder_io else 0)
    o, lse = vsa.vsa_sparse_attn_fwd(q.to(d), k.to(d), v.to(d), g, layout, masks, tiles, scale=scale, flags=f)
    torch.cuda.synchronize()
    return o, lse, tiles


def assert_close(got, ref, dtype, what=""):
    got = got.float().cpu().numpy().astype(np.float64) if torch.is_tensor(got) else got
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    if dtype == "f32":
        assert err.max() <= F32_MAX_ABS, f"{what}: max |err| {err.max():.3e} > {F32_MAX_ABS}"
    else:
        assert err.max() <= BF16_MAX_ABS, f"{what}: max |err| {err.max():.3e} > {BF16_MAX_ABS}"
        assert err.mean() <= BF16_MEAN_ABS, f"{what}: mean |err| {err.mean():.3e} > {BF16_MEAN_ABS}"
    return err.max(), err.mean()


def oracle_lists(cls_row):
    return (np.flatnonzero(cls_row == oracle.FULL), np.flatnonzero(cls_row == oracle.BOUNDARY))


def check_lists_against(tiles, u, q_tiles, ref_cls):
    """Bit-exact comparison of the GPU class rows and lists of unique mask u."""
    n_full = tiles["n_full"][u].cpu().numpy()
    n_bnd = tiles["n_bnd"][u].cpu().numpy()
    fi = tiles["full_idx"][u]
    bi = tiles["bnd_idx"][u]
    cls = tiles["cls"][u] if tiles["cls"] is not None else None
    for j, qt in enumerate(q_tiles):
        rf, rb = oracle_lists(ref_cls[j])
        if cls is not None:
            got = cls[qt].cpu().numpy()
            assert np.array_equal(got, ref_cls[j]), f"class row of q-tile {qt} differs"
        assert n_full[qt] == len(rf) and n_bnd[qt] == len(rb), f"list lengths of q-tile {qt}"
        assert np.array_equal(fi[qt, : len(rf)].cpu().numpy(), rf), f"full list of q-tile {qt}"
        assert np.array_equal(bi[qt, : len(rb)].cpu().numpy(), rb), f"boundary list of q-tile {qt}"
