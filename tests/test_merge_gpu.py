"""Merging partial attention results on the GPU against the oracle's log-sum-exp merge
(DSA study guide, section 18).  fp32 outputs within 1e-5; bf16 outputs within the
parity bf16 tolerance (max-abs 2e-2, mean-abs 1e-3); lse within 1e-5."""
import numpy as np
import pytest
import torch

import block_sparse_spatio_amd as vsa
import oracle
import workloads as W
from tests.gpu_helpers import assert_close, dev, run_attention, say

pytestmark = pytest.mark.gpu


def _parts(n, B, S, H, D, dtype, seed, empty_frac=0.2):
    rng = np.random.default_rng(seed)
    o = [torch.from_numpy(rng.standard_normal((B, S, H, D)).astype(np.float32)) for _ in range(n)]
    if dtype == "bf16":
        o = [t.to(torch.bfloat16) for t in o]
    lse = []
    for i in range(n):
        x = rng.normal(0.0, 3.0, (B, H, S)).astype(np.float32)
        x[rng.random((B, H, S)) < empty_frac] = -np.inf  # parts without kept keys
        lse.append(torch.from_numpy(x))
    lse[0][0, 0, :3] = -np.inf
    for t in lse:  # rows empty in every part
        t[0, 0, 0] = -np.inf
    return o, lse


@pytest.mark.parametrize("n,D,dtype", [(1, 128, "bf16"), (2, 128, "bf16"), (3, 64, "bf16"), (5, 128, "f32"),
                                       (16, 64, "f32")])
def test_merge_random_parts(gpu_lib, n, D, dtype):
    B, S, H = 2, 37, 3
    o, lse = _parts(n, B, S, H, D, dtype, seed=n * 10 + D)
    say(f"merge n={n} D={D} {dtype}")
    d = dev()
    og, lg = vsa.vsa_merge_partials([t.to(d) for t in o], [t.to(d) for t in lse])
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.merge_partials(o, lse)
    assert_close(og, ref_o, dtype, f"merge n={n}")
    lg = lg.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(lg), np.isneginf(ref_l))
    fin = np.isfinite(ref_l)
    assert np.abs(lg[fin] - ref_l[fin]).max() <= 1e-5
    assert torch.all(og.cpu()[0, 0, 0] == 0)


def test_merge_in_place(gpu_lib):
    o, lse = _parts(3, 1, 50, 2, 128, "bf16", seed=4)
    d = dev()
    od, ld = [t.to(d) for t in o], [t.to(d) for t in lse]
    og, lg = vsa.vsa_merge_partials(od, ld, o=od[0], lse=ld[0])
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.merge_partials(o, lse)
    assert_close(od[0], ref_o, "bf16", "in place")
    fin = np.isfinite(ref_l)
    assert np.abs(ld[0].cpu().numpy()[fin] - ref_l[fin]).max() <= 1e-5


def test_merge_of_key_partition_is_full_attention(gpu_lib):
    """Attention under the three masks 'dt = r (mod 3)' partitions every key set;
    merging the three GPU results equals GPU and oracle attention over all keys."""
    g = W.grid(7, 9, 10)
    S = W.seq_len(g)
    classes = [W.mask_stripe(1, r, 3, 1, 0, 1, sink_frames=0) for r in range(3)]
    q, k, v = W.qkv(1, S, 2, 128, "bf16", seed=21)
    parts = [run_attention(q, k, v, g, "frame", [m, m], 128, 64, flags=vsa.VSA_FWD_WRITE_LSE)[:2]
             for m in classes]
    og, lg = vsa.vsa_merge_partials([p[0] for p in parts], [p[1] for p in parts])
    full_o, full_l, _ = run_attention(q, k, v, g, "frame", [W.mask_all()] * 2, 128, 64,
                                      flags=vsa.VSA_FWD_WRITE_LSE)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attention(q, k, v, g, "frame", [W.mask_all()] * 2)
    assert_close(og, ref_o, "bf16", "merged partition vs oracle")
    assert np.abs(lg.cpu().numpy() - ref_l).max() <= 5e-3
    assert (og.float() - full_o.float()).abs().max().item() <= 2e-2
