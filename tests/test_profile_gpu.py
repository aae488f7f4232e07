"""Head profiler on the GPU against the oracle: errors within 1% relative (fp32
accumulation of bf16-rounded probabilities against fp64), routes equal wherever the
oracle's margin between the candidates exceeds that tolerance, and the GPU's own
route is the argmin of the GPU's own errors."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import dev, say

pytestmark = pytest.mark.gpu

REL = 1e-2


def _check(err_g, route_g, err_o, route_o):
    err_g = err_g.cpu().numpy().astype(np.float64)
    route_g = route_g.cpu().numpy()
    assert np.all(err_g[:, 0] == 0)
    assert np.allclose(err_g, err_o, rtol=REL, atol=1e-4), np.abs(err_g - err_o).max()
    for h in range(err_g.shape[0]):
        assert route_g[h] == 1 + int(np.argmin(err_g[h, 1:]))
        e = np.sort(err_o[h, 1:])
        if len(e) < 2 or e[1] - e[0] > 3 * REL * e[1]:
            assert route_g[h] == route_o[h], (h, err_g[h], err_o[h])


def _coded(g, H, D, by, alpha, seed):
    rng = np.random.default_rng(seed)
    S = W.seq_len(g)
    t, y, x = oracle.token_coords(g, "frame", np.arange(S))
    key = (y * g["Wg"] + x) if by == "position" else t
    codes = rng.standard_normal((key.max() + 1, H, D))
    codes /= np.linalg.norm(codes, axis=-1, keepdims=True)
    qk = torch.from_numpy(alpha * codes[key][None]).to(torch.bfloat16)
    v = torch.from_numpy(rng.standard_normal((1, S, H, D))).to(torch.bfloat16)
    return qk, qk.clone(), v


@pytest.mark.parametrize("by,winner", [("position", 2), ("frame", 1)])
def test_profiler_constructed_winner(gpu_lib, by, winner):
    g = W.grid(8, 12, 12)
    q, k, v = _coded(g, 4, 128, by, 12.0, 3)
    S = W.seq_len(g)
    idx = W.sample_rows(S, 48, 4, 5)
    cands = [W.mask_all(), W.mask_spatial(1), W.mask_temporal(4)]
    d = dev()
    err, route = gpu_lib.vsa_profile_heads(q.to(d), k.to(d), v.to(d), g, "frame",
                                           torch.from_numpy(idx).to(d), cands)
    torch.cuda.synchronize()
    assert torch.all(route.cpu() == winner)
    err_o, route_o = oracle.profile_heads(q, k, v, g, "frame", idx, cands)
    _check(err, route, err_o, route_o)


@pytest.mark.parametrize("n,nc", [(16, 2), (20, 3), (32, 4), (64, 3), (100, 4), (128, 2), (200, 2), (256, 3)])
def test_profiler_iid_small(gpu_lib, n, nc):
    g = W.grid(6, 12, 14)
    S = W.seq_len(g)
    q, k, v = W.qkv(2, S, 3, 128, "bf16", seed=n)
    idx = W.sample_rows(S, n, 3, n + 1)
    cands = [W.mask_all(), W.mask_spatial(1), W.mask_temporal(3), W.mask_stripe(1, 0, 2, 3, 0, 14)][:nc]
    d = dev()
    say(f"profiler iid n={n} n_cand={nc}")
    err, route = gpu_lib.vsa_profile_heads(q.to(d), k.to(d), v.to(d), g, "frame",
                                           torch.from_numpy(idx).to(d), cands)
    torch.cuda.synchronize()
    err_o, route_o = oracle.profile_heads(q, k, v, g, "frame", idx, cands)
    _check(err, route, err_o, route_o)


def test_profiler_full_config(gpu_lib):
    cfg = W.config("stripe_route")
    g = cfg["grid"]
    S = W.seq_len(g)
    say("profiler full config stripe_route")
    q, k, v = W.qkv(cfg["B"], S, cfg["H"], cfg["D"], "bf16", seed=cfg["seed"])
    idx = W.sample_rows(S, cfg["n_samples"], cfg["H"], cfg["seed"] + 1)
    d = dev()
    err, route = gpu_lib.vsa_profile_heads(q.to(d), k.to(d), v.to(d), g, "frame",
                                           torch.from_numpy(idx).to(d), cfg["candidates"])
    torch.cuda.synchronize()
    heads = list(range(0, cfg["H"], 5))
    err_o, route_o = oracle.profile_heads(q[:, :, heads], k[:, :, heads], v[:, :, heads], g, "frame",
                                          idx[heads], cfg["candidates"])
    _check(err[heads], route[heads], err_o, route_o)
