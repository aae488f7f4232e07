"""Tile-major reorder on the GPU: bit-exact against the oracle's permutation."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import dev, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("g,dtype,H,D", [
    (W.grid(4, 8, 8, (2, 4, 4)), "bf16", 2, 64),
    (W.grid(6, 6, 10, (3, 2, 5)), "f32", 3, 128),
    (W.grid(30, 48, 80, (6, 8, 8)), "bf16", 24, 128),
])
def test_reorder_matches_permutation(gpu_lib, g, dtype, H, D):
    S = W.seq_len(g)
    say(f"reorder grid={g} {dtype} H={H} D={D}")
    x = W.qkv(1, S, H, D, dtype, seed=4)[0]
    xd = x.to(dev())
    y = gpu_lib.vsa_reorder_tokens(xd, g)
    z = gpu_lib.vsa_reorder_tokens(y, g, inverse=True)
    torch.cuda.synchronize()
    perm = torch.from_numpy(oracle.tile_major_permutation(g))
    assert torch.equal(y.cpu(), x[:, perm])
    assert torch.equal(z.cpu(), x)


@pytest.mark.parametrize("g,dtype,layouts,D", [
    (W.grid(4, 8, 8, (2, 4, 4)), "bf16", ["frame", "position", "tile", "position"], 64),
    (W.grid(5, 6, 7), "f32", ["position", "frame", "position"], 128),
    (W.grid(1, 6, 7), "bf16", ["position", "frame"], 64),  # one frame: position-major is frame order
    (W.grid(21, 45, 80), "bf16", ["frame"] * 4 + ["position"] * 4, 128),
])
def test_reorder_heads_matches_permutation(gpu_lib, g, dtype, layouts, D):
    S, H = W.seq_len(g), len(layouts)
    say(f"reorder heads grid={g} {dtype} layouts={layouts} D={D}")
    x = W.qkv(1, S, H, D, dtype, seed=5)[0]
    xd = x.to(dev())
    y = gpu_lib.vsa_reorder_heads(xd, g, layouts)
    z = gpu_lib.vsa_reorder_heads(y, g, layouts, inverse=True)
    torch.cuda.synchronize()
    y = y.cpu()
    for h, lay in enumerate(layouts):
        perm = torch.from_numpy(oracle.layout_permutation(g, lay))
        assert torch.equal(y[:, :, h], x[:, perm, h]), (h, lay)
    assert torch.equal(z.cpu(), x)


@pytest.mark.parametrize("g,dtype,H,D", [
    (W.grid(3, 5, 7, (2, 2, 4)), "bf16", 2, 64),
    (W.grid(5, 6, 10, (2, 4, 4)), "f32", 3, 128),
    (W.grid(21, 45, 80, (3, 8, 16)), "bf16", 4, 128),
])
def test_reorder_padded_matches_permutation(gpu_lib, g, dtype, H, D):
    """Frame-major -> tile-major over the padded grid (zero padding rows) and back."""
    S = W.seq_len(g)
    say(f"reorder padded grid={g} {dtype} H={H} D={D}")
    x = W.qkv(1, S, H, D, dtype, seed=6)[0]
    y = gpu_lib.vsa_reorder_heads(x.to(dev()), g, ["padded"] * H)
    z = gpu_lib.vsa_reorder_heads(y, g, ["padded"] * H, inverse=True)
    torch.cuda.synchronize()
    perm = oracle.layout_permutation(g, "padded")
    assert y.shape[1] == len(perm) == oracle.seq_len(g, "padded")
    ref = torch.from_numpy(oracle.reorder_tokens(x.float().numpy(), g, layout="padded")).to(x.dtype)
    assert torch.equal(y.cpu(), ref)
    assert torch.equal(z.cpu(), x)
