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
