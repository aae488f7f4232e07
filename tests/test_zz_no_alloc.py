"""The allocation-free forward (vsa_sparse_attn_fwd_noalloc) against the forward with a
caller workspace (vsa_sparse_attn_fwd_ex): the same kernels, so the same output bit for
bit, on two calls in a row on one GPU, the second with a smaller input (the scratch
keeps the first call's contents and must not leak into the second).  Both calls go
through the C ABI with every output allocated beforehand."""
import pytest
import torch

import block_sparse_spatio_amd as vsa
import workloads as W
from tests.gpu_helpers import dev, say

pytestmark = pytest.mark.gpu


def _case(big):
    if big:  # B 2, 4 heads of 128 channels, a position-major head reordered inside the call
        g = W.grid(6, 16, 16)
        masks = [W.mask_spatial(1), W.with_head_layout(W.mask_temporal(2), "position"),
                 W.mask_stripe(2, 1, 3, 3, 0, 16), W.mask_all()]
        return g, "frame", masks, 2, 128, 128, True
    g = W.grid(4, 8, 9)  # 288 tokens: a ragged tail; 2 heads of 64 channels
    return g, "frame", [W.mask_temporal(1), W.mask_box(0, 2, 2, sink_frames=1)], 1, 64, 64, False


@pytest.mark.parametrize("order", ["big_then_small", "small_then_big_then_small"])
def test_noalloc_matches_workspace_forward(gpu_lib, order):
    d = dev()
    seq = [True, False] if order == "big_then_small" else [False, True, False]
    for i, big in enumerate(seq):
        g, layout, masks, B, D, Bq, reorder = _case(big)
        S = W.seq_len(g)
        H = len(masks)
        q, k, v = (x.to(d) for x in W.qkv(B, S, H, D, "bf16", seed=40 + i))
        flags = vsa.VSA_FWD_WRITE_LSE | (vsa.VSA_FWD_REORDER_IO if reorder else 0)
        tiles = vsa.vsa_classify_tiles(g, layout, masks, Bq, 64, device=d, with_cls=False)
        words = vsa.vsa_boundary_words(g, layout, masks, tiles) if big else None
        o_ref, lse_ref = vsa.vsa_sparse_attn_fwd(q, k, v, g, layout, masks, tiles, flags=flags, words=words)
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, H, S), float("nan"), dtype=torch.float32, device=d)
        torch.cuda.synchronize()
        say(f"noalloc call {i}: {'big' if big else 'small'} B={B} S={S} H={H} D={D} Bq={Bq} reorder={reorder}")
        vsa.vsa_sparse_attn_fwd_noalloc(q, k, v, g, layout, masks, tiles, o, lse=lse, flags=flags, words=words)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), f"call {i}: o differs"
        assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32)), f"call {i}: lse differs"
