"""Sampled-query head profiler and router (oracle; test infrastructure).

Sparse VideoGen routes each head at run time (Sparse VideoGen on TPU, "how to
accelerate attention"): it samples a few queries, computes their outputs under full
attention and under each candidate sparse mask, and routes the head to the mask
whose output deviates least from the full one.  The routing result is one flag per
head, with fixed tensor shapes (same page, "supporting dynamic routing with fixed
tensor shapes").  The sample is a small fraction of the sequence (video-DiT
attention blog, section 7.3: 1-2% of N).

Readings taken where the pages are silent:
* deviation = Frobenius norm of (o_candidate - o_full) over the sampled rows, every
  batch item and every channel; candidate 0 is the reference (full attention);
* the sample indices are an explicit input, shared by every batch item;
* route[h] = the candidate index c >= 1 with the smallest deviation, the lowest
  index on a tie.
"""
from __future__ import annotations

import numpy as np

from .attention import attention


def profile_heads(q, k, v, grid, layout, sample_idx, candidates, scale=None):
    """q, k, v: [B, S, H, D]; sample_idx: int [H, n]; candidates: list of descriptor
    dicts, candidates[0] being the reference.  Returns err fp64 [H, n_cand] and
    route int32 [H]."""
    B, S, H, D = q.shape
    sample_idx = np.asarray(sample_idx)
    n_cand = len(candidates)
    err = np.zeros((H, n_cand), dtype=np.float64)
    for h in range(H):
        rows = sample_idx[h]
        outs = []
        for c in range(n_cand):
            masks = [candidates[c]] * H
            o, _ = attention(q, k, v, grid, layout, masks, scale=scale, rows=rows, heads=[h])
            outs.append(o)
        for c in range(n_cand):
            err[h, c] = np.sqrt(np.sum((outs[c] - outs[0]) ** 2))
    route = np.zeros(H, dtype=np.int32)
    for h in range(H):
        best = 1
        for c in range(2, n_cand):
            if err[h, c] < err[h, best]:
                best = c
        route[h] = best
    return err, route
