"""Merge of partial attention results over disjoint key sets (oracle; test
infrastructure).

DSA study guide, section 18 ("why online softmax can merge blocks"): for one query,
the full softmax needs the maximum m and the exponential sum l over all kept keys.
A partial result over a key subset carries its own (m_i, l_i) and its normalised
output o_i.  With the new maximum m' = max_i m_i every part is rescaled by
exp(m_i - m') and the rescaled sums are added; the result equals one softmax over
the union of the subsets, in any order of arrival.

In terms of the log-sum-exp statistic lse_i = m_i + ln l_i that the forward pass
returns:

    m'  = max_i lse_i
    w_i = exp(lse_i - m')          (0 for a part with no kept key, lse_i = -inf)
    lse = m' + ln(sum_i w_i)
    o   = sum_i w_i o_i / sum_i w_i

A row where every part is empty keeps the forward pass's convention: o = 0,
lse = -inf.  fp64 throughout.
"""
from __future__ import annotations

import numpy as np


def merge_partials(o_parts, lse_parts):
    """o_parts: list of n arrays [B, S, H, D]; lse_parts: list of n arrays [B, H, S]
    (natural log, -inf for a row without kept keys).  Returns (o [B, S, H, D],
    lse [B, H, S]) in fp64."""
    o_parts = [np.asarray(_f64(o), dtype=np.float64) for o in o_parts]
    lse_parts = [np.asarray(_f64(x), dtype=np.float64) for x in lse_parts]
    n = len(o_parts)
    if n == 0:
        raise ValueError("at least one part")
    lse_stack = np.stack(lse_parts)                      # [n, B, H, S]
    m = lse_stack.max(axis=0)                            # [B, H, S]
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(lse_stack - m_safe[None])                 # exp(-inf) = 0 for empty parts
    wsum = w.sum(axis=0)
    wsum_safe = np.where(empty, 1.0, wsum)
    lse = np.where(empty, -np.inf, m_safe + np.log(wsum_safe))
    o = np.zeros_like(o_parts[0])
    for i in range(n):
        wi = np.transpose(w[i] / wsum_safe, (0, 2, 1))[..., None]          # [B, S, H, 1]
        kept = np.transpose(np.isfinite(lse_stack[i]), (0, 2, 1))[..., None]
        o += wi * np.where(kept, o_parts[i], 0.0)   # an empty part adds nothing, whatever its o
    o[np.transpose(empty, (0, 2, 1))] = 0.0
    return o, lse


def _f64(x):
    if hasattr(x, "detach"):
        import torch
        return x.detach().to("cpu").to(torch.float64).numpy()
    return x
