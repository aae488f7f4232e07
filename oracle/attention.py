"""Masked softmax attention from its definition (oracle; test infrastructure).

For one head (Sliding Tile Attention explainer, method section 2, eq. (1)):

    S = Q K^T * scale,   A = softmax(S + M),   O = A V

with M = 0 on kept pairs and -inf on dropped ones, scale = 1/sqrt(d) by default.
Block skipping and the full/boundary split must leave this result unchanged
(Sparse VideoGen on TPU: skipped tiles hold no kept pair; the two tile paths give
the same output and are merged with their softmax statistics), so the oracle does
not tile: it materialises the score rows, applies the boolean mask and normalises.

Also returned: the log-sum-exp per row, lse = m + ln(sum_j exp(s_j - m)), the
statistic that lets partial results over disjoint key sets be merged (DSA guide
section 18, "why online softmax can merge blocks").

A row with no kept key (impossible with a sink or an all-keep mask) is defined as
o = 0 and lse = -inf; the pages do not cover it.

All arithmetic is fp64.  Inputs are widened exactly (bf16 and fp32 values are
exactly representable in fp64).
"""
from __future__ import annotations

import numpy as np

from .coords import is_real, token_coords
from .classify import rounded_keep_rows
from .masks import keep_matrix


def attention_rows(q, k, v, keep, scale):
    """Masked softmax attention for query rows q [n, D] against k, v [S, D], given the
    boolean keep matrix [n, S].  Returns o [n, D] and lse [n] in fp64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = (q @ k.T) * scale
    s = np.where(keep, s, -np.inf)
    m = s.max(axis=1)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    p = np.exp(s - m_safe[:, None])
    l = p.sum(axis=1)
    l_safe = np.where(empty, 1.0, l)
    o = (p @ v) / l_safe[:, None]
    o[empty] = 0.0
    lse = np.where(empty, -np.inf, m_safe + np.log(l_safe))
    return o, lse


def attention(q, k, v, grid, layout, masks, scale=None, rows=None, heads=None, block=128, round_tiles=None):
    """Masked attention for tensors q, k, v of shape [B, S, H, D] (any float dtype).

    masks: list of H descriptor dicts, one per head.
    layout: the order of the positions of q, k, v (for "padded", S is the padded length
             and padding keys are never kept; padding rows are computed like the others).
    rows:  optional int array of executed query positions (default: all S).
    heads: optional list of heads (default: all).
    round_tiles: optional (Bq, Bk): attend under the tile-aligned (B3) rounding of each
             mask (oracle.classify.rounded_keep_rows) instead of the exact mask.
    Returns o [B, len(rows), len(heads), D] fp64 and lse [B, len(heads), len(rows)] fp64."""
    B, S, H, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = list(range(H)) if heads is None else list(heads)
    ck = token_coords(grid, layout, np.arange(S))
    real_k = is_real(grid, *ck)  # padding keys of the padded layout are never kept
    o = np.zeros((B, len(rows), len(heads), D), dtype=np.float64)
    lse = np.zeros((B, len(heads), len(rows)), dtype=np.float64)
    for hi, h in enumerate(heads):
        kh = [_f64(k[b, :, h]) for b in range(B)]
        vh = [_f64(v[b, :, h]) for b in range(B)]
        qh = [_f64(q[b, :, h]) for b in range(B)]
        for r0 in range(0, len(rows), block):
            r = rows[r0:r0 + block]
            if round_tiles is None:
                keep = keep_matrix(masks[h], grid, token_coords(grid, layout, r), ck) & real_k[None, :]
            else:
                keep = rounded_keep_rows(grid, layout, masks[h], round_tiles[0], round_tiles[1], r)
            for b in range(B):
                ob, lb = attention_rows(qh[b][r], kh[b], vh[b], keep, scale)
                o[b, r0:r0 + len(r), hi] = ob
                lse[b, hi, r0:r0 + len(r)] = lb
    return o, lse


def _f64(x):
    if hasattr(x, "detach"):  # a torch tensor: widen exactly, then hand to numpy
        x = x.detach().to("cpu")
        import torch
        return x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)
