"""The CPU oracle's attention on sampled rows of full-size workloads, spread over a
process pool (test infrastructure; imports only numpy and the oracle).

The full-size parity tests compare every query tile of a workload, several rows each,
on several heads: minutes of single-core oracle time (materialising the mask rows
dominates).  Each task is one (batch item, head): its query rows and that head's keys
and values go to a worker (spawned, so it shares nothing with a process that uses the
GPU), which runs oracle.attention on them unchanged with one BLAS thread.
"""
from __future__ import annotations

import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

import oracle


def _init():
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)


def _task(args):
    b, h, qr, kh, vh, g, layout, mask, rows, round_tiles = args
    # the oracle takes [B, S, H, D] and the query rows at their positions: place the
    # sampled rows in a zero tensor (only those rows are read)
    q = np.zeros((1, kh.shape[0], 1, kh.shape[1]), dtype=np.float32)
    q[0, rows, 0] = qr
    o, lse = oracle.attention(q, kh[None, :, None, :], vh[None, :, None, :], g, layout, [mask], rows=rows,
                              round_tiles=round_tiles)
    return b, h, o[0, :, 0], lse[0, 0]


def workers():
    """Pool size: the host's cores, at most 16 (one GPU's share of a GPU machine)."""
    return max(1, min(16, os.cpu_count() or 1))


def _f32_bhsd(x):
    """[B, S, H, D] tensor or array -> float32 [B, H, S, D] array (bf16 widens exactly)."""
    if hasattr(x, "detach"):
        return x.detach().float().cpu().permute(0, 2, 1, 3).contiguous().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32).transpose(0, 2, 1, 3))


def attention_rows(q, k, v, g, layout, masks, rows, pairs, round_tiles=None):
    """Oracle output and lse of query positions `rows` for each (batch item, head) in
    `pairs`.  q, k, v: [B, S, H, D] tensors or arrays.  Returns
    {(b, h): (o [len(rows), D] fp64, lse [len(rows)] fp64)}."""
    rows = np.asarray(rows, dtype=np.int64)
    qa, ka, va = _f32_bhsd(q), _f32_bhsd(k), _f32_bhsd(v)
    tasks = [(b, h, qa[b, h][rows], ka[b, h], va[b, h], g, layout, masks[h], rows, round_tiles) for b, h in pairs]
    out = {}
    ctx = mp.get_context("spawn")
    with ProcessPoolExecutor(min(workers(), len(tasks)), mp_context=ctx, initializer=_init) as ex:
        for b, h, o, lse in ex.map(_task, tasks):
            out[(b, h)] = (o, lse)
    return out


def _profile_task(args):
    h, qh, kh, vh, g, layout, idx, cands = args
    err, route = oracle.profile_heads(qh[:, :, None, :], kh[:, :, None, :], vh[:, :, None, :], g, layout,
                                      idx[None, :], cands)
    return h, err[0], int(route[0])


def profile_heads(q, k, v, g, layout, sample_idx, cands, heads):
    """oracle.profile_heads for each head in `heads`, one head per task.  q, k, v:
    [B, S, H, D]; sample_idx: int [H, n].  Returns (err fp64 [len(heads), n_cand], route
    int32 [len(heads)])."""
    qa, ka, va = _f32_bhsd(q), _f32_bhsd(k), _f32_bhsd(v)
    idx = np.asarray(sample_idx)
    tasks = [(h, qa[:, h], ka[:, h], va[:, h], g, layout, idx[h], cands) for h in heads]
    err = np.zeros((len(heads), len(cands)))
    route = np.zeros(len(heads), dtype=np.int32)
    pos = {h: i for i, h in enumerate(heads)}
    ctx = mp.get_context("spawn")
    with ProcessPoolExecutor(min(workers(), len(tasks)), mp_context=ctx, initializer=_init) as ex:
        for h, e, r in ex.map(_profile_task, tasks):
            err[pos[h]] = e
            route[pos[h]] = r
    return err, route
