"""Benchmark of the block-sparse video attention hot path on one MI355X.

One step = one pass of the path over one batch of synthetic input: tile
classification of the layer's masks (vsa_classify_tiles), the element masks of the
listed boundary tiles (vsa_boundary_words, bf16 unless --no-mask-words), and the
sparse attention forward that reads them (vsa_sparse_attn_fwd_ex).  The default workload is the Wan-2.1-14B
720p-shaped mixed-head layer (21 x 45 x 80 = 75,600 tokens, 40 heads, d = 128,
bf16, heads 0-19 spatial and 20-39 temporal with a frame-0 sink, tiles 128 x 64).

Prints one JSON line.  `value` is effective TFLOP/s over executed tiles
(4*D FLOP per executed (query, key) pair, the pages' convention) for the whole
step; the roofline block reports the attention kernel alone against the bf16
dense MFMA peak, timed with HIP events on the stream it runs on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA (no structured sparsity)
PEAK_HBM_GBS = 8000.0
METRIC = "sparse-attn ms/call + effective TFLOP/s at 75.6K tokens; % of bf16 MFMA peak"
ATTN_SOURCES = ["attn_bf16.hip", "lds_pipe.h", "vsa_geom.h"]


def kernel_hash():
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(os.path.join(ROOT, "block_sparse_spatio_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# FLOP accounting
# ---------------------------------------------------------------------------
def executed_pairs(tiles, head_map, B, S):
    """Sum over heads and batch of |R|*|C| over the listed (executed) tiles."""
    import torch
    Bq, Bk, nQ, nK = tiles["Bq"], tiles["Bk"], tiles["nQ"], tiles["nK"]
    rows = torch.full((nQ,), Bq, dtype=torch.int64)
    rows[-1] = S - (nQ - 1) * Bq
    last_cols = S - (nK - 1) * Bk
    nf = tiles["n_full"].cpu().long()
    nb = tiles["n_bnd"].cpu().long()
    # a tail key tile is never FULL; it is the last entry of a boundary list when listed
    bi = tiles["bnd_idx"].cpu()
    idx = (nb - 1).clamp(min=0)
    last = torch.gather(bi, 2, idx.unsqueeze(-1)).squeeze(-1).long()
    has_tail = (nb > 0) & (last == nK - 1)
    cols = (nf + nb) * Bk - has_tail.long() * (Bk - last_cols)
    per_slot = (cols * rows.unsqueeze(0)).sum(dim=1)  # [U]
    total = 0
    for h in range(len(head_map)):
        total += int(per_slot[head_map[h]])
    return total * B


def kept_pairs(g, masks, B):
    """Exact kept (query, key) pairs of frame-major coordinate masks, counted per frame
    pair from per-axis difference histograms (measurement accounting)."""
    T, Hg, Wg = g["T"], g["Hg"], g["Wg"]
    HW = Hg * Wg
    total = 0
    cache = {}
    for m in masks:
        key = tuple(sorted(m.items()))
        if key in cache:
            total += cache[key]
            continue
        sink = m["sink_frames"]
        if m["kind"] == "all":
            c = (T * HW) ** 2
        elif m["kind"] == "box":
            def axis(n, r):
                if r < 0:
                    return n * n
                d = np.arange(-(n - 1), n)
                return int(np.sum((n - np.abs(d))[np.abs(d) <= r]))
            within = axis(Hg, m["rh"]) * axis(Wg, m["rw"])
            c = 0
            for tq in range(T):
                for tk in range(T):
                    if tk < sink:
                        c += HW * HW
                    elif m["rt"] < 0 or abs(tk - tq) <= m["rt"]:
                        c += within
        elif m["kind"] == "stripe":
            ds = np.arange(-(HW - 1), HW)
            intra = (np.abs(ds - m["So"]) % m["Ss"]) <= m["Sw"] - 1
            n_intra = int(np.sum((HW - np.abs(ds))[intra]))
            c = 0
            for tq in range(T):
                for tk in range(T):
                    if tk < sink:
                        c += HW * HW
                    elif (abs(tk - tq - m["To"]) % m["Ts"]) <= m["Tw"] - 1:
                        c += n_intra
        elif m["kind"] == "sta":
            # the window is a product over axes: count (query, key) coordinate pairs per
            # axis (tiles counted over the axis padded up to whole tiles)
            c = 1
            for N, b, w in ((T, g["tile_t"], m["win_t"]), (Hg, g["tile_h"], m["win_h"]), (Wg, g["tile_w"], m["win_w"])):
                n = -(-N // b)
                a = np.arange(N) // b
                start = np.minimum(np.maximum(a - w // 2, 0), max(n - w, 0))
                c *= int(((a[None, :] >= start[:, None]) & (a[None, :] < start[:, None] + w)).sum())
        else:
            raise ValueError(m["kind"])
        cache[key] = c
        total += c
    return total * B


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the same workload
# ---------------------------------------------------------------------------
def cpu_baseline(cfg, q, k, v, tiles, head_map, budget_s=12.0):
    import oracle
    from threadpoolctl import threadpool_info

    g, masks = cfg["grid"], cfg["masks"]
    S = g["T"] * g["Hg"] * g["Wg"]
    Bq, Bk, nQ, nK = tiles["Bq"], tiles["Bk"], tiles["nQ"], tiles["nK"]
    nf = tiles["n_full"].cpu().numpy()
    nb = tiles["n_bnd"].cpu().numpy()
    # heads of both kinds, query tiles spread over the sequence
    uniq = sorted(set(head_map))
    heads = [head_map.index(u) for u in uniq][:4]
    rng = np.random.default_rng(0)
    order = rng.permutation(nQ)
    work = 0
    rows_done = 0
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < budget_s and i < nQ:
        qt = int(order[i])
        i += 1
        rows = np.arange(qt * Bq, min(S, (qt + 1) * Bq))
        oracle.attention(q[:1], k[:1], v[:1], g, "frame", masks, rows=rows, heads=heads)
        for h in heads:
            u = head_map[h]
            work += (int(nf[u, qt]) + int(nb[u, qt])) * Bk * len(rows) * 4 * cfg["D"]
        rows_done += len(rows) * len(heads)
    dt = time.perf_counter() - t0
    threads = 1
    for info in threadpool_info():
        if info.get("user_api") == "blas":
            threads = max(threads, int(info.get("num_threads", 1)))
    return {"value": work / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows_done} query rows ({len(heads)} heads x {i} query tiles of {Bq}) of batch 0, "
                      f"fp64 NumPy, {dt:.1f} s; work counted as executed-tile FLOP of those rows"}


# ---------------------------------------------------------------------------
def traffic_from_profiles(khash, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, when it was
    taken on the current kernel source and on this workload in its default run; else
    None."""
    path = os.path.join(ROOT, "profiles", "attn_bf16_wan_mixed_traffic.json")
    if workload is None or not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_hash") != khash or rec.get("workload") != workload:
        return None
    return rec.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="wan_mixed")
    ap.add_argument("--Bq", type=int, default=None)
    ap.add_argument("--flags", type=int, default=0, help="extra VSA_FWD_* flags (e.g. 1 = B1 ablation)")
    ap.add_argument("--round-tiles", action="store_true",
                    help="tile-aligned rounding of the masks (B3): rounded lists, forward with VSA_FWD_TILE_ALIGNED")
    ap.add_argument("--temporal-layout", choices=("frame", "position"), default="frame",
                    help="executed order of the temporal heads of wan_mixed: position = each spatial "
                         "position's frames contiguous, reordered inside the call (frame-major I/O)")
    ap.add_argument("--head-layouts", choices=("workload", "auto"), default="workload",
                    help="auto: give every head the order (frame-, position- or tile-major over a "
                         "(1, Hg, w) grid tile) in which the classifier's lists cost least; q/k/v/o stay "
                         "frame-major")
    ap.add_argument("--no-mask-words", action="store_true",
                    help="let the forward derive the boundary tiles' element masks itself instead of "
                         "precomputing them in the step (vsa_boundary_words)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the comparison runs (all-keep dense; position-major temporal heads)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run the tile-major reorder (a plain row copy) over a MIB-sized tensor, "
                         "5 times: the known-size kernel that calibrates HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by head with no exchange; see the design notes)", file=sys.stderr)
        return 2

    import torch

    import block_sparse_spatio_amd as vsa
    import workloads as W
    from block_sparse_spatio_amd.layouts import choose_head_layouts

    vsa.load()
    dev = torch.device("cuda:0")
    if args.copy_probe:
        gp = W.grid(30, 48, 80, (6, 8, 8))
        Sp = W.seq_len(gp)
        Hp = max(1, (args.copy_probe << 20) // (Sp * 128 * 2))
        x = torch.randn((1, Sp, Hp, 128), device=dev).to(torch.bfloat16)
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        for _ in range(5):
            vsa.vsa_reorder_tokens(x, gp, dst=y)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": x.numel() * 2, "copy_probe_bytes_written": y.numel() * 2,
                          "launches": 5}), flush=True)
        return 0
    cfg = W.config(args.config)
    g, layout, masks = cfg["grid"], cfg["layout"], cfg["masks"]
    if args.temporal_layout == "position":
        if "position_masks" not in cfg:
            print(f"--temporal-layout position needs a workload with temporal heads (wan_mixed), not {args.config}",
                  file=sys.stderr)
            return 2
        masks = cfg["position_masks"]
    B, H, D = cfg["B"], cfg["H"], cfg["D"]
    S = W.seq_len(g)
    Bq = args.Bq or cfg["Bq"]
    Bk = cfg["Bk"]
    if args.head_layouts == "auto":
        if layout != "frame":
            print(f"--head-layouts auto needs a frame-major workload, not {args.config}", file=sys.stderr)
            return 2
        g, masks = choose_head_layouts(g, masks, Bq, Bk, dev)
    head_lays = W.head_layouts(masks, layout)
    reorder = any(x != "frame" for x in head_lays)
    flags = args.flags | (vsa.VSA_FWD_REORDER_IO if reorder else 0) | (vsa.VSA_FWD_TILE_ALIGNED if args.round_tiles else 0)
    print(f"[bench] {args.config}: B={B} S={S} H={H} D={D} Bq={Bq} Bk={Bk} drawing inputs", file=sys.stderr,
          flush=True)
    q, k, v = W.qkv(B, S, H, D, cfg["dtype"], seed=cfg["seed"])
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty_like(qd)
    head_map, U = vsa.vsa_unique_masks(masks)
    tiles = vsa.alloc_tile_lists(g, masks, Bq, Bk, dev, with_cls=False, layout=layout)
    S_exec = vsa.vsa_seq_len(g, layout)  # executed length (padded grids are longer)
    ws_bytes = vsa.vsa_fwd_workspace_bytes(B, S_exec, H, D, vsa.VSA_BF16 if cfg["dtype"] == "bf16" else vsa.VSA_F32,
                                           flags)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    stream = torch.cuda.current_stream(dev)
    # the boundary tiles' element masks, computed in every step into the compact table
    # (one entry per listed boundary tile, rows indexed by the classifier's prefix sum of
    # the list lengths); the masks are static per shape, so the table is sized once here,
    # from one classification, and the timed step reads nothing back to the host
    use_words = cfg["dtype"] == "bf16" and not args.round_tiles and not args.no_mask_words
    words = None
    if use_words:
        vsa.vsa_classify_tiles(g, layout, masks, Bq, Bk, out=tiles, stream=stream)
        words = vsa.vsa_boundary_words(g, layout, masks, tiles, stream=stream)
        n_entries = int(words["words"].shape[0])

    # the sampled-query profiler is part of the step when the workload routes heads
    profile = "candidates" in cfg
    if profile:
        sidx = torch.from_numpy(W.sample_rows(S, cfg["n_samples"], H, cfg["seed"] + 1)).to(dev)
        pws = torch.empty(vsa.vsa_profile_workspace_bytes(B, S, H, D, cfg["n_samples"], len(cfg["candidates"])),
                          dtype=torch.uint8, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if profile:
            vsa.vsa_profile_heads(qd, kd, vd, g, layout, sidx, cfg["candidates"], workspace=pws, stream=stream)
        if ev is not None:
            ev[3].record(stream)
        vsa.vsa_classify_tiles(g, layout, masks, Bq, Bk, out=tiles, stream=stream, round_tiles=args.round_tiles)
        if ev is not None:
            ev[1].record(stream)
        if use_words:
            vsa.vsa_boundary_words(g, layout, masks, tiles, out=words["words"], stream=stream, n_entries=n_entries)
        if ev is not None:
            ev[4].record(stream)
        vsa.vsa_sparse_attn_fwd(qd, kd, vd, g, layout, masks, tiles, flags=flags, o=o, workspace=ws, stream=stream,
                                words=words)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    prof_ms = [e[0].elapsed_time(e[3]) for e in evs]
    cls_ms = [e[3].elapsed_time(e[1]) for e in evs]
    words_ms = [e[1].elapsed_time(e[4]) for e in evs]
    fwd_ms = [e[4].elapsed_time(e[2]) for e in evs]
    attn_ms = float(np.mean(fwd_ms))

    f_exec = 4.0 * D * executed_pairs(tiles, head_map, B, S_exec)
    n_full_tiles = int(tiles["n_full"][torch.as_tensor(head_map, device=dev).long()].sum())
    n_bnd_tiles = int(tiles["n_bnd"][torch.as_tensor(head_map, device=dev).long()].sum())
    f_kept = 4.0 * D * kept_pairs(g, masks, B)
    f_dense = 4.0 * D * float(S) * S * H * B
    value = f_exec / (ms_step * 1e-3) / 1e12
    achieved = f_exec / (attn_ms * 1e-3) / 1e12

    dense = {}
    if not args.no_dense:
        all_masks = [W.mask_all()] * H
        # dense attention in the call's layout (a frame-major call needs no reorder)
        dflags = flags & ~vsa.VSA_FWD_REORDER_IO if layout == "frame" else flags
        dt_tiles = vsa.vsa_classify_tiles(g, layout, all_masks, Bq, Bk, device=dev, with_cls=False)
        for _ in range(2):
            vsa.vsa_sparse_attn_fwd(qd, kd, vd, g, layout, all_masks, dt_tiles, flags=dflags, o=o, workspace=ws)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n_dense = 3
        e0.record(stream)
        for _ in range(n_dense):
            vsa.vsa_sparse_attn_fwd(qd, kd, vd, g, layout, all_masks, dt_tiles, flags=dflags, o=o, workspace=ws)
        e1.record(stream)
        torch.cuda.synchronize()
        d_ms = e0.elapsed_time(e1) / n_dense
        dense = {"dense_ms_per_call": round(d_ms, 3), "speedup_vs_dense": round(d_ms / attn_ms, 3),
                 "dense_tflops": round(f_dense / (d_ms * 1e-3) / 1e12, 1)}
        del dt_tiles

    extra = {}
    if profile:
        extra["profile_ms"] = round(float(np.mean(prof_ms)), 4)
        extra["profile_kv_gbs"] = round(2.0 * B * S * H * D * 2 / (np.mean(prof_ms) * 1e-3) / 1e9, 1)
    if reorder:
        # the per-head token reorder alone, on one tensor: HBM GB/s (read + write); the
        # destination holds the executed order (the padded length for a padded grid)
        y = torch.empty((B, S_exec, H, D), dtype=qd.dtype, device=dev)
        vsa.vsa_reorder_heads(qd, g, head_lays, dst=y, stream=stream)
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        r0.record(stream)
        for _ in range(5):
            vsa.vsa_reorder_heads(qd, g, head_lays, dst=y, stream=stream)
        r1.record(stream)
        torch.cuda.synchronize()
        r_ms = r0.elapsed_time(r1) / 5
        extra["reorder_ms_per_tensor"] = round(r_ms, 4)
        extra["reorder_gbs"] = round((qd.numel() + y.numel()) * qd.element_size() / (r_ms * 1e-3) / 1e9, 1)
        del y

    if "position_masks" in cfg and args.temporal_layout == "frame" and not args.round_tiles and not args.no_dense:
        # the same layer with its temporal heads attended position-major (reorder of
        # q, k, v and o inside the call): classify + forward per step, and the forward alone
        pm = cfg["position_masks"]
        pm_tiles = vsa.alloc_tile_lists(g, pm, Bq, Bk, dev, with_cls=False, layout=layout)
        pm_flags = flags | vsa.VSA_FWD_REORDER_IO
        pm_ws = torch.empty(vsa.vsa_fwd_workspace_bytes(B, S, H, D, vsa.VSA_BF16, pm_flags), dtype=torch.uint8,
                            device=dev)
        pm_words = None
        if use_words:
            vsa.vsa_classify_tiles(g, layout, pm, Bq, Bk, out=pm_tiles, stream=stream)
            pm_words = vsa.vsa_boundary_words(g, layout, pm, pm_tiles, stream=stream)
            pm_entries = int(pm_words["words"].shape[0])

        def pm_step():
            vsa.vsa_classify_tiles(g, layout, pm, Bq, Bk, out=pm_tiles, stream=stream)
            if use_words:
                vsa.vsa_boundary_words(g, layout, pm, pm_tiles, out=pm_words["words"], stream=stream,
                                       n_entries=pm_entries)
            vsa.vsa_sparse_attn_fwd(qd, kd, vd, g, layout, pm, pm_tiles, flags=pm_flags, o=o, workspace=pm_ws,
                                    stream=stream, words=pm_words)

        for _ in range(2):
            pm_step()
        p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n_pm = 5
        p0.record(stream)
        for _ in range(n_pm):
            pm_step()
        p1.record(stream)
        torch.cuda.synchronize()
        pm_ms = p0.elapsed_time(p1) / n_pm
        hm_pm, _ = vsa.vsa_unique_masks(pm)
        pm_exec = 4.0 * D * executed_pairs(pm_tiles, hm_pm, B, S)
        extra["temporal_heads_position_major"] = {
            "ms_per_step": round(pm_ms, 4), "speedup_vs_frame_major": round(ms_step / pm_ms, 3),
            "executed_tflop": round(pm_exec / 1e12, 3),
            "note": "heads 20-39 attended in position-major order, q/k/v/o reordered inside the call"}
        del pm_tiles, pm_ws, pm_words

    # merging two partial results of this shape (LSE merge): HBM GB/s of the
    # algorithmic traffic (2 parts read + 1 output written, with their LSE rows)
    pa = torch.randn_like(qd)
    pb = torch.randn_like(qd)
    la = torch.randn((B, H, S), dtype=torch.float32, device=dev)
    lb = torch.randn((B, H, S), dtype=torch.float32, device=dev)
    mo = torch.empty_like(qd)
    ml = torch.empty_like(la)
    vsa.vsa_merge_partials([pa, pb], [la, lb], o=mo, lse=ml, stream=stream)
    m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    m0.record(stream)
    for _ in range(5):
        vsa.vsa_merge_partials([pa, pb], [la, lb], o=mo, lse=ml, stream=stream)
    m1.record(stream)
    torch.cuda.synchronize()
    m_ms = m0.elapsed_time(m1) / 5
    extra["merge2_ms"] = round(m_ms, 4)
    extra["merge2_gbs"] = round((3.0 * qd.numel() * qd.element_size() + 3.0 * la.numel() * 4) / (m_ms * 1e-3) / 1e9, 1)
    del pa, pb, la, lb, mo, ml

    khash = kernel_hash()
    # the counters were taken on the workload's default run (its Bq, flags, orders and
    # the precomputed mask words)
    default_run = (args.Bq is None and args.flags == 0 and not args.round_tiles and args.temporal_layout == "frame"
                   and args.head_layouts == "workload" and not args.no_mask_words)
    traffic = traffic_from_profiles(khash, args.config if default_run else None)
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic",
        "config": {"workload": args.config, "B": B, "S": S, "H": H, "D": D, "grid": [g["T"], g["Hg"], g["Wg"]],
                   "layout": layout, "Bq": Bq, "Bk": Bk, "masks": sorted({m["kind"] for m in masks}),
                   "unique_masks": U, "flags": flags, "tile_rounding": bool(args.round_tiles),
                   "head_layouts": {x: head_lays.count(x) for x in sorted(set(head_lays))},
                   "grid_tile": [g.get("tile_t", 0), g.get("tile_h", 0), g.get("tile_w", 0)]},
        "attn_ms_per_call": round(attn_ms, 4),
        "attn_ms_p10_p90": [round(float(np.percentile(fwd_ms, 10)), 4), round(float(np.percentile(fwd_ms, 90)), 4)],
        "classify_ms": round(float(np.mean(cls_ms)), 4),
        "mask_words": use_words,
        "mask_words_ms": round(float(np.mean(words_ms)), 4) if use_words else None,
        "mask_words_table_mib": round(words["words"].numel() * 4 / 2**20, 1) if use_words else None,
        "boundary_tile_frac": round(n_bnd_tiles / max(1, n_full_tiles + n_bnd_tiles), 5),
        **extra,
        "tflops_executed_attn": round(achieved, 2),
        "pct_of_bf16_peak": round(100.0 * achieved / PEAK_BF16_TFLOPS, 2),
        "tflops_kept": round(f_kept / (attn_ms * 1e-3) / 1e12, 2),
        "tflops_dense_equiv": round(f_dense / (attn_ms * 1e-3) / 1e12, 2),
        "executed_tflop": round(f_exec / 1e12, 3),
        "kept_tflop": round(f_kept / 1e12, 3),
        "dense_tflop": round(f_dense / 1e12, 3),
        **dense,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "kernel": "attn_fwd_bf16_kernel", "kernel_hash": khash},
    }
    if not args.no_cpu and not reorder:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(cfg, q, k, v, tiles, head_map)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
