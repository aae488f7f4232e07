"""Write tests/golden/class_maps_full.json: the oracle's tile classes of every distinct
mask of the full-size workloads, in every token order those workloads run in.

Test infrastructure.  This script calls only the CPU oracle (``oracle``) and the
shape/mask records of ``workloads``; nothing here comes from the HIP library.  For
each case and each distinct mask descriptor it stores

  sha256   SHA-256 of the class map, uint8 [nQ, nK] in C order (0 empty, 1 full,
           2 boundary; Sparse VideoGen on TPU, "logical sparsity is not physical
           sparsity"), so a GPU class map can be compared bit for bit;
  n_full, n_bnd   per query tile, run-length coded as "value*count" tokens, so that a
           mismatch can be located by query tile;
  heads    the heads of the case that use the descriptor.

The lists of FULL and BOUNDARY key tiles are the ascending positions of those classes
in each map row, so the map fixes them too.

Usage:  python tests/golden/make_class_goldens.py [--jobs N] [--only CASE ...]
(about half an hour on 8 cores: the stripe layer has 36 distinct masks in two orders).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ProcessPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads as W  # noqa: E402
from oracle.classify import classify_qtile  # noqa: E402

OUT = os.path.join(ROOT, "tests", "golden", "class_maps_full.json")
CHUNK = 48  # query tiles per task


def stripe_orders(masks):
    """The stripe layer's per-head orders under the fixed rule used by the tests: a stripe
    whose spatial period is one row (S_s = Wg = 80) runs tile-major over one-column tiles
    1 x 45 x 1 (each frame read column by column, so the column band is contiguous), the
    others position-major."""
    return [W.with_head_layout(m, "tile" if m["Ss"] == 80 else "position") for m in masks]


def cases():
    """(name, grid, call layout, masks, Bq, Bk, round_tiles) of every full-size case."""
    out = []
    c = W.config("wan_mixed")
    out.append(("wan_mixed/frame", c["grid"], "frame", c["masks"], 128, 64, False))
    out.append(("wan_mixed/position", c["grid"], "frame", c["position_masks"], 128, 64, False))
    out.append(("wan_mixed/frame/b3", c["grid"], "frame", c["masks"], 128, 64, True))
    c = W.config("wan_single")
    for bq in c["Bq_sweep"]:
        out.append((f"wan_single/bq{bq}", c["grid"], "frame", c["masks"], bq, 64, False))
    out.append(("wan_single/bq128/b3", c["grid"], "frame", c["masks"], 128, 64, True))
    out.append(("wan_single/bq128/all", c["grid"], "frame", c["extra_masks"], 128, 64, False))
    c = W.config("sta_hunyuan")
    out.append(("sta_hunyuan", c["grid"], "tile", c["masks"], 128, 64, False))
    c = W.config("wan_sta_padded")
    out.append(("wan_sta_padded", c["grid"], "padded", c["masks"], 128, 64, False))
    c = W.config("stripe_route")
    out.append(("stripe_route/frame", c["grid"], "frame", c["masks"], 128, 64, False))
    g = W.grid(21, 45, 80, (1, 45, 1))
    out.append(("stripe_route/column_position", g, "frame", stripe_orders(c["masks"]), 128, 64, False))
    return out


def distinct(masks, layout):
    """Distinct (descriptor, executed order) pairs and the heads using each, in first-use order."""
    seen = {}
    for h, m in enumerate(masks):
        lay = m.get("head_layout", layout)
        key = json.dumps(dict(m, head_layout=lay), sort_keys=True)
        seen.setdefault(key, []).append(h)
    return [(json.loads(k), heads) for k, heads in seen.items()]


def _task(args):
    g, lay, desc, Bq, Bk, rnd, q0, q1 = args
    S = oracle.seq_len(g, lay)
    desc = {k: v for k, v in desc.items() if k != "head_layout"}
    return q0, np.stack([classify_qtile(g, lay, desc, S, Bq, Bk, qt, rnd) for qt in range(q0, q1)])


def rle(a):
    toks, i = [], 0
    a = [int(x) for x in a]
    while i < len(a):
        j = i
        while j < len(a) and a[j] == a[i]:
            j += 1
        toks.append(f"{a[i]}*{j - i}" if j - i > 1 else f"{a[i]}")
        i = j
    return " ".join(toks)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=max(1, (os.cpu_count() or 2) - 1))
    ap.add_argument("--only", nargs="*", default=None)
    args = ap.parse_args()
    old = {}
    if os.path.exists(OUT):
        with open(OUT) as f:
            old = {c["case"]: c for c in json.load(f)["cases"]}
    result = dict(old)
    with ProcessPoolExecutor(args.jobs) as ex:
        for name, g, layout, masks, Bq, Bk, rnd in cases():
            if args.only is not None and name not in args.only:
                continue
            t0 = time.time()
            entries = []
            for desc, heads in distinct(masks, layout):
                lay = desc["head_layout"]
                S = oracle.seq_len(g, lay)
                nQ, nK = -(-S // Bq), -(-S // Bk)
                cls = np.zeros((nQ, nK), dtype=np.uint8)
                tasks = [(g, lay, desc, Bq, Bk, rnd, q0, min(nQ, q0 + CHUNK)) for q0 in range(0, nQ, CHUNK)]
                for q0, rows in ex.map(_task, tasks):
                    cls[q0:q0 + rows.shape[0]] = rows
                entries.append({"desc": desc, "heads": heads, "nQ": nQ, "nK": nK,
                                "sha256": hashlib.sha256(np.ascontiguousarray(cls).tobytes()).hexdigest(),
                                "n_full": rle((cls == oracle.FULL).sum(1)),
                                "n_bnd": rle((cls == oracle.BOUNDARY).sum(1))})
            result[name] = {"case": name, "grid": g, "layout": layout, "Bq": Bq, "Bk": Bk, "round_tiles": rnd,
                            "masks": entries}
            print(f"{name}: {len(entries)} distinct masks, {time.time() - t0:.0f} s", flush=True)
            order = [c[0] for c in cases()]
            with open(OUT, "w") as f:
                json.dump({"note": "oracle tile classes of the full-size workloads; written by "
                                   "tests/golden/make_class_goldens.py",
                           "cases": [result[n] for n in order if n in result]}, f, indent=1)
                f.write("\n")


if __name__ == "__main__":
    main()
