"""Seeded synthetic inputs and the workload shapes used by tests and the benchmark.

This module holds no attention, mask or classification arithmetic.  It only
describes shapes and mask *parameters* (plain dicts) and draws random tensors
from seeded generators.  Both the CPU oracle (``oracle/``) and the HIP path
(``block_sparse_spatio_amd``) receive what this module produces; neither
imports the other, and neither imports this module.

Shapes follow the pages' workloads:
  * Wan-2.1-14B 720p latent grid 21 x 45 x 80 = 75,600 tokens, 40 heads, d=128
    (video-DiT attention blog, section on token counts; PSA notes, worked example);
  * HunyuanVideo 720p grid 30 x 48 x 80 = 115,200 tokens, 24 heads, d=128
    (Sliding Tile Attention explainer, Table 2 setup);
  * the TPU kernel measurement at 75.6K tokens, 10 heads, d=128
    (Sparse VideoGen on TPU, "implementing sparse attention on TPU").
The pages measured real models on prompt suites; no such data exists here, so
Q, K and V are iid N(0, 1) stand-ins of the same shapes.
"""
from __future__ import annotations

import numpy as np
import torch

# ---------------------------------------------------------------------------
# mask parameter records (plain dicts; the kind is a string)
# ---------------------------------------------------------------------------
_FIELDS = ("sink_frames", "rt", "rh", "rw", "Tw", "To", "Ts", "Sw", "So", "Ss",
           "win_t", "win_h", "win_w")


def _desc(kind, **kw):
    d = {"kind": kind}
    for f in _FIELDS:
        d[f] = int(kw.pop(f, 0))
    if kw:
        raise TypeError(f"unknown mask fields {sorted(kw)}")
    return d


def mask_all():
    """Keep every (query, key) pair: dense attention."""
    return _desc("all")


def mask_box(rt=-1, rh=-1, rw=-1, sink_frames=0):
    """Coordinate box |dt|<=rt, |dy|<=rh, |dx|<=rw (-1 = unbounded), OR key frame < sink_frames."""
    return _desc("box", rt=rt, rh=rh, rw=rw, sink_frames=sink_frames)


def mask_spatial(rt=1, sink_frames=1):
    """Spatial head: same or adjacent frames, whole frames, plus the first-frame sink."""
    return mask_box(rt=rt, rh=-1, rw=-1, sink_frames=sink_frames)


def mask_temporal(r=4, sink_frames=1):
    """Temporal head: |dy|,|dx| <= r in every frame, plus the first-frame sink."""
    return mask_box(rt=-1, rh=r, rw=r, sink_frames=sink_frames)


def mask_stripe(Tw, To, Ts, Sw, So, Ss, sink_frames=1):
    """PSA six-tuple stripe mask, plus the first-frame sink."""
    return _desc("stripe", Tw=Tw, To=To, Ts=Ts, Sw=Sw, So=So, Ss=Ss, sink_frames=sink_frames)


def mask_sta(win_t, win_h, win_w, sink_frames=0):
    """Sliding-tile window measured in tiles (tile size is part of the grid)."""
    return _desc("sta", win_t=win_t, win_h=win_h, win_w=win_w, sink_frames=sink_frames)


def with_head_layout(mask, layout):
    """The same mask on a head that runs in its own token order: "frame", "tile" or
    "position" (the library's head_layout; the mask itself is defined on coordinates)."""
    if layout not in ("frame", "tile", "position"):
        raise ValueError(f"unknown layout {layout!r}")
    return dict(mask, head_layout=layout)


def head_layouts(masks, layout):
    """Executed order of every head: its own head_layout, else the call's layout."""
    return [m.get("head_layout", layout) for m in masks]


def grid(T, Hg, Wg, tile=(0, 0, 0)):
    return {"T": int(T), "Hg": int(Hg), "Wg": int(Wg),
            "tile_t": int(tile[0]), "tile_h": int(tile[1]), "tile_w": int(tile[2])}


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------
def draw_stripe_tuples(H, seed):
    """Seeded per-head PSA six-tuples: each field independent and uniform over its set
    (T_w in {1,2,3}, T_o in {0,1}, T_s in {3,7,21}, S_w in {1..4}, S_o = 0, S_s in {80,3600})."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(H):
        Tw = int(rng.choice([1, 2, 3]))
        To = int(rng.choice([0, 1]))
        Ts = int(rng.choice([3, 7, 21]))
        Sw = int(rng.choice([1, 2, 3, 4]))
        Ss = int(rng.choice([80, 3600]))
        out.append(mask_stripe(Tw, To, Ts, Sw, 0, Ss, sink_frames=1))
    return out


def config(name):
    """Return the workload record for one of the five named configurations."""
    if name == "tiny":
        return dict(name="tiny", seed=1000, B=1, grid=grid(4, 8, 8), layout="frame",
                    H=2, D=64, dtype="f32", Bq=32, Bk=32,
                    masks=[mask_spatial(rt=1), mask_temporal(r=1)],
                    extra_masks=[mask_all(), mask_all()])
    if name == "wan_mixed":
        H = 40
        return dict(name="wan_mixed", seed=1001, B=1, grid=grid(21, 45, 80), layout="frame",
                    H=H, D=128, dtype="bf16", Bq=128, Bk=64,
                    masks=[mask_spatial(rt=1)] * 20 + [mask_temporal(r=4)] * 20,
                    # temporal heads gathered position-major (each position's frames
                    # contiguous), spatial heads in frame order
                    position_masks=[mask_spatial(rt=1)] * 20
                    + [with_head_layout(mask_temporal(r=4), "position")] * 20)
    if name == "wan_single":
        H = 10
        return dict(name="wan_single", seed=1002, B=1, grid=grid(21, 45, 80), layout="frame",
                    H=H, D=128, dtype="bf16", Bq=128, Bk=64, Bq_sweep=(64, 128, 256),
                    masks=[mask_spatial(rt=3)] * H, extra_masks=[mask_all()] * H)
    if name == "sta_hunyuan":
        H = 24
        return dict(name="sta_hunyuan", seed=1003, B=1, grid=grid(30, 48, 80, (6, 8, 8)),
                    layout="tile", H=H, D=128, dtype="bf16", Bq=128, Bk=64,
                    masks=[mask_sta(3, 3, 3)] * H)
    if name == "wan_sta_padded":
        # sliding tiles on the Wan 2.1 720p latent: the 3 x 8 x 16 block of the PSA notes'
        # worked example does not divide H = 45, so the grid is padded to 21 x 48 x 80
        H = 40
        return dict(name="wan_sta_padded", seed=1005, B=1, grid=grid(21, 45, 80, (3, 8, 16)),
                    layout="padded", H=H, D=128, dtype="bf16", Bq=128, Bk=64,
                    masks=[mask_sta(3, 3, 3)] * H)
    if name == "stripe_route":
        H = 40
        return dict(name="stripe_route", seed=1004, B=2, grid=grid(21, 45, 80), layout="frame",
                    H=H, D=128, dtype="bf16", Bq=128, Bk=64,
                    masks=draw_stripe_tuples(H, 1004), n_samples=64,
                    candidates=[mask_all(), mask_spatial(rt=1), mask_temporal(r=4)])
    raise KeyError(name)


CONFIG_NAMES = ("tiny", "wan_mixed", "wan_single", "sta_hunyuan", "stripe_route")


def seq_len(g):
    return g["T"] * g["Hg"] * g["Wg"]


# ---------------------------------------------------------------------------
# seeded tensors
# ---------------------------------------------------------------------------
def qkv(B, S, H, D, dtype="bf16", seed=0, device="cpu"):
    """Q, K, V iid N(0,1) of shape [B, S, H, D], drawn in that order from one seeded
    CPU generator in fp32; bf16 is the round-to-nearest-even cast of those values.
    Drawing always happens on the CPU so the values do not depend on the device."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    out = []
    for _ in range(3):
        x = torch.randn((B, S, H, D), generator=g, dtype=torch.float32)
        if dtype == "bf16":
            x = x.to(torch.bfloat16)
        elif dtype != "f32":
            raise ValueError(dtype)
        out.append(x.to(device) if device != "cpu" else x)
    return tuple(out)


def sample_rows(S, n, H, seed):
    """Per-head query sample indices, uniform without replacement from [0, S), sorted,
    shape [H, n] int32 (shared across the batch)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    idx = np.stack([np.sort(rng.choice(S, size=n, replace=False)) for _ in range(H)])
    return idx.astype(np.int32)
