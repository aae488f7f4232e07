"""ctypes binding of libvsa (include/vsa.h).

Argument marshalling only: every step of the path runs in the HIP library.  The
functions keep the C names; tensors are PyTorch device tensors (memory and streams
only), masks are ``workloads``-style dicts or ``vsa_mask_desc`` structs.  A missing
library raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvsa.so")

VSA_OK, VSA_ERR_INVALID_ARG, VSA_ERR_UNSUPPORTED, VSA_ERR_WORKSPACE, VSA_ERR_HIP = 0, -1, -2, -3, -4
VSA_BF16, VSA_F32 = 0, 1
VSA_LAYOUT_FRAME_MAJOR, VSA_LAYOUT_TILE_MAJOR, VSA_LAYOUT_POSITION_MAJOR, VSA_LAYOUT_TILE_PADDED = 0, 1, 2, 3
VSA_HEAD_LAYOUT_CALL, VSA_HEAD_LAYOUT_FRAME, VSA_HEAD_LAYOUT_TILE, VSA_HEAD_LAYOUT_POSITION = 0, 1, 2, 3
VSA_MASK_ALL, VSA_MASK_BOX, VSA_MASK_STRIPE, VSA_MASK_STA = 0, 1, 2, 3
VSA_TILE_EMPTY, VSA_TILE_FULL, VSA_TILE_BOUNDARY = 0, 1, 2
VSA_FWD_FORCE_MASK, VSA_FWD_REORDER_IO, VSA_FWD_WRITE_LSE, VSA_FWD_TILE_ALIGNED = 1, 2, 4, 8
VSA_CLASSIFY_ROUND_TILES = 1
VSA_WORDS_COMPACT = -1

_KINDS = {"all": VSA_MASK_ALL, "box": VSA_MASK_BOX, "stripe": VSA_MASK_STRIPE, "sta": VSA_MASK_STA}
_LAYOUTS = {"frame": VSA_LAYOUT_FRAME_MAJOR, "tile": VSA_LAYOUT_TILE_MAJOR, "position": VSA_LAYOUT_POSITION_MAJOR,
            "padded": VSA_LAYOUT_TILE_PADDED}
_HEAD_LAYOUTS = {"call": VSA_HEAD_LAYOUT_CALL, "frame": VSA_HEAD_LAYOUT_FRAME, "tile": VSA_HEAD_LAYOUT_TILE,
                 "position": VSA_HEAD_LAYOUT_POSITION}
_MASK_FIELDS = ("kind", "sink_frames", "rt", "rh", "rw", "Tw", "To", "Ts", "Sw", "So", "Ss",
                "win_t", "win_h", "win_w", "head_layout")


class vsa_grid(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("T", "Hg", "Wg", "tile_t", "tile_h", "tile_w")]


class vsa_mask_desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in _MASK_FIELDS]


class vsa_tile_lists(ctypes.Structure):
    _fields_ = [("cls", ctypes.c_void_p), ("n_full", ctypes.c_void_p), ("n_bnd", ctypes.c_void_p),
                ("full_idx", ctypes.c_void_p), ("bnd_idx", ctypes.c_void_p), ("bnd_offs", ctypes.c_void_p)]


class VsaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"libvsa status {status}: {message}")
        self.status = status


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32

_SIGNATURES = {
    "vsa_last_error": (ctypes.c_char_p, []),
    "vsa_unique_masks": (_I, [ctypes.POINTER(vsa_mask_desc), _I, ctypes.POINTER(_I), ctypes.POINTER(_I)]),
    "vsa_tile_counts": (_I, [ctypes.POINTER(vsa_grid), _I, _I, ctypes.POINTER(_I), ctypes.POINTER(_I)]),
    "vsa_seq_len": (_I, [ctypes.POINTER(vsa_grid), _I, ctypes.POINTER(_I)]),
    "vsa_tile_lists_bytes": (_I, [ctypes.POINTER(vsa_grid), _I, _I, _I, _I, ctypes.POINTER(ctypes.c_size_t)]),
    "vsa_tile_lists_carve": (_I, [ctypes.POINTER(vsa_grid), _I, _I, _I, _I, _P, ctypes.POINTER(vsa_tile_lists)]),
    "vsa_classify_tiles": (_I, [ctypes.POINTER(vsa_grid), _I, ctypes.POINTER(vsa_mask_desc), _I, _I, _I,
                                ctypes.POINTER(vsa_tile_lists), _P]),
    "vsa_classify_tiles_ex": (_I, [ctypes.POINTER(vsa_grid), _I, ctypes.POINTER(vsa_mask_desc), _I, _I, _I, _I,
                                   ctypes.POINTER(vsa_tile_lists), _P]),
    "vsa_fwd_workspace_bytes": (_I, [_I, _I, _I, _I, _I, _I, ctypes.POINTER(ctypes.c_size_t)]),
    "vsa_sparse_attn_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, ctypes.POINTER(vsa_grid), _I,
                                 ctypes.POINTER(vsa_mask_desc), ctypes.POINTER(vsa_tile_lists), _I, _I,
                                 ctypes.c_float, _I, _P, ctypes.c_size_t, _P]),
    "vsa_sparse_attn_fwd_ex": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, ctypes.POINTER(vsa_grid), _I,
                                    ctypes.POINTER(vsa_mask_desc), ctypes.POINTER(vsa_tile_lists), _I, _I,
                                    ctypes.c_float, _I, _P, _I, _P, ctypes.c_size_t, _P]),
    "vsa_sparse_attn_fwd_noalloc": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, ctypes.POINTER(vsa_grid), _I,
                                         ctypes.POINTER(vsa_mask_desc), ctypes.POINTER(vsa_tile_lists), _I, _I,
                                         ctypes.c_float, _I, _P, _I, _P]),
    "vsa_boundary_words": (_I, [ctypes.POINTER(vsa_grid), _I, ctypes.POINTER(vsa_mask_desc), _I, _I, _I,
                                ctypes.POINTER(vsa_tile_lists), _P, _I, _P]),
    "vsa_reorder_tokens": (_I, [_P, _P, _I, _I, _I, _I, ctypes.POINTER(vsa_grid), _I, _P]),
    "vsa_reorder_heads": (_I, [_P, _P, _I, _I, _I, _I, ctypes.POINTER(vsa_grid), ctypes.POINTER(_I), _I, _P]),
    "vsa_merge_partials": (_I, [ctypes.POINTER(_P), ctypes.POINTER(_P), _I, _P, _P, _I, _I, _I, _I, _I, _P]),
    "vsa_profile_workspace_bytes": (_I, [_I, _I, _I, _I, _I, _I, ctypes.POINTER(ctypes.c_size_t)]),
    "vsa_profile_heads": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, ctypes.POINTER(vsa_grid), _I, _P, _I,
                               ctypes.POINTER(vsa_mask_desc), _I, _P, _P, ctypes.c_float, _P,
                               ctypes.c_size_t, _P]),
}


def load(path=None):
    """Load libvsa.so (built in-tree by __graft_entry__.build()).  Raises if missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libvsa.so not found at {p}: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _check(status):
    if status != VSA_OK:
        raise VsaError(status, load().vsa_last_error().decode())


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
def make_grid(g):
    if isinstance(g, vsa_grid):
        return g
    return vsa_grid(g["T"], g["Hg"], g["Wg"], g.get("tile_t", 0), g.get("tile_h", 0), g.get("tile_w", 0))


def make_masks(masks):
    arr = (vsa_mask_desc * len(masks))()
    for i, m in enumerate(masks):
        if isinstance(m, vsa_mask_desc):
            arr[i] = m
            continue
        vals = dict(m)
        kind = vals["kind"]
        vals["kind"] = _KINDS[kind] if isinstance(kind, str) else int(kind)
        hl = vals.get("head_layout", 0)
        vals["head_layout"] = _HEAD_LAYOUTS[hl] if isinstance(hl, str) else int(hl)
        arr[i] = vsa_mask_desc(*[int(vals.get(f, 0)) for f in _MASK_FIELDS])
    return arr


def _layout(layout):
    return _LAYOUTS[layout] if isinstance(layout, str) else int(layout)


def _dtype(t):
    if t.dtype == torch.bfloat16:
        return VSA_BF16
    if t.dtype == torch.float32:
        return VSA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------
def vsa_last_error():
    return load().vsa_last_error().decode()


def vsa_unique_masks(masks):
    arr = make_masks(masks)
    hm = (_I * len(masks))()
    nu = _I()
    _check(load().vsa_unique_masks(arr, len(masks), hm, ctypes.byref(nu)))
    return list(hm), nu.value


def vsa_tile_counts(grid, Bq, Bk):
    nq, nk = _I(), _I()
    _check(load().vsa_tile_counts(ctypes.byref(make_grid(grid)), Bq, Bk, ctypes.byref(nq), ctypes.byref(nk)))
    return nq.value, nk.value


def vsa_seq_len(grid, layout):
    """Executed sequence length of a layout (T*Hg*Wg, or the padded grid's size)."""
    s = _I()
    _check(load().vsa_seq_len(ctypes.byref(make_grid(grid)), _layout(layout), ctypes.byref(s)))
    return s.value


def vsa_tile_lists_bytes(grid, layout, n_unique, Bq, Bk):
    """Bytes of one allocation holding every array of the tile lists (vsa_tile_lists_carve)."""
    n = ctypes.c_size_t()
    _check(load().vsa_tile_lists_bytes(ctypes.byref(make_grid(grid)), _layout(layout), n_unique, Bq, Bk,
                                       ctypes.byref(n)))
    return n.value


def alloc_tile_lists(grid, masks, Bq, Bk, device, with_cls=True, layout="frame"):
    """Tile lists for these masks in one device allocation, carved by the library
    (vsa_tile_lists_bytes / vsa_tile_lists_carve); returns a dict of tensor views."""
    S = vsa_seq_len(grid, layout)
    nQ, nK = -(-S // Bq), -(-S // Bk)
    head_map, U = vsa_unique_masks(masks)
    nbytes = vsa_tile_lists_bytes(grid, layout, U, Bq, Bk)
    buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    pad = (-buf.data_ptr()) % 256
    st = vsa_tile_lists()
    _check(load().vsa_tile_lists_carve(ctypes.byref(make_grid(grid)), _layout(layout), U, Bq, Bk,
                                       ctypes.c_void_p(buf.data_ptr() + pad), ctypes.byref(st)))

    def view(ptr, dtype, shape):
        off = ptr - buf.data_ptr()
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        return buf[off:off + n].view(dtype).view(shape)

    return {
        "cls": view(st.cls, torch.uint8, (U, nQ, nK)) if with_cls else None,
        "n_full": view(st.n_full, torch.int32, (U, nQ)),
        "n_bnd": view(st.n_bnd, torch.int32, (U, nQ)),
        "full_idx": view(st.full_idx, torch.int32, (U, nQ, nK)),
        "bnd_idx": view(st.bnd_idx, torch.int32, (U, nQ, nK)),
        "bnd_offs": view(st.bnd_offs, torch.int64, (U * nQ + 1,)),
        "head_map": head_map, "n_unique": U, "nQ": nQ, "nK": nK, "Bq": Bq, "Bk": Bk, "_buf": buf,
    }


def _lists_struct(t):
    return vsa_tile_lists(*[(t[n].data_ptr() if t.get(n) is not None else None)
                            for n in ("cls", "n_full", "n_bnd", "full_idx", "bnd_idx", "bnd_offs")])


def vsa_classify_tiles(grid, layout, masks, Bq, Bk, out=None, device="cuda", stream=None, with_cls=True,
                       round_tiles=False):
    """Classify tiles; returns the dict of device tensors (allocated when out is None).
    round_tiles: tile-aligned rounding (vsa_classify_tiles_ex, VSA_CLASSIFY_ROUND_TILES)."""
    if out is None:
        out = alloc_tile_lists(grid, masks, Bq, Bk, device, with_cls, layout)
    dev = out["n_full"].device
    arr = make_masks(masks)
    st = _lists_struct(out)
    flags = VSA_CLASSIFY_ROUND_TILES if round_tiles else 0
    _check(load().vsa_classify_tiles_ex(ctypes.byref(make_grid(grid)), _layout(layout), arr, len(masks), Bq, Bk,
                                        flags, ctypes.byref(st), _stream(stream, dev)))
    return out


def vsa_fwd_workspace_bytes(B, S, H, D, dtype, flags):
    n = ctypes.c_size_t()
    _check(load().vsa_fwd_workspace_bytes(B, S, H, D, dtype, flags, ctypes.byref(n)))
    return n.value


def vsa_boundary_words(grid, layout, masks, tiles, cap="compact", out=None, stream=None, n_entries=None):
    """Element masks of the listed boundary tiles for the bf16 forward.
    cap="compact" (default): one entry per listed boundary tile, list row r from entry
    tiles["bnd_offs"][r] (VSA_WORDS_COMPACT); the table size is the total of the lists,
    read back from the device (waits for the classification) unless n_entries gives it.
    cap=int: entries per list row (a forward derives the masks of entries past it);
    cap=None: the longest boundary list (also read back).  Returns {"words": int32
    device tensor (uint32 bit patterns) of shape [n_entries, Bq/32, 64] (compact) or
    [U, nQ, cap, Bq/32, 64], "cap": cap (VSA_WORDS_COMPACT when compact)}."""
    U, nQ, nK, Bq = tiles["n_unique"], tiles["nQ"], tiles["nK"], tiles["Bq"]
    dev = tiles["n_bnd"].device
    if cap == "compact":
        if tiles.get("bnd_offs") is None:
            raise ValueError("the compact table needs tile lists with bnd_offs")
        if n_entries is None:
            n_entries = int(tiles["bnd_offs"][-1])
        cap = VSA_WORDS_COMPACT
        shape = (max(1, int(n_entries)), Bq // 32, 64)
    else:
        if cap is None:
            cap = max(1, int(tiles["n_bnd"].max()))
        cap = int(cap)
        shape = (U, nQ, cap, Bq // 32, 64)
    if out is None:
        out = torch.empty(shape, dtype=torch.int32, device=dev)
    if tuple(out.shape) != shape or out.dtype != torch.int32 or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous int32 tensor of shape {shape}")
    st = _lists_struct(tiles)
    _check(load().vsa_boundary_words(ctypes.byref(make_grid(grid)), _layout(layout), make_masks(masks), len(masks),
                                     Bq, tiles["Bk"], ctypes.byref(st), _ptr(out), cap, _stream(stream, dev)))
    return {"words": out, "cap": cap}


def vsa_sparse_attn_fwd(q, k, v, grid, layout, masks, tiles, scale=0.0, flags=0, o=None, lse=None,
                        workspace=None, stream=None, words=None):
    """Block-sparse attention forward; q, k, v contiguous [B, S, H, D] on one device (S the
    executed length, or T*Hg*Wg with VSA_FWD_REORDER_IO).  words: the result of
    vsa_boundary_words for these lists (bf16 only; vsa_sparse_attn_fwd_ex).
    Returns (o, lse) with lse None unless VSA_FWD_WRITE_LSE is in flags."""
    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous [B, S, H, D]")
    B, S, H, D = q.shape
    dt = _dtype(q)
    for t in (k, v):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("q, k, v must have one shape and dtype")
    if o is None:
        o = torch.empty_like(q)
    if o.shape != q.shape or o.dtype != q.dtype or not o.is_contiguous():
        raise ValueError("o must be a contiguous tensor shaped like q")
    if (flags & VSA_FWD_WRITE_LSE) and lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    if lse is not None and (tuple(lse.shape) != (B, H, S) or lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError(f"lse must be a contiguous float32 tensor of shape {(B, H, S)}")
    need = vsa_fwd_workspace_bytes(B, vsa_seq_len(grid, layout), H, D, dt, flags)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _lists_struct(tiles)
    if words is None:
        _check(load().vsa_sparse_attn_fwd(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), dt, B, S, H, D, ctypes.byref(make_grid(grid)),
            _layout(layout), make_masks(masks), ctypes.byref(st), tiles["Bq"], tiles["Bk"], float(scale),
            flags, _ptr(workspace), ws_bytes, _stream(stream, q.device)))
    else:
        w = words["words"]
        if words["cap"] == VSA_WORDS_COMPACT:
            ok = w.dim() == 3 and tuple(w.shape[1:]) == (tiles["Bq"] // 32, 64) and tiles.get("bnd_offs") is not None
        else:
            ok = tuple(w.shape) == (tiles["n_unique"], tiles["nQ"], words["cap"], tiles["Bq"] // 32, 64)
        if not ok:
            raise ValueError("words do not match the tile lists")
        _check(load().vsa_sparse_attn_fwd_ex(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), dt, B, S, H, D, ctypes.byref(make_grid(grid)),
            _layout(layout), make_masks(masks), ctypes.byref(st), tiles["Bq"], tiles["Bk"], float(scale),
            flags, _ptr(w), words["cap"], _ptr(workspace), ws_bytes, _stream(stream, q.device)))
    return o, (lse if flags & VSA_FWD_WRITE_LSE else None)


def vsa_sparse_attn_fwd_noalloc(q, k, v, grid, layout, masks, tiles, o, lse=None, scale=0.0, flags=0, words=None,
                                stream=None):
    """The forward with its workspace in the library's static per-GPU scratch
    (vsa_sparse_attn_fwd_noalloc): the caller passes every output buffer (o, and lse with
    VSA_FWD_WRITE_LSE), and nothing is allocated on either side of the call."""
    for t in (q, k, v, o):
        if not t.is_contiguous():
            raise ValueError("q, k, v and o must be contiguous [B, S, H, D]")
    B, S, H, D = q.shape
    for t in (k, v, o):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("q, k, v and o must have one shape and dtype")
    if (flags & VSA_FWD_WRITE_LSE) and (lse is None or tuple(lse.shape) != (B, H, S)
                                        or lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError(f"VSA_FWD_WRITE_LSE needs lse, a contiguous float32 tensor of shape {(B, H, S)}")
    w, cap = (None, 0) if words is None else (words["words"], words["cap"])
    st = _lists_struct(tiles)
    _check(load().vsa_sparse_attn_fwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _dtype(q), B, S, H, D, ctypes.byref(make_grid(grid)),
        _layout(layout), make_masks(masks), ctypes.byref(st), tiles["Bq"], tiles["Bk"], float(scale), flags,
        _ptr(w), cap, _stream(stream, q.device)))
    return o, lse


def vsa_merge_partials(o_parts, lse_parts, o=None, lse=None, stream=None):
    """Merge partial results over disjoint key subsets.  o_parts: list of [B, S, H, D]
    device tensors (one dtype); lse_parts: list of float32 [B, H, S].  Returns (o, lse)."""
    n = len(o_parts)
    if n != len(lse_parts):
        raise ValueError("o_parts and lse_parts differ in length")
    B, S, H, D = o_parts[0].shape
    for t in list(o_parts) + list(lse_parts):
        if not t.is_contiguous():
            raise ValueError("parts must be contiguous")
    for t in o_parts:
        if t.shape != o_parts[0].shape or t.dtype != o_parts[0].dtype:
            raise ValueError("o_parts must share one shape and dtype")
    for t in lse_parts:
        if tuple(t.shape) != (B, H, S) or t.dtype != torch.float32:
            raise ValueError(f"lse_parts must be float32 tensors of shape {(B, H, S)}")
    if o is None:
        o = torch.empty_like(o_parts[0])
    if lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=o_parts[0].device)
    if o.shape != o_parts[0].shape or o.dtype != o_parts[0].dtype or not o.is_contiguous():
        raise ValueError("o must be a contiguous tensor shaped like the parts")
    if tuple(lse.shape) != (B, H, S) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError(f"lse must be a contiguous float32 tensor of shape {(B, H, S)}")
    op = (_P * n)(*[_ptr(t) for t in o_parts])
    lp = (_P * n)(*[_ptr(t) for t in lse_parts])
    _check(load().vsa_merge_partials(op, lp, n, _ptr(o), _ptr(lse), _dtype(o_parts[0]), B, S, H, D,
                                     _stream(stream, o_parts[0].device)))
    return o, lse


def vsa_reorder_tokens(src, grid, inverse=False, dst=None, stream=None):
    if not src.is_contiguous():
        raise ValueError("src must be contiguous [B, S, H, D]")
    B, S, H, D = src.shape
    if S != grid["T"] * grid["Hg"] * grid["Wg"]:
        raise ValueError(f"src holds {S} positions, the grid {grid['T'] * grid['Hg'] * grid['Wg']}")
    if dst is None:
        dst = torch.empty_like(src)
    if dst.shape != src.shape or dst.dtype != src.dtype or not dst.is_contiguous():
        raise ValueError("dst must be a contiguous tensor shaped like src")
    _check(load().vsa_reorder_tokens(_ptr(src), _ptr(dst), _dtype(src), B, H, D, ctypes.byref(make_grid(grid)),
                                     1 if inverse else 0, _stream(stream, src.device)))
    return dst


def vsa_reorder_heads(src, grid, layouts, inverse=False, dst=None, stream=None):
    """Per-head reorder of src [B, S, H, D]; layouts: H layout names or VSA_LAYOUT_* values.
    With the padded layout (all heads) dst has the padded length, or T*Hg*Wg when inverse."""
    if not src.is_contiguous():
        raise ValueError("src must be contiguous [B, S, H, D]")
    B, S, H, D = src.shape
    if len(layouts) != H:
        raise ValueError(f"{len(layouts)} layouts for {H} heads")
    if _layout(layouts[0]) != VSA_LAYOUT_TILE_PADDED and S != grid["T"] * grid["Hg"] * grid["Wg"]:
        raise ValueError(f"src holds {S} positions, the grid {grid['T'] * grid['Hg'] * grid['Wg']}")
    S_dst = S
    if _layout(layouts[0]) == VSA_LAYOUT_TILE_PADDED:
        S_src = vsa_seq_len(grid, "padded") if inverse else grid["T"] * grid["Hg"] * grid["Wg"]
        if S != S_src:
            raise ValueError(f"src holds {S} positions, the padded reorder reads {S_src}")
        S_dst = grid["T"] * grid["Hg"] * grid["Wg"] if inverse else vsa_seq_len(grid, "padded")
    if dst is None:
        dst = torch.empty((B, S_dst, H, D), dtype=src.dtype, device=src.device)
    if tuple(dst.shape) != (B, S_dst, H, D) or dst.dtype != src.dtype or not dst.is_contiguous():
        raise ValueError(f"dst must be a contiguous {src.dtype} tensor of shape {(B, S_dst, H, D)}")
    lay = (_I * H)(*[_layout(x) for x in layouts])
    _check(load().vsa_reorder_heads(_ptr(src), _ptr(dst), _dtype(src), B, H, D, ctypes.byref(make_grid(grid)),
                                    lay, 1 if inverse else 0, _stream(stream, src.device)))
    return dst


def vsa_profile_workspace_bytes(B, S, H, D, n_samples, n_cand):
    n = ctypes.c_size_t()
    _check(load().vsa_profile_workspace_bytes(B, S, H, D, n_samples, n_cand, ctypes.byref(n)))
    return n.value


def vsa_profile_heads(q, k, v, grid, layout, sample_idx, cands, scale=0.0, workspace=None, stream=None):
    """Sampled-query profiler; sample_idx int32 [H, n] on the device.  Returns (err [H, n_cand] f32,
    route [H] int32) device tensors."""
    B, S, H, D = q.shape
    n = sample_idx.shape[1]
    nc = len(cands)
    err = torch.empty((H, nc), dtype=torch.float32, device=q.device)
    route = torch.empty((H,), dtype=torch.int32, device=q.device)
    need = vsa_profile_workspace_bytes(B, S, H, D, n, nc)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check(load().vsa_profile_heads(
        _ptr(q), _ptr(k), _ptr(v), _dtype(q), B, S, H, D, ctypes.byref(make_grid(grid)), _layout(layout),
        _ptr(sample_idx.contiguous()), n, make_masks(cands), nc, _ptr(err), _ptr(route), float(scale),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream, q.device)))
    return err, route


def default_scale(D):
    return 1.0 / math.sqrt(D)
