"""The C ABI: the library loads, exports every symbol include/vsa.h declares, and its
host-only helpers and argument validation work without a GPU (no compute calls)."""
import ctypes
import os
import re

import pytest

import block_sparse_spatio_amd as vsa
import workloads as W
from block_sparse_spatio_amd import _lib
from tests.conftest import ROOT


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "vsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vsa_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = vsa.load()
    names = _declared_functions()
    assert {"vsa_classify_tiles", "vsa_sparse_attn_fwd", "vsa_profile_heads"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib._SIGNATURES), "binding and header disagree"


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "vsa.h"\nint main(void){ vsa_grid g = {1,1,1,0,0,0}; (void)g; return 0; }\n')
    r = os.system(f"gcc -std=c99 -Wall -Werror -I{ROOT}/include -c {src} -o {tmp_path}/t.o")
    assert r == 0


def test_struct_layouts_match_header():
    assert ctypes.sizeof(_lib.vsa_grid) == 24
    assert ctypes.sizeof(_lib.vsa_mask_desc) == 60
    assert ctypes.sizeof(_lib.vsa_tile_lists) == 48


def test_unique_masks_and_counts():
    masks = [W.mask_spatial(1)] * 3 + [W.mask_temporal(4)] * 2 + [W.mask_spatial(1)]
    hm, u = vsa.vsa_unique_masks(masks)
    assert u == 2 and hm == [0, 0, 0, 1, 1, 0]
    assert vsa.vsa_tile_counts(W.grid(21, 45, 80), 128, 64) == (591, 1182)
    assert vsa.vsa_tile_counts(W.grid(30, 48, 80), 128, 64) == (900, 1800)
    # the padded layout: 21 x 45 x 80 with 3 x 8 x 16 tiles runs on 21 x 48 x 80
    assert vsa.vsa_seq_len(W.grid(21, 45, 80, (3, 8, 16)), "padded") == 80640
    assert vsa.vsa_seq_len(W.grid(21, 45, 80), "frame") == 75600
    assert vsa.vsa_seq_len(W.grid(30, 48, 80, (6, 8, 8)), "padded") == 115200


def test_workspace_sizes():
    sched = 3328  # the per-call schedule of the bf16 grid
    vt = 24 * 128 * 115200 * 2 + sched  # V^T, S already a multiple of 64
    assert vsa.vsa_fwd_workspace_bytes(1, 115200, 24, 128, vsa.VSA_BF16, 0) == vt
    assert vsa.vsa_fwd_workspace_bytes(2, 100, 3, 64, vsa.VSA_BF16, 0) == 2 * 3 * 64 * 128 * 2 + sched
    assert vsa.vsa_fwd_workspace_bytes(2, 100, 3, 64, vsa.VSA_F32, 0) == 0
    assert vsa.vsa_fwd_workspace_bytes(1, 115200, 24, 128, vsa.VSA_BF16, vsa.VSA_FWD_REORDER_IO) \
        == 115200 * 24 * 128 * 2 + vt  # k reordered; q, v gathered, o scattered
    assert vsa.vsa_fwd_workspace_bytes(2, 100, 3, 64, vsa.VSA_F32, vsa.VSA_FWD_REORDER_IO) \
        == 3 * 2 * 100 * 3 * 64 * 4
    assert vsa.vsa_profile_workspace_bytes(2, 75600, 40, 128, 64, 3) > 0


class _Fake:
    """Stand-in tensor: the validation paths below fail before any pointer is used."""
    def __init__(self, shape, dtype):
        import torch
        self.shape = shape
        self.dtype = dtype
        self.device = torch.device("cpu")

    def is_contiguous(self):
        return True

    def data_ptr(self):
        return 0x1000


def _call_fwd(**over):
    import torch
    lib = vsa.load()
    g = over.pop("grid", W.grid(4, 8, 8))
    masks = over.pop("masks", [W.mask_spatial(1), W.mask_temporal(1)])
    args = dict(q=0x1000, k=0x2000, v=0x3000, o=0x4000, lse=None, dtype=vsa.VSA_BF16, B=1, S=256, H=2, D=64,
                layout=0, Bq=64, Bk=64, scale=0.0, flags=0, ws=0xA000, ws_bytes=1 << 40)
    args.update(over)
    lists = _lib.vsa_tile_lists(0x5000, 0x6000, 0x7000, 0x8000, 0x9000, None)
    arr = _lib.make_masks(masks)
    st = lib.vsa_sparse_attn_fwd(args["q"], args["k"], args["v"], args["o"], args["lse"], args["dtype"],
                                 args["B"], args["S"], args["H"], args["D"], ctypes.byref(_lib.make_grid(g)),
                                 args["layout"], arr, ctypes.byref(lists), args["Bq"], args["Bk"],
                                 args["scale"], args["flags"], args["ws"], args["ws_bytes"], None)
    del torch
    return st, vsa.vsa_last_error()


@pytest.mark.parametrize("over,status,needle", [
    (dict(S=255), -1, "S=255"),
    (dict(D=96), -2, "D=96"),
    (dict(dtype=7), -1, "dtype"),
    (dict(Bq=96), -2, "Bq=96"),
    (dict(q=None), -1, "non-NULL"),
    (dict(o=0x1000), -1, "alias"),
    (dict(flags=64), -1, "flag"),
    (dict(flags=4), -1, "lse"),
    (dict(flags=2), -1, "not frame-major"),
    (dict(flags=2, masks=[W.mask_spatial(1), dict(W.mask_temporal(1), head_layout="position")], ws_bytes=1000),
     -3, "workspace"),
    (dict(masks=[dict(W.mask_all(), head_layout=7), W.mask_all()]), -1, "head_layout"),
    (dict(masks=[dict(W.mask_all(), head_layout="tile"), W.mask_all()]), -1, "tile"),
    (dict(grid=W.grid(3, 5, 7, (2, 2, 4)), layout=3, S=105), -1, "positions"),  # padded: S = 192
    (dict(grid=W.grid(3, 5, 7, (2, 2, 4)), layout=3, S=192, ws_bytes=10), -3, "workspace"),
    (dict(grid=W.grid(3, 5, 7, (2, 2, 4)), layout=3, S=105, flags=2, ws_bytes=10), -3, "workspace"),
    (dict(grid=W.grid(3, 5, 7, (2, 2, 4)), layout=3, S=192, flags=2), -1, "frame-major I/O"),
    (dict(grid=W.grid(3, 5, 7, (2, 2, 4)), layout=3, S=192,
          masks=[W.mask_all(), W.with_head_layout(W.mask_all(), "frame")]), -1, "every head"),
    (dict(grid=W.grid(3, 5, 7), layout=3, S=105), -1, "tile"),
    (dict(flags=2, layout=1, grid=W.grid(4, 8, 8, (2, 4, 4)), ws_bytes=1000), -3, "workspace"),
    (dict(ws=None, ws_bytes=0), -3, "workspace"),
    (dict(ws=0xA008), -1, "aligned"),
    (dict(grid=W.grid(4, 8, 8, (3, 4, 4)), layout=1), -1, "divide"),
    (dict(masks=[W.mask_stripe(1, 0, 0, 1, 0, 5), W.mask_all()]), -1, "period"),
    (dict(masks=[W.mask_sta(1, 1, 1), W.mask_all()]), -1, "tile"),
    (dict(masks=[dict(W.mask_all(), rt=3), W.mask_all()]), -1, "ALL"),
    (dict(masks=[dict(W.mask_all(), kind=9), W.mask_all()]), -1, "kind"),
    (dict(scale=float("nan")), -1, "scale"),
])
def test_fwd_validation(over, status, needle):
    st, msg = _call_fwd(**over)
    assert st == status, msg
    assert needle in msg


def test_fwd_size_limits_enqueue_nothing():
    """Kernel-side limits are checked before anything is enqueued: S*H*D at or above
    2^31 (32-bit offsets inside a batch item) and B above 65535 (a grid dimension) are
    UNSUPPORTED.  The pointers are not device memory, so an enqueued launch or copy
    could not have returned this status."""
    g = W.grid(64, 64, 64)  # 262144 tokens; 64 heads of 128 channels: 2^31 elements
    masks = [W.mask_all()] * 64
    st, msg = _call_fwd(grid=g, S=262144, H=64, D=128, masks=masks)
    assert st == -2 and "2^31" in msg, msg
    st, msg = _call_fwd(grid=g, S=262144, H=64, D=128, masks=masks, dtype=vsa.VSA_F32, Bq=64, Bk=64)
    assert st == -2 and "2^31" in msg, msg
    st, msg = _call_fwd(B=65536)
    assert st == -2 and "65535" in msg, msg
    # the padded layout counts its padded length
    gp = W.grid(63, 64, 64, (2, 1, 1))
    st, msg = _call_fwd(grid=gp, layout=3, S=64 * 64 * 64, H=64, D=128, masks=masks)
    assert st == -2 and "2^31" in msg, msg


def test_noalloc_rejects_oversized_call():
    """The allocation-free forward refuses a call whose workspace exceeds the static
    scratch before anything is enqueued (the pointers are not device memory), and
    validates its arguments like the forward with a workspace."""
    lib = vsa.load()
    g = W.grid(21, 45, 80)  # 40 heads of 128 channels: V^T alone is 774 MB
    masks = _lib.make_masks([W.mask_spatial(1)] * 40)
    lists = _lib.vsa_tile_lists(0x5000, 0x6000, 0x7000, 0x8000, 0x9000, None)
    call = lambda **o: lib.vsa_sparse_attn_fwd_noalloc(  # noqa: E731
        0x1000, 0x2000, 0x3000, o.get("o", 0x4000), None, vsa.VSA_BF16, 1, 75600, 40, o.get("D", 128),
        ctypes.byref(_lib.make_grid(g)), 0, masks, ctypes.byref(lists), 128, 64, 0.0, 0, None, 0, None)
    assert call() == -3 and "static scratch" in vsa.vsa_last_error()
    assert call(o=0x1000) == -1 and "alias" in vsa.vsa_last_error()
    assert call(D=96) == -2


def test_tile_lists_bytes_and_carve():
    """One allocation for every array of the tile lists: sizes and 256-byte aligned
    offsets in struct order, bnd_offs with U*nQ + 1 entries."""
    lib = vsa.load()
    g = _lib.make_grid(W.grid(21, 45, 80))
    n = ctypes.c_size_t()
    assert lib.vsa_tile_lists_bytes(ctypes.byref(g), 0, 2, 128, 64, ctypes.byref(n)) == 0
    nQ, nK, U = 591, 1182, 2
    a = lambda x: (x + 255) // 256 * 256  # noqa: E731
    sizes = [a(U * nQ * nK), a(U * nQ * 4), a(U * nQ * 4), a(U * nQ * nK * 4), a(U * nQ * nK * 4), a((U * nQ + 1) * 8)]
    assert n.value == sum(sizes)
    out = _lib.vsa_tile_lists()
    base = 0x10000000
    assert lib.vsa_tile_lists_carve(ctypes.byref(g), 0, 2, 128, 64, base, ctypes.byref(out)) == 0
    offs = [out.cls, out.n_full, out.n_bnd, out.full_idx, out.bnd_idx, out.bnd_offs]
    assert offs == [base + sum(sizes[:i]) for i in range(6)]
    assert lib.vsa_tile_lists_carve(ctypes.byref(g), 0, 2, 128, 64, base + 8, ctypes.byref(out)) == -1
    assert "aligned" in vsa.vsa_last_error()
    assert lib.vsa_tile_lists_bytes(ctypes.byref(g), 0, 0, 128, 64, ctypes.byref(n)) == -1
    assert lib.vsa_tile_lists_bytes(ctypes.byref(g), 0, 2, 0, 64, ctypes.byref(n)) == -1
    # the padded layout sizes the lists by its padded length
    gp = _lib.make_grid(W.grid(21, 45, 80, (3, 8, 16)))
    assert lib.vsa_tile_lists_bytes(ctypes.byref(gp), 3, 1, 128, 64, ctypes.byref(n)) == 0
    assert n.value == a(630 * 1260) + 2 * a(630 * 4) + 2 * a(630 * 1260 * 4) + a(631 * 8)


def test_classify_validation():
    lib = vsa.load()
    arr = _lib.make_masks([W.mask_spatial(1)])
    lists = _lib.vsa_tile_lists(None, None, None, None, None, None)
    st = lib.vsa_classify_tiles(ctypes.byref(_lib.make_grid(W.grid(4, 8, 8))), 0, arr, 1, 64, 64,
                                ctypes.byref(lists), None)
    assert st == -1 and "non-NULL" in vsa.vsa_last_error()
    lists = _lib.vsa_tile_lists(0x10, 0x20, 0x30, 0x40, 0x50, None)
    st = lib.vsa_classify_tiles(ctypes.byref(_lib.make_grid(W.grid(0, 8, 8))), 0, arr, 1, 64, 64,
                                ctypes.byref(lists), None)
    assert st == -1 and "positive" in vsa.vsa_last_error()
    st = lib.vsa_classify_tiles(ctypes.byref(_lib.make_grid(W.grid(4, 8, 8))), 0, arr, 1, 0, 64,
                                ctypes.byref(lists), None)
    assert st == -1
    many = _lib.make_masks([W.mask_box(i, -1, -1) for i in range(65)])
    st = lib.vsa_classify_tiles(ctypes.byref(_lib.make_grid(W.grid(70, 2, 2))), 0, many, 65, 64, 64,
                                ctypes.byref(lists), None)
    assert st == -2 and "distinct" in vsa.vsa_last_error()


def test_profile_validation():
    lib = vsa.load()
    g = _lib.make_grid(W.grid(4, 8, 8))
    cands = _lib.make_masks([W.mask_all(), W.mask_spatial(1), W.mask_temporal(1)])
    err = ctypes.c_void_p(0x10)
    st = lib.vsa_profile_heads(0x1, 0x2, 0x3, vsa.VSA_F32, 1, 256, 2, 64, ctypes.byref(g), 0, 0x4, 8,
                               cands, 3, err, 0x5, 0.0, 0x6, 1 << 20, None)
    assert st == -2 and "bf16" in vsa.vsa_last_error()
    st = lib.vsa_profile_heads(0x1, 0x2, 0x3, vsa.VSA_BF16, 1, 256, 2, 64, ctypes.byref(g), 0, 0x4, 8,
                               cands, 3, err, 0x5, 0.0, 0x6, 16, None)
    assert st == -3
    st = lib.vsa_profile_heads(0x1, 0x2, 0x3, vsa.VSA_BF16, 1, 256, 2, 64, ctypes.byref(g), 0, 0x4, 300,
                               cands, 3, err, 0x5, 0.0, 0x6, 1 << 30, None)
    assert st == -1
    moved = _lib.make_masks([W.mask_all(), W.mask_spatial(1), dict(W.mask_temporal(1), head_layout="position")])
    st = lib.vsa_profile_heads(0x1, 0x2, 0x3, vsa.VSA_BF16, 1, 256, 2, 64, ctypes.byref(g), 0, 0x4, 8,
                               moved, 3, err, 0x5, 0.0, 0x6, 1 << 30, None)
    assert st == -2 and "call's layout" in vsa.vsa_last_error()
    gp = _lib.make_grid(W.grid(4, 8, 8, (2, 4, 4)))
    st = lib.vsa_profile_heads(0x1, 0x2, 0x3, vsa.VSA_BF16, 1, 256, 2, 64, ctypes.byref(gp), 3, 0x4, 8,
                               cands, 3, err, 0x5, 0.0, 0x6, 1 << 30, None)
    assert st == -2 and "padded" in vsa.vsa_last_error()


def test_reorder_validation():
    lib = vsa.load()
    g = _lib.make_grid(W.grid(4, 8, 8))
    st = lib.vsa_reorder_tokens(0x1, 0x2, vsa.VSA_BF16, 1, 2, 64, ctypes.byref(g), 0, None)
    assert st == -1 and "tile" in vsa.vsa_last_error()
    g = _lib.make_grid(W.grid(4, 8, 8, (2, 4, 4)))
    st = lib.vsa_reorder_tokens(0x1, 0x1, vsa.VSA_BF16, 1, 2, 64, ctypes.byref(g), 0, None)
    assert st == -1 and "alias" in vsa.vsa_last_error()
    I4 = ctypes.c_int32 * 4
    g = _lib.make_grid(W.grid(4, 8, 8))
    st = lib.vsa_reorder_heads(0x1, 0x2, vsa.VSA_BF16, 1, 4, 64, ctypes.byref(g), I4(0, 2, 5, 0), 0, None)
    assert st == -1 and "unknown layout" in vsa.vsa_last_error()
    st = lib.vsa_reorder_heads(0x1, 0x2, vsa.VSA_BF16, 1, 4, 64, ctypes.byref(g), I4(0, 2, 1, 0), 0, None)
    assert st == -1 and "tile" in vsa.vsa_last_error()
    # 4 heads of 4 bf16 channels: a 16-byte chunk holds two heads, fine only when they move alike
    st = lib.vsa_reorder_heads(0x1, 0x2, vsa.VSA_BF16, 1, 4, 4, ctypes.byref(g), I4(0, 2, 2, 0), 0, None)
    assert st == -2 and "D*element" in vsa.vsa_last_error()
    st = lib.vsa_reorder_heads(0x1, 0x2, vsa.VSA_BF16, 1, 4, 64, ctypes.byref(g), None, 0, None)
    assert st == -1 and "layouts" in vsa.vsa_last_error()
    gp = _lib.make_grid(W.grid(3, 5, 7, (2, 2, 4)))
    st = lib.vsa_reorder_heads(0x1, 0x2, vsa.VSA_BF16, 1, 4, 64, ctypes.byref(gp), I4(3, 3, 0, 3), 0, None)
    assert st == -1 and "every head" in vsa.vsa_last_error()


def _call_merge(n=2, o_ok=True, lse_ok=True, D=128, dtype=0, S=10, out=0x9000, misalign=False):
    lib = vsa.load()
    P = ctypes.c_void_p
    op = (P * max(n, 1))(*([0x1000 + (8 if misalign else 0)] * max(n, 1) if o_ok else [None] * max(n, 1)))
    lp = (P * max(n, 1))(*([0x2000] * max(n, 1) if lse_ok else [None] * max(n, 1)))
    st = lib.vsa_merge_partials(op, lp, n, out, None, dtype, 1, S, 2, D, None)
    return st, vsa.vsa_last_error()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(n=0), -1, "n_parts"),
    (dict(n=17), -1, "n_parts"),
    (dict(o_ok=False), -1, "NULL"),
    (dict(lse_ok=False), -1, "NULL"),
    (dict(D=96), -2, "D=96"),
    (dict(dtype=5), -1, "dtype"),
    (dict(S=0), -1, "positive"),
    (dict(out=None), -1, "non-NULL"),
    (dict(misalign=True), -1, "aligned"),
])
def test_merge_validation(kw, status, needle):
    st, msg = _call_merge(**kw)
    assert st == status, msg
    assert needle in msg


def test_classify_ex_validation():
    lib = vsa.load()
    arr = _lib.make_masks([W.mask_spatial(1)])
    lists = _lib.vsa_tile_lists(0x10, 0x20, 0x30, 0x40, 0x50, None)
    g = ctypes.byref(_lib.make_grid(W.grid(4, 8, 8)))
    st = lib.vsa_classify_tiles_ex(g, 0, arr, 1, 64, 64, 2, ctypes.byref(lists), None)
    assert st == -1 and "flag" in vsa.vsa_last_error()
    st = lib.vsa_classify_tiles_ex(g, 0, arr, 1, 64, 128, vsa.VSA_CLASSIFY_ROUND_TILES, ctypes.byref(lists), None)
    assert st == -2 and "Bk <= 64" in vsa.vsa_last_error()


def _call_fwd_ex(words, cap, **over):
    lib = vsa.load()
    g = W.grid(4, 8, 8)
    arr = _lib.make_masks([W.mask_spatial(1), W.mask_temporal(1)])
    args = dict(dtype=vsa.VSA_BF16, flags=0, Bq=64)
    args.update(over)
    lists = _lib.vsa_tile_lists(0x5000, 0x6000, 0x7000, 0x8000, 0x9000, None)
    st = lib.vsa_sparse_attn_fwd_ex(0x1000, 0x2000, 0x3000, 0x4000, None, args["dtype"], 1, 256, 2, 64,
                                    ctypes.byref(_lib.make_grid(g)), 0, arr, ctypes.byref(lists), args["Bq"], 64,
                                    0.0, args["flags"], words, cap, 0xA000, 1 << 40, None)
    return st, vsa.vsa_last_error()


@pytest.mark.parametrize("words,cap,over,status,needle", [
    (None, 3, {}, -1, "both set"),
    (0xB000, 0, {}, -1, "both set"),
    (0xB000, -2, {}, -1, "both set"),
    (None, -1, {}, -1, "both set"),
    (0xB000, -1, {}, -1, "bnd_offs"),  # the compact table needs the list offsets
    (0xB000, 5, {}, -1, "above the 4 key tiles"),
    (0xB004, 2, {}, -1, "aligned"),
    (0xB000, 2, dict(dtype=vsa.VSA_F32), -2, "bf16 only"),
    (0xB000, 2, dict(flags=vsa.VSA_FWD_TILE_ALIGNED), -1, "TILE_ALIGNED"),
])
def test_fwd_ex_validation(words, cap, over, status, needle):
    st, msg = _call_fwd_ex(words, cap, **over)
    assert st == status, msg
    assert needle in msg


def test_boundary_words_validation():
    lib = vsa.load()
    arr = _lib.make_masks([W.mask_spatial(1), W.mask_stripe(1, 0, 2, 1, 0, 5)])
    g = ctypes.byref(_lib.make_grid(W.grid(4, 8, 8)))
    lists = _lib.vsa_tile_lists(0x10, 0x20, 0x30, 0x40, 0x50, None)
    cases = [
        (dict(Bk=32), -2, "Bk 64"),
        (dict(Bq=32), -2, "Bq 64/128/256"),
        (dict(cap=5), -1, "above the 4 key tiles"),
        (dict(cap=-2), -1, "negative"),
        (dict(cap=-1), -1, "bnd_offs"),  # VSA_WORDS_COMPACT without list offsets
        (dict(words=None), -1, "words is NULL"),
        (dict(words=0x1008), -1, "aligned"),
        (dict(lists=_lib.vsa_tile_lists(0x10, 0x20, None, 0x40, 0x50, None)), -1, "non-NULL"),
        (dict(grid=ctypes.byref(_lib.make_grid(W.grid(0, 8, 8)))), -1, "positive"),
    ]
    for over, status, needle in cases:
        a = dict(grid=g, Bq=64, Bk=64, lists=lists, words=0x1000, cap=2)
        a.update(over)
        st = lib.vsa_boundary_words(a["grid"], 0, arr, 2, a["Bq"], a["Bk"], ctypes.byref(a["lists"]), a["words"],
                                    a["cap"], None)
        msg = vsa.vsa_last_error()
        assert st == status and needle in msg, (over, st, msg)


def test_binding_rejects_mis_sized_outputs():
    """The binding checks tensor shapes before any pointer reaches the library (the C
    ABI cannot see allocation sizes): a destination shorter than the padded order is an
    error, not a write past its end."""
    import torch
    g = W.grid(3, 5, 7, (2, 2, 4))  # 105 tokens, 192 positions padded
    x = torch.zeros((1, 105, 2, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="dst must be"):
        vsa.vsa_reorder_heads(x, g, ["padded", "padded"], dst=torch.zeros_like(x))
    with pytest.raises(ValueError, match="padded reorder reads"):
        vsa.vsa_reorder_heads(x, g, ["padded", "padded"], inverse=True)
    with pytest.raises(ValueError, match="src holds"):
        vsa.vsa_reorder_tokens(torch.zeros((1, 99, 2, 64)), W.grid(4, 5, 5, (2, 5, 5)))
    q = torch.zeros((1, 105, 2, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="o must be"):
        vsa.vsa_sparse_attn_fwd(q, q, q, g, "frame", [W.mask_all()] * 2, {"Bq": 64, "Bk": 64},
                                o=torch.zeros((1, 104, 2, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="lse_parts"):
        vsa.vsa_merge_partials([q, q], [torch.zeros((1, 2, 104)), torch.zeros((1, 2, 105))])
    tiles = {"cls": None, "n_full": torch.zeros((1, 2), dtype=torch.int32), "n_bnd": torch.zeros((1, 2), dtype=torch.int32),
             "full_idx": torch.zeros((1, 2, 2), dtype=torch.int32), "bnd_idx": torch.zeros((1, 2, 2), dtype=torch.int32),
             "n_unique": 1, "nQ": 2, "nK": 2, "Bq": 64, "Bk": 64}
    with pytest.raises(ValueError, match="out must be"):
        vsa.vsa_boundary_words(W.grid(2, 8, 8), "frame", [W.mask_all()], tiles, cap=2,
                               out=torch.zeros((1, 2, 1, 2, 64), dtype=torch.int32))
    q2 = torch.zeros((1, 128, 1, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="words do not match"):
        vsa.vsa_sparse_attn_fwd(q2, q2, q2, W.grid(2, 8, 8), "frame", [W.mask_all()], tiles,
                                words={"words": torch.zeros((1, 2, 2, 4, 64), dtype=torch.int32), "cap": 2})
