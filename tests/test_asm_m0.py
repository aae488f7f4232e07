"""The LDS DMA helpers write m0 inside inline asm without naming it as clobbered (the
compiler reserves m0 and refuses it in a clobber list).  That is sound only while no
other instruction of those kernels reads m0.  This builds the kernels that use the
helpers to gfx950 assembly (hipcc, no GPU needed) and checks that every reference to m0
is an `s_mov_b32 m0, <SGPR>` (an s register or a half of VCC, which the compiler may
also hand to an "s" operand) immediately followed by the global_load_lds it addresses."""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "block_sparse_spatio_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["attn_bf16.hip", "profile.hip"]


def _asm(src, out):
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-S",
           os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return open(out).read()


@pytest.mark.skipif(not os.path.exists(HIPCC),
                    reason="needs hipcc")
def test_m0_written_only_by_the_dma_helpers(tmp_path):
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        texts = list(ex.map(lambda s: _asm(s, str(tmp_path / (s + ".s"))), SOURCES))
    for src, text in zip(SOURCES, texts):
        lines = [ln.split(";")[0].strip() for ln in text.splitlines()]
        lines = [ln for ln in lines if ln and not ln.startswith(".") and not ln.endswith(":")]
        n_dma = 0
        for i, ln in enumerate(lines):
            if re.search(r"\bm0\b", ln):
                assert re.fullmatch(r"s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi)", ln), f"{src}: m0 referenced by '{ln}'"
                assert lines[i + 1].startswith("global_load_lds_dword"), f"{src}: '{ln}' followed by '{lines[i + 1]}'"
                n_dma += 1
        assert n_dma > 0, src
