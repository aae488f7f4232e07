"""The geometry of the GPU path (csrc/vsa_classify_geom.h, csrc/vsa_geom.h), built for the host
with g++ and checked against brute-force enumeration (tests/geometry_check.cpp): tile
classes, kept-pair counts and the 64-key row masks of every mask kind in every token
order, on random small grids.  Needs g++ and the ROCm headers, no GPU."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "block_sparse_spatio_amd", "csrc")
ROCM_INC = "/opt/rocm/include"


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if shutil.which("g++") is None or not os.path.isdir(ROCM_INC):
        pytest.skip("needs g++ and the ROCm headers")
    exe = str(tmp_path_factory.mktemp("geom") / "geometry_check")
    cmd = ["g++", "-O2", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INC, "-I", CSRC,
           os.path.join(HERE, "geometry_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


@pytest.mark.parametrize("seed,focus", [(1, False), (2, False), (7, True), (8, True)])
def test_geometry_against_brute_force(checker, seed, focus):
    args = [checker, "250", str(seed)] + (["focus"] if focus else [])
    r = subprocess.run(args, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-2000:]
    assert "bad 0; mask bits" in r.stdout and r.stdout.strip().endswith("bad 0"), r.stdout
