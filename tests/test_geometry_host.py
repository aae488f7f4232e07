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


def _build(tmp_path_factory, name, flags):
    if shutil.which("g++") is None or not os.path.isdir(ROCM_INC):
        pytest.skip("needs g++ and the ROCm headers")
    exe = str(tmp_path_factory.mktemp("geom") / name)
    cmd = ["g++", *flags, "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INC, "-I", CSRC,
           os.path.join(HERE, "geometry_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    return _build(tmp_path_factory, "geometry_check", ["-O2"])


@pytest.fixture(scope="module")
def checker_sanitized(tmp_path_factory):
    """The same check built with AddressSanitizer and UndefinedBehaviorSanitizer (host
    code only): out-of-bounds accesses of the box arrays, signed overflow in the
    interval arithmetic, shifts past the word width and the like abort the run."""
    return _build(tmp_path_factory, "geometry_check_asan",
                  ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                   "-fno-sanitize-recover=all"])


def _run(exe, trials, seed, focus):
    args = [exe, str(trials), str(seed)] + (["focus"] if focus else [])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run(args, capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "bad 0; mask bits" in r.stdout and r.stdout.strip().endswith("bad 0"), r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]


@pytest.mark.parametrize("seed,focus", [(1, False), (2, False), (7, True), (8, True)])
def test_geometry_against_brute_force(checker, seed, focus):
    _run(checker, 250, seed, focus)


@pytest.mark.parametrize("seed,focus", [(3, False), (9, True)])
def test_geometry_sanitized(checker_sanitized, seed, focus):
    _run(checker_sanitized, 60, seed, focus)
