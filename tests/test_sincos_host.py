"""The kernels' rope sin/cos (qkv_bias_rope_amd/csrc/qkv_sincos.h), built for
the host, against the definition the oracle uses: f32(sin((double)a)) and
f32(cos((double)a)) from the C library.

Every operation in the header is written out (fused multiply-adds called
explicitly, no contraction left to a compiler), so the host build computes the
bits the device does.  Checked: every angle f32(pos * inv[i]) for positions
below 65536 with the inverse-frequency tables of theta 1e6 (head_dim 128 and
64) and 1e4 (128), 4M random angles in (-2^20, 2^20), and the f32 values at
and beside k*pi/2 for every quadrant below 2^20 (where the reduction cancels
most).  All must agree bit for bit.  A copy of the header with one series
term dropped must not (the harness can see an error).
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c", "sincos_check.cpp")
HDR_DIR = os.path.join(ROOT, "qkv_bias_rope_amd", "csrc")


def _build(out, hdr_dir):
    subprocess.run(["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-D__host__=", "-D__device__=",
                    "-I", hdr_dir, SRC, "-o", out], check=True)
    return out


def _run(exe, mode):
    out = subprocess.run([exe, mode], capture_output=True, text=True, check=True, timeout=300).stdout
    name, n, bad, maxulp = out.split()
    return int(n), int(bad), int(maxulp)


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    return _build(str(tmp_path_factory.mktemp("sincos") / "sincos_check"), HDR_DIR)


@pytest.mark.parametrize("mode,count", [("rope", 10485760), ("random", 4000000), ("quadrant", 2002632)])
def test_rope_sincos_matches_libm(exe, mode, count):
    n, bad, maxulp = _run(exe, mode)
    assert n == count
    assert bad == 0, f"{mode}: {bad} of {n} angles differ (max {maxulp} ulp)"


def test_harness_sees_a_dropped_term(tmp_path):
    text = open(os.path.join(HDR_DIR, "qkv_sincos.h")).read()
    old = "s23 = std::fma(kS9, z, kS7)"
    assert text.count(old) == 1
    (tmp_path / "qkv_sincos.h").write_text(text.replace(old, "s23 = kS7"))
    exe = _build(str(tmp_path / "planted"), str(tmp_path))
    n, bad, maxulp = _run(exe, "random")
    assert bad > 1000 and maxulp >= 1
