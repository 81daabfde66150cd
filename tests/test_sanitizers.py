"""CPU sanitizer runs of the host code (no GPU).

AddressSanitizer + UndefinedBehaviorSanitizer builds of
  * the oracle (oracle/qkv_oracle.c), driven by the oracle's pin tests, and
  * the library's host-only part (qkv_bias_rope_amd/csrc/qkv_host.cpp:
    argument checks, launch planner, inverse-frequency tables; plain C++),
    driven by the host cases of tests/test_abi_host.py,
each in a child process with the sanitizer runtimes preloaded ahead of
whatever the environment already preloads.  Any report aborts the child
(-fno-sanitize-recover=all), so a clean exit means no out-of-bounds access,
use of freed memory or undefined behaviour on those paths.  Leak checking is
off: the interpreter itself does not free everything at exit.  One planted
error per build (made in a copy of the source, on the CPU) shows the runs
would catch one.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_SRC = os.path.join(ROOT, "qkv_bias_rope_amd", "csrc", "qkv_host.cpp")
ORACLE_SRC = os.path.join(ROOT, "oracle", "qkv_oracle.c")
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all", "-shared", "-fPIC"]
ORACLE_PINS = ["tests/test_oracle_pins.py", "tests/test_oracle_norm_pins.py",
               "tests/test_oracle_rope_variants.py", "tests/test_oracle_proj_pins.py",
               "tests/test_oracle_fp8_pins.py"]


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


ASAN, UBSAN = _runtime("libasan.so"), _runtime("libubsan.so")
pytestmark = pytest.mark.skipif(not (ASAN and UBSAN), reason="gcc sanitizer runtimes not found")


def _build_oracle(src, out):
    subprocess.run(["gcc", "-std=c11", "-ffp-contract=off", "-fno-fast-math", *SAN, src, "-lm",
                    "-o", out], check=True)
    return out


def _build_host(src, out):
    subprocess.run(["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.dirname(HOST_SRC), src, "-o", out], check=True)
    return out


def _child(files, extra_env, select=None):
    env = dict(os.environ)
    pre = [ASAN, UBSAN] + ([env["LD_PRELOAD"]] if env.get("LD_PRELOAD") else [])
    env["LD_PRELOAD"] = ":".join(pre)
    env["ASAN_OPTIONS"] = "detect_leaks=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    env.update(extra_env)
    # -s: a sanitizer report goes straight to stderr (the run ends at the report)
    cmd = [sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider", "-m", "not gpu", *files]
    if select:
        cmd += ["-k", select]
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)


@pytest.fixture(scope="module")
def sandir(tmp_path_factory):
    return str(tmp_path_factory.mktemp("sanitize"))


@pytest.fixture(scope="module")
def oracle_san(sandir):
    return _build_oracle(ORACLE_SRC, os.path.join(sandir, "liboracle_san.so"))


def test_oracle_pins_clean_under_sanitizers(oracle_san):
    r = _child(ORACLE_PINS, {"QKV_ORACLE_LIB": oracle_san})
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "Sanitizer" not in r.stderr, tail


def test_host_code_clean_under_sanitizers(sandir, oracle_san):
    lib = _build_host(HOST_SRC, os.path.join(sandir, "libqkv_host_san.so"))
    r = _child(["tests/test_abi_host.py"], {"QKV_HOST_LIB": lib, "QKV_ORACLE_LIB": oracle_san})
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "Sanitizer" not in r.stderr, tail


def _plant(src, old, new, path):
    text = open(src).read()
    assert text.count(old) == 1, old
    with open(path, "w") as f:
        f.write(text.replace(old, new))
    return path


def test_planted_host_overflow_is_caught(sandir, oracle_san):
    """The pointer checks walk one entry past their table: a stack read out of
    bounds on every validated launch."""
    src = _plant(HOST_SRC, "    for (auto &e : ptrs) {",
                 "    for (size_t ie = 0; ie <= sizeof ptrs / sizeof ptrs[0]; ++ie) {\n"
                 "        auto &e = ptrs[ie];",
                 os.path.join(sandir, "qkv_host_planted.cpp"))
    lib = _build_host(src, os.path.join(sandir, "libqkv_host_planted.so"))
    r = _child(["tests/test_abi_host.py"], {"QKV_HOST_LIB": lib, "QKV_ORACLE_LIB": oracle_san},
               select="valid_args_ok")
    assert r.returncode != 0
    assert "stack-buffer-overflow" in r.stderr, (r.stdout + r.stderr)[-3000:]


def test_planted_oracle_overflow_is_caught(sandir):
    """add_bias reads the bias one element past its end."""
    src = _plant(ORACLE_SRC, "            x[t * ld + j] = x[t * ld + j] + b[j];",
                 "            x[t * ld + j] = x[t * ld + j] + b[j + (j + 1 == width)];",
                 os.path.join(sandir, "qkv_oracle_planted.c"))
    lib = _build_oracle(src, os.path.join(sandir, "liboracle_planted.so"))
    r = _child(["tests/test_oracle_pins.py"], {"QKV_ORACLE_LIB": lib})
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr, (r.stdout + r.stderr)[-3000:]
