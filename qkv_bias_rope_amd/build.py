"""Compile the HIP libraries in-tree:
  csrc/qkv_epilogue.hip, qkv_unfused.hip, qkv_proj.hip, qkv_host.cpp
    -> libqkv_epilogue.so
  csrc/hbm_probe.hip -> libqkv_probe.so (the benchmark's floor and ceiling
  kernels; not part of the epilogue library).

hipcc cross-compiles for gfx950 without a GPU.  Flags: -O3, no fast-math
(denormals and IEEE rounding stay as HIP's defaults), packed FP32 ops off.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", f)
        for f in ("qkv_epilogue.hip", "qkv_unfused.hip", "qkv_proj.hip", "qkv_host.cpp")]
HOST_SRC = os.path.join(PKG, "csrc", "qkv_host.cpp")   # the host-only part (no HIP)
HDRS = [os.path.join(ROOT, "include", "qkv_epilogue.h"), os.path.join(PKG, "csrc", "qkv_internal.h"),
        os.path.join(PKG, "csrc", "qkv_plan.h")]
LIB = os.path.join(PKG, "libqkv_epilogue.so")
PROBE_SRC = os.path.join(PKG, "csrc", "hbm_probe.hip")
PROBE_LIB = os.path.join(PKG, "libqkv_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def _compile(srcs, out, verbose):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), *srcs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Always recompile both libraries (the build check must compile),
    atomically replacing each."""
    _compile(SRCS, LIB, verbose)
    _compile([PROBE_SRC], PROBE_LIB, verbose)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB) or not os.path.exists(PROBE_LIB):
        return True
    t = min(os.path.getmtime(LIB), os.path.getmtime(PROBE_LIB))
    return any(os.path.getmtime(p) > t for p in (*SRCS, *HDRS, PROBE_SRC))


if __name__ == "__main__":
    print(build(verbose=True))
