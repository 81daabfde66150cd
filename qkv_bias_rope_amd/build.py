"""Compile the HIP library in-tree: csrc/*.hip -> libqkv_epilogue.so.

hipcc cross-compiles for gfx950 without a GPU.  Flags: -O3, no fast-math
(denormals and IEEE rounding stay as HIP's defaults), packed FP32 ops off.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", f) for f in ("qkv_epilogue.hip", "qkv_unfused.hip", "qkv_proj.hip")]
HDRS = [os.path.join(ROOT, "include", "qkv_epilogue.h"), os.path.join(PKG, "csrc", "qkv_internal.h")]
LIB = os.path.join(PKG, "libqkv_epilogue.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False) -> str:
    """Always recompile (the build check must compile), atomically replace."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), *SRCS, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in (*SRCS, *HDRS))


if __name__ == "__main__":
    print(build(verbose=True))
