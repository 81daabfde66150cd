"""ctypes binding of libqkv_probe.so: the benchmark's reference kernels.

These set the floor (an empty kernel) and the ceilings (a streaming copy, an
in-place add, a read-only pass, and a row-scatter pass that moves the batched
decode's bytes)
that the epilogue's timings are read against on the same device.  They are
measurement tools, not part of the epilogue; only the benchmark and its tests
load them.  Argument marshalling only; every entry point returns 0 or a
negative code.

Memory policy of the copy/add/rows kernels: 0 plain loads and stores, 1
non-temporal loads and stores, 2 non-temporal loads and non-temporal
device-scope stores (written through the L2 as they are issued), 3
non-temporal loads and device-scope stores without the non-temporal bit (in
the row pass only the cache rows take these; the rows keep 2's: the
epilogue's combination).
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (bind to torch's HIP runtime, as the epilogue binding does)

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqkv_probe.so")

_P = ctypes.c_void_p
_I = ctypes.c_int
_LL = ctypes.c_longlong


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    lib.qkv_probe_grid.argtypes = [_LL, _I, _I]
    lib.qkv_probe_grid.restype = _LL
    lib.qkv_probe_empty.argtypes = [_I, _I, _P]
    lib.qkv_probe_empty.restype = _I
    lib.qkv_probe_empty_args.argtypes = [_I, _I, _P]
    lib.qkv_probe_empty_args.restype = _I
    lib.qkv_probe_copy.argtypes = [_P, _P, _LL, _I, _I, _I, _P]
    lib.qkv_probe_copy.restype = _I
    lib.qkv_probe_add.argtypes = [_P, _LL, _I, _I, _I, _P]
    lib.qkv_probe_add.restype = _I
    lib.qkv_probe_read.argtypes = [_P, _LL, _P, _I, _I, _I, _P]
    lib.qkv_probe_read.restype = _I
    lib.qkv_probe_rows.argtypes = [_P, _P, _LL, _LL, _LL, _LL, _P, _P, _LL, _P, _P, _I, _I, _I, _I,
                                   _P]
    lib.qkv_probe_rows.restype = _I
    return lib


lib = _load()
EXPORTS = ("qkv_probe_grid", "qkv_probe_empty", "qkv_probe_empty_args", "qkv_probe_copy", "qkv_probe_add",
           "qkv_probe_read", "qkv_probe_rows")


def _s(stream):
    if stream is None:
        return None
    return stream if isinstance(stream, int) else stream.cuda_stream


def grid(n16: int, block: int, vpt: int) -> int:
    return lib.qkv_probe_grid(n16, block, vpt)


def empty(grid_: int, block: int, stream=None) -> int:
    return lib.qkv_probe_empty(grid_, block, _s(stream))


def empty_args(grid_: int, block: int, stream=None) -> int:
    """An empty kernel that takes 1280 bytes of arguments (about an epilogue
    launch's)."""
    return lib.qkv_probe_empty_args(grid_, block, _s(stream))


POLICIES = (0, 1, 2)


def copy(dst, src, block=256, vpt=1, policy=2, stream=None) -> int:
    """dst = src for two float32 device tensors of equal size (a multiple of 4)."""
    assert dst.numel() == src.numel() and dst.numel() % 4 == 0
    return lib.qkv_probe_copy(dst.data_ptr(), src.data_ptr(), dst.numel() // 4, block, vpt,
                              policy, _s(stream))


def add(buf, block=256, vpt=1, policy=2, stream=None) -> int:
    """buf += 1 in place for a float32 device tensor (numel a multiple of 4)."""
    assert buf.numel() % 4 == 0
    return lib.qkv_probe_add(buf.data_ptr(), buf.numel() // 4, block, vpt, policy, _s(stream))


def read_out_numel(n16: int, block: int, vpt: int) -> int:
    """Floats the per-wave sums of a read launch take."""
    return grid(n16, block, vpt) * block // 64


def read(src, out, block=256, vpt=1, policy=1, stream=None) -> int:
    """Read every element of a float32 device tensor (numel a multiple of 4);
    out (float32, at least read_out_numel(src.numel() // 4, block, vpt)
    elements) receives the per-wave sums.  Policy 0 plain or 1 non-temporal
    loads."""
    assert src.numel() % 4 == 0 and src.dtype == torch.float32 and out.dtype == torch.float32
    n16 = src.numel() // 4
    assert out.numel() >= read_out_numel(n16, block, vpt)
    return lib.qkv_probe_read(src.data_ptr(), n16, out.data_ptr(), block, vpt, policy, _s(stream))


def rows(x, b, kv_col, nkt, pos, slot, n_ctx, kc, vc, block=256, tpb=1, policy=2,
         stream=None) -> int:
    """x[t] += b in place for x [nt][width] float32; columns [kv_col, kv_col+nkt)
    of row t also go to kc[slot[t]*n_ctx + pos[t]] and the next nkt columns to
    vc (float32 or float16 caches of nkt-wide rows).  The caller guarantees
    that every row index is inside the caches."""
    nt, width = x.shape
    assert b.numel() == width and pos.numel() == nt and (slot is None or slot.numel() == nt)
    assert kc.dtype == vc.dtype and kc.shape[-1] == nkt and vc.shape[-1] == nkt
    f16 = 1 if kc.dtype == torch.float16 else 0
    return lib.qkv_probe_rows(x.data_ptr(), b.data_ptr(), nt, width, kv_col, nkt, pos.data_ptr(),
                              None if slot is None else slot.data_ptr(), n_ctx, kc.data_ptr(),
                              vc.data_ptr(), f16, block, tpb, policy, _s(stream))
