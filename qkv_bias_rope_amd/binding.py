"""ctypes binding of libqkv_epilogue.so (the C ABI in include/qkv_epilogue.h).

Argument marshalling only: every step of the epilogue runs in the HIP kernels
of the library.  The functions keep the C names and return the C codes; the
``Epilogue`` class wraps them for torch tensors and raises on errors.  PyTorch
is used for nothing but device memory (``data_ptr``) and the current stream.

If the library is not built this module raises at import time: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

# Load torch first: its wheel bundles the HIP runtime (SONAME libamdhip64.so.7)
# and this library must bind to that same runtime instance, not load a second
# copy from /opt/rocm (two runtimes in one process do not share device state).
import torch  # noqa: F401

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqkv_epilogue.so")

from .abi import *  # noqa: F401,F403  (the C ABI's constants, structures and builders)
from .abi import (EXPORTS, HostApi, QkvEpilogueArgs, QkvEpilogueConfig, QkvError,  # noqa: F401
                  QkvProjArgs, _P, _addr, _row_stride, _stream_addr, bind, make_args,
                  make_proj_args)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc --offload-arch=gfx950)")
    return bind(ctypes.CDLL(LIB_PATH))


lib = _load()
_host = HostApi(lib)


# ---- the C entry points, same names ----------------------------------------

def qkv_epilogue_create(device: int = 0, n_ctx: int = 4096, stream=None):
    """Returns (rc, handle); handle is an opaque integer (0 on failure)."""
    h = _P()
    cfg = QkvEpilogueConfig(device, n_ctx, _stream_addr(stream))
    rc = lib.qkv_epilogue_create(ctypes.byref(h), ctypes.byref(cfg))
    return rc, (h.value or 0)


def qkv_epilogue_run(h, q, k, v, bq, bk, bv, pos, kcache, vcache, nt, n_head, n_kv_head,
                     head_dim, theta, cache_dtype) -> int:
    return lib.qkv_epilogue_run(h, _addr(q), _addr(k), _addr(v), _addr(bq), _addr(bk),
                                _addr(bv), _addr(pos), _addr(kcache), _addr(vcache),
                                nt, n_head, n_kv_head, head_dim, theta, cache_dtype)


def qkv_epilogue_run_ex(h, args: QkvEpilogueArgs) -> int:
    return lib.qkv_epilogue_run_ex(h, ctypes.byref(args))


def qkv_epilogue_run_unfused(h, args: QkvEpilogueArgs) -> int:
    return lib.qkv_epilogue_run_unfused(h, ctypes.byref(args))


def qkv_epilogue_run_qk_norm(h, args: QkvEpilogueArgs, w_q, w_k, eps: float) -> int:
    return lib.qkv_epilogue_run_qk_norm(h, ctypes.byref(args), _addr(w_q), _addr(w_k), eps)


def qkv_epilogue_run_proj(h, args: QkvProjArgs) -> int:
    return lib.qkv_epilogue_run_proj(h, ctypes.byref(args))


def qkv_epilogue_run_proj_noalloc(h, args: QkvProjArgs) -> int:
    return lib.qkv_epilogue_run_proj_noalloc(h, ctypes.byref(args))


def qkv_epilogue_status(h) -> int:
    return lib.qkv_epilogue_status(h)


def qkv_epilogue_last_error(h) -> str:
    r = lib.qkv_epilogue_last_error(h)
    return r.decode() if r else ""


def qkv_epilogue_destroy(h) -> None:
    lib.qkv_epilogue_destroy(h)


qkv_epilogue_inv_freq = _host.qkv_epilogue_inv_freq
qkv_epilogue_inv_freq_scaled = _host.qkv_epilogue_inv_freq_scaled
qkv_epilogue_check_args = _host.qkv_epilogue_check_args
qkv_epilogue_plan = _host.qkv_epilogue_plan


# ---- torch convenience ------------------------------------------------------

def _section_rows(t, width, name, nt):
    """Raise unless section t holds nt rows of width elements: a contiguous
    1-D tensor of nt*width elements, or a 2-D [nt][width] view with unit
    column stride."""
    if t.dim() == 1:
        if t.stride(0) != 1 or t.numel() != nt * width:
            raise ValueError(f"{name}: a 1-D section must be contiguous with nt*width = "
                             f"{nt}*{width} elements, has {t.numel()}")
    elif t.dim() == 2:
        if t.shape[0] != nt or t.shape[1] != width or t.stride(1) != 1:
            raise ValueError(f"{name}: shape {tuple(t.shape)} (column stride {t.stride(1)}), "
                             f"expected [{nt}][{width}] with unit column stride")
    else:
        raise ValueError(f"{name}: need a 1-D tensor or a 2-D [nt][width] view")


def check_extents(q, k, v, bq, bk, bv, pos, slot, kcache, vcache, *, n_head, n_kv_head,
                  head_dim, n_ctx, n_slots):
    """Host-side extent checks of one launch (the C ABI takes bare pointers and
    cannot check them): q/k/v hold nt = pos.numel() rows of their section
    widths, the biases (when given) one row each, slot nt entries, and each
    cache is a contiguous tensor of at least n_slots*n_ctx rows of
    n_kv_head*head_dim elements.  Raises ValueError before anything is
    launched."""
    nt = int(pos.numel())
    nqt, nkt = n_head * head_dim, n_kv_head * head_dim
    for name, t, width in (("q", q, nqt), ("k", k, nkt), ("v", v, nkt)):
        _section_rows(t, width, name, nt)
    for name, t, width in (("bq", bq, nqt), ("bk", bk, nkt), ("bv", bv, nkt)):
        if t is not None and (t.numel() != width or not t.is_contiguous()):
            raise ValueError(f"{name}: need {width} contiguous elements, has {t.numel()}")
    if slot is not None and slot.numel() != nt:
        raise ValueError(f"slot has {slot.numel()} entries, pos has {nt}")
    need = n_slots * n_ctx * nkt
    for name, t in (("kcache", kcache), ("vcache", vcache)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.numel() < need:
            raise ValueError(f"{name} holds {t.numel()} elements, the launch addresses "
                             f"n_slots*n_ctx*nkt = {n_slots}*{n_ctx}*{nkt} = {need}")


def _check_device(device, **tensors):
    for name, t in tensors.items():
        if t is not None and (not t.is_cuda or t.device.index != device):
            raise TypeError(f"{name} must be a tensor on cuda:{device}, got {t.device}")


class Epilogue:
    """A handle bound to one device.  ``run`` launches on torch's current
    stream and raises QkvError on a non-zero return."""

    def __init__(self, device: int = 0, n_ctx: int = 4096):
        rc, h = qkv_epilogue_create(device, n_ctx, None)
        if rc != QKV_OK:
            raise QkvError(rc, f"qkv_epilogue_create(device={device}, n_ctx={n_ctx}) failed")
        self.h = h
        self.device = device
        self.n_ctx = n_ctx

    def run(self, q, k, v, bq, bk, bv, pos, kcache, vcache, *, n_head, n_kv_head, head_dim,
            theta=1.0e6, slot=None, n_ctx=None, n_slots=None, stream=None, **kw):
        import torch
        if kcache.dtype == torch.float32:
            cd = QKV_CACHE_F32
        elif kcache.dtype == torch.float16:
            cd = QKV_CACHE_F16
        else:
            raise TypeError(f"cache dtype must be float32 or float16, got {kcache.dtype}")
        if vcache.dtype != kcache.dtype:
            raise TypeError("kcache and vcache must share a dtype")
        for name, t in (("q", q), ("k", k), ("v", v), ("bq", bq), ("bk", bk), ("bv", bv)):
            if t.dtype != torch.float32:
                raise TypeError(f"{name} must be float32")
        for name, t in (("pos", pos), ("slot", slot)):
            if t is not None and (t.dtype != torch.int32 or not t.is_contiguous()):
                raise TypeError(f"{name} must be a contiguous int32 tensor")
        check_extents(q, k, v, bq, bk, bv, pos, slot, kcache, vcache, n_head=n_head,
                      n_kv_head=n_kv_head, head_dim=head_dim, n_ctx=n_ctx or self.n_ctx,
                      n_slots=n_slots or 1)
        _check_device(self.device, q=q, k=k, v=v, bq=bq, bk=bk, bv=bv, pos=pos, slot=slot,
                      kcache=kcache, vcache=vcache)
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        a = make_args(q, k, v, bq, bk, bv, pos, kcache, vcache, n_head=n_head,
                      n_kv_head=n_kv_head, head_dim=head_dim, theta=theta, cache_dtype=cd,
                      slot=slot, n_ctx=n_ctx or 0, n_slots=n_slots or 0, stream=stream,
                      use_stream=True, **kw)
        rc = qkv_epilogue_run_ex(self.h, a)
        if rc != QKV_OK:
            raise QkvError(rc, qkv_epilogue_last_error(self.h))

    def run_proj(self, x, w, q, k, v, bq, bk, bv, pos, kcache, vcache, *, n_head, n_kv_head,
                 head_dim, theta=1.0e6, w_k=None, w_v=None, slot=None, n_ctx=None, n_slots=None,
                 rope_style=QKV_ROPE_NEOX, freq_scale=0.0, w_scale=None, stream=None):
        """The projection feeding the epilogue: x [nt][hidden] as a bfloat16
        device tensor, the weights (w [nqt+2*nkt][hidden] concat, or w/w_k/w_v
        per section) bfloat16 -- or float8_e4m3fn with w_scale, a float32
        [nqt+2*nkt] tensor of row scales; q, k, v are the float32 outputs;
        biases may be None."""
        import torch
        if kcache.dtype == torch.float32:
            cd = QKV_CACHE_F32
        elif kcache.dtype == torch.float16:
            cd = QKV_CACHE_F16
        else:
            raise TypeError(f"cache dtype must be float32 or float16, got {kcache.dtype}")
        if vcache.dtype != kcache.dtype:
            raise TypeError("kcache and vcache must share a dtype")
        if (w_k is None) != (w_v is None):
            raise TypeError("w_k and w_v go together")
        if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
            raise TypeError("x must be a 2-D bfloat16 tensor with unit column stride")
        wdt = w.dtype
        if wdt not in (torch.bfloat16, torch.float8_e4m3fn):
            raise TypeError(f"w must be bfloat16 or float8_e4m3fn, got {wdt}")
        for name, t in (("w", w), ("w_k", w_k), ("w_v", w_v)):
            if t is not None and (t.dtype != wdt or t.dim() != 2):
                raise TypeError(f"{name} must be a 2-D tensor of the weights' dtype {wdt}")
        w8 = wdt == torch.float8_e4m3fn
        if w8 != (w_scale is not None):
            raise TypeError("w_scale goes with float8_e4m3fn weights, and only with them")
        if w8 and (w_scale.dtype != torch.float32 or not w_scale.is_contiguous()
                   or w_scale.numel() != (n_head + 2 * n_kv_head) * head_dim):
            raise TypeError("w_scale must be a contiguous float32 tensor of nqt + 2*nkt scales")
        for name, t in (("w", w), ("w_k", w_k), ("w_v", w_v)):
            if t is not None and not t.is_contiguous():
                raise TypeError(f"{name} must be contiguous")
        for name, t in (("q", q), ("k", k), ("v", v), ("bq", bq), ("bk", bk), ("bv", bv)):
            if t is not None and t.dtype != torch.float32:
                raise TypeError(f"{name} must be float32")
        for name, t in (("pos", pos), ("slot", slot)):
            if t is not None and (t.dtype != torch.int32 or not t.is_contiguous()):
                raise TypeError(f"{name} must be a contiguous int32 tensor")
        hidden = x.shape[1]
        if w.shape[1] != hidden or any(t is not None and t.shape[1] != hidden for t in (w_k, w_v)):
            raise ValueError("x and the weights must share the hidden size")
        nt = int(pos.numel())
        nqt, nkt = n_head * head_dim, n_kv_head * head_dim
        if x.shape[0] != nt:
            raise ValueError(f"x has {x.shape[0]} rows, pos has {nt} tokens")
        if w_k is None:
            if w.shape[0] != nqt + 2 * nkt:
                raise ValueError(f"w has {w.shape[0]} rows, the concat q|k|v weights need "
                                 f"nqt + 2*nkt = {nqt + 2 * nkt}")
        else:
            for name, t, rows in (("w", w, nqt), ("w_k", w_k, nkt), ("w_v", w_v, nkt)):
                if t.shape[0] != rows:
                    raise ValueError(f"{name} has {t.shape[0]} rows, expected {rows}")
        check_extents(q, k, v, bq, bk, bv, pos, slot, kcache, vcache, n_head=n_head,
                      n_kv_head=n_kv_head, head_dim=head_dim, n_ctx=n_ctx or self.n_ctx,
                      n_slots=n_slots or 1)
        _check_device(self.device, x=x, w=w, w_k=w_k, w_v=w_v, w_scale=w_scale, q=q, k=k, v=v,
                      bq=bq, bk=bk, bv=bv, pos=pos, slot=slot, kcache=kcache, vcache=vcache)
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        epi = make_args(q, k, v, bq, bk, bv, pos, kcache, vcache, n_head=n_head,
                        n_kv_head=n_kv_head, head_dim=head_dim, theta=theta, cache_dtype=cd,
                        slot=slot, n_ctx=n_ctx or 0, n_slots=n_slots or 0, stream=stream,
                        use_stream=True, nt=int(pos.numel()), rope_style=rope_style,
                        freq_scale=freq_scale)
        ld_x = x.stride(0) if x.stride(0) != hidden else 0
        rc = qkv_epilogue_run_proj(self.h, make_proj_args(
            x, w, hidden, epi, ld_x=ld_x, w_k=w_k, w_v=w_v,
            w_format=QKV_WEIGHT_E4M3 if w8 else QKV_WEIGHT_BF16, w_scale=w_scale))
        if rc != QKV_OK:
            raise QkvError(rc, qkv_epilogue_last_error(self.h))

    def status(self) -> int:
        return qkv_epilogue_status(self.h)

    def last_error(self) -> str:
        return qkv_epilogue_last_error(self.h)

    def close(self):
        if self.h:
            qkv_epilogue_destroy(self.h)
            self.h = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
