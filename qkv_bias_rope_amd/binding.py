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

QKV_OK = 0
QKV_ERR_INVALID_ARG = -1
QKV_ERR_ALIAS = -2
QKV_ERR_UNSUPPORTED = -3
QKV_ERR_HIP = -4
QKV_ERR_POSITION_RANGE = -5
ERR_NAMES = {0: "QKV_OK", -1: "QKV_ERR_INVALID_ARG", -2: "QKV_ERR_ALIAS",
             -3: "QKV_ERR_UNSUPPORTED", -4: "QKV_ERR_HIP", -5: "QKV_ERR_POSITION_RANGE"}
QKV_CACHE_F32 = 0
QKV_CACHE_F16 = 1
QKV_ROPE_NEOX = 0
QKV_ROPE_INTERLEAVED = 1
QKV_WEIGHT_BF16 = 0
QKV_WEIGHT_E4M3 = 1
QKV_MAX_HEAD_DIM = 512

EXPORTS = ("qkv_epilogue_create", "qkv_epilogue_run", "qkv_epilogue_run_ex",
           "qkv_epilogue_run_unfused", "qkv_epilogue_run_qk_norm",
           "qkv_epilogue_status", "qkv_epilogue_last_error", "qkv_epilogue_destroy",
           "qkv_epilogue_inv_freq", "qkv_epilogue_inv_freq_scaled", "qkv_epilogue_check_args",
           "qkv_epilogue_plan", "qkv_epilogue_run_proj", "qkv_epilogue_run_proj_noalloc")

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_F = ctypes.c_float


class QkvEpilogueConfig(ctypes.Structure):
    _fields_ = [("device", _I), ("n_ctx", _I64), ("stream", _P)]


class QkvEpilogueArgs(ctypes.Structure):
    _fields_ = [
        ("q", _P), ("k", _P), ("v", _P),
        ("bq", _P), ("bk", _P), ("bv", _P),
        ("pos", _P), ("slot", _P),
        ("kcache", _P), ("vcache", _P),
        ("ld_q", _I64), ("ld_k", _I64), ("ld_v", _I64),
        ("n_ctx", _I64), ("n_slots", _I64),
        ("nt", _I), ("n_head", _I), ("n_kv_head", _I), ("head_dim", _I),
        ("theta", _F),
        ("cache_dtype", _I), ("rope_style", _I),
        ("stream", _P), ("use_stream", _I),
        ("freq_scale", _F),
    ]


class QkvProjArgs(ctypes.Structure):
    _fields_ = [("x", _P), ("w", _P), ("hidden", _I), ("ld_x", _I64),
                ("epi", QkvEpilogueArgs), ("w_k", _P), ("w_v", _P), ("w_format", _I),
                ("w_scale", _P)]


class QkvEpiloguePlan(ctypes.Structure):
    _fields_ = [("vec_width", _I), ("units_per_token", _I), ("units_per_thread", _I),
                ("block", _I), ("col_blocks", _I), ("tokens_per_block", _I), ("grid", _I64),
                ("lds_bytes", _I)]


class QkvError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{ERR_NAMES.get(code, code)}: {msg}")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc --offload-arch=gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.qkv_epilogue_create.argtypes = [ctypes.POINTER(_P), ctypes.POINTER(QkvEpilogueConfig)]
    lib.qkv_epilogue_create.restype = _I
    lib.qkv_epilogue_run.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                     _I, _I, _I, _I, _F, _I]
    lib.qkv_epilogue_run.restype = _I
    lib.qkv_epilogue_run_ex.argtypes = [_P, ctypes.POINTER(QkvEpilogueArgs)]
    lib.qkv_epilogue_run_ex.restype = _I
    lib.qkv_epilogue_run_unfused.argtypes = [_P, ctypes.POINTER(QkvEpilogueArgs)]
    lib.qkv_epilogue_run_unfused.restype = _I
    lib.qkv_epilogue_run_qk_norm.argtypes = [_P, ctypes.POINTER(QkvEpilogueArgs), _P, _P, _F]
    lib.qkv_epilogue_run_qk_norm.restype = _I
    lib.qkv_epilogue_status.argtypes = [_P]
    lib.qkv_epilogue_status.restype = _I
    lib.qkv_epilogue_last_error.argtypes = [_P]
    lib.qkv_epilogue_last_error.restype = ctypes.c_char_p
    lib.qkv_epilogue_destroy.argtypes = [_P]
    lib.qkv_epilogue_destroy.restype = None
    lib.qkv_epilogue_inv_freq.argtypes = [_F, _I, _P]
    lib.qkv_epilogue_inv_freq.restype = _I
    lib.qkv_epilogue_inv_freq_scaled.argtypes = [_F, _F, _I, _P]
    lib.qkv_epilogue_inv_freq_scaled.restype = _I
    lib.qkv_epilogue_check_args.argtypes = [ctypes.POINTER(QkvEpilogueArgs), ctypes.c_char_p,
                                            ctypes.c_size_t]
    lib.qkv_epilogue_check_args.restype = _I
    lib.qkv_epilogue_plan.argtypes = [ctypes.POINTER(QkvEpilogueArgs),
                                      ctypes.POINTER(QkvEpiloguePlan)]
    lib.qkv_epilogue_plan.restype = _I
    lib.qkv_epilogue_run_proj.argtypes = [_P, ctypes.POINTER(QkvProjArgs)]
    lib.qkv_epilogue_run_proj.restype = _I
    lib.qkv_epilogue_run_proj_noalloc.argtypes = [_P, ctypes.POINTER(QkvProjArgs)]
    lib.qkv_epilogue_run_proj_noalloc.restype = _I
    return lib


lib = _load()


def _addr(x):
    """Device address of a tensor (data_ptr) or a raw integer address."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


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


def make_proj_args(x, w, hidden, epi: QkvEpilogueArgs, ld_x=0, w_k=None, w_v=None,
                   w_format=QKV_WEIGHT_BF16, w_scale=None) -> QkvProjArgs:
    """Build the run_proj argument block: bf16 activations x and concat weight
    rows w (tensors, or raw addresses) -- or, with w_k and w_v, the q, k and v
    weights as three matrices -- the contraction length and the epilogue block
    whose q/k/v are the outputs.  w_format QKV_WEIGHT_E4M3: one-byte E4M3
    weights with the f32 row scales w_scale."""
    pa = QkvProjArgs()
    pa.x, pa.w = _addr(x), _addr(w)
    pa.w_k, pa.w_v = _addr(w_k), _addr(w_v)
    pa.w_format, pa.w_scale = w_format, _addr(w_scale)
    pa.hidden = hidden
    pa.ld_x = ld_x
    pa.epi = epi
    return pa


def qkv_epilogue_status(h) -> int:
    return lib.qkv_epilogue_status(h)


def qkv_epilogue_last_error(h) -> str:
    r = lib.qkv_epilogue_last_error(h)
    return r.decode() if r else ""


def qkv_epilogue_destroy(h) -> None:
    lib.qkv_epilogue_destroy(h)


def qkv_epilogue_inv_freq(theta: float, head_dim: int, out_addr: int) -> int:
    return lib.qkv_epilogue_inv_freq(theta, head_dim, out_addr)


def qkv_epilogue_inv_freq_scaled(theta: float, freq_scale: float, head_dim: int,
                                 out_addr: int) -> int:
    return lib.qkv_epilogue_inv_freq_scaled(theta, freq_scale, head_dim, out_addr)


def qkv_epilogue_check_args(args: QkvEpilogueArgs):
    """Returns (rc, message)."""
    buf = ctypes.create_string_buffer(512)
    rc = lib.qkv_epilogue_check_args(ctypes.byref(args), buf, len(buf))
    return rc, buf.value.decode()


def qkv_epilogue_plan(args: QkvEpilogueArgs):
    """Returns (rc, QkvEpiloguePlan)."""
    p = QkvEpiloguePlan()
    rc = lib.qkv_epilogue_plan(ctypes.byref(args), ctypes.byref(p))
    return rc, p


# ---- torch convenience ------------------------------------------------------

def _stream_addr(stream):
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _row_stride(t, width, name):
    """Row stride (elements) of a [nt][width] section view, 0 when dense."""
    if t.dim() == 1:
        return 0
    if t.dim() != 2 or t.stride(-1) != 1:
        raise ValueError(f"{name}: need a 1-D tensor or a 2-D view with unit column stride")
    if t.shape[-1] != width:
        raise ValueError(f"{name}: rows hold {t.shape[-1]} elements, expected {width}")
    return 0 if t.shape[0] <= 1 else t.stride(0)


def make_args(q, k, v, bq, bk, bv, pos, kcache, vcache, *, n_head, n_kv_head, head_dim,
              theta, cache_dtype, nt=None, slot=None, n_ctx=0, n_slots=0, ld_q=None,
              ld_k=None, ld_v=None, rope_style=QKV_ROPE_NEOX, stream=None,
              use_stream=False, freq_scale=0.0) -> QkvEpilogueArgs:
    """Build the run_ex argument block.  Tensors (or raw addresses) are taken as
    they are; strides come from 2-D tensor views unless given."""
    nqt, nkt = n_head * head_dim, n_kv_head * head_dim
    if nt is None:
        nt = int(pos.numel())
    if ld_q is None:
        ld_q = 0 if (q is None or isinstance(q, int)) else _row_stride(q, nqt, "q")
    if ld_k is None:
        ld_k = 0 if (k is None or isinstance(k, int)) else _row_stride(k, nkt, "k")
    if ld_v is None:
        ld_v = 0 if (v is None or isinstance(v, int)) else _row_stride(v, nkt, "v")
    a = QkvEpilogueArgs()
    a.q, a.k, a.v = _addr(q), _addr(k), _addr(v)
    a.bq, a.bk, a.bv = _addr(bq), _addr(bk), _addr(bv)
    a.pos, a.slot = _addr(pos), _addr(slot)
    a.kcache, a.vcache = _addr(kcache), _addr(vcache)
    a.ld_q, a.ld_k, a.ld_v = ld_q, ld_k, ld_v
    a.n_ctx, a.n_slots = n_ctx, n_slots
    a.nt, a.n_head, a.n_kv_head, a.head_dim = nt, n_head, n_kv_head, head_dim
    a.theta = theta
    a.cache_dtype = cache_dtype
    a.rope_style = rope_style
    a.stream = _stream_addr(stream)
    a.use_stream = 1 if use_stream else 0
    a.freq_scale = freq_scale
    return a


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
        [nqt+2*nkt] tensor of row scales (1-4 tokens); q, k, v are the float32
        outputs; biases may be None."""
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
