"""The C ABI of include/qkv_epilogue.h as ctypes declarations, with no torch
dependency: return codes and constants, the argument structures, argument
builders, and typed calls of the host-only entry points (argument checks,
launch plan, inverse-frequency tables) on any loaded build of the library.
qkv_bias_rope_amd.binding loads the product library on top of this module;
the sanitizer tests load a host-only build of the same source through it.
Argument marshalling only.
"""
from __future__ import annotations

import ctypes

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



HOST_EXPORTS = ("qkv_epilogue_inv_freq", "qkv_epilogue_inv_freq_scaled", "qkv_epilogue_check_args",
                "qkv_epilogue_plan")


def bind(lib):
    """Declare argument and result types of the entry points `lib` exports
    (a build may export only the host-only ones)."""
    if hasattr(lib, "qkv_epilogue_create"):
        lib.qkv_epilogue_create.argtypes = [ctypes.POINTER(_P), ctypes.POINTER(QkvEpilogueConfig)]
    if hasattr(lib, "qkv_epilogue_create"):
        lib.qkv_epilogue_create.restype = _I
    if hasattr(lib, "qkv_epilogue_run"):
        lib.qkv_epilogue_run.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                         _I, _I, _I, _I, _F, _I]
    if hasattr(lib, "qkv_epilogue_run"):
        lib.qkv_epilogue_run.restype = _I
    if hasattr(lib, "qkv_epilogue_run_ex"):
        lib.qkv_epilogue_run_ex.argtypes = [_P, ctypes.POINTER(QkvEpilogueArgs)]
    if hasattr(lib, "qkv_epilogue_run_ex"):
        lib.qkv_epilogue_run_ex.restype = _I
    if hasattr(lib, "qkv_epilogue_run_unfused"):
        lib.qkv_epilogue_run_unfused.argtypes = [_P, ctypes.POINTER(QkvEpilogueArgs)]
    if hasattr(lib, "qkv_epilogue_run_unfused"):
        lib.qkv_epilogue_run_unfused.restype = _I
    if hasattr(lib, "qkv_epilogue_run_qk_norm"):
        lib.qkv_epilogue_run_qk_norm.argtypes = [_P, ctypes.POINTER(QkvEpilogueArgs), _P, _P, _F]
    if hasattr(lib, "qkv_epilogue_run_qk_norm"):
        lib.qkv_epilogue_run_qk_norm.restype = _I
    if hasattr(lib, "qkv_epilogue_status"):
        lib.qkv_epilogue_status.argtypes = [_P]
    if hasattr(lib, "qkv_epilogue_status"):
        lib.qkv_epilogue_status.restype = _I
    if hasattr(lib, "qkv_epilogue_last_error"):
        lib.qkv_epilogue_last_error.argtypes = [_P]
    if hasattr(lib, "qkv_epilogue_last_error"):
        lib.qkv_epilogue_last_error.restype = ctypes.c_char_p
    if hasattr(lib, "qkv_epilogue_destroy"):
        lib.qkv_epilogue_destroy.argtypes = [_P]
    if hasattr(lib, "qkv_epilogue_destroy"):
        lib.qkv_epilogue_destroy.restype = None
    if hasattr(lib, "qkv_epilogue_inv_freq"):
        lib.qkv_epilogue_inv_freq.argtypes = [_F, _I, _P]
    if hasattr(lib, "qkv_epilogue_inv_freq"):
        lib.qkv_epilogue_inv_freq.restype = _I
    if hasattr(lib, "qkv_epilogue_inv_freq_scaled"):
        lib.qkv_epilogue_inv_freq_scaled.argtypes = [_F, _F, _I, _P]
    if hasattr(lib, "qkv_epilogue_inv_freq_scaled"):
        lib.qkv_epilogue_inv_freq_scaled.restype = _I
    if hasattr(lib, "qkv_epilogue_check_args"):
        lib.qkv_epilogue_check_args.argtypes = [ctypes.POINTER(QkvEpilogueArgs), ctypes.c_char_p,
                                                ctypes.c_size_t]
    if hasattr(lib, "qkv_epilogue_check_args"):
        lib.qkv_epilogue_check_args.restype = _I
    if hasattr(lib, "qkv_epilogue_plan"):
        lib.qkv_epilogue_plan.argtypes = [ctypes.POINTER(QkvEpilogueArgs),
                                          ctypes.POINTER(QkvEpiloguePlan)]
    if hasattr(lib, "qkv_epilogue_plan"):
        lib.qkv_epilogue_plan.restype = _I
    if hasattr(lib, "qkv_epilogue_run_proj"):
        lib.qkv_epilogue_run_proj.argtypes = [_P, ctypes.POINTER(QkvProjArgs)]
    if hasattr(lib, "qkv_epilogue_run_proj"):
        lib.qkv_epilogue_run_proj.restype = _I
    if hasattr(lib, "qkv_epilogue_run_proj_noalloc"):
        lib.qkv_epilogue_run_proj_noalloc.argtypes = [_P, ctypes.POINTER(QkvProjArgs)]
    if hasattr(lib, "qkv_epilogue_run_proj_noalloc"):
        lib.qkv_epilogue_run_proj_noalloc.restype = _I
    return lib


def _addr(x):
    """Device address of a tensor (data_ptr) or a raw integer address."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


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


class HostApi:
    """The host-only entry points of one loaded build, typed."""

    def __init__(self, lib):
        self.lib = lib

    def qkv_epilogue_inv_freq(self, theta: float, head_dim: int, out_addr: int) -> int:
        return self.lib.qkv_epilogue_inv_freq(theta, head_dim, out_addr)

    def qkv_epilogue_inv_freq_scaled(self, theta: float, freq_scale: float, head_dim: int,
                                     out_addr: int) -> int:
        return self.lib.qkv_epilogue_inv_freq_scaled(theta, freq_scale, head_dim, out_addr)

    def qkv_epilogue_check_args(self, args: QkvEpilogueArgs):
        """Returns (rc, message)."""
        buf = ctypes.create_string_buffer(512)
        rc = self.lib.qkv_epilogue_check_args(ctypes.byref(args), buf, len(buf))
        return rc, buf.value.decode()

    def qkv_epilogue_plan(self, args: QkvEpilogueArgs):
        """Returns (rc, QkvEpiloguePlan)."""
        p = QkvEpiloguePlan()
        rc = self.lib.qkv_epilogue_plan(ctypes.byref(args), ctypes.byref(p))
        return rc, p


def load_host(path: str) -> HostApi:
    """A build of the library (or of its host-only part) at `path`, with its
    host-only entry points typed."""
    return HostApi(bind(ctypes.CDLL(path)))
