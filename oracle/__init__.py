"""CPU oracle of the attention-input epilogue (numpy front end of qkv_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark may import this package; the product path (the HIP library and
its Python binding) never does.  It shares no code with the HIP path.

The C file holds the arithmetic; this module only compiles it (gcc, -O2,
-ffp-contract=off, no fast-math), loads it with ctypes and marshals numpy
arrays.  The steps follow the unfused chain described on the page "73 · D3-8 —
G4 FusedQKV ported to CUDA", §2 and §3.2 Excerpt A: add_bias on q, k, v; rope
(NeoX pairing) on q, then k; store K, then store V.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qkv_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CACHE_F32 = 0
CACHE_F16 = 1


def build(force: bool = False) -> str:
    """Compile qkv_oracle.c into liboracle.so next to it."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
            "-Wall", "-Wextra", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _bind(lib):
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    F = ctypes.c_float
    lib.oracle_add_bias.argtypes = [P, P, I64, I64, I64]
    lib.oracle_add_bias.restype = None
    lib.oracle_inv_freq.argtypes = [F, I, P]
    lib.oracle_inv_freq.restype = None
    lib.oracle_rope_neox.argtypes = [P, I64, I64, I, I, P, P]
    lib.oracle_rope_neox.restype = None
    lib.oracle_f32_to_f16.argtypes = [F]
    lib.oracle_f32_to_f16.restype = ctypes.c_uint16
    lib.oracle_store_rows.argtypes = [P, I64, I64, I64, P, P, I64, I64, I, P, P]
    lib.oracle_store_rows.restype = I64
    lib.oracle_scatter_rows.argtypes = [P, I64, I64, I, I64, P, P]
    lib.oracle_scatter_rows.restype = None
    lib.oracle_qkv_epilogue.argtypes = [
        P, P, P, I64, I64, I64, P, P, P, P, P, I64, I, I, I, F, I64, I64, I, I, F, P, P, P]
    lib.oracle_qkv_epilogue.restype = I64
    lib.oracle_rms_norm_heads.argtypes = [P, I64, I64, I, I, P, F]
    lib.oracle_rms_norm_heads.restype = None
    lib.oracle_qkv_norm_epilogue.argtypes = [
        P, P, P, I64, I64, I64, P, P, P, P, P, F, P, P, I64, I, I, I, F, I64, I64, I, I, F, P, P, P]
    lib.oracle_inv_freq_scaled.argtypes = [F, F, I, P]
    lib.oracle_inv_freq_scaled.restype = None
    lib.oracle_rope_interleaved.argtypes = [P, I64, I64, I, I, P, P]
    lib.oracle_rope_interleaved.restype = None
    lib.oracle_proj_bf16.argtypes = [P, I64, P, I64, I64, I64, P, I64]
    lib.oracle_proj_bf16.restype = None
    lib.oracle_e4m3_decode.argtypes = [P, I64, P]
    lib.oracle_e4m3_decode.restype = None
    lib.oracle_proj_fp8w.argtypes = [P, I64, P, P, I64, I64, I64, P, I64]
    lib.oracle_proj_fp8w.restype = None
    lib.oracle_qkv_norm_epilogue.restype = I64
    return lib


class using_library:
    """Context manager: route every oracle call to another build of the C file
    (used by the tests that plant mistakes in a copy of the oracle)."""

    def __init__(self, path):
        self.lib = _bind(ctypes.CDLL(path))

    def __enter__(self):
        global _lib
        self.saved = _load()
        _lib = self.lib
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _load():
    """The oracle library: liboracle.so built next to the source, or, when
    QKV_ORACLE_LIB names one, another build of the same C file (the sanitizer
    test runs the pins against an AddressSanitizer/UBSan build this way)."""
    global _lib
    if _lib is None:
        alt = os.environ.get("QKV_ORACLE_LIB")
        if alt:
            lib = _bind(ctypes.CDLL(alt))
        else:
            build()
            lib = _bind(ctypes.CDLL(_LIB))
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _f32(a, name):
    if not (isinstance(a, np.ndarray) and a.dtype == np.float32 and a.flags.c_contiguous):
        raise TypeError(f"{name} must be a C-contiguous float32 numpy array")
    return a


def _i32(a, name):
    if not (isinstance(a, np.ndarray) and a.dtype == np.int32 and a.flags.c_contiguous):
        raise TypeError(f"{name} must be a C-contiguous int32 numpy array")
    return a


# ---- single steps -----------------------------------------------------------

def add_bias(x, b, nt, width, ld):
    """Step O1 in place on x (rows of stride ld)."""
    _f32(x, "x"), _f32(b, "b")
    assert x.size >= (nt - 1) * ld + width if nt else True
    _load().oracle_add_bias(_ptr(x), _ptr(b), nt, width, ld)


def inv_freq(theta: float, head_dim: int) -> np.ndarray:
    """Step O2: the [head_dim/2] f32 inverse frequencies."""
    out = np.zeros(head_dim // 2, dtype=np.float32)
    _load().oracle_inv_freq(theta, head_dim, _ptr(out))
    return out


ROPE_NEOX = 0
ROPE_INTERLEAVED = 1


def inv_freq_scaled(theta: float, freq_scale: float, head_dim: int) -> np.ndarray:
    """Step O2 with a frequency scale: f32(freq_scale * theta^(-2i/hd))."""
    out = np.zeros(head_dim // 2, dtype=np.float32)
    _load().oracle_inv_freq_scaled(theta, freq_scale, head_dim, _ptr(out))
    return out


def rope_interleaved(x, nt, ld, n_heads, head_dim, pos, inv):
    """Step O3' (pairs (2i, 2i+1)) in place on x."""
    _f32(x, "x"), _i32(pos, "pos"), _f32(inv, "inv")
    assert pos.size >= nt and inv.size >= head_dim // 2
    if nt:
        assert x.size >= (nt - 1) * ld + n_heads * head_dim
    _load().oracle_rope_interleaved(_ptr(x), nt, ld, n_heads, head_dim, _ptr(pos), _ptr(inv))


def rope_neox(x, nt, ld, n_heads, head_dim, pos, inv):
    """Step O3 in place on x."""
    _f32(x, "x"), _i32(pos, "pos"), _f32(inv, "inv")
    assert pos.size >= nt and inv.size >= head_dim // 2
    if nt:
        assert x.size >= (nt - 1) * ld + n_heads * head_dim
    _load().oracle_rope_neox(_ptr(x), nt, ld, n_heads, head_dim, _ptr(pos), _ptr(inv))


def rms_norm_heads(x, nt, ld, n_heads, head_dim, w, eps):
    """Step N (per-head RMS norm) in place on x."""
    _f32(x, "x"), _f32(w, "w")
    assert w.size >= head_dim
    if nt:
        assert x.size >= (nt - 1) * ld + n_heads * head_dim
    _load().oracle_rms_norm_heads(_ptr(x), nt, ld, n_heads, head_dim, _ptr(w), eps)


def f32_to_f16_bits(values) -> np.ndarray:
    """binary16 round-to-nearest-even bit patterns of float32 values."""
    lib = _load()
    flat = np.asarray(values, dtype=np.float32).ravel()
    return np.array([lib.oracle_f32_to_f16(float(v)) for v in flat], dtype=np.uint16)


def store_rows(x, nt, ld, nkt, pos, slot, n_ctx, n_slots, cache_dtype):
    """Step O4 (one of K or V): returns (row_ids[int64 nt], rows[nt][nkt], rejected)."""
    _f32(x, "x"), _i32(pos, "pos")
    if slot is not None:
        _i32(slot, "slot")
    row_ids = np.zeros(nt, dtype=np.int64)
    rows = np.zeros((nt, nkt), dtype=np.float32 if cache_dtype == CACHE_F32 else np.uint16)
    bad = _load().oracle_store_rows(_ptr(x), nt, ld, nkt, _ptr(pos), _ptr(slot),
                                    n_ctx, n_slots, cache_dtype, _ptr(row_ids), _ptr(rows))
    return row_ids, rows, int(bad)


def scatter_rows(cache, row_ids, rows):
    """Write [nt][nkt] rows into a dense [n_rows][nkt] cache array (in place)."""
    assert cache.flags.c_contiguous and rows.flags.c_contiguous and cache.dtype == rows.dtype
    nkt = cache.shape[-1]
    n_rows = cache.size // nkt
    row_ids = np.ascontiguousarray(row_ids, dtype=np.int64)
    _load().oracle_scatter_rows(_ptr(cache), n_rows, nkt, cache.itemsize, row_ids.size,
                                _ptr(row_ids), _ptr(rows))


# ---- the whole chain --------------------------------------------------------

def qkv_epilogue(q, k, v, bq, bk, bv, pos, *, n_head, n_kv_head, head_dim, theta,
                 n_ctx, cache_dtype, slot=None, n_slots=1, ld_q=None, ld_k=None, ld_v=None,
                 rope_style=ROPE_NEOX, freq_scale=1.0):
    """Run the unfused chain in place on q, k, v (float32 numpy arrays).

    q holds nt rows of stride ld_q (default n_head*head_dim), k and v rows of
    stride ld_k / ld_v (default n_kv_head*head_dim); the three may be views of
    one concat buffer.  Returns (row_ids, krows, vrows, rejected): the cache row
    each token's K/V went to (-1 if rejected) and the [nt][nkt] rows in the
    cache dtype (float32, or uint16 binary16 bits).
    """
    nt = int(pos.size)
    nqt = n_head * head_dim
    nkt = n_kv_head * head_dim
    ld_q = nqt if ld_q is None else ld_q
    ld_k = nkt if ld_k is None else ld_k
    ld_v = nkt if ld_v is None else ld_v
    for name, a in (("q", q), ("k", k), ("v", v), ("bq", bq), ("bk", bk), ("bv", bv)):
        if not (isinstance(a, np.ndarray) and a.dtype == np.float32):
            raise TypeError(f"{name} must be float32")
    _i32(pos, "pos")
    if slot is not None:
        _i32(slot, "slot")
    assert bq.size >= nqt and bk.size >= nkt and bv.size >= nkt
    row_ids = np.zeros(nt, dtype=np.int64)
    rdt = np.float32 if cache_dtype == CACHE_F32 else np.uint16
    krows = np.zeros((nt, nkt), dtype=rdt)
    vrows = np.zeros((nt, nkt), dtype=rdt)

    def base(a, ld, width, name):
        # a is a 1-D float32 view starting at the section's first element; it
        # must hold nt rows of stride ld (a view of a concat buffer qualifies).
        if a.ndim != 1 or not a.flags.c_contiguous:
            raise TypeError(f"{name} must be a 1-D contiguous float32 view")
        if nt and a.size < (nt - 1) * ld + width:
            raise ValueError(f"{name} holds {a.size} elements, needs {(nt - 1) * ld + width}")
        return a.ctypes.data

    bad = _load().oracle_qkv_epilogue(
        base(q, ld_q, nqt, "q"), base(k, ld_k, nkt, "k"), base(v, ld_v, nkt, "v"), ld_q, ld_k, ld_v,
        _ptr(bq), _ptr(bk), _ptr(bv), _ptr(pos), _ptr(slot), nt,
        n_head, n_kv_head, head_dim, theta, n_ctx, n_slots, cache_dtype, rope_style, freq_scale,
        _ptr(row_ids), _ptr(krows), _ptr(vrows))
    if bad < 0:
        raise ValueError("oracle: head_dim must be positive and even")
    return row_ids, krows, vrows, int(bad)


def qkv_norm_epilogue(q, k, v, bq, bk, bv, wq, wk, eps, pos, *, n_head, n_kv_head, head_dim,
                      theta, n_ctx, cache_dtype, slot=None, n_slots=1, ld_q=None, ld_k=None,
                      ld_v=None, rope_style=ROPE_NEOX, freq_scale=1.0):
    """The q/k-norm variant of the chain (biases may be None).  Same returns as
    qkv_epilogue."""
    nt = int(pos.size)
    nqt = n_head * head_dim
    nkt = n_kv_head * head_dim
    ld_q = nqt if ld_q is None else ld_q
    ld_k = nkt if ld_k is None else ld_k
    ld_v = nkt if ld_v is None else ld_v
    for name, a in (("q", q), ("k", k), ("v", v), ("wq", wq), ("wk", wk)):
        if not (isinstance(a, np.ndarray) and a.dtype == np.float32):
            raise TypeError(f"{name} must be float32")
    for name, a in (("bq", bq), ("bk", bk), ("bv", bv)):
        if a is not None and not (isinstance(a, np.ndarray) and a.dtype == np.float32):
            raise TypeError(f"{name} must be float32 or None")
    _i32(pos, "pos")
    if slot is not None:
        _i32(slot, "slot")
    assert wq.size >= head_dim and wk.size >= head_dim
    row_ids = np.zeros(nt, dtype=np.int64)
    rdt = np.float32 if cache_dtype == CACHE_F32 else np.uint16
    krows = np.zeros((nt, nkt), dtype=rdt)
    vrows = np.zeros((nt, nkt), dtype=rdt)
    for name, a, ld, width in (("q", q, ld_q, nqt), ("k", k, ld_k, nkt), ("v", v, ld_v, nkt)):
        if a.ndim != 1 or not a.flags.c_contiguous:
            raise TypeError(f"{name} must be a 1-D contiguous float32 view")
        if nt and a.size < (nt - 1) * ld + width:
            raise ValueError(f"{name} holds {a.size} elements, needs {(nt - 1) * ld + width}")
    bad = _load().oracle_qkv_norm_epilogue(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, ld_q, ld_k, ld_v,
        _ptr(bq), _ptr(bk), _ptr(bv), _ptr(wq), _ptr(wk), eps, _ptr(pos), _ptr(slot), nt,
        n_head, n_kv_head, head_dim, theta, n_ctx, n_slots, cache_dtype, rope_style, freq_scale,
        _ptr(row_ids), _ptr(krows), _ptr(vrows))
    if bad < 0:
        raise ValueError("oracle: head_dim must be positive and even")
    return row_ids, krows, vrows, int(bad)


def proj_bf16(x_bits, w_bits):
    """Step P: y = x @ w.T with bfloat16 inputs (uint16 bit arrays [nt][hidden]
    and [n_out][hidden]), exact products, double sum, one rounding to f32."""
    for name, a in (("x", x_bits), ("w", w_bits)):
        if not (isinstance(a, np.ndarray) and a.dtype == np.uint16 and a.ndim == 2
                and a.flags.c_contiguous):
            raise TypeError(f"{name} must be a C-contiguous 2-D uint16 (bfloat16 bits) array")
    nt, hidden = x_bits.shape
    n_out, h2 = w_bits.shape
    assert h2 == hidden
    y = np.zeros((nt, n_out), np.float32)
    _load().oracle_proj_bf16(_ptr(x_bits), hidden, _ptr(w_bits), nt, n_out, hidden, _ptr(y), n_out)
    return y


def e4m3_values(codes):
    """The real value (float64; NaN for 0x7f / 0xff) of each OCP E4M3 code
    (uint8 array)."""
    codes = np.ascontiguousarray(codes, np.uint8)
    out = np.zeros(codes.shape, np.float64)
    _load().oracle_e4m3_decode(_ptr(codes), codes.size, _ptr(out))
    return out


def proj_fp8w(x_bits, w_codes, scale):
    """Step P with 8-bit float weights: y[t][n] = f32(scale[n] * sum_k x[t][k]
    * e4m3(w[n][k])), x bfloat16 bits [nt][hidden], w uint8 E4M3 codes
    [n_out][hidden], scale float32 [n_out]; exact products, double sum."""
    if not (isinstance(x_bits, np.ndarray) and x_bits.dtype == np.uint16 and x_bits.ndim == 2
            and x_bits.flags.c_contiguous):
        raise TypeError("x must be a C-contiguous 2-D uint16 (bfloat16 bits) array")
    if not (isinstance(w_codes, np.ndarray) and w_codes.dtype == np.uint8 and w_codes.ndim == 2
            and w_codes.flags.c_contiguous):
        raise TypeError("w must be a C-contiguous 2-D uint8 (E4M3 codes) array")
    nt, hidden = x_bits.shape
    n_out, h2 = w_codes.shape
    assert h2 == hidden
    scale = np.ascontiguousarray(scale, np.float32)
    assert scale.shape == (n_out,)
    y = np.zeros((nt, n_out), np.float32)
    _load().oracle_proj_fp8w(_ptr(x_bits), hidden, _ptr(w_codes), _ptr(scale), nt, n_out, hidden,
                             _ptr(y), n_out)
    return y
