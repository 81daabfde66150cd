"""Pins of the oracle's per-head RMS norm (the q/k-norm variant of the chain,
named on the page "06 · Assign + fusion" §3.2 as QkNorm / FusedQkvNorm without
a formula; the reading is y = x / sqrt(mean(x^2) + eps) * w per head).

Independent checks only: hand-worked and decimal closed forms, exact
power-of-two scale invariance, the mean-square invariant, numpy's
linalg.norm, per-head independence, and the whole variant at pos 0 and at
large positions against numpy double-precision computations of the
definition.
"""
import math
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle
from qkv_bias_rope_amd import workloads as wl

getcontext().prec = 50


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def dec_f32(d):
    from test_oracle_pins import dec_to_f32
    return dec_to_f32(d)


def test_handworked_3_4():
    # x = [3, 4, 0, 0]: mean square 25/4, rms 2.5 -> [1.2, 1.6, 0, 0] (eps 0, w 1)
    x = np.array([3, 4, 0, 0], np.float32)
    oracle.rms_norm_heads(x, 1, 4, 1, 4, np.ones(4, np.float32), 0.0)
    want = np.array([dec_f32(Decimal(3) / Decimal("2.5")), dec_f32(Decimal(4) / Decimal("2.5")), 0, 0],
                    np.float32)
    assert np.array_equal(bits(x), bits(want))
    # weights scale element-wise: w = [2, 0.5, 7, 7] -> [2.4, 0.8, 0, 0]
    x = np.array([3, 4, 0, 0], np.float32)
    oracle.rms_norm_heads(x, 1, 4, 1, 4, np.array([2, 0.5, 7, 7], np.float32), 0.0)
    want = np.array([dec_f32(Decimal("2.4")), dec_f32(Decimal("0.8")), 0, 0], np.float32)
    assert np.array_equal(bits(x), bits(want))
    # eps = 0.75: mean square 6.25 + 0.75 = 7 -> [3/sqrt 7, 4/sqrt 7, 0, 0]
    x = np.array([3, 4, 0, 0], np.float32)
    oracle.rms_norm_heads(x, 1, 4, 1, 4, np.ones(4, np.float32), 0.75)
    s7 = Decimal(7).sqrt()
    want = np.array([dec_f32(3 / s7), dec_f32(4 / s7), 0, 0], np.float32)
    assert np.array_equal(bits(x), bits(want))


@pytest.mark.parametrize("c,eps", [(0.5, 1e-6), (-3.0, 1e-6), (1e-3, 1e-6), (2.0, 0.0), (1e-4, 1e-6)])
def test_constant_vector_closed_form(c, eps):
    hd = 64
    rng = np.random.default_rng(1)
    w = (1 + 0.1 * rng.standard_normal(hd)).astype(np.float32)
    x = np.full(hd, c, np.float32)
    oracle.rms_norm_heads(x, 1, hd, 1, hd, w, eps)
    cd, ed = Decimal(float(np.float32(c))), Decimal(float(np.float32(eps)))
    r = cd / (cd * cd + ed).sqrt()
    want = np.array([dec_f32(Decimal(float(wj)) * r) for wj in w], np.float32)
    diff = np.abs(x.astype(np.float64) - want.astype(np.float64))
    assert np.all(diff <= np.spacing(np.abs(want)).astype(np.float64))   # within 1 ulp
    assert np.sum(diff > 0) <= 2


def test_power_of_two_scale_invariance_is_exact():
    """With eps 0, scaling a head by 2^k scales every square by 4^k and the
    root by 2^k exactly, so the output is identical bit for bit."""
    rng = np.random.default_rng(2)
    hd, nh = 128, 5
    w = (1 + 0.1 * rng.standard_normal(hd)).astype(np.float32)
    x = rng.standard_normal(nh * hd).astype(np.float32)
    a = x.copy()
    oracle.rms_norm_heads(a, 1, nh * hd, nh, hd, w, 0.0)
    for k in (-20, -3, 1, 7, 30):
        b = (x * np.float32(2.0 ** k)).astype(np.float32)
        oracle.rms_norm_heads(b, 1, nh * hd, nh, hd, w, 0.0)
        assert np.array_equal(bits(a), bits(b)), k


def test_mean_square_invariant():
    """With unit weights the output's mean square is ms/(ms + eps)."""
    rng = np.random.default_rng(3)
    hd, nh = 128, 8
    for eps in (0.0, 1e-6, 0.5):
        x = (rng.standard_normal(nh * hd) * 0.3).astype(np.float32)
        ms = (x.astype(np.float64).reshape(nh, hd) ** 2).mean(axis=1)
        y = x.copy()
        oracle.rms_norm_heads(y, 1, nh * hd, nh, hd, np.ones(hd, np.float32), eps)
        got = (y.astype(np.float64).reshape(nh, hd) ** 2).mean(axis=1)
        assert np.allclose(got, ms / (ms + np.float64(np.float32(eps))), rtol=4e-7, atol=0)


def test_matches_linalg_norm():
    rng = np.random.default_rng(4)
    hd, nh, nt = 96, 6, 3
    w = (1 + 0.1 * rng.standard_normal(hd)).astype(np.float32)
    x = rng.standard_normal((nt, nh, hd)).astype(np.float32)
    eps = np.float32(1e-6)
    y = x.copy().ravel()
    oracle.rms_norm_heads(y, nt, nh * hd, nh, hd, w, float(eps))
    rms = np.linalg.norm(x.astype(np.float64), axis=2, keepdims=True) / math.sqrt(hd)
    want = x / np.sqrt(rms ** 2 + np.float64(eps)) * w.astype(np.float64)
    err = np.abs(y.reshape(nt, nh, hd) - want)
    assert np.all(err <= np.spacing(np.abs(want).astype(np.float32)).astype(np.float64))


def test_heads_are_independent_and_stride_respected():
    rng = np.random.default_rng(5)
    hd, nh, ld = 64, 4, 4 * 64 + 16
    w = (1 + 0.1 * rng.standard_normal(hd)).astype(np.float32)
    x = rng.standard_normal(2 * ld).astype(np.float32)
    a = x.copy()
    oracle.rms_norm_heads(a, 2, ld, nh, hd, w, 1e-6)
    b = x.copy()
    b[2 * hd:3 * hd] *= 5           # change head 2 of token 0
    oracle.rms_norm_heads(b, 2, ld, nh, hd, w, 1e-6)
    t0 = slice(0, nh * hd)
    assert np.array_equal(bits(a[0:2 * hd]), bits(b[0:2 * hd]))
    assert np.array_equal(bits(a[3 * hd:nh * hd]), bits(b[3 * hd:nh * hd]))
    assert np.array_equal(bits(a[ld:]), bits(b[ld:]))
    assert np.array_equal(a[nh * hd:ld], x[nh * hd:ld])   # padding untouched


def _variant(w_, nt, pos, bias=True, layer=0, cache_dtype=wl.CACHE_F32):
    d = wl.draw_layer(w_, layer, nt=nt)
    nw = wl.draw_norm_weights(w_, layer)
    d["pos"] = np.asarray(pos, np.int32)
    q, k, v = (d[n].copy().ravel() for n in ("q", "k", "v"))
    rid, kr, vr, bad = oracle.qkv_norm_epilogue(
        q, k, v, d["bq"] if bias else None, d["bk"] if bias else None, d["bv"] if bias else None,
        nw["wq"], nw["wk"], wl.QK_NORM_EPS, d["pos"], n_head=w_.n_head, n_kv_head=w_.n_kv_head,
        head_dim=w_.head_dim, theta=w_.theta, n_ctx=w_.n_ctx, cache_dtype=cache_dtype,
        slot=d["slot"], n_slots=w_.n_slots)
    return d, nw, q.reshape(nt, -1), k.reshape(nt, -1), v.reshape(nt, -1), rid, kr, vr


def _normed(x, b, wvec, heads, hd, eps):
    """numpy double precision: f32 bias add, then per-head RMS norm."""
    xb = (x + b[None, :]).astype(np.float32) if b is not None else x
    h = xb.astype(np.float64).reshape(xb.shape[0], heads, hd)
    ms = (h ** 2).mean(axis=2, keepdims=True)
    return h / np.sqrt(ms + np.float64(np.float32(eps))) * wvec.astype(np.float64)


@pytest.mark.parametrize("bias", [True, False])
def test_variant_at_pos0_is_bias_then_norm(bias):
    w_ = wl.DECODE_14B
    d, nw, q, k, v, rid, kr, vr = _variant(w_, 3, [0, 0, 0], bias=bias)
    for name, x, b, wv, heads in (("q", d["q"], d["bq"], nw["wq"], w_.n_head),
                                  ("k", d["k"], d["bk"], nw["wk"], w_.n_kv_head)):
        want = _normed(x, b if bias else None, wv, heads, w_.head_dim, wl.QK_NORM_EPS)
        got = (q if name == "q" else k).reshape(want.shape).astype(np.float64)
        assert np.all(np.abs(got - want) <= np.spacing(np.abs(want).astype(np.float32))), name
    want_v = (d["v"] + d["bv"][None, :]).astype(np.float32) if bias else d["v"]
    assert np.array_equal(bits(v), bits(want_v))          # v: bias only, never normalised
    assert np.array_equal(bits(kr), bits(k)) and np.array_equal(bits(vr), bits(v))


def test_variant_rotates_after_norm():
    """At large positions each pair of the output is the complex rotation of the
    normalised pair (norm with the weights first, then NeoX rope)."""
    from test_oracle_pins import dec_inv_freq
    w_ = wl.BATCHED_DECODE_14B
    pos = np.array([1, 32767, 777, 20000], np.int32)
    d, nw, q, k, v, rid, kr, vr = _variant(w_, 4, pos)
    inv = dec_inv_freq(w_.theta, w_.head_dim)
    ang = (pos.astype(np.float32)[:, None] * inv[None, :]).astype(np.float32).astype(np.float64)
    half = w_.head_dim // 2
    for x, b, wv, heads, out in ((d["q"], d["bq"], nw["wq"], w_.n_head, q),
                                 (d["k"], d["bk"], nw["wk"], w_.n_kv_head, k)):
        n = _normed(x, b, wv, heads, w_.head_dim, wl.QK_NORM_EPS)
        z = (n[..., :half] + 1j * n[..., half:]) * np.exp(1j * ang)[:, None, :]
        o = out.reshape(n.shape).astype(np.float64)
        mag = np.abs(z)
        tol = mag * 2.0 ** -22 + 2 * np.spacing(np.abs(z.real).astype(np.float32))
        assert np.all(np.abs(o[..., :half] - z.real) <= tol)
        tol = mag * 2.0 ** -22 + 2 * np.spacing(np.abs(z.imag).astype(np.float32))
        assert np.all(np.abs(o[..., half:] - z.imag) <= tol)
