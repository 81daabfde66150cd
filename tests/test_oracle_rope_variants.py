"""Pins of the oracle's rope variants: interleaved (GPT-J) pairing and a
frequency scale.  The page "06 · Assign + fusion" §3.2 names the rotary style
other than NeoX; the page "73 · D3-8" §3.2 Excerpt A multiplies the frequency
by freq_scale.  Checks: a hand-worked interleaved case, interleaved == NeoX on
the de-interleaved vector (bit for bit), numpy complex multiply at large
positions, the scaled inverse frequencies against decimal arithmetic, scale 1
== unscaled, and scale 2^-k at position p == scale 1 at p / 2^k (exact)."""
import os
from decimal import Decimal

import numpy as np
import pytest

import oracle
from qkv_bias_rope_amd import workloads as wl
from test_oracle_pins import dec_inv_freq, dec_sincos, dec_to_f32

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def test_interleaved_handworked_1h4d():
    want = []
    for line in open(os.path.join(GOLDEN, "rope_interleaved_1h4d.txt")):
        if line.startswith("#") or not line.strip():
            continue
        want.append(np.float32(float(line.split()[1])))
    want = np.array(want, np.float32)
    s0, c0 = dec_sincos(Decimal(1))
    s1, c1 = dec_sincos(Decimal(float(np.float32(1e-3))))
    closed = np.array([dec_to_f32(c0), dec_to_f32(s0), dec_to_f32(-s1), dec_to_f32(c1)])
    assert np.array_equal(bits(closed), bits(want))
    x = np.array([1, 0, 0, 1], np.float32)
    oracle.rope_interleaved(x, 1, 4, 1, 4, np.array([1], np.int32), oracle.inv_freq(1e6, 4))
    assert np.array_equal(bits(x), bits(want))


def _deinterleave(x, heads, hd):
    h = x.reshape(x.shape[0], heads, hd)
    return np.ascontiguousarray(np.concatenate([h[..., 0::2], h[..., 1::2]], axis=2))


def _interleave(y, heads, hd):
    h = y.reshape(y.shape[0], heads, hd)
    out = np.empty_like(h)
    out[..., 0::2] = h[..., : hd // 2]
    out[..., 1::2] = h[..., hd // 2:]
    return out


@pytest.mark.parametrize("hd", [4, 64, 128])
def test_interleaved_is_permuted_neox(hd):
    """Pairs (2i, 2i+1) rotated = NeoX on the vector with the even elements in
    the first half and the odd ones in the second, permuted back."""
    rng = np.random.default_rng(hd)
    nt, heads = 5, 3
    x = rng.standard_normal((nt, heads * hd)).astype(np.float32)
    pos = rng.integers(0, 40000, nt).astype(np.int32)
    inv = oracle.inv_freq(1e6, hd)
    a = x.copy().ravel()
    oracle.rope_interleaved(a, nt, heads * hd, heads, hd, pos, inv)
    d = _deinterleave(x, heads, hd).ravel()
    oracle.rope_neox(d, nt, heads * hd, heads, hd, pos, inv)
    b = _interleave(d.reshape(nt, -1), heads, hd).ravel()
    assert np.array_equal(bits(a), bits(b))


def test_interleaved_complex_multiply():
    hd, heads = 128, 4
    pos = np.array([0, 1, 4095, 32767], np.int32)
    rng = np.random.default_rng(9)
    x = rng.standard_normal((4, heads * hd)).astype(np.float32)
    a = x.copy().ravel()
    oracle.rope_interleaved(a, 4, heads * hd, heads, hd, pos, oracle.inv_freq(1e6, hd))
    inv = dec_inv_freq(1e6, hd)
    ang = (pos.astype(np.float32)[:, None] * inv[None, :]).astype(np.float32).astype(np.float64)
    h = x.astype(np.float64).reshape(4, heads, hd)
    z = (h[..., 0::2] + 1j * h[..., 1::2]) * np.exp(1j * ang)[:, None, :]
    o = a.reshape(4, heads, hd).astype(np.float64)
    mag = np.abs(z)
    assert np.all(np.abs(o[..., 0::2] - z.real) <= mag * 2.0 ** -23 + np.spacing(np.abs(z.real).astype(np.float32)))
    assert np.all(np.abs(o[..., 1::2] - z.imag) <= mag * 2.0 ** -23 + np.spacing(np.abs(z.imag).astype(np.float32)))


@pytest.mark.parametrize("scale", [0.25, 0.5, 1.0 / 3.0, 2.0, 0.125])
@pytest.mark.parametrize("hd", [64, 128])
def test_scaled_inv_freq_matches_decimal(scale, hd):
    got = oracle.inv_freq_scaled(1e6, scale, hd)
    s = Decimal(float(np.float32(scale)))
    lt = Decimal(1e6).ln()
    want = np.array([dec_to_f32(s * (-(Decimal(2 * i) / Decimal(hd)) * lt).exp())
                     for i in range(hd // 2)], np.float32)
    assert np.array_equal(bits(got), bits(want))


def test_scale_one_is_unscaled():
    for hd in (4, 64, 128, 96):
        assert np.array_equal(bits(oracle.inv_freq_scaled(1e6, 1.0, hd)), bits(oracle.inv_freq(1e6, hd)))


@pytest.mark.parametrize("style", [oracle.ROPE_NEOX, oracle.ROPE_INTERLEAVED])
def test_power_of_two_scale_equals_scaled_position(style):
    """inv*2^-k is exact, and f32(p * inv * 2^-k) = f32((p / 2^k) * inv) when
    2^k divides p, so the whole chain at scale 2^-k and position p equals the
    chain at scale 1 and position p / 2^k, bit for bit."""
    w = wl.DECODE_14B
    for k in (1, 2, 3):
        p = np.array([8 * 37, 8 * 511, 8 * 1, 8 * 4000], np.int32)
        d = wl.draw_layer(w, 0, nt=4)
        outs = []
        for pos, scale in ((p, 2.0 ** -k), (p // (2 ** k), 1.0)):
            q, kk, v = (d[n].copy().ravel() for n in ("q", "k", "v"))
            oracle.qkv_epilogue(q, kk, v, d["bq"], d["bk"], d["bv"], pos.astype(np.int32),
                                n_head=w.n_head, n_kv_head=w.n_kv_head, head_dim=w.head_dim,
                                theta=w.theta, n_ctx=1 << 16, cache_dtype=wl.CACHE_F32,
                                rope_style=style, freq_scale=scale)
            outs.append((q, kk, v))
        for a, b in zip(*outs):
            assert np.array_equal(bits(a), bits(b)), k


def test_chain_style_and_scale_are_applied():
    """The chain with interleaved pairing equals add_bias then rope_interleaved;
    with scale 0.5 the angles halve (checked at pos 2 vs pos 1 above); here the
    chain's q at pos 0 is bias-only for either style."""
    w = wl.TINY_DECODE
    d = wl.draw_layer(w, 0, nt=2)
    for style in (oracle.ROPE_NEOX, oracle.ROPE_INTERLEAVED):
        q, k, v = (d[n].copy().ravel() for n in ("q", "k", "v"))
        oracle.qkv_epilogue(q, k, v, d["bq"], d["bk"], d["bv"], np.zeros(2, np.int32),
                            n_head=w.n_head, n_kv_head=w.n_kv_head, head_dim=w.head_dim,
                            theta=w.theta, n_ctx=32, cache_dtype=0, rope_style=style,
                            freq_scale=0.5)
        assert np.array_equal(bits(q), bits((d["q"] + d["bq"][None, :]).astype(np.float32).ravel()))
    # interleaved differs from NeoX at a nonzero position
    outs = []
    for style in (oracle.ROPE_NEOX, oracle.ROPE_INTERLEAVED):
        q, k, v = (d[n].copy().ravel() for n in ("q", "k", "v"))
        oracle.qkv_epilogue(q, k, v, d["bq"], d["bk"], d["bv"], np.array([3, 9], np.int32),
                            n_head=w.n_head, n_kv_head=w.n_kv_head, head_dim=w.head_dim,
                            theta=w.theta, n_ctx=32, cache_dtype=0, rope_style=style)
        outs.append(q)
    assert not np.array_equal(outs[0], outs[1])
