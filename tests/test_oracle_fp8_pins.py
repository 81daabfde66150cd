"""Pins of the oracle's 8-bit-float-weight projection (the concat q|k|v matmul
of page "73 · D3-8" §2 with weights stored as OCP E4M3 codes and one f32
scale per weight row): the code table against torch's own float8_e4m3fn
conversion and against closed forms of the encoding, exact rational
arithmetic on a small case, the same values through the bfloat16 projection,
and the scale applied once per row."""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import torch

import oracle
from qkv_bias_rope_amd import workloads as wl
from test_oracle_pins import dec_to_f32

getcontext().prec = 60

ALL = np.arange(256, dtype=np.uint8)


def _finite_codes(rng, shape):
    """Random E4M3 codes, NaN patterns (0x7f, 0xff) excluded."""
    c = rng.integers(0, 254, shape).astype(np.uint8)
    return np.where(c >= 0x7f, c + 1, c).astype(np.uint8)


def test_code_table_matches_torch():
    want = torch.from_numpy(ALL.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = oracle.e4m3_values(ALL)
    nan = np.isnan(want)
    assert np.array_equal(np.nonzero(nan)[0], [0x7f, 0xff])
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan].astype(np.float64))
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_code_table_closed_forms():
    v = oracle.e4m3_values(ALL)
    assert v[0x00] == 0.0 and not np.signbit(v[0x00])
    assert v[0x80] == 0.0 and np.signbit(v[0x80])
    assert v[0x38] == 1.0                       # exponent field 7 = bias
    assert v[0x7e] == 448.0                     # largest finite: 1.75 * 2^8
    assert v[0x01] == 2.0 ** -9                 # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9             # largest subnormal
    assert v[0x08] == 2.0 ** -6                 # smallest normal
    assert v[0x3c] == 1.5 and v[0x40] == 2.0
    # the positive finite codes increase strictly; the sign bit negates
    pos = v[:0x7f]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(v[0x80:0xff], -pos)
    # each binade holds 8 evenly spaced values
    for e in range(1, 15):
        b = pos[8 * e: 8 * e + 8]
        assert np.all(np.diff(b) == 2.0 ** (e - 10))


def test_exact_rational_small():
    rng = np.random.default_rng(21)
    x = wl.bf16_bits(rng.standard_normal((3, 64)).astype(np.float32))
    w = _finite_codes(rng, (5, 64))
    s = (rng.uniform(0.5, 2.0, 5) * 2.0 ** -6).astype(np.float32)
    y = oracle.proj_fp8w(x, w, s)
    xf = wl.bf16_to_f32(x)
    wv = torch.from_numpy(w.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    for t in range(3):
        for n in range(5):
            exact = Fraction(float(s[n])) * sum(Fraction(float(a)) * Fraction(float(b))
                                                for a, b in zip(xf[t], wv[n]))
            want = dec_to_f32(Decimal(exact.numerator) / Decimal(exact.denominator))
            assert y[t, n] == want, (t, n, y[t, n], want)


def test_equals_bf16_projection_of_the_decoded_values():
    """Every E4M3 value is a bfloat16 value; with unit scales the 8-bit
    projection equals the oracle's bfloat16 projection of the decoded weights
    bit for bit."""
    rng = np.random.default_rng(22)
    x = wl.bf16_bits(rng.standard_normal((4, 256)).astype(np.float32))
    w = _finite_codes(rng, (40, 256))
    dec = oracle.e4m3_values(w).astype(np.float32)
    wb = wl.bf16_bits(dec)
    assert np.array_equal(wl.bf16_to_f32(wb), dec)
    y8 = oracle.proj_fp8w(x, w, np.ones(40, np.float32))
    y16 = oracle.proj_bf16(x, wb)
    assert np.array_equal(y8.view(np.uint32), y16.view(np.uint32))


def test_scale_applies_once_per_row():
    """Power-of-two scales scale the rows exactly; a row's scale touches only
    its own output."""
    rng = np.random.default_rng(23)
    x = wl.bf16_bits(rng.standard_normal((2, 128)).astype(np.float32))
    w = _finite_codes(rng, (6, 128))
    one = oracle.proj_fp8w(x, w, np.ones(6, np.float32))
    s = np.array([1, 2, 0.5, 2.0 ** -7, 8, 1], np.float32)
    y = oracle.proj_fp8w(x, w, s)
    assert np.array_equal(y, one * s)
    s2 = np.ones(6, np.float32)
    s2[3] = 0.0
    y2 = oracle.proj_fp8w(x, w, s2)
    assert np.all(y2[:, 3] == 0) and np.array_equal(np.delete(y2, 3, 1), np.delete(one, 3, 1))


def test_single_code_rows_decode_exactly():
    """One-hot activations pick single weights: with unit scales the output is
    the code's value, for every finite code."""
    codes = np.array([c for c in range(256) if c not in (0x7f, 0xff)], np.uint8)
    hidden = 64
    w = np.zeros((codes.size, hidden), np.uint8)
    w[:, 5] = codes
    x = np.zeros((1, hidden), np.uint16)
    x[0, 5] = 0x3f80                            # bfloat16 1.0
    y = oracle.proj_fp8w(x, w, np.ones(codes.size, np.float32))
    want = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    assert np.array_equal(y[0], want)
