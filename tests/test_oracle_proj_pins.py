"""Pins of the oracle's bfloat16 projection step (the concat q|k|v matmul that
feeds the epilogue; page "73 · D3-8" §2 and Excerpt C): exact rational
arithmetic on a small case, identity weights, row permutation, and numpy's
float64 matmul of the same values."""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

import oracle
from qkv_bias_rope_amd import workloads as wl
from test_oracle_pins import dec_to_f32

getcontext().prec = 60


def _bf(a):
    return wl.bf16_bits(np.asarray(a, np.float32))


def test_exact_rational_small():
    rng = np.random.default_rng(11)
    x = _bf(rng.standard_normal((3, 64)))
    w = _bf(rng.standard_normal((5, 64)) * 0.2)
    y = oracle.proj_bf16(x, w)
    xf, wf = wl.bf16_to_f32(x), wl.bf16_to_f32(w)
    for t in range(3):
        for n in range(5):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(xf[t], wf[n]))
            want = dec_to_f32(Decimal(exact.numerator) / Decimal(exact.denominator))
            assert y[t, n] == want, (t, n, y[t, n], want)


def test_identity_weights_copy_the_input():
    rng = np.random.default_rng(12)
    hidden = 96
    x = _bf(rng.standard_normal((4, hidden)))
    w = _bf(np.eye(hidden, dtype=np.float32))
    y = oracle.proj_bf16(x, w)
    assert np.array_equal(y.view(np.uint32), wl.bf16_to_f32(x).view(np.uint32))


def test_row_permutation_permutes_outputs():
    rng = np.random.default_rng(13)
    x = _bf(rng.standard_normal((5, 128)))
    w = _bf(rng.standard_normal((40, 128)) * 0.1)
    perm = rng.permutation(40)
    y = oracle.proj_bf16(x, w)
    yp = oracle.proj_bf16(x, np.ascontiguousarray(w[perm]))
    assert np.array_equal(yp.view(np.uint32), y[:, perm].view(np.uint32))


def test_matches_numpy_float64_matmul():
    w_ = wl.DECODE_7B
    d = wl.draw_projection(w_, 3584, nt=4)
    y = oracle.proj_bf16(d["x"], d["w"][:512])
    ref = (wl.bf16_to_f32(d["x"]).astype(np.float64) @ wl.bf16_to_f32(d["w"][:512]).astype(np.float64).T)
    err = np.abs(y.astype(np.float64) - ref)
    # one rounding to f32 (half an ulp) plus numpy's own summation error
    assert np.all(err <= np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64))
    assert np.mean(y == ref.astype(np.float32)) > 0.999
