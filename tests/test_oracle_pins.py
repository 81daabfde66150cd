"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

None of these re-type the oracle's formulas: each checks the oracle against a
closed form, an invariant, an independent high-precision computation (Python
``decimal``), a library routine (numpy complex128, numpy float16) or a
hand-worked case.  The op is the one on the page "73 · D3-8 — G4 FusedQKV
ported to CUDA" (§2, §3.2 Excerpt A) with the KV layout of "07 · The
allocator" (§2.5).
"""
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle
from qkv_bias_rope_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
getcontext().prec = 60


# ---- independent high-precision helpers (decimal) ---------------------------

def _dec_pi():
    # Machin: pi = 16 atan(1/5) - 4 atan(1/239)
    def atan_inv(n):
        x = Decimal(1) / n
        x2 = x * x
        term, total, k = x, x, 1
        while True:
            term *= -x2
            d = term / (2 * k + 1)
            if abs(d) < Decimal(10) ** -58:
                break
            total += d
            k += 1
        return total
    return 16 * atan_inv(5) - 4 * atan_inv(239)


PI = _dec_pi()


def dec_sincos(a: Decimal):
    """sin and cos of a decimal angle by range reduction and Taylor series."""
    two_pi = 2 * PI
    r = a - two_pi * (a / two_pi).to_integral_value(rounding="ROUND_FLOOR")
    s, c = Decimal(0), Decimal(0)
    term = r  # sin series
    k = 1
    s = term
    while abs(term) > Decimal(10) ** -55:
        term *= -r * r / ((2 * k) * (2 * k + 1))
        s += term
        k += 1
    term = Decimal(1)
    c = term
    k = 1
    while abs(term) > Decimal(10) ** -55:
        term *= -r * r / ((2 * k - 1) * (2 * k))
        c += term
        k += 1
    return s, c


def dec_to_f32(d: Decimal) -> np.float32:
    """The f32 nearest to a decimal value (ties to even), found by comparing
    the decimal with the neighbouring f32 values exactly."""
    f = np.float32(float(d))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = min(cands, key=lambda c: (abs(Decimal(float(c)) - d),
                                     int(np.array([c]).view(np.uint32)[0]) & 1))
    return np.float32(best)


def dec_inv_freq(theta, head_dim):
    lt = Decimal(theta).ln()
    return np.array([dec_to_f32((-(Decimal(2 * i) / Decimal(head_dim)) * lt).exp())
                     for i in range(head_dim // 2)], dtype=np.float32)


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32 if a.dtype == np.float32 else np.uint16)


# ---- O2: inverse frequencies ------------------------------------------------

@pytest.mark.parametrize("head_dim", [4, 6, 8, 64, 96, 128, 256])
@pytest.mark.parametrize("theta", [1.0e6, 1.0e4, 5.0e5])
def test_inv_freq_matches_decimal(theta, head_dim):
    got = oracle.inv_freq(theta, head_dim)
    want = dec_inv_freq(theta, head_dim)
    assert np.array_equal(bits(got), bits(want)), (got, want)


def test_inv_freq_closed_forms():
    inv = oracle.inv_freq(1.0e6, 4)
    assert inv[0] == np.float32(1.0)
    assert inv[1] == np.float32(1.0e-3)                 # 1e6^(-1/2)
    assert oracle.inv_freq(1.0e6, 128)[32] == np.float32(1.0e-3)
    assert oracle.inv_freq(1.0e6, 64)[16] == np.float32(1.0e-3)
    inv = oracle.inv_freq(1.0e6, 128)
    assert np.all(np.diff(inv.astype(np.float64)) < 0)   # strictly decreasing


# ---- f16 conversion ---------------------------------------------------------

def _read_f16_table():
    rows = []
    with open(os.path.join(GOLDEN, "f16_rne_table.txt")) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            a, b = line.split()[:2]
            rows.append((int(a, 16), int(b, 16)))
    return rows


def test_f16_golden_table():
    rows = _read_f16_table()
    f = np.array([r[0] for r in rows], dtype=np.uint32).view(np.float32)
    want = np.array([r[1] for r in rows], dtype=np.uint16)
    got = oracle.f32_to_f16_bits(f)
    assert np.array_equal(got, want), [(hex(a), hex(b), hex(c)) for a, b, c in
                                       zip(f.view(np.uint32), want, got) if b != c]
    # the table itself agrees with numpy's binary16 conversion
    with np.errstate(over="ignore"):
        assert np.array_equal(f.astype(np.float16).view(np.uint16), want)


def test_f16_matches_numpy_over_ranges():
    rng = np.random.default_rng(123)
    parts = [
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(5000) * 1e-5).astype(np.float32),      # subnormal range
        (rng.standard_normal(5000) * 3e4).astype(np.float32),       # near overflow
        rng.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ]
    # exact ties: f16 grid midpoints
    h = rng.integers(0, 0x7bff, 5000).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float32).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float32).astype(np.float64)
    parts.append(((lo + hi) / 2).astype(np.float32))
    x = np.concatenate(parts)
    x = x[~np.isnan(x)]
    got = oracle.f32_to_f16_bits(x)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def test_f16_nan_stays_nan():
    got = oracle.f32_to_f16_bits(np.array([np.nan, -np.nan], dtype=np.float32))
    assert np.all((got & 0x7c00) == 0x7c00) and np.all((got & 0x03ff) != 0)


# ---- O3: rope ---------------------------------------------------------------

def test_handworked_1h4d():
    want = []
    with open(os.path.join(GOLDEN, "rope_handworked_1h4d.txt")) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            idx, val = line.split()[:2]
            want.append(np.float32(float(val)))
    want = np.array(want, dtype=np.float32)
    # the golden decimals are the f32 nearest to the closed forms
    a1 = np.float32(np.float32(1.0e-3) * np.float32(1.0))
    closed = [dec_to_f32(Decimal(repr(math.cos(1.0)))), None, None, None]
    s1, c1 = dec_sincos(Decimal(float(a1)))
    s0, c0 = dec_sincos(Decimal(1))
    closed = np.array([dec_to_f32(c0), dec_to_f32(-s1), dec_to_f32(s0), dec_to_f32(c1)])
    assert np.array_equal(bits(closed), bits(want))

    x = np.array([1, 0, 0, 1], dtype=np.float32)
    inv = oracle.inv_freq(1.0e6, 4)
    oracle.rope_neox(x, 1, 4, 1, 4, np.array([1], dtype=np.int32), inv)
    assert np.array_equal(bits(x), bits(want)), (x, want)

    # through the whole chain (zero bias) the q and k sections give the same
    q = np.array([1, 0, 0, 1], dtype=np.float32)
    k = q.copy()
    v = np.array([3, -2, 0.5, 7], dtype=np.float32)
    z = np.zeros(4, dtype=np.float32)
    rid, kr, vr, bad = oracle.qkv_epilogue(q, k, v, z, z, z, np.array([1], np.int32),
                                           n_head=1, n_kv_head=1, head_dim=4, theta=1.0e6,
                                           n_ctx=2, cache_dtype=oracle.CACHE_F32)
    assert bad == 0 and rid.tolist() == [1]
    assert np.array_equal(bits(q), bits(want)) and np.array_equal(bits(k), bits(want))
    assert np.array_equal(v, [3, -2, 0.5, 7])
    assert np.array_equal(bits(kr[0]), bits(want)) and np.array_equal(vr[0], v)


def _chain(w, nt=None, pos=None, cache_dtype=None, layer=0):
    d = wl.draw_layer(w, layer, nt=nt)
    if pos is not None:
        d["pos"] = np.asarray(pos, dtype=np.int32)
    x = {n: d[n].copy() for n in ("q", "k", "v")}
    cd = w.cache_dtypes[0] if cache_dtype is None else cache_dtype
    rid, kr, vr, bad = oracle.qkv_epilogue(
        x["q"].ravel(), x["k"].ravel(), x["v"].ravel(), d["bq"], d["bk"], d["bv"], d["pos"],
        n_head=w.n_head, n_kv_head=w.n_kv_head, head_dim=w.head_dim, theta=w.theta,
        n_ctx=w.n_ctx, cache_dtype=cd, slot=d["slot"], n_slots=w.n_slots)
    return d, x, rid, kr, vr, bad


@pytest.mark.parametrize("w", [wl.TINY_DECODE, wl.DECODE_7B])
def test_pos0_is_bias_only(w):
    """At position 0 every angle is 0 (cos 1, sin 0), so q and k only get their
    bias: the result must be exactly f32(x + b); v is f32(v + b) at any pos."""
    d, x, rid, kr, vr, bad = _chain(w, nt=3, pos=[0, 0, 0], cache_dtype=oracle.CACHE_F32)
    assert bad == 0
    for n, b in (("q", "bq"), ("k", "bk"), ("v", "bv")):
        want = (d[n] + d[b][None, :]).astype(np.float32)
        assert np.array_equal(bits(x[n]), bits(want)), n
    assert np.array_equal(bits(kr), bits(x["k"])) and np.array_equal(bits(vr), bits(x["v"]))
    assert rid.tolist() == [0, 0, 0]


def test_v_is_bias_only_at_any_position():
    w = wl.DECODE_7B
    d, x, *_ = _chain(w, nt=4, pos=[1, 77, 4095, 2000])
    assert np.array_equal(bits(x["v"]), bits((d["v"] + d["bv"][None, :]).astype(np.float32)))


def _pairs(a, n_heads, hd):
    a = a.reshape(a.shape[0], n_heads, hd).astype(np.float64)
    return a[..., : hd // 2], a[..., hd // 2:]


@pytest.mark.parametrize("w", [wl.TINY_DECODE, wl.DECODE_14B])
def test_norm_preserved(w):
    pos = [1, 4095 % w.n_ctx, 31, 17]
    d, x, *_ = _chain(w, nt=4, pos=pos)
    for n, b, heads in (("q", "bq", w.n_head), ("k", "bk", w.n_kv_head)):
        xb = (d[n] + d[b][None, :]).astype(np.float32)
        x0, x1 = _pairs(xb, heads, w.head_dim)
        r0, r1 = _pairs(x[n], heads, w.head_dim)
        n_in = x0 * x0 + x1 * x1
        n_out = r0 * r0 + r1 * r1
        # each output is within half an f32 ulp of the exact rotation of
        # f32 inputs by f32-rounded cos/sin (|c|,|s| <= 1, c^2+s^2 = 1 +- 2^-23)
        tol = n_in * 4 * 2.0 ** -23 + 1e-30
        assert np.all(np.abs(n_out - n_in) <= tol), (n, np.max(np.abs(n_out - n_in) / (n_in + 1e-30)))


def test_matches_complex_multiply_large_angles():
    """Each rotated pair equals (x0 + i x1) * exp(i a) with a = f32(pos * inv),
    computed with numpy complex128 and the decimal-pinned inverse frequencies,
    up to the rounding of cos/sin to f32 and of the output to f32."""
    w = wl.BATCHED_DECODE_14B
    pos = np.array([0, 1, 2, 1000, 4095, 32767, 32766, 12345], dtype=np.int32)
    d, x, rid, kr, vr, bad = _chain(w, nt=8, pos=pos, cache_dtype=oracle.CACHE_F32)
    inv = dec_inv_freq(w.theta, w.head_dim)
    ang = (pos.astype(np.float32)[:, None] * inv[None, :]).astype(np.float32)  # f32 product
    for n, b, heads in (("q", "bq", w.n_head), ("k", "bk", w.n_kv_head)):
        xb = (d[n] + d[b][None, :]).astype(np.float32)
        x0, x1 = _pairs(xb, heads, w.head_dim)
        z = (x0 + 1j * x1) * np.exp(1j * ang.astype(np.float64))[:, None, :]
        r0, r1 = _pairs(x[n], heads, w.head_dim)
        mag = np.sqrt(x0 * x0 + x1 * x1)
        # cos/sin each rounded to f32 (<= 2^-24 abs) and the output rounded
        # to f32 (<= half an ulp): a bound of |x|*2^-23 + ulp(out)
        tol = mag * 2.0 ** -23 + np.spacing(np.abs(z.real).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(r0 - z.real) <= tol)
        tol = mag * 2.0 ** -23 + np.spacing(np.abs(z.imag).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(r1 - z.imag) <= tol)


def test_cos_sin_match_decimal_at_large_positions():
    """A unit pair (1, 0) rotated by angle a comes out as (cos a, sin a).  With
    f32 angles up to 32767 rad, compare with decimal sin/cos rounded to f32."""
    hd = 128
    inv = dec_inv_freq(1.0e6, hd)
    mismatches = 0
    for p in (32767, 30001, 4095, 1):
        x = np.zeros(hd, dtype=np.float32)
        x[: hd // 2] = 1.0
        oracle.rope_neox(x, 1, hd, 1, hd, np.array([p], np.int32), oracle.inv_freq(1.0e6, hd))
        for i in range(hd // 2):
            a = np.float32(np.float32(p) * inv[i])
            s, c = dec_sincos(Decimal(float(a)))
            wc, ws = dec_to_f32(c), dec_to_f32(s)
            for got, want in ((x[i], wc), (x[i + hd // 2], ws)):
                if got != want:
                    mismatches += 1
                    # only a double-rounding case may differ, by one f32 ulp
                    assert abs(float(got) - float(want)) <= float(np.spacing(np.abs(want)))
    assert mismatches <= 2


def test_rotations_compose_additively():
    w = wl.TINY_DECODE
    hd = w.head_dim
    rng = np.random.default_rng(7)
    inv = oracle.inv_freq(w.theta, hd)
    for p1, p2 in ((3, 5), (100, 27), (999, 1), (0, 64)):
        x = rng.standard_normal((1, 6 * hd), dtype=np.float32)
        a = x.copy().ravel()
        oracle.rope_neox(a, 1, 6 * hd, 6, hd, np.array([p1], np.int32), inv)
        oracle.rope_neox(a, 1, 6 * hd, 6, hd, np.array([p2], np.int32), inv)
        b = x.copy().ravel()
        oracle.rope_neox(b, 1, 6 * hd, 6, hd, np.array([p1 + p2], np.int32), inv)
        ang = lambda p: (np.float32(p) * inv).astype(np.float32)
        sp = lambda a_: np.spacing(np.abs(a_)).astype(np.float64)
        dang = 0.5 * (sp(ang(p1)) + sp(ang(p2)) + sp(ang(p1 + p2)))
        x0, x1 = _pairs(x, 6, hd)
        mag = np.sqrt(x0 * x0 + x1 * x1)[0]
        tol = mag * (dang[None, :] + 8 * 2.0 ** -24)
        a0, a1 = _pairs(a.reshape(1, -1), 6, hd)
        b0, b1 = _pairs(b.reshape(1, -1), 6, hd)
        assert np.all(np.abs(a0 - b0)[0] <= tol) and np.all(np.abs(a1 - b1)[0] <= tol), (p1, p2)


# ---- O4: store --------------------------------------------------------------

def test_store_bruteforce_tiny():
    """Tiny decode at position 5 into a zeroed 32-row f32 cache: exactly row 5 of
    K and V changes and holds the returned k and v sections."""
    w = wl.TINY_DECODE
    d, x, rid, kr, vr, bad = _chain(w)
    assert bad == 0 and rid.tolist() == [5]
    kc = np.zeros((w.n_ctx, w.nkt), np.float32)
    vc = np.zeros((w.n_ctx, w.nkt), np.float32)
    oracle.scatter_rows(kc, rid, kr)
    oracle.scatter_rows(vc, rid, vr)
    changed_k = np.nonzero(np.any(kc != 0, axis=1))[0].tolist()
    changed_v = np.nonzero(np.any(vc != 0, axis=1))[0].tolist()
    assert changed_k == [5] and changed_v == [5]
    assert np.array_equal(bits(kc[5]), bits(x["k"][0]))
    assert np.array_equal(bits(vc[5]), bits(x["v"][0]))


def test_store_f16_rows_are_rne_of_outputs():
    w = wl.DECODE_7B
    d, x, rid, kr, vr, bad = _chain(w, nt=2, pos=[10, 4000], cache_dtype=oracle.CACHE_F16)
    assert rid.tolist() == [10, 4000]
    assert np.array_equal(kr, x["k"].astype(np.float16).view(np.uint16))
    assert np.array_equal(vr, x["v"].astype(np.float16).view(np.uint16))


def test_slot_rows_and_range_errors():
    w = wl.BATCHED_DECODE_14B
    nt = 6
    d = wl.draw_layer(w, 0, nt=nt)
    pos = np.array([0, 32767, 32768, -1, 5, 7], np.int32)
    slot = np.array([0, 3, 1, 2, 256, 255], np.int32)
    q, k, v = d["q"].ravel().copy(), d["k"].ravel().copy(), d["v"].ravel().copy()
    rid, kr, vr, bad = oracle.qkv_epilogue(
        q, k, v, d["bq"], d["bk"], d["bv"], pos, n_head=w.n_head, n_kv_head=w.n_kv_head,
        head_dim=w.head_dim, theta=w.theta, n_ctx=32768, cache_dtype=oracle.CACHE_F32,
        slot=slot, n_slots=256)
    assert bad == 3
    assert rid.tolist() == [0, 3 * 32768 + 32767, -1, -1, -1, 255 * 32768 + 7]
    # rejected tokens are still biased and roped: position 32768 token matches
    # the same token computed alone with a valid slot
    q2, k2, v2 = (d[n][2].copy() for n in ("q", "k", "v"))
    oracle.qkv_epilogue(q2, k2, v2, d["bq"], d["bk"], d["bv"], np.array([32768], np.int32),
                        n_head=w.n_head, n_kv_head=w.n_kv_head, head_dim=w.head_dim,
                        theta=w.theta, n_ctx=1 << 20, cache_dtype=oracle.CACHE_F32)
    assert np.array_equal(bits(q.reshape(nt, -1)[2]), bits(q2))


def test_tokens_are_independent():
    """A multi-token call equals the same tokens run one at a time."""
    w = wl.DECODE_7B
    pos = [3, 4000, 17, 2048, 1]
    d, x, rid, kr, vr, bad = _chain(w, nt=5, pos=pos)
    for t, p in enumerate(pos):
        q1, k1, v1 = (d[n][t].copy() for n in ("q", "k", "v"))
        r1, kr1, vr1, _ = oracle.qkv_epilogue(
            q1, k1, v1, d["bq"], d["bk"], d["bv"], np.array([p], np.int32),
            n_head=w.n_head, n_kv_head=w.n_kv_head, head_dim=w.head_dim, theta=w.theta,
            n_ctx=w.n_ctx, cache_dtype=w.cache_dtypes[0])
        assert np.array_equal(bits(x["q"][t]), bits(q1))
        assert np.array_equal(bits(x["k"][t]), bits(k1))
        assert np.array_equal(kr[t], kr1[0]) and np.array_equal(vr[t], vr1[0])
        assert rid[t] == p


def test_concat_rows_equal_separate_buffers():
    """The concat q|k|v layout (section views with the row stride of the
    concat buffer) gives the same results as three separate buffers."""
    w = wl.DECODE_14B
    nt = 3
    d = wl.draw_layer(w, 0, nt=nt)
    d["pos"] = np.array([5, 100, 4095], np.int32)
    buf = wl.concat_rows(d["q"], d["k"], d["v"])
    pad = np.full((nt, 8), 123.0, np.float32)          # extra columns stay untouched
    buf = np.ascontiguousarray(np.concatenate([buf, pad], axis=1))
    ld = buf.shape[1]
    flat = buf.ravel()
    nqt, nkt = w.nqt, w.nkt
    rid, kr, vr, _ = oracle.qkv_epilogue(
        flat[:], flat[nqt:], flat[nqt + nkt:], d["bq"], d["bk"], d["bv"], d["pos"],
        n_head=w.n_head, n_kv_head=w.n_kv_head, head_dim=w.head_dim, theta=w.theta,
        n_ctx=w.n_ctx, cache_dtype=oracle.CACHE_F16, ld_q=ld, ld_k=ld, ld_v=ld)
    q, k, v = d["q"].ravel().copy(), d["k"].ravel().copy(), d["v"].ravel().copy()
    rid2, kr2, vr2, _ = oracle.qkv_epilogue(
        q, k, v, d["bq"], d["bk"], d["bv"], d["pos"], n_head=w.n_head, n_kv_head=w.n_kv_head,
        head_dim=w.head_dim, theta=w.theta, n_ctx=w.n_ctx, cache_dtype=oracle.CACHE_F16)
    out = buf.reshape(nt, ld)
    assert np.array_equal(bits(out[:, :nqt]), bits(q.reshape(nt, -1)))
    assert np.array_equal(bits(out[:, nqt:nqt + nkt]), bits(k.reshape(nt, -1)))
    assert np.array_equal(bits(out[:, nqt + nkt:nqt + 2 * nkt]), bits(v.reshape(nt, -1)))
    assert np.all(out[:, nqt + 2 * nkt:] == 123.0)
    assert np.array_equal(kr, kr2) and np.array_equal(vr, vr2) and np.array_equal(rid, rid2)


def test_odd_head_dim_rejected():
    q = np.zeros(6, np.float32)
    with pytest.raises(ValueError):
        oracle.qkv_epilogue(q, q.copy(), q.copy(), q, q, q, np.array([0], np.int32),
                            n_head=2, n_kv_head=2, head_dim=3, theta=1e6, n_ctx=4,
                            cache_dtype=0)
