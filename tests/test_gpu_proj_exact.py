"""Exact pins of the projection that feeds the epilogue.

With small-integer inputs the projection has one correct answer whatever the
summation order: x and w in {-3..3} are exact in bfloat16 (and in E4M3), every
product is an integer of magnitude <= 9, and every partial sum over hidden =
5120 terms is an integer below 2^16, so each f32 addition is exact and the
GPU's sums equal the oracle's (exact double sums rounded once) bit for bit, on
every launch form: the weight-streaming kernel (1-4 tokens), the MFMA kernel
with k split (256 tokens) and data-parallel (4096 tokens), with bf16 and with
E4M3 weights.  At position 0 (cos 1, sin 0) with no bias the epilogue passes
those values through, so q/k/v and the cache rows must equal the oracle's bit
for bit; this pins the indexing of x, of the q|k|v weight rows and of the
outputs exactly.

Page "73 · D3-8 — G4 FusedQKV ported to CUDA", §2 and §4 (i), shows the concat
matmul equal bit for bit to three separate matmuls; here the same holds for
the launch fed one concat weight matrix or three matrices, on random inputs.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from qkv_bias_rope_amd import binding as B
from qkv_bias_rope_amd import workloads as wl

from parity_helpers import DEV, say
from test_gpu_proj import ProjCase, _run

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def handle():
    rc, h = B.qkv_epilogue_create(0, 4096, None)
    assert rc == B.QKV_OK, rc
    yield h
    B.qkv_epilogue_destroy(h)


def _int_bits(rng, shape):
    return wl.bf16_bits(rng.integers(-3, 4, size=shape).astype(np.float32))


def _e4m3_codes(rng, shape):
    vals = rng.integers(-3, 4, size=shape).astype(np.float32)
    return torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _exact_case(nt, hidden, seed, cd, weights="concat", wfmt="bf16", sample=None, pos_zero=True):
    """14B geometry, integer inputs, no bias.  pos_zero: every token at
    position 0 in a slot of its own (distinct cache rows, identity rotation);
    else distinct random positions of one sequence."""
    if pos_zero:
        w = wl.Workload(f"exact_{nt}", 40, 8, 128, nt=nt, n_ctx=2, n_slots=nt, layers=1, seed=seed,
                        cache_dtypes=(cd,), pos_mode="fixed", fixed_pos=0)
    else:
        w = wl.Workload(f"exact_rope_{nt}", 40, 8, 128, nt=nt, n_ctx=4096, n_slots=1, layers=1,
                        seed=seed, cache_dtypes=(cd,), pos_mode="uniform")
    c = ProjCase(w, hidden=hidden, bias=False, weights=weights, wfmt=wfmt, sample=sample,
                 pos=None if pos_zero else
                 np.random.default_rng(seed).permutation(w.n_ctx)[:nt].astype(np.int32))
    rng = np.random.default_rng(seed + 1)
    N = w.nqt + 2 * w.nkt
    c.d["x"] = _int_bits(rng, (nt, hidden))
    if wfmt == "e4m3":
        c.d["w8"] = _e4m3_codes(rng, (N, hidden))
        c.d["wscale"] = np.ones(N, np.float32)
    else:
        c.d["w"] = _int_bits(rng, (N, hidden))
    return c


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.float16 else torch.int32).cpu().numpy()


def _check_exact(c, label):
    s = c.sample
    idx = torch.from_numpy(s.astype(np.int64)).to(DEV)
    for name in ("q", "k", "v"):
        got = getattr(c, "g_" + name).index_select(0, idx).cpu().numpy()
        want = c.o[name].reshape(len(s), -1)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), \
            f"{label} {name}: {int((got != want).sum())} elements differ from the oracle"
    rid = c.o["rid"]
    assert (rid >= 0).all()
    ridx = torch.from_numpy(rid.astype(np.int64)).to(DEV)
    for nm, cache, want in (("K", c.kc, c.o["kr"]), ("V", c.vc, c.o["vr"])):
        got = _bits(cache.index_select(0, ridx))
        assert np.array_equal(got.view(want.dtype), want), f"{label} {nm} cache rows differ"
    say(f"  {label}: q/k/v and cache rows bit-equal to the oracle on {len(s)} tokens")


@pytest.mark.parametrize("cd", [wl.CACHE_F16, wl.CACHE_F32])
@pytest.mark.parametrize("nt", [1, 2, 3, 4])
def test_exact_gemv(handle, nt, cd):
    c = _exact_case(nt, 5120, 100 + nt, cd)
    assert _run(handle, c, f"exact_gemv_{nt}") == B.QKV_OK
    _check_exact(c, f"exact_gemv_{nt}")
    c.check(f"exact_gemv_{nt}")


@pytest.mark.parametrize("nt", [1, 4])
def test_exact_gemv_e4m3(handle, nt):
    c = _exact_case(nt, 5120, 110 + nt, wl.CACHE_F16, wfmt="e4m3")
    assert _run(handle, c, f"exact_e4m3_{nt}") == B.QKV_OK
    _check_exact(c, f"exact_e4m3_{nt}")


@pytest.mark.parametrize("weights", ["concat", "three"])
def test_exact_ksplit_256(handle, weights):
    """256 tokens at hidden 5120: the MFMA kernel with k split (partials summed
    by the second kernel in split order)."""
    sample = np.unique(np.r_[0, 1, 127, 128, 255, np.random.default_rng(5).integers(0, 256, 27)])
    c = _exact_case(256, 5120, 120, wl.CACHE_F16, weights=weights, sample=sample)
    assert _run(handle, c, f"exact_ksplit_{weights}") == B.QKV_OK
    _check_exact(c, f"exact_ksplit_{weights}")
    c.check(f"exact_ksplit_{weights}")


def test_exact_data_parallel_4096(handle):
    """4096 tokens at hidden 5120: the data-parallel MFMA kernel with the
    epilogue on its accumulators; sampled tokens against the oracle, every
    cache row's address checked."""
    sample = np.unique(np.r_[0, 255, 256, 4095, np.random.default_rng(6).integers(0, 4096, 44)])
    c = _exact_case(4096, 5120, 130, wl.CACHE_F32, sample=sample)
    assert _run(handle, c, "exact_dp_4096") == B.QKV_OK
    _check_exact(c, "exact_dp_4096")
    c.check("exact_dp_4096")


@pytest.mark.parametrize("weights", ["concat", "three"])
def test_exact_e4m3_ksplit_256(handle, weights):
    """E4M3 weights (codes of -3..3, scales 1) on the k-split MFMA path: the
    codes converted to bf16 in the fragment reads, the partials summed, then
    scaled -- bit-equal to the oracle."""
    sample = np.unique(np.r_[0, 1, 127, 128, 255, np.random.default_rng(7).integers(0, 256, 27)])
    c = _exact_case(256, 5120, 160, wl.CACHE_F16, weights=weights, wfmt="e4m3", sample=sample)
    assert _run(handle, c, f"exact_e4m3_ksplit_{weights}") == B.QKV_OK
    _check_exact(c, f"exact_e4m3_ksplit_{weights}")
    c.check(f"exact_e4m3_ksplit_{weights}")


def test_exact_e4m3_data_parallel_4096(handle):
    """E4M3 weights on the data-parallel MFMA kernel (4096 tokens, hidden
    5120): sampled tokens bit-equal to the oracle, every cache row's address."""
    sample = np.unique(np.r_[0, 255, 256, 4095, np.random.default_rng(8).integers(0, 4096, 44)])
    c = _exact_case(4096, 5120, 170, wl.CACHE_F32, wfmt="e4m3", sample=sample)
    assert _run(handle, c, "exact_e4m3_dp_4096") == B.QKV_OK
    _check_exact(c, "exact_e4m3_dp_4096")
    c.check("exact_e4m3_dp_4096")


@pytest.mark.parametrize("nt", [4, 256])
def test_exact_sums_then_rope(handle, nt):
    """Exact projection at random positions: q and k may differ from the
    oracle only by the epilogue's own rounding bar, v and the V cache not at
    all (the accumulation error term is zero here)."""
    c = _exact_case(nt, 5120, 140 + nt, wl.CACHE_F16, pos_zero=False)
    assert _run(handle, c, f"exact_rope_{nt}") == B.QKV_OK
    s = torch.from_numpy(c.sample.astype(np.int64)).to(DEV)
    for name in ("q", "k", "v"):
        got = getattr(c, "g_" + name).index_select(0, s).cpu().numpy().astype(np.float64)
        want = c.o[name].reshape(got.shape).astype(np.float64)
        if name == "v":
            assert np.array_equal(got, want)
        else:
            err = np.abs(got - want)
            assert (err <= 2e-6 + 1e-6 * np.abs(want)).all(), (name, float(err.max()))
    c.check(f"exact_rope_{nt}")


@pytest.mark.parametrize("cd", [wl.CACHE_F16, wl.CACHE_F32])
@pytest.mark.parametrize("nt", [1, 3, 4, 256, 1030])
def test_concat_equals_three_matrices(handle, nt, cd):
    """One launch fed the concat q|k|v weight rows and one fed three separate
    matrices (copies of the same rows) give the same q/k/v and cache rows bit
    for bit, on random N(0,1)-scale inputs: the layout changes where the rows
    are read from, never the order of the sums."""
    w = wl.Workload(f"concat3_{nt}", 40, 8, 128, nt=nt, n_ctx=4096, n_slots=1, layers=1,
                    seed=150 + nt, cache_dtypes=(cd,), pos_mode="uniform")
    pos = np.random.default_rng(150 + nt).permutation(w.n_ctx)[:nt].astype(np.int32)
    outs = []
    for weights in ("concat", "three"):
        c = ProjCase(w, hidden=5120 if nt <= 256 else 1024, weights=weights, pos=pos,
                     sample=np.arange(min(nt, 4)))
        c.run_oracle().upload()
        assert c.run_gpu(handle) == B.QKV_OK, B.qkv_epilogue_last_error(handle)
        assert B.qkv_epilogue_status(handle) == B.QKV_OK
        torch.cuda.synchronize()
        outs.append([_bits(t) for t in (c.g_q, c.g_k, c.g_v, c.kc, c.vc)])
        if weights == "concat":
            c.check(f"concat3_{nt}")
    for name, a, b in zip(("q", "k", "v", "kcache", "vcache"), *outs):
        assert np.array_equal(a, b), f"{name}: concat and three-matrix launches differ"
    say(f"  concat3_{nt}: bit-equal")
