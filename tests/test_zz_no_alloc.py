"""qkv_epilogue_run_proj_noalloc, the allocation-free projection entry point,
through the C ABI: on the same inputs it must give what qkv_epilogue_run_proj
gives, bit for bit (the same kernels and launch plan; only the workspace
differs), on two calls in a row, the second smaller than the first, so a
stale workspace from the first call would show; and the first call's outputs
are also held to the oracle's bound.  Requests beyond its static workspace
are rejected with nothing launched."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from qkv_bias_rope_amd import binding as B
from qkv_bias_rope_amd import workloads as wl

from parity_helpers import DEV, say
from test_gpu_proj import ProjCase

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def handle():
    rc, h = B.qkv_epilogue_create(0, 4096, None)
    assert rc == B.QKV_OK, rc
    yield h
    B.qkv_epilogue_destroy(h)


def _snapshot(c):
    torch.cuda.synchronize()
    return [t.clone() for t in (c.g_q, c.g_k, c.g_v, c.kc, c.vc)]


def _same(a, b):
    for x, y in zip(a, b):
        if x.dtype == torch.float16:
            assert torch.equal(x.view(torch.int16), y.view(torch.int16))
        else:
            assert torch.equal(x.view(torch.int32), y.view(torch.int32))


def _case(nt, hidden, seed, sample=None, wfmt="bf16"):
    """Distinct random positions: tokens sharing a cache row race for it (a
    caller error), which would make the two entry points' rows differ."""
    w = wl.Workload(f"noalloc_{nt}", 40, 8, 128, nt=nt, n_ctx=4096, n_slots=1, layers=1,
                    seed=seed, pos_mode="uniform")
    pos = np.random.default_rng(seed).permutation(w.n_ctx)[:nt].astype(np.int32)
    return ProjCase(w, hidden=hidden, sample=sample, pos=pos, wfmt=wfmt)


@pytest.mark.parametrize("sizes", [((256, 5120), (40, 1024)), ((1030, 1024), (300, 512))])
@pytest.mark.parametrize("wfmt", ["bf16", "e4m3"])
def test_noalloc_matches_run_proj_two_calls(handle, sizes, wfmt):
    """First pair: 256 tokens at hidden 5120 (k split four ways: table, rows
    and 29 MB of partial sums in the workspace), then 40 tokens at hidden 1024.
    Second pair: 1030 tokens (data-parallel: table and rows only), then 300
    tokens split at hidden 512.  With bf16 and with E4M3 weights."""
    cases = []
    for i, (nt, hid) in enumerate(sizes):
        sample = None if nt <= 300 else np.unique(np.r_[0, nt - 1, np.arange(0, nt, 37)])
        c = _case(nt, hid, 40 + i, sample, wfmt=wfmt)
        say(f"[noalloc] nt={nt} hidden={hid} weights={wfmt}: run_proj")
        c.run_oracle().upload()
        assert c.run_gpu(handle) == B.QKV_OK, B.qkv_epilogue_last_error(handle)
        assert B.qkv_epilogue_status(handle) == B.QKV_OK
        cases.append((c, _snapshot(c)))
    # the two calls in a row through the allocation-free entry point
    for c, _ in cases:
        c.upload()   # fresh outputs (NaN) and caches (sentinel)
    for c, _ in cases:
        say(f"[noalloc] nt={c.nt} hidden={c.hidden}: run_proj_noalloc")
        rc = B.qkv_epilogue_run_proj_noalloc(handle, c.args())
        assert rc == B.QKV_OK, B.qkv_epilogue_last_error(handle)
    assert B.qkv_epilogue_status(handle) == B.QKV_OK
    for c, ref in cases:
        _same(_snapshot(c), ref)
        c.check(f"noalloc_{c.nt}")


def test_noalloc_repeat_smaller_after_larger(handle):
    """The same pair again on one handle after the previous test's calls:
    the static workspace keeps the last call's contents, and nothing read
    depends on them."""
    big, small = _case(256, 5120, 50), _case(64, 2048, 51)
    for c in (big, small):
        c.run_oracle().upload()
        assert B.qkv_epilogue_run_proj_noalloc(handle, c.args()) == B.QKV_OK, \
            B.qkv_epilogue_last_error(handle)
    assert B.qkv_epilogue_status(handle) == B.QKV_OK
    torch.cuda.synchronize()
    for c in (big, small):
        c.check(f"noalloc_seq_{c.nt}")


def test_noalloc_decode_matches(handle):
    """1-4 tokens take the weight-streaming kernel, which uses no workspace."""
    for nt in (1, 4):
        c = _case(nt, 5120, 60 + nt)
        c.run_oracle().upload()
        assert c.run_gpu(handle) == B.QKV_OK
        ref = _snapshot(c)
        c.upload()
        assert B.qkv_epilogue_run_proj_noalloc(handle, c.args()) == B.QKV_OK
        _same(_snapshot(c), ref)
        c.check(f"noalloc_decode_{nt}")


def test_noalloc_rejects_oversize(handle):
    """65600 tokens of a one-head shape need a 33.6 MB cos/sin table alone:
    QKV_ERR_UNSUPPORTED, with a message naming both sizes, and no output
    touched."""
    nt, hid, hd = 65600, 64, 128
    w = wl.Workload("noalloc_big", 1, 1, hd, nt=nt, n_ctx=nt, n_slots=1, layers=1, seed=70,
                    pos_mode="arange")
    x = torch.zeros(nt, hid, dtype=torch.bfloat16, device=DEV)
    wt = torch.zeros(3 * hd, hid, dtype=torch.bfloat16, device=DEV)
    q, k, v = (torch.full((nt, hd), float("nan"), device=DEV) for _ in range(3))
    pos = torch.arange(nt, dtype=torch.int32, device=DEV)
    kc = torch.full((nt, hd), 7.0, dtype=torch.float16, device=DEV)
    vc = torch.full_like(kc, 7.0)
    epi = B.make_args(q, k, v, None, None, None, pos, kc, vc, n_head=1, n_kv_head=1, head_dim=hd,
                      theta=w.theta, cache_dtype=B.QKV_CACHE_F16, n_ctx=nt,
                      stream=torch.cuda.current_stream(), use_stream=True, nt=nt)
    rc = B.qkv_epilogue_run_proj_noalloc(handle, B.make_proj_args(x, wt, hid, epi))
    msg = B.qkv_epilogue_last_error(handle)
    assert rc == B.QKV_ERR_UNSUPPORTED, (rc, msg)
    assert "workspace" in msg and "33554432" in msg, msg
    torch.cuda.synchronize()
    assert bool(torch.isnan(q).all()) and bool((kc == 7.0).all()) and bool((vc == 7.0).all())
