"""The library used from C with no Python in the process: tests/c/abi_decode
(built by __graft_entry__.build()) calls qkv_epilogue_run on inputs this test
writes, and its outputs are checked against the oracle like the Python-path
parity tests (same bounds, bit-exact v and cache rows)."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from parity_helpers import ABS_TOL, REL_TOL
from qkv_bias_rope_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c", "abi_decode")

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("w,cd", [
    (wl.TINY_DECODE, wl.CACHE_F32),
    (wl.Workload("c_consumer_7b", 28, 4, 128, nt=7, n_ctx=512, n_slots=1, layers=1, seed=31,
                 pos_mode="uniform"), wl.CACHE_F16),
])
def test_c_program_matches_oracle(tmp_path, w, cd):
    if not os.path.exists(EXE):
        pytest.fail("tests/c/abi_decode is not built: run __graft_entry__.build()")
    d = wl.draw_layer(w, 0)
    nt = int(d["pos"].size)
    # distinct positions so each cache row has one writer
    pos = np.arange(nt, dtype=np.int32) * 3 + 1 if nt > 1 else d["pos"].astype(np.int32)
    cdt = np.float16 if cd == wl.CACHE_F16 else np.float32
    kc0 = np.zeros((w.n_ctx, w.nkt), cdt)
    vc0 = np.zeros((w.n_ctx, w.nkt), cdt)
    hdr = np.array([nt, w.n_head, w.n_kv_head, w.head_dim, w.n_ctx, cd], np.int32)
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(fin, "wb") as f:
        f.write(hdr.tobytes())
        f.write(np.float32(w.theta).tobytes())
        for n in ("q", "k", "v", "bq", "bk", "bv"):
            f.write(np.ascontiguousarray(d[n], np.float32).tobytes())
        f.write(pos.tobytes())
        f.write(kc0.tobytes())
        f.write(vc0.tobytes())
    print(f"[c-consumer] {w.name}: nt={nt} cache={'f16' if cd else 'f32'}", flush=True)
    r = subprocess.run([EXE, str(fin), str(fout)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr

    q, k, v = (d[n].astype(np.float32).copy() for n in ("q", "k", "v"))
    rid, kr, vr, bad = oracle.qkv_epilogue(
        q.ravel(), k.ravel(), v.ravel(), d["bq"], d["bk"], d["bv"], pos,
        n_head=w.n_head, n_kv_head=w.n_kv_head, head_dim=w.head_dim, theta=w.theta,
        n_ctx=w.n_ctx, cache_dtype=cd)
    assert bad == 0
    raw = open(fout, "rb").read()
    sizes = [nt * w.nqt * 4, nt * w.nkt * 4, nt * w.nkt * 4]
    offs = np.cumsum([0] + sizes)
    gq, gk, gv = (np.frombuffer(raw[offs[i]:offs[i + 1]], np.float32).reshape(nt, -1) for i in range(3))
    cbytes = w.n_ctx * w.nkt * np.dtype(cdt).itemsize
    gkc = np.frombuffer(raw[offs[3]:offs[3] + cbytes], cdt).reshape(w.n_ctx, w.nkt)
    gvc = np.frombuffer(raw[offs[3] + cbytes:offs[3] + 2 * cbytes], cdt).reshape(w.n_ctx, w.nkt)
    for name, got, want in (("q", gq, q.reshape(nt, -1)), ("k", gk, k.reshape(nt, -1))):
        err = np.abs(got.astype(np.float64) - want.astype(np.float64))
        assert np.all(err <= ABS_TOL + REL_TOL * np.abs(want)), (name, float(err.max()))
    assert np.array_equal(gv.view(np.uint32), v.reshape(nt, -1).view(np.uint32))
    # exactly the oracle's rows changed: K holds the token's own k output in the
    # cache type, V the oracle's v row bit for bit
    bits = np.uint16 if cd == wl.CACHE_F16 else np.uint32
    assert np.array_equal(rid, pos.astype(np.int64))
    for cache in (gkc, gvc):
        changed = np.nonzero(np.any(cache.view(bits) != 0, axis=1))[0]
        assert np.array_equal(changed, np.sort(pos))
    for t in range(nt):
        assert np.array_equal(gkc[pos[t]].view(bits), gk[t].astype(cdt).view(bits))
        assert np.array_equal(gvc[pos[t]].view(bits), vr[t].view(bits))


def test_c_decode_loop_runs():
    """tests/c/decode_loop, the decode step the benchmark issues from C: a few
    steps of the 7B shape end with the status call clean and a JSON line of
    positive timings; bad arguments are refused."""
    exe = os.path.join(ROOT, "tests", "c", "decode_loop")
    if not os.path.exists(exe):
        pytest.fail("tests/c/decode_loop is not built: run __graft_entry__.build()")
    import json
    r = subprocess.run([exe, "28", "4", "128", "28", "5", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    d = json.loads(r.stdout.strip().splitlines()[-1])
    assert d["layers"] == 28 and d["steps"] == 5
    assert d["us_per_layer"] > 0 and d["host_issue_us_per_call"] > 0
    bad = subprocess.run([exe, "28", "4", "128", "0", "5", "2"], capture_output=True, text=True, timeout=60)
    assert bad.returncode != 0 and "bad arguments" in bad.stderr
