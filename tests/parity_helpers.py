"""Shared helpers of the GPU parity tests: run one case through the C ABI and
through the CPU oracle on the same seeded inputs, and compare.

Tolerances (the op's stated bar):
  * q and k: |gpu - oracle| <= 2e-6 + 1e-6*|oracle| per element;
  * v and the V cache: bit-exact;
  * K cache: f32 rows bit-equal to the GPU's own k output and within the q/k
    tolerance of the oracle; f16 rows within 1 binary16 ulp of the oracle's;
  * addressing: the set of cache rows that changed equals the set the oracle
    wrote, and every other row still holds the sentinel fill;
  * tokens that share a cache row (a caller error the op leaves unordered):
    each element of the row equals that element from one of them.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from qkv_bias_rope_amd import binding as B
from qkv_bias_rope_amd import workloads as wl

ABS_TOL = 2e-6
REL_TOL = 1e-6
SENTINEL_F32 = 0x5A5A5A5A
SENTINEL_F16 = 0x5A5A

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def torch_cache_dtype(cd):
    return torch.float32 if cd == wl.CACHE_F32 else torch.float16


def new_cache(rows, nkt, cd):
    """A [rows][nkt] device cache filled with the sentinel bit pattern."""
    if cd == wl.CACHE_F32:
        c = torch.empty((rows, nkt), dtype=torch.float32, device=DEV)
        c.view(torch.int32).fill_(SENTINEL_F32)
    else:
        c = torch.empty((rows, nkt), dtype=torch.float16, device=DEV)
        c.view(torch.int16).fill_(SENTINEL_F16)
    return c


def changed_rows(cache, cd, chunk_rows=1 << 16):
    """Indices of rows that differ anywhere from the sentinel (computed on the
    device, chunked so huge caches need little extra memory)."""
    iv = cache.view(torch.int32 if cd == wl.CACHE_F32 else torch.int16)
    sent = SENTINEL_F32 if cd == wl.CACHE_F32 else SENTINEL_F16
    if cd == wl.CACHE_F16:
        sent = sent - (1 << 16) if sent >= (1 << 15) else sent
    out = []
    for r0 in range(0, iv.shape[0], chunk_rows):
        blk = iv[r0:r0 + chunk_rows]
        idx = torch.nonzero((blk != sent).any(dim=1)).flatten()
        if idx.numel():
            out.append(idx.cpu().numpy().astype(np.int64) + r0)
    return np.concatenate(out) if out else np.zeros(0, np.int64)


def tensors_bitwise_equal(a, b, chunk=1 << 28):
    """Byte equality of two same-shaped device tensors, chunked on the device."""
    ia = a.reshape(-1).view(torch.uint8)
    ib = b.reshape(-1).view(torch.uint8)
    if ia.numel() != ib.numel():
        return False
    for i in range(0, ia.numel(), chunk):
        if not torch.equal(ia[i:i + chunk], ib[i:i + chunk]):
            return False
    return True


def qk_close(got, want):
    got = got.astype(np.float64)
    want = want.astype(np.float64)
    err = np.abs(got - want)
    ok = err <= ABS_TOL + REL_TOL * np.abs(want)
    max_abs = float(err.max()) if err.size else 0.0
    rel = err / np.maximum(np.abs(want), 1e-30)
    max_rel = float(rel.max()) if rel.size else 0.0
    return bool(ok.all()), max_abs, max_rel, int((~ok).sum())


def f16_ulp_diff(a_bits, b_bits):
    """|a - b| in binary16 ulps, via the ordered integer image of the bits."""
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, 0x8000 - x, x)   # negatives mirror below 0
    return np.abs(ordered(a_bits) - ordered(b_bits))


class Case:
    """One launch: inputs drawn for workload w, run on the GPU and the oracle."""

    def __init__(self, w, layer=0, nt=None, pos=None, slot=None, cache_dtype=None, form="separate",
                 n_ctx=None, n_slots=None, inputs=None, misalign=0, norm=False, bias=True,
                 style=0, freq_scale=1.0):
        self.w = w
        self.style = style              # 0 NeoX, 1 interleaved pairs
        self.freq_scale = freq_scale
        self.norm = norm            # q/k-norm variant (run_qk_norm)
        self.bias = bias            # False: no biases (NULL), only with norm
        if norm:
            self.nw = wl.draw_norm_weights(w, layer)
            self.eps = wl.QK_NORM_EPS
        self.cd = w.cache_dtypes[0] if cache_dtype is None else cache_dtype
        d = wl.draw_layer(w, layer, nt=nt) if inputs is None else inputs
        if pos is not None:
            d["pos"] = np.asarray(pos, dtype=np.int32)
        if slot is not None:
            d["slot"] = np.asarray(slot, dtype=np.int32)
        self.d = d
        self.nt = int(d["pos"].size)
        self.form = form
        self.n_ctx = w.n_ctx if n_ctx is None else n_ctx
        self.n_slots = w.n_slots if n_slots is None else n_slots
        self.misalign = misalign   # elements to shift every section by (forces the scalar path)

    # -- oracle --
    def run_oracle(self):
        w, d = self.w, self.d
        q, k, v = (d[n].copy() for n in ("q", "k", "v"))
        if self.norm:
            b = (d["bq"], d["bk"], d["bv"]) if self.bias else (None, None, None)
            rid, kr, vr, bad = oracle.qkv_norm_epilogue(
                q.ravel(), k.ravel(), v.ravel(), *b, self.nw["wq"], self.nw["wk"], self.eps,
                d["pos"], n_head=w.n_head, n_kv_head=w.n_kv_head, head_dim=w.head_dim,
                theta=w.theta, n_ctx=self.n_ctx, cache_dtype=self.cd, slot=d["slot"],
                n_slots=self.n_slots, rope_style=self.style, freq_scale=self.freq_scale)
        else:
            rid, kr, vr, bad = oracle.qkv_epilogue(
                q.ravel(), k.ravel(), v.ravel(), d["bq"], d["bk"], d["bv"], d["pos"],
                n_head=w.n_head, n_kv_head=w.n_kv_head, head_dim=w.head_dim, theta=w.theta,
                n_ctx=self.n_ctx, cache_dtype=self.cd, slot=d["slot"], n_slots=self.n_slots,
                rope_style=self.style, freq_scale=self.freq_scale)
        self.o_q, self.o_k, self.o_v = q, k, v
        self.o_rows, self.o_krows, self.o_vrows, self.o_bad = rid, kr, vr, bad
        return self

    # -- gpu --
    def upload(self, kcache=None, vcache=None):
        w, d = self.w, self.d
        nqt, nkt, nt = w.nqt, w.nkt, self.nt
        m = self.misalign
        if self.form == "concat":
            buf = np.concatenate([d["q"], d["k"], d["v"]], axis=1)
            flat = np.zeros(buf.size + m, np.float32)
            flat[m:] = buf.ravel()
            self.g_buf = torch.from_numpy(flat).to(DEV)
            ld = nqt + 2 * nkt
            base = self.g_buf[m:].view(nt, ld)
            self.g_q, self.g_k, self.g_v = base[:, :nqt], base[:, nqt:nqt + nkt], base[:, nqt + nkt:]
        else:
            def up(a):
                flat = np.zeros(a.size + m, np.float32)
                flat[m:] = a.ravel()
                t = torch.from_numpy(flat).to(DEV)
                return t, t[m:].view(a.shape)
            self._q, self.g_q = up(d["q"])
            self._k, self.g_k = up(d["k"])
            self._v, self.g_v = up(d["v"])
        self.g_bq, self.g_bk, self.g_bv = (torch.from_numpy(d[n]).to(DEV) for n in ("bq", "bk", "bv"))
        if not self.bias:
            self.g_bq = self.g_bk = self.g_bv = None
        if self.norm:
            self.g_wq = torch.from_numpy(self.nw["wq"]).to(DEV)
            self.g_wk = torch.from_numpy(self.nw["wk"]).to(DEV)
        self.g_pos = torch.from_numpy(d["pos"]).to(DEV)
        self.g_slot = None if d["slot"] is None else torch.from_numpy(d["slot"]).to(DEV)
        rows = self.n_slots * self.n_ctx
        self.kc = new_cache(rows, nkt, self.cd) if kcache is None else kcache
        self.vc = new_cache(rows, nkt, self.cd) if vcache is None else vcache
        return self

    def run_gpu(self, h, entry="run_ex", stream=None):
        w = self.w
        if entry == "run":
            assert self.form == "separate" and self.g_slot is None
            rc = B.qkv_epilogue_run(h, self.g_q, self.g_k, self.g_v, self.g_bq, self.g_bk,
                                    self.g_bv, self.g_pos, self.kc, self.vc, self.nt, w.n_head,
                                    w.n_kv_head, w.head_dim, w.theta, self.cd)
        else:
            a = self.args(stream)
            if self.norm:
                rc = B.qkv_epilogue_run_qk_norm(h, a, self.g_wq, self.g_wk, self.eps)
            else:
                rc = (B.qkv_epilogue_run_unfused if entry == "unfused" else B.qkv_epilogue_run_ex)(h, a)
        return rc

    def args(self, stream=None):
        w = self.w
        return B.make_args(self.g_q, self.g_k, self.g_v, self.g_bq, self.g_bk, self.g_bv,
                           self.g_pos, self.kc, self.vc, n_head=w.n_head, n_kv_head=w.n_kv_head,
                           head_dim=w.head_dim, theta=w.theta, cache_dtype=self.cd,
                           slot=self.g_slot, n_ctx=self.n_ctx, n_slots=self.n_slots,
                           stream=stream if stream is not None else torch.cuda.current_stream(),
                           use_stream=True, nt=self.nt, rope_style=self.style,
                           freq_scale=self.freq_scale)

    def download(self):
        self.r_q = self.g_q.cpu().numpy().reshape(self.nt, -1)
        self.r_k = self.g_k.cpu().numpy().reshape(self.nt, -1)
        self.r_v = self.g_v.cpu().numpy().reshape(self.nt, -1)
        return self

    # -- comparison --
    def check(self, check_untouched=True, label=""):
        w = self.w
        nt = self.nt
        oq = self.o_q.reshape(nt, -1)
        ok_ = self.o_k.reshape(nt, -1)
        ov = self.o_v.reshape(nt, -1)
        res = {}
        for name, got, want in (("q", self.r_q, oq), ("k", self.r_k, ok_)):
            ok, ma, mr, nbad = qk_close(got, want)
            res[name] = (ma, mr, int((got.view(np.uint32) != want.view(np.uint32)).sum()))
            assert ok, f"{label} {name}: {nbad} elements beyond tolerance (max abs {ma:.3g}, max rel {mr:.3g})"
        assert np.array_equal(self.r_v.view(np.uint32), ov.view(np.uint32)), f"{label} v not bit-exact"

        valid = self.o_rows >= 0
        rows = self.o_rows[valid]
        if check_untouched:
            for nm, cache in (("K", self.kc), ("V", self.vc)):
                ch = changed_rows(cache, self.cd)
                assert np.array_equal(np.sort(ch), np.sort(np.unique(rows))), \
                    f"{label} {nm} cache: changed rows {ch[:8]} != oracle rows {np.sort(rows)[:8]}"
        if rows.size:
            idx = torch.from_numpy(rows).to(DEV)
            gk = self.kc.index_select(0, idx).cpu().numpy()
            gv = self.vc.index_select(0, idx).cpu().numpy()
            rk = self.r_k[valid]
            if self.cd == wl.CACHE_F32:
                ok_k = gk.view(np.uint32) == rk.view(np.uint32)
                err = np.abs(gk.astype(np.float64) - self.o_krows[valid].astype(np.float64))
                ok_k &= err <= ABS_TOL + REL_TOL * np.abs(self.o_krows[valid])
                ok_v = gv.view(np.uint32) == self.o_vrows[valid].view(np.uint32)
            else:
                gkb = gk.view(np.uint16)
                ok_k = f16_ulp_diff(gkb, self.o_krows[valid]) <= 1
                # the f16 K row is also the RNE image of the GPU's own k output
                # (outputs beyond the f16 range round to inf on purpose)
                with np.errstate(over="ignore"):
                    ok_k &= gkb == rk.astype(np.float16).view(np.uint16)
                ok_v = gv.view(np.uint16) == self.o_vrows[valid]
            # Tokens sharing a cache row (duplicate positions) race: each element
            # of the row holds the value of one of the colliding tokens, so per
            # element one token of the group matches.
            uniq, inv = np.unique(rows, return_inverse=True)
            for name, ok in (("K", ok_k), ("V", ok_v)):
                grp_ok = np.zeros((uniq.size, ok.shape[1]), bool)
                np.logical_or.at(grp_ok, inv, ok)
                bad = uniq[~grp_ok.all(axis=1)]
                assert bad.size == 0, f"{label} {name} cache rows {bad[:8]} hold values of no token writing them"
        return res
