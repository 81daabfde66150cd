"""GPU parity of the projection-fed epilogue (qkv_epilogue_run_proj) against
the CPU oracle: y = x w^T on bfloat16 inputs (oracle.proj_bf16, exact double
sum), then the epilogue chain (oracle.qkv_epilogue) on the q|k|v sections of y.

Tolerance, derived from the arithmetic.  Every bfloat16 product is exact in
float32, so the GPU differs from the oracle only in how it sums.  Each f32
addition of the running sum a_j errs by at most 2^-24 |a_j|, with signs that
vary from step to step, so the accumulated error behaves like a random walk:
with g products per accumulator step and product RMS sigma, its standard
deviation is about 2^-24 K sigma / sqrt(6 g) (4.4e-7 at hidden 5120 and the
14B scale, where 4.5e-7 RMS is measured).  The bound per element of y is eight
times a looser form of that, B = 8 * 2^-24 * sqrt(K) * R with
R = sqrt(sum_k (x_k w_k)^2) (so sqrt(K) R = K sigma): about 77 standard
deviations, which no rounding reaches, while a misplaced or dropped product
(or k tile) moves an output by ~R or more and fails it.  The rotation mixes
the two elements of a pair with weights |cos|, |sin| <= 1, so a rotated
element gets B(j) + B(partner); on top comes the epilogue's own bar
(2e-6 + 1e-6 |ref|).  The RMS of the error over a case must also stay below
1e-4.  tests/test_gpu_proj_exact.py pins the sums themselves bit for bit with
integer inputs.  Caches are checked structurally: every written row equals
the GPU's own k / v output of that token (f32 bit-equal, or its binary16 RNE
image), and exactly the oracle's rows change.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from qkv_bias_rope_amd import binding as B
from qkv_bias_rope_amd import workloads as wl

from parity_helpers import DEV, changed_rows, new_cache, say

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24
RMS_TOL = 1e-4
KSTAT = 8.0     # multiples of the random-walk scale in the per-element bound


@pytest.fixture(scope="module")
def handle():
    rc, h = B.qkv_epilogue_create(0, 4096, None)
    assert rc == B.QKV_OK, rc
    yield h
    B.qkv_epilogue_destroy(h)


class ProjCase:
    def __init__(self, w, hidden, nt=None, cache_dtype=None, form="separate", bias=True,
                 pos=None, slot=None, sample=None, ld_x_pad=0, misalign=0, weights="concat",
                 style=B.QKV_ROPE_NEOX, freq_scale=1.0, wfmt="bf16"):
        self.w, self.hidden = w, hidden
        d = wl.draw_projection(w, hidden, nt=nt)
        if pos is not None:
            d["pos"] = np.asarray(pos, np.int32)
        if slot is not None:
            d["slot"] = np.asarray(slot, np.int32)
        self.d = d
        self.nt = int(d["pos"].size)
        self.cd = w.cache_dtypes[0] if cache_dtype is None else cache_dtype
        self.form, self.bias = form, bias
        self.ld_x_pad = ld_x_pad
        self.misalign = misalign   # shift every output section by this many floats
        self.weights = weights     # "concat" [N][hidden], or "three" q, k, v matrices
        self.style, self.freq_scale = style, freq_scale
        self.wfmt = wfmt           # "bf16", or "e4m3": 8-bit float codes with row scales
        if wfmt == "e4m3":
            d["w8"], d["wscale"] = wl.draw_e4m3_weights(w.nqt + 2 * w.nkt, hidden, w.seed)
        # tokens the oracle recomputes (all of them unless a sample is given)
        self.sample = np.arange(self.nt) if sample is None else np.asarray(sample)

    # -- oracle on the sampled tokens --
    def run_oracle(self):
        w, d, s = self.w, self.d, self.sample
        nqt, nkt = w.nqt, w.nkt
        xs = np.ascontiguousarray(d["x"][s])
        x2 = wl.bf16_to_f32(xs).astype(np.float64) ** 2
        if self.wfmt == "e4m3":
            y = oracle.proj_fp8w(xs, d["w8"], d["wscale"])
            w2 = oracle.e4m3_values(d["w8"]) ** 2
            R = np.sqrt(x2 @ w2.T) * np.abs(d["wscale"].astype(np.float64))
        else:
            y = oracle.proj_bf16(xs, d["w"])
            R = np.sqrt(x2 @ (wl.bf16_to_f32(d["w"]).astype(np.float64) ** 2).T)
        q = np.ascontiguousarray(y[:, :nqt])
        k = np.ascontiguousarray(y[:, nqt:nqt + nkt])
        v = np.ascontiguousarray(y[:, nqt + nkt:])
        if self.bias:
            b = (d["bq"], d["bk"], d["bv"])
        else:
            b = (np.zeros(nqt, np.float32), np.zeros(nkt, np.float32), np.zeros(nkt, np.float32))
        slot = None if d["slot"] is None else np.ascontiguousarray(d["slot"][s])
        rid, kr, vr, bad = oracle.qkv_epilogue(
            q.ravel(), k.ravel(), v.ravel(), *b, np.ascontiguousarray(d["pos"][s]),
            n_head=w.n_head, n_kv_head=w.n_kv_head, head_dim=w.head_dim, theta=w.theta,
            n_ctx=w.n_ctx, cache_dtype=self.cd, slot=slot, n_slots=w.n_slots,
            rope_style=self.style, freq_scale=self.freq_scale)
        self.o = dict(q=q, k=k, v=v, R=R, rid=rid, kr=kr, vr=vr)
        # the cache rows of every token (addressing only: the chain on zeros)
        zq = np.zeros(self.nt * nqt, np.float32)
        zk = np.zeros(self.nt * nkt, np.float32)
        zv = np.zeros(self.nt * nkt, np.float32)
        self.all_rows, _, _, self.n_bad = oracle.qkv_epilogue(
            zq, zk, zv, np.zeros(nqt, np.float32), np.zeros(nkt, np.float32),
            np.zeros(nkt, np.float32), d["pos"], n_head=w.n_head, n_kv_head=w.n_kv_head,
            head_dim=w.head_dim, theta=w.theta, n_ctx=w.n_ctx, cache_dtype=self.cd,
            slot=d["slot"], n_slots=w.n_slots)
        return self

    # -- gpu --
    def upload(self):
        w, d = self.w, self.d
        nqt, nkt, nt = w.nqt, w.nkt, self.nt
        ldx = self.hidden + self.ld_x_pad
        xp = np.zeros((nt, ldx), np.uint16)
        xp[:, :self.hidden] = d["x"]
        self.g_x = torch.from_numpy(xp.view(np.int16)).to(DEV)
        self.ld_x = ldx if self.ld_x_pad else 0
        wsrc = d["w8"] if self.wfmt == "e4m3" else d["w"].view(np.int16)
        self.g_w = torch.from_numpy(wsrc).to(DEV)
        self.g_wk = self.g_wv = None
        self.g_scale = torch.from_numpy(d["wscale"]).to(DEV) if self.wfmt == "e4m3" else None
        if self.weights == "three":
            # three allocations, v first so the sections are not laid out in order
            wq, wk, wv = (wsrc[a:b] for a, b in ((0, nqt), (nqt, nqt + nkt), (nqt + nkt, nqt + 2 * nkt)))
            self.g_wv = torch.from_numpy(np.ascontiguousarray(wv)).to(DEV)
            self.g_wk = torch.from_numpy(np.ascontiguousarray(wk)).to(DEV)
            self.g_w = torch.from_numpy(np.ascontiguousarray(wq)).to(DEV)
        m = self.misalign
        if self.form == "concat":
            n = nqt + 2 * nkt
            self._buf = torch.full((nt * n + m,), float("nan"), device=DEV)
            self.g_buf = self._buf[m:].view(nt, n)
            self.g_q = self.g_buf[:, :nqt]
            self.g_k = self.g_buf[:, nqt:nqt + nkt]
            self.g_v = self.g_buf[:, nqt + nkt:]
        else:
            def full(width):
                flat = torch.full((nt * width + m,), float("nan"), device=DEV)
                return flat, flat[m:].view(nt, width)
            self._q, self.g_q = full(nqt)
            self._k, self.g_k = full(nkt)
            self._v, self.g_v = full(nkt)
        if self.bias:
            self.g_b = [torch.from_numpy(d[n]).to(DEV) for n in ("bq", "bk", "bv")]
        else:
            self.g_b = [None, None, None]
        self.g_pos = torch.from_numpy(d["pos"]).to(DEV)
        self.g_slot = None if d["slot"] is None else torch.from_numpy(d["slot"]).to(DEV)
        rows = w.n_slots * w.n_ctx
        self.kc = new_cache(rows, nkt, self.cd)
        self.vc = new_cache(rows, nkt, self.cd)
        return self

    def args(self):
        w = self.w
        epi = B.make_args(self.g_q, self.g_k, self.g_v, *self.g_b, self.g_pos, self.kc, self.vc,
                          n_head=w.n_head, n_kv_head=w.n_kv_head, head_dim=w.head_dim,
                          theta=w.theta, cache_dtype=self.cd, slot=self.g_slot, n_ctx=w.n_ctx,
                          n_slots=w.n_slots, stream=torch.cuda.current_stream(),
                          use_stream=True, nt=self.nt, rope_style=self.style,
                          freq_scale=self.freq_scale)
        fmt = B.QKV_WEIGHT_E4M3 if self.wfmt == "e4m3" else B.QKV_WEIGHT_BF16
        return B.make_proj_args(self.g_x, self.g_w, self.hidden, epi, ld_x=self.ld_x, w_k=self.g_wk,
                                w_v=self.g_wv, w_format=fmt, w_scale=self.g_scale)

    def run_gpu(self, h):
        return B.qkv_epilogue_run_proj(h, self.args())

    # -- comparison --
    def check(self, label=""):
        w, s = self.w, self.sample
        nqt, nkt, hd, half = w.nqt, w.nkt, w.head_dim, w.head_dim // 2
        idx = torch.from_numpy(s.astype(np.int64)).to(DEV)
        got = {n: t.index_select(0, idx).cpu().numpy() for n, t in
               (("q", self.g_q), ("k", self.g_k), ("v", self.g_v))}
        K = self.hidden
        bnd = KSTAT * U32 * np.sqrt(K) * self.o["R"]
        secs = {"q": bnd[:, :nqt], "k": bnd[:, nqt:nqt + nkt], "v": bnd[:, nqt + nkt:]}
        for name in ("q", "k", "v"):
            g = got[name].astype(np.float64)
            o = self.o[name].astype(np.float64)
            b = secs[name]
            if name != "v" and self.style == B.QKV_ROPE_INTERLEAVED:
                # partner of column j: j ^ 1
                bh = b.reshape(b.shape[0], -1, 2)
                b = (bh + bh[:, :, ::-1]).reshape(b.shape)
            elif name != "v":
                # partner of column j inside its head: j +- half
                bh = b.reshape(b.shape[0], -1, 2, half)
                b = (bh + bh[:, :, ::-1, :]).reshape(b.shape)
            tol = 2e-6 + 1e-6 * np.abs(o) + b
            err = np.abs(g - o)
            nbad = int((err > tol).sum())
            rms = float(np.sqrt(np.mean(err ** 2))) if err.size else 0.0
            say(f"  {label} {name}: max err {err.max():.3g}, rms {rms:.3g}, "
                f"max bound {tol.max():.3g}")
            assert np.isfinite(g).all(), f"{label} {name}: non-finite outputs"
            assert nbad == 0, f"{label} {name}: {nbad} elements beyond the accumulation bound"
            assert rms <= RMS_TOL, f"{label} {name}: rms error {rms:.3g} > {RMS_TOL}"

        # addressing: exactly the oracle's rows change
        rows_all = self.all_rows[self.all_rows >= 0]
        for nm, cache in (("K", self.kc), ("V", self.vc)):
            ch = changed_rows(cache, self.cd)
            assert np.array_equal(np.sort(ch), np.unique(rows_all)), \
                f"{label} {nm} cache: changed rows differ from the oracle's"
        # contents: each sampled token's row is the store of its own k / v
        rid = self.all_rows[s]
        ok = rid >= 0
        if ok.any():
            ridx = torch.from_numpy(rid[ok]).to(DEV)
            for nm, cache, mine in (("K", self.kc, got["k"]), ("V", self.vc, got["v"])):
                c = cache.index_select(0, ridx).cpu().numpy()
                if self.cd == wl.CACHE_F32:
                    eq = c.view(np.uint32) == mine[ok].view(np.uint32)
                else:
                    eq = c.view(np.uint16) == mine[ok].astype(np.float16).view(np.uint16)
                # tokens sharing a row (equal positions) race: per element, the
                # row holds the store of one of them
                uniq, inv = np.unique(rid[ok], return_inverse=True)
                grp = np.zeros((uniq.size, eq.shape[1]), bool)
                np.logical_or.at(grp, inv, eq)
                assert grp.all(), \
                    f"{label} {nm} cache rows are not the store of the tokens' own outputs"


def _run(h, c, label):
    say(f"[proj] {label}: nt={c.nt} hidden={c.hidden} N={c.w.nqt + 2 * c.w.nkt} "
        f"hd={c.w.head_dim} cache={'f16' if c.cd else 'f32'} form={c.form} weights={c.wfmt}")
    c.run_oracle().upload()
    rc = c.run_gpu(h)
    assert rc == B.QKV_OK, B.qkv_epilogue_last_error(h)
    st = B.qkv_epilogue_status(h)
    torch.cuda.synchronize()
    return st


SMALL_14B = wl.Workload("proj_small_14b", 40, 8, 128, nt=300, n_ctx=4096, n_slots=1, layers=1,
                        seed=11, pos_mode="arange")
SMALL_7B = wl.Workload("proj_small_7b", 28, 4, 128, nt=130, n_ctx=4096, n_slots=1, layers=1,
                       seed=12, cache_dtypes=(wl.CACHE_F32,))
SMALL_05B = wl.Workload("proj_small_0.5b", 14, 2, 64, nt=257, n_ctx=512, n_slots=1, layers=1,
                        seed=13, cache_dtypes=(wl.CACHE_F32,))


@pytest.mark.parametrize("cd", [wl.CACHE_F16, wl.CACHE_F32])
def test_proj_prefill_small_14b(handle, cd):
    """300 tokens, 14B geometry: two 256 x 128 token tiles (the second ragged,
    44 tokens), k split in two, the summing epilogue."""
    c = ProjCase(SMALL_14B, hidden=1024, cache_dtype=cd)
    assert _run(handle, c, "small_14b") == B.QKV_OK
    c.check("small_14b")


def test_proj_concat_outputs_7b(handle):
    """Outputs as views of one concat q|k|v buffer (row stride N), 7B width."""
    c = ProjCase(SMALL_7B, hidden=3584, form="concat")
    assert _run(handle, c, "concat_7b") == B.QKV_OK
    c.check("concat_7b")


def test_proj_head_dim_64_no_bias(handle):
    """hd 64 (a wave's 64 outputs are one whole head) and NULL biases, 0.5B
    geometry (1152 outputs: 9 column blocks of 128), k split 7 ways."""
    c = ProjCase(SMALL_05B, hidden=896, bias=False)
    assert _run(handle, c, "hd64_nobias") == B.QKV_OK
    c.check("hd64_nobias")


def test_proj_padded_activation_rows(handle):
    """x rows with a stride larger than hidden."""
    c = ProjCase(SMALL_05B, hidden=512, nt=70, ld_x_pad=24)
    assert _run(handle, c, "ldx_pad") == B.QKV_OK
    c.check("ldx_pad")


@pytest.mark.parametrize("nt", [1, 2, 3, 4, 5, 8])
def test_proj_decode_gemv(handle, nt):
    """1-4 tokens take the weight-streaming kernel (one NeoX pair per wave),
    5 and 8 the k-split MFMA path on 64-token tiles; 14B decode geometry."""
    c = ProjCase(wl.DECODE_14B, hidden=5120, nt=nt)
    assert _run(handle, c, f"gemv_nt{nt}") == B.QKV_OK
    c.check(f"gemv_nt{nt}")


@pytest.mark.parametrize("nt", [4, 7])
def test_proj_gemv_hd64_slots(handle, nt):
    """hd 64 and per-token cache slots on the GEMV (4 tokens) and on the
    k-split MFMA path (7 tokens)."""
    w = wl.Workload("proj_gemv_slots", 14, 2, 64, nt=nt, n_ctx=64, n_slots=8, layers=1, seed=14,
                    cache_dtypes=(wl.CACHE_F16,))
    c = ProjCase(w, hidden=896)
    assert _run(handle, c, f"gemv_slots_{nt}") == B.QKV_OK
    c.check(f"gemv_slots_{nt}")


def test_proj_nine_tokens(handle):
    """Nine tokens of the 7B geometry on the MFMA path: one ragged 64-token
    tile per 256 outputs, k split 14 ways."""
    c = ProjCase(wl.DECODE_7B, hidden=3584, nt=9)
    assert _run(handle, c, "nt9") == B.QKV_OK
    c.check("nt9")


def test_proj_out_of_range_position(handle):
    """A token with a bad position: its q/k/v are still written, no cache row,
    and the status reports the range error (GEMV and MFMA paths)."""
    for nt in (3, 6, 40):
        pos = np.arange(nt, dtype=np.int32) * 7
        pos[1] = 4096 + 5   # beyond n_ctx
        c = ProjCase(wl.DECODE_14B, hidden=512, nt=nt, pos=pos)
        st = _run(handle, c, f"bad_pos_nt{nt}")
        assert st == B.QKV_ERR_POSITION_RANGE, st
        assert c.n_bad == 1
        c.check(f"bad_pos_nt{nt}")


def test_proj_long_ragged_hd64_no_bias(handle):
    """hd 64, 1100 tokens of the 0.5B geometry (too few tiles to fill the
    chip): 256 x 128 tiles with a ragged last token tile (1100 = 4*256 + 76),
    k split 4 ways."""
    w = wl.Workload("proj_long_0.5b", 14, 2, 64, nt=1100, n_ctx=2048, n_slots=1, layers=1,
                    seed=16, cache_dtypes=(wl.CACHE_F32,), pos_mode="arange")
    c = ProjCase(w, hidden=512, bias=False)
    assert _run(handle, c, "long_hd64") == B.QKV_OK
    c.check("long_hd64")


def test_proj_long_concat_14b(handle):
    """The data-parallel 128 x 128 launch (1030 tokens) writing views of one
    concat q|k|v buffer."""
    w = wl.Workload("proj_long_14b", 40, 8, 128, nt=1030, n_ctx=4096, n_slots=1, layers=1,
                    seed=17, pos_mode="uniform")
    c = ProjCase(w, hidden=256, form="concat")
    assert _run(handle, c, "long_concat") == B.QKV_OK
    c.check("long_concat")


def test_proj_long_misaligned_outputs(handle):
    """Outputs off 16-byte alignment: the data-parallel launch takes the
    epilogue's scalar stores."""
    w = wl.Workload("proj_long_mis", 40, 8, 128, nt=1030, n_ctx=4096, n_slots=1, layers=1,
                    seed=18, pos_mode="arange")
    c = ProjCase(w, hidden=256, misalign=1)
    assert _run(handle, c, "long_misaligned") == B.QKV_OK
    c.check("long_misaligned")


def test_proj_prefill_full_size_sampled(handle):
    """4096 tokens x hidden 5120, the prefill launch the benchmark times;
    the oracle recomputes a sample of tokens (both ends of every tile edge
    region and random ones), addressing is checked for all tokens."""
    rng = np.random.default_rng(7)
    sample = np.unique(np.concatenate([[0, 1, 127, 128, 2047, 4094, 4095],
                                       rng.integers(0, 4096, 41)]))
    c = ProjCase(wl.PREFILL_14B, hidden=5120, sample=sample)
    assert _run(handle, c, "prefill_full") == B.QKV_OK
    c.check("prefill_full")


def test_proj_batched_full_size_sampled(handle):
    """256 sequences, one token each, slot per sequence, hidden 5120."""
    rng = np.random.default_rng(8)
    sample = np.unique(np.concatenate([[0, 127, 128, 255], rng.integers(0, 256, 28)]))
    c = ProjCase(wl.BATCHED_DECODE_14B, hidden=5120, sample=sample)
    assert _run(handle, c, "batched_full") == B.QKV_OK
    c.check("batched_full")


def test_proj_rejects_unsupported(handle):
    """Requests outside the projection path's limits fail before any launch."""
    c = ProjCase(SMALL_05B, hidden=512, nt=8).upload()
    base = c.args()
    a = c.args()
    a.epi.rope_style = 2     # no such style
    assert B.qkv_epilogue_run_proj(handle, a) == B.QKV_ERR_UNSUPPORTED
    a = c.args()
    a.hidden = 100
    assert B.qkv_epilogue_run_proj(handle, a) == B.QKV_ERR_INVALID_ARG
    a = c.args()
    a.ld_x = 500
    assert B.qkv_epilogue_run_proj(handle, a) == B.QKV_ERR_INVALID_ARG
    a = c.args()
    a.x = c.g_q.data_ptr()   # activations overlapping the q output
    assert B.qkv_epilogue_run_proj(handle, a) == B.QKV_ERR_ALIAS
    a = c.args()
    a.w = c.kc.data_ptr()    # weights overlapping the K cache
    assert B.qkv_epilogue_run_proj(handle, a) == B.QKV_ERR_ALIAS
    a = c.args()
    a.x = c.g_x.data_ptr() + 2   # misaligned
    assert B.qkv_epilogue_run_proj(handle, a) == B.QKV_ERR_INVALID_ARG
    # head_dim 96 (widths not multiples of 128 either)
    w96 = wl.Workload("hd96", 4, 4, 96, nt=8, n_ctx=64, n_slots=1, layers=1, seed=15,
                      cache_dtypes=(wl.CACHE_F32,))
    c96 = ProjCase(w96, hidden=256).upload()
    assert B.qkv_epilogue_run_proj(handle, c96.args()) == B.QKV_ERR_UNSUPPORTED
    # three weight matrices: both k and v needed; none may overlap an output
    c3 = ProjCase(SMALL_05B, hidden=512, nt=8, weights="three").upload()
    a = c3.args()
    a.w_v = None
    assert B.qkv_epilogue_run_proj(handle, a) == B.QKV_ERR_INVALID_ARG
    a = c3.args()
    a.w_k = c3.g_v.data_ptr()   # the k weights overlapping the v output
    assert B.qkv_epilogue_run_proj(handle, a) == B.QKV_ERR_ALIAS
    a = c3.args()
    a.w_v = c3.vc.data_ptr()    # the v weights overlapping the V cache
    assert B.qkv_epilogue_run_proj(handle, a) == B.QKV_ERR_ALIAS
    a = c3.args()
    a.w_k = c3.g_wk.data_ptr() + 8   # misaligned
    assert B.qkv_epilogue_run_proj(handle, a) == B.QKV_ERR_INVALID_ARG
    # nothing was launched: the outputs still hold their NaN fill
    torch.cuda.synchronize()
    assert torch.isnan(c.g_q).all() and torch.isnan(c96.g_q).all() and torch.isnan(c3.g_q).all()
    assert B.qkv_epilogue_run_proj(handle, base) == B.QKV_OK
    assert B.qkv_epilogue_status(handle) == B.QKV_OK


def test_proj_split_head_groups_ragged(handle):
    """hd 64, 1900 tokens of the 0.5B geometry: k split 3 ways on 256 x 128
    tiles, and the summing kernel takes 4 heads per thread, so its last group
    holds the remaining 2 of the 18 heads; sampled tokens."""
    # unique positions: the cache check of sampled tokens cannot see a race
    # won by a token outside the sample
    w = wl.Workload("proj_groups_0.5b", 14, 2, 64, nt=1900, n_ctx=2048, n_slots=1, layers=1,
                    seed=24, cache_dtypes=(wl.CACHE_F16,), pos_mode="arange")
    rng = np.random.default_rng(9)
    sample = np.unique(np.concatenate([[0, 255, 256, 1899], rng.integers(0, 1900, 28)]))
    c = ProjCase(w, hidden=512, sample=sample)
    assert _run(handle, c, "groups_hd64") == B.QKV_OK
    c.check("groups_hd64")


@pytest.mark.parametrize("nt", [40, 300, 1030])
@pytest.mark.parametrize("wfmt", ["bf16", "e4m3"])
def test_proj_repeat_is_bitwise_identical(handle, nt, wfmt):
    """The k-split partials are added in split order and every tile sums its
    k steps in one order, so a repeated launch reproduces q/k/v bit for bit
    (40 and 300 tokens split k, 1030 run data-parallel), with bf16 and with
    E4M3 weights; the first result is also checked against the oracle."""
    w = wl.Workload("proj_repeat", 40, 8, 128, nt=nt, n_ctx=4096, n_slots=1, layers=1,
                    seed=25, pos_mode="arange")
    c = ProjCase(w, hidden=1024, wfmt=wfmt)
    assert _run(handle, c, f"repeat_{nt}") == B.QKV_OK
    first = [t.clone() for t in (c.g_q, c.g_k, c.g_v)]
    for _ in range(3):
        assert c.run_gpu(handle) == B.QKV_OK
        torch.cuda.synchronize()
        for a, b in zip(first, (c.g_q, c.g_k, c.g_v)):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"repeat_{nt}: results differ"
    c.check(f"repeat_{nt}")


@pytest.mark.parametrize("nt", [64, 150, 258, 400, 520, 1000, 1300, 1800])
def test_proj_plan_switches(handle, nt):
    """Every tile shape of the launch plan, split and data-parallel, at the
    14B width with hidden 2048 (the cost model's picks): 64 tokens on
    128 x 128 tiles with k split 4 ways, 150 on 64 x 256 split 3 ways, 258
    on 256 x 128 split 2 ways, 400 data-parallel 128 x 128, 520 data-
    parallel 64 x 256, 1000 data-parallel 256 x 128, 1300 data-parallel
    256 x 192 (three pair groups per wave; 112 groups leave the last tile
    one group), 1800 data-parallel 256 x 256.  The oracle recomputes both
    ends of every 256-token block and a random sample; the cache addressing
    is checked for all tokens (distinct positions: each sampled token's
    cache row is its own)."""
    w = wl.Workload("proj_plan", 40, 8, 128, nt=nt, n_ctx=4096, n_slots=1, layers=1,
                    seed=19, pos_mode="uniform")
    rng = np.random.default_rng(nt + 19)
    ends = np.r_[np.arange(0, nt, 256), np.arange(255, nt, 256), nt - 1]
    c = ProjCase(w, hidden=2048, sample=np.unique(np.r_[ends, rng.integers(0, nt, 24)]),
                 pos=rng.permutation(w.n_ctx)[:nt].astype(np.int32))
    assert _run(handle, c, f"plan_{nt}") == B.QKV_OK
    c.check(f"plan_{nt}")


def test_proj_split_256x256_sampled(handle):
    """700 tokens, hidden 5120: 256 x 256 tiles with k split 3 ways (the
    plan between the small-batch and the data-parallel shapes); the oracle
    recomputes sampled tokens, addressing is checked for all."""
    w = wl.Workload("proj_split_big", 40, 8, 128, nt=700, n_ctx=4096, n_slots=1, layers=1,
                    seed=26, pos_mode="arange")
    rng = np.random.default_rng(10)
    sample = np.unique(np.concatenate([[0, 255, 256, 511, 512, 699], rng.integers(0, 700, 26)]))
    c = ProjCase(w, hidden=5120, sample=sample)
    assert _run(handle, c, "split_256x256") == B.QKV_OK
    c.check("split_256x256")


def test_proj_split_256x192(handle):
    """660 tokens, hidden 3072: 256 x 192 tiles (three pair groups per wave)
    with k split 2 ways, so the partial tiles of every group go through the
    summing kernel."""
    w = wl.Workload("proj_split_g3", 40, 8, 128, nt=660, n_ctx=4096, n_slots=1, layers=1,
                    seed=27, pos_mode="uniform")
    c = ProjCase(w, hidden=3072)
    assert _run(handle, c, "split_256x192") == B.QKV_OK
    c.check("split_256x192")


def test_proj_hd64_256x192(handle):
    """hd 64 on 256 x 192 tiles (a wave's three pair groups are three whole
    heads; 64 groups leave the last tile one), 2100 tokens, hidden 1024, f32
    cache, data-parallel with the fused epilogue."""
    w = wl.Workload("proj_hd64_g3", 48, 8, 64, nt=2100, n_ctx=4096, n_slots=1, layers=1,
                    seed=28, cache_dtypes=(wl.CACHE_F32,), pos_mode="uniform")
    c = ProjCase(w, hidden=1024)
    assert _run(handle, c, "hd64_256x192") == B.QKV_OK
    c.check("hd64_256x192")


@pytest.mark.parametrize("nt", [1, 3, 40, 1100])
def test_proj_three_weight_matrices(handle, nt):
    """The q, k, v weights as three separate matrices (the page's layers that
    cannot share a concat matrix), in one launch: the GEMV (1 and 3 tokens),
    the k-split MFMA path (40) and the data-parallel one (1100), 14B widths."""
    w = wl.Workload("proj_three_w", 40, 8, 128, nt=nt, n_ctx=4096, n_slots=1, layers=1,
                    seed=29, pos_mode="uniform")
    c = ProjCase(w, hidden=1024, weights="three")
    assert _run(handle, c, f"three_w_{nt}") == B.QKV_OK
    c.check(f"three_w_{nt}")


def _random_shape(seed):
    """A seeded random projection case inside the path's limits: head_dim 64 or
    128, q and k/v widths multiples of 128, hidden a multiple of 64, 1-700
    tokens, either cache type, concat or three weight matrices, biases or none,
    one sequence or per-token slots, NeoX or interleaved pairing, a frequency
    scale or none."""
    rng = np.random.default_rng(1000 + seed)
    hd = int(rng.choice([64, 128]))
    step = 128 // hd                              # heads per 128 columns
    n_head = step * int(rng.integers(1, 13))
    n_kv_head = step * int(rng.integers(1, 5))
    nt = int(rng.choice([int(rng.integers(1, 5)), int(rng.integers(5, 80)), int(rng.integers(80, 700))]))
    hidden = 64 * int(rng.integers(1, 25))
    slots = int(rng.choice([1, 4]))
    cd = int(rng.choice([wl.CACHE_F32, wl.CACHE_F16]))
    w = wl.Workload(f"proj_rand_{seed}", n_head, n_kv_head, hd, nt=nt, n_ctx=1024, n_slots=slots,
                    layers=1, seed=40 + seed, cache_dtypes=(cd,), pos_mode="uniform")
    kw = dict(hidden=hidden, bias=bool(rng.integers(0, 2)), weights=str(rng.choice(["concat", "three"])))
    kw["style"] = int(rng.integers(0, 2))
    kw["freq_scale"] = float(rng.choice([1.0, 0.25]))
    return w, kw


@pytest.mark.parametrize("seed", range(40))
def test_proj_random_shapes(handle, seed):
    """Seeded random shapes across the launch plans (GEMV, k-split and
    data-parallel MFMA tiles of every shape), both head dims, both cache
    types, both weight layouts, with or without biases and slots, both
    pairings."""
    w, kw = _random_shape(seed)
    c = ProjCase(w, **kw)
    assert _run(handle, c, f"rand_{seed}") == B.QKV_OK
    c.check(f"rand_{seed}")


@pytest.mark.parametrize("seed", range(40, 64))
def test_proj_random_shapes_e4m3(handle, seed):
    """The same seeded random shapes with E4M3 weights and row scales: the
    GEMV for 1-4 tokens, the k-split and data-parallel MFMA tiles (E4M3
    stages, converted fragments, scales in the fused epilogue or in the
    summing kernel) for more."""
    w, kw = _random_shape(seed)
    c = ProjCase(w, wfmt="e4m3", **kw)
    assert _run(handle, c, f"rand_e4m3_{seed}") == B.QKV_OK
    c.check(f"rand_e4m3_{seed}")


@pytest.mark.parametrize("weights", ["concat", "three"])
def test_proj_python_wrapper(weights):
    """Epilogue.run_proj (the checked torch-tensor wrapper of the same entry
    point) on a 40-token 14B batch, against the oracle (three matrices with
    interleaved pairing); wrong dtypes raise before any launch."""
    w = wl.Workload("proj_wrapper", 40, 8, 128, nt=40, n_ctx=1024, n_slots=1, layers=1,
                    seed=32, pos_mode="uniform")
    style = B.QKV_ROPE_INTERLEAVED if weights == "three" else B.QKV_ROPE_NEOX
    c = ProjCase(w, hidden=512, weights=weights, style=style)
    c.run_oracle().upload()
    ep = B.Epilogue(0, w.n_ctx)
    bf = torch.bfloat16
    wk = None if c.g_wk is None else c.g_wk.view(bf)
    wv = None if c.g_wv is None else c.g_wv.view(bf)
    with pytest.raises(TypeError):
        ep.run_proj(c.g_x.view(bf).float(), c.g_w.view(bf), c.g_q, c.g_k, c.g_v, *c.g_b, c.g_pos, c.kc,
                    c.vc, n_head=w.n_head, n_kv_head=w.n_kv_head, head_dim=w.head_dim, theta=w.theta,
                    w_k=wk, w_v=wv)
    ep.run_proj(c.g_x.view(bf), c.g_w.view(bf), c.g_q, c.g_k, c.g_v, *c.g_b, c.g_pos, c.kc, c.vc,
                n_head=w.n_head, n_kv_head=w.n_kv_head, head_dim=w.head_dim, theta=w.theta,
                w_k=wk, w_v=wv, rope_style=style)
    assert ep.status() == B.QKV_OK, ep.last_error()
    torch.cuda.synchronize()
    c.check(f"wrapper_{weights}")
    ep.close()


def test_proj_long_slots_f32_cache(handle):
    """The fused long-prompt path with per-token cache slots (32 sequences)
    and an f32 cache; equal (slot, position) pairs are allowed to race."""
    w = wl.Workload("proj_long_slots", 40, 8, 128, nt=1100, n_ctx=64, n_slots=32, layers=1,
                    seed=20, cache_dtypes=(wl.CACHE_F32,), pos_mode="uniform")
    c = ProjCase(w, hidden=128)
    assert _run(handle, c, "long_slots") == B.QKV_OK
    c.check("long_slots")


@pytest.mark.parametrize("nt", [3, 40, 1030])
def test_proj_minimal_hidden(handle, nt):
    """hidden = 64 (one 64-deep k stage, fewer than the LDS ring's depth) on the
    GEMV, a small batch (k too short to split) and the data-parallel launch."""
    w = wl.Workload("proj_hidden64", 40, 8, 128, nt=nt, n_ctx=2048, n_slots=1, layers=1,
                    seed=21, pos_mode="arange")
    c = ProjCase(w, hidden=64)
    assert _run(handle, c, f"hidden64_{nt}") == B.QKV_OK
    c.check(f"hidden64_{nt}")


def _refresh_inputs(c, rep):
    """New activations and positions written into a case's device buffers."""
    rng = np.random.default_rng(5000 + rep)
    x = wl.bf16_bits(rng.standard_normal(c.d["x"].shape, dtype=np.float32))
    pos = rng.integers(0, c.w.n_ctx, size=c.nt, dtype=np.int32)
    c.d["x"] = x
    c.d["pos"] = pos
    ldx = c.g_x.shape[1]
    xp = np.zeros((c.nt, ldx), np.uint16)
    xp[:, :c.hidden] = x
    c.g_x.copy_(torch.from_numpy(xp.view(np.int16)).to(DEV))
    c.g_pos.copy_(torch.from_numpy(pos).to(DEV))
    for cache in (c.kc, c.vc):   # back to the sentinel so addressing is checked again
        fresh = new_cache(cache.shape[0], cache.shape[1], c.cd)
        cache.copy_(fresh)


def _graph_replays(handle, cases, reps=2):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):            # warm-up outside capture (sizes the workspace)
        for c in cases:
            assert B.qkv_epilogue_run_proj(handle, c.args()) == 0
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for c in cases:
            assert B.qkv_epilogue_run_proj(handle, c.args()) == 0
    torch.cuda.synchronize()
    for rep in range(reps):
        for c in cases:
            _refresh_inputs(c, rep * 100 + cases.index(c))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert B.qkv_epilogue_status(handle) == 0
        for i, c in enumerate(cases):
            c.run_oracle()
            c.check(f"graph replay {rep} call {i}")


@pytest.mark.parametrize("wfmt", ["bf16", "e4m3"])
def test_proj_graph_capture_decode_layers(handle, wfmt):
    """Six one-token layers (alternating concat and separate outputs) captured
    into one HIP graph and replayed with new activations and positions, with
    bf16 and with E4M3 weights."""
    cases = []
    for layer in range(6):
        c = ProjCase(wl.DECODE_14B, hidden=5120, nt=1, wfmt=wfmt,
                     form="concat" if layer % 2 == 0 else "separate")
        c.upload()
        cases.append(c)
    _graph_replays(handle, cases)


@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")
def test_proj_workspace_growth_refused_in_capture():
    """On a fresh handle a long-prompt call needs workspace: during stream
    capture it is refused (INVALID_ARG, nothing launched, the capture stays
    usable); outside capture the same call grows the workspace and runs."""
    rc, h = B.qkv_epilogue_create(0, 4096)
    assert rc == 0
    try:
        w = wl.Workload("proj_capture_grow", 40, 8, 128, nt=300, n_ctx=4096, n_slots=1, layers=1,
                        seed=24, pos_mode="uniform")
        c = ProjCase(w, hidden=256)
        c.run_oracle().upload()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            assert B.qkv_epilogue_run_proj(h, c.args()) == B.QKV_ERR_INVALID_ARG
        assert "outside stream capture" in B.qkv_epilogue_last_error(h)
        torch.cuda.synchronize()
        assert torch.isnan(c.g_q).all()
        assert B.qkv_epilogue_run_proj(h, c.args()) == B.QKV_OK
        assert B.qkv_epilogue_status(h) == B.QKV_OK
        torch.cuda.synchronize()
        c.check("grown outside capture")
    finally:
        B.qkv_epilogue_destroy(h)


@pytest.mark.parametrize("wfmt", ["bf16", "e4m3"])
def test_proj_graph_capture_split_and_fused(handle, wfmt):
    """A k-split call (300 tokens) and a data-parallel call (1100 tokens)
    captured after a warm-up call; no allocation happens in the capture.
    With bf16 and with E4M3 weights."""
    w1 = wl.Workload("proj_graph_split", 40, 8, 128, nt=300, n_ctx=4096, n_slots=1, layers=1,
                     seed=22, pos_mode="uniform")
    w2 = wl.Workload("proj_graph_long", 40, 8, 128, nt=1100, n_ctx=4096, n_slots=1, layers=1,
                     seed=23, pos_mode="uniform")
    cases = [ProjCase(w1, hidden=256, wfmt=wfmt).upload(), ProjCase(w2, hidden=256, wfmt=wfmt).upload()]
    _graph_replays(handle, cases)


@pytest.mark.parametrize("geom,nt", [("14b", 1), ("14b", 3), ("14b", 40), ("14b", 300), ("14b", 1030),
                                     ("0.5b", 2), ("0.5b", 257), ("0.5b", 1100)])
def test_proj_interleaved(handle, geom, nt):
    """Interleaved (GPT-J) pairs (2i, 2i+1): the GEMV (1-3 tokens) takes
    adjacent weight rows as a pair; MFMA launches of 40-1100 tokens, with or
    without a k split as the plan picks, rotate inside each lane's four
    consecutive outputs or pair adjacent columns in the summing kernel; hd
    128, and hd 64 with a frequency scale."""
    if geom == "14b":
        w = wl.Workload("proj_il_14b", 40, 8, 128, nt=nt, n_ctx=4096, n_slots=1, layers=1,
                        seed=60 + nt, pos_mode="uniform")
        c = ProjCase(w, hidden=512, style=B.QKV_ROPE_INTERLEAVED)
    else:
        w = wl.Workload("proj_il_0.5b", 14, 2, 64, nt=nt, n_ctx=2048, n_slots=1, layers=1,
                        seed=70 + nt, cache_dtypes=(wl.CACHE_F16,), pos_mode="arange")
        c = ProjCase(w, hidden=896, style=B.QKV_ROPE_INTERLEAVED, freq_scale=0.25)
    assert _run(handle, c, f"interleaved_{geom}_{nt}") == B.QKV_OK
    c.check(f"interleaved_{geom}_{nt}")


def test_proj_interleaved_full_size_sampled(handle):
    """4096 tokens x hidden 5120 with interleaved pairing (the largest tile
    shape), sampled tokens against the oracle."""
    rng = np.random.default_rng(11)
    sample = np.unique(np.concatenate([[0, 255, 256, 4095], rng.integers(0, 4096, 28)]))
    c = ProjCase(wl.PREFILL_14B, hidden=5120, sample=sample, style=B.QKV_ROPE_INTERLEAVED)
    assert _run(handle, c, "interleaved_full") == B.QKV_OK
    c.check("interleaved_full")


# ---- 8-bit float (E4M3) weights: the weight-streaming kernel, 1-4 tokens ----

@pytest.mark.parametrize("nt", [1, 2, 3, 4])
def test_proj_e4m3_decode_14b(handle, nt):
    """E4M3 weights with row scales on the 14B decode geometry at its real
    hidden size (the GEMV streams 36.7 MB of weights)."""
    c = ProjCase(wl.DECODE_14B, hidden=5120, nt=nt, wfmt="e4m3")
    assert _run(handle, c, f"e4m3_nt{nt}") == B.QKV_OK
    c.check(f"e4m3_nt{nt}")


@pytest.mark.parametrize("weights,style,nt", [("three", B.QKV_ROPE_NEOX, 1), ("concat", B.QKV_ROPE_INTERLEAVED, 3),
                                              ("three", B.QKV_ROPE_INTERLEAVED, 4)])
def test_proj_e4m3_layouts(handle, weights, style, nt):
    """E4M3 weights as three matrices and with interleaved pairing, 7B
    geometry (hidden 3584: 112 chunks per wave, two per lane)."""
    c = ProjCase(wl.DECODE_7B, hidden=3584, nt=nt, wfmt="e4m3", weights=weights, style=style)
    assert _run(handle, c, f"e4m3_{weights}_{style}_{nt}") == B.QKV_OK
    c.check(f"e4m3_{weights}_{style}_{nt}")


@pytest.mark.parametrize("geom,weights,style,hidden", [
    ("7b", "three", B.QKV_ROPE_NEOX, 4096),          # two chunks per lane
    ("7b", "three", B.QKV_ROPE_INTERLEAVED, 4160),   # three, last step partly masked
    ("14b", "concat", B.QKV_ROPE_INTERLEAVED, 8192),  # four
])
def test_proj_e4m3_two_pairs_per_wave_layouts(handle, geom, weights, style, hidden):
    """4 tokens at hidden >= 4096 run the GEMV with two NeoX/interleaved pairs
    per wave: the three-matrix layout, interleaved pairing and each unroll
    depth of that instance."""
    w = wl.DECODE_7B if geom == "7b" else wl.DECODE_14B
    c = ProjCase(w, hidden=hidden, nt=4, wfmt="e4m3", weights=weights, style=style)
    label = f"e4m3_p2_{geom}_{weights}_{style}_{hidden}"
    assert _run(handle, c, label) == B.QKV_OK
    c.check(label)


@pytest.mark.parametrize("hidden", [4096, 4160])
def test_proj_e4m3_two_pairs_per_wave_hd64(handle, hidden):
    """head_dim 64 at 4 tokens and hidden >= 4096 (two pairs per wave), slots,
    no bias; 4160 leaves the last step partly masked."""
    w = wl.Workload("proj_e4m3_hd64_p2", 14, 2, 64, nt=4, n_ctx=64, n_slots=8, layers=1, seed=35,
                    cache_dtypes=(wl.CACHE_F16,))
    c = ProjCase(w, hidden=hidden, wfmt="e4m3", bias=False)
    assert _run(handle, c, f"e4m3_p2_hd64_{hidden}") == B.QKV_OK
    c.check(f"e4m3_p2_hd64_{hidden}")


@pytest.mark.parametrize("hidden", [64, 896, 1088])
def test_proj_e4m3_hd64_ragged_hidden(handle, hidden):
    """hd 64 with hidden sizes that leave the last step partly masked (64:
    2 of 64 lanes busy; 896: 28 chunks per wave; 1088: 34), slots, no bias."""
    w = wl.Workload("proj_e4m3_hd64", 14, 2, 64, nt=3, n_ctx=64, n_slots=8, layers=1, seed=33,
                    cache_dtypes=(wl.CACHE_F16,))
    c = ProjCase(w, hidden=hidden, wfmt="e4m3", bias=False)
    assert _run(handle, c, f"e4m3_hd64_{hidden}") == B.QKV_OK
    c.check(f"e4m3_hd64_{hidden}")


def test_proj_e4m3_every_code_exact(handle):
    """One-hot activations pick single weights, so every v output is one
    decoded code times its row's scale plus the bias: bit-equal to the
    oracle.  The v rows at the picked columns hold every finite E4M3 code."""
    w = wl.Workload("proj_e4m3_codes", 2, 2, 64, nt=4, n_ctx=64, n_slots=1, layers=1, seed=34,
                    cache_dtypes=(wl.CACHE_F32,), pos_mode="arange")
    hidden = 64
    c = ProjCase(w, hidden=hidden, wfmt="e4m3")
    cols = np.array([3, 20, 41, 62])
    x = np.zeros((4, hidden), np.uint16)
    x[np.arange(4), cols] = 0x3f80                     # bfloat16 1.0
    c.d["x"] = x
    finite = np.array([v for v in range(256) if v not in (0x7F, 0xFF)], np.uint8)
    nqt, nkt = w.nqt, w.nkt
    vblock = np.resize(finite, (nkt, 4))               # 128 rows x 4 columns = 512 slots
    c.d["w8"][nqt + nkt:, cols] = vblock
    assert np.isin(finite, c.d["w8"][nqt + nkt:][:, cols]).all()
    assert _run(handle, c, "e4m3_codes") == B.QKV_OK
    c.check("e4m3_codes")
    got_v = c.g_v.cpu().numpy()
    assert np.array_equal(got_v.view(np.uint32), c.o["v"].view(np.uint32)), "v differs from the oracle"


@pytest.mark.parametrize("nt", [4, 5])
def test_proj_e4m3_rejections(handle, nt):
    """E4M3 weights, on the GEMV (4 tokens) and the MFMA path (5): the
    scales are required, aligned and read-only; an unknown format is
    unsupported.  Nothing is launched for a rejected call."""
    c = ProjCase(SMALL_05B, hidden=512, nt=nt, wfmt="e4m3").upload()
    a = c.args()
    a.w_scale = None
    assert B.qkv_epilogue_run_proj(handle, a) == B.QKV_ERR_INVALID_ARG
    a = c.args()
    a.w_scale = c.g_scale.data_ptr() + 2
    assert B.qkv_epilogue_run_proj(handle, a) == B.QKV_ERR_INVALID_ARG
    a = c.args()
    a.w_scale = c.g_k.data_ptr()                    # scales overlapping the k output
    assert B.qkv_epilogue_run_proj(handle, a) == B.QKV_ERR_ALIAS
    a = c.args()
    a.w_format = 7
    assert B.qkv_epilogue_run_proj(handle, a) == B.QKV_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.isnan(c.g_q).all()
    assert B.qkv_epilogue_run_proj(handle, c.args()) == B.QKV_OK
    assert B.qkv_epilogue_status(handle) == B.QKV_OK


# ---- E4M3 weights on the MFMA kernel, 5+ tokens -------------------------------

@pytest.mark.parametrize("nt", [5, 64, 150, 258, 400, 520, 1000, 1300, 1800])
def test_proj_e4m3_mfma_plan_switches(handle, nt):
    """E4M3 weights through every tile shape the plan picks for them, k
    split and data-parallel, at the 14B width with hidden 2048: the codes
    land in LDS as bytes, each fragment read turns 8 of them into bf16, the
    epilogue (or the split path's summing kernel) applies the row scales.
    The oracle recomputes both ends of every 256-token block and a random
    sample (its E4M3 decode costs ~0.1 s per token at this width); the cache
    addressing is checked for all tokens.  Distinct positions, so that every
    sampled token's cache row is its own."""
    w = wl.Workload("proj_plan_e4m3", 40, 8, 128, nt=nt, n_ctx=4096, n_slots=1, layers=1,
                    seed=36, pos_mode="uniform")
    rng = np.random.default_rng(nt)
    ends = np.r_[np.arange(0, nt, 256), np.arange(255, nt, 256), nt - 1]
    sample = np.unique(np.r_[ends, rng.integers(0, nt, 16)]) if nt > 40 else None
    c = ProjCase(w, hidden=2048, wfmt="e4m3", sample=sample,
                 pos=rng.permutation(w.n_ctx)[:nt].astype(np.int32))
    assert _run(handle, c, f"e4m3_plan_{nt}") == B.QKV_OK
    c.check(f"e4m3_plan_{nt}")


@pytest.mark.parametrize("weights,style,nt", [("three", B.QKV_ROPE_NEOX, 40), ("three", B.QKV_ROPE_NEOX, 1030),
                                              ("concat", B.QKV_ROPE_INTERLEAVED, 40),
                                              ("three", B.QKV_ROPE_INTERLEAVED, 1030)])
def test_proj_e4m3_mfma_layouts(handle, weights, style, nt):
    """Three weight matrices and interleaved pairing on the MFMA kernel with
    E4M3 weights, split (40 tokens) and data-parallel (1030), 7B geometry."""
    rng = np.random.default_rng(nt)
    c = ProjCase(wl.DECODE_7B, hidden=3584, nt=nt, wfmt="e4m3", weights=weights, style=style,
                 sample=np.unique(np.r_[0, nt - 1, rng.integers(0, nt, 30)]),
                 pos=rng.permutation(wl.DECODE_7B.n_ctx)[:nt].astype(np.int32))
    assert _run(handle, c, f"e4m3_mfma_{weights}_{style}_{nt}") == B.QKV_OK
    c.check(f"e4m3_mfma_{weights}_{style}_{nt}")


@pytest.mark.parametrize("nt", [40, 1030])
def test_proj_e4m3_mfma_hd64(handle, nt):
    """head_dim 64 with slots and no bias on the MFMA kernel, E4M3 weights."""
    w = wl.Workload("proj_e4m3_hd64_mm", 14, 2, 64, nt=nt, n_ctx=512, n_slots=4, layers=1, seed=37,
                    cache_dtypes=(wl.CACHE_F16,))
    rng = np.random.default_rng(nt + 1)
    sample = np.unique(np.r_[0, nt - 1, rng.integers(0, nt, 30)])
    rows = rng.permutation(w.n_slots * w.n_ctx)[:nt]         # distinct (slot, position) rows
    c = ProjCase(w, hidden=896, wfmt="e4m3", bias=False, sample=sample,
                 pos=(rows % w.n_ctx).astype(np.int32), slot=(rows // w.n_ctx).astype(np.int32))
    assert _run(handle, c, f"e4m3_mfma_hd64_{nt}") == B.QKV_OK
    c.check(f"e4m3_mfma_hd64_{nt}")


def test_proj_e4m3_prefill_full_size_sampled(handle):
    """4096 tokens x hidden 5120 with E4M3 weights: the data-parallel
    256 x 256 tiles, three stages of LDS; sampled tokens, every row address."""
    rng = np.random.default_rng(38)
    sample = np.unique(np.concatenate([[0, 1, 255, 256, 2047, 4095], rng.integers(0, 4096, 42)]))
    c = ProjCase(wl.PREFILL_14B, hidden=5120, sample=sample, wfmt="e4m3")
    assert _run(handle, c, "e4m3_prefill_full") == B.QKV_OK
    c.check("e4m3_prefill_full")


def test_proj_e4m3_batched_full_size_sampled(handle):
    """256 sequences, one token each, slot per sequence, hidden 5120, E4M3
    weights: the k-split path, row scales applied after the partials' sum."""
    rng = np.random.default_rng(39)
    sample = np.unique(np.concatenate([[0, 127, 128, 255], rng.integers(0, 256, 28)]))
    c = ProjCase(wl.BATCHED_DECODE_14B, hidden=5120, sample=sample, wfmt="e4m3")
    assert _run(handle, c, "e4m3_batched_full") == B.QKV_OK
    c.check("e4m3_batched_full")


@pytest.mark.parametrize("nt,hidden", [(40, 64), (64, 1024)])
def test_proj_e4m3_every_code_exact_mfma(handle, nt, hidden):
    """The one-hot test on the MFMA kernel: fused epilogue (40 tokens,
    hidden 64, no split) and the k-split path (64 tokens, hidden 1024).  Each
    v output is one decoded code times its row's scale plus the bias, equal
    to the oracle bit for bit; the picked columns of the v rows hold every
    finite E4M3 code."""
    w = wl.Workload(f"proj_e4m3_codes_mm{nt}", 2, 2, 64, nt=nt, n_ctx=128, n_slots=1, layers=1, seed=40,
                    cache_dtypes=(wl.CACHE_F32,), pos_mode="arange")
    c = ProjCase(w, hidden=hidden, wfmt="e4m3")
    rng = np.random.default_rng(41)
    cols = rng.integers(0, hidden, nt)
    x = np.zeros((nt, hidden), np.uint16)
    x[np.arange(nt), cols] = 0x3f80                    # bfloat16 1.0
    c.d["x"] = x
    finite = np.array([v for v in range(256) if v not in (0x7F, 0xFF)], np.uint8)
    nqt, nkt = w.nqt, w.nkt
    ucols = np.unique(cols)
    vblock = np.resize(finite, (nkt, ucols.size))
    c.d["w8"][nqt + nkt:, ucols] = vblock
    assert np.isin(finite, c.d["w8"][nqt + nkt:][:, ucols]).all()
    assert _run(handle, c, f"e4m3_codes_mm{nt}") == B.QKV_OK
    c.check(f"e4m3_codes_mm{nt}")
    got_v = c.g_v.cpu().numpy()
    assert np.array_equal(got_v.view(np.uint32), c.o["v"].view(np.uint32)), "v differs from the oracle"


def test_proj_e4m3_python_wrapper():
    """Epilogue.run_proj with float8_e4m3fn weight tensors and the scale
    tensor; a missing scale raises before any launch."""
    w = wl.DECODE_14B
    c = ProjCase(w, hidden=1024, nt=2, wfmt="e4m3", weights="three")
    c.run_oracle().upload()
    ep = B.Epilogue(0, w.n_ctx)
    f8, bf = torch.float8_e4m3fn, torch.bfloat16
    ws = [t.view(f8) for t in (c.g_w, c.g_wk, c.g_wv)]
    with pytest.raises(TypeError):
        ep.run_proj(c.g_x.view(bf), *ws[:1], c.g_q, c.g_k, c.g_v, *c.g_b, c.g_pos, c.kc, c.vc,
                    n_head=w.n_head, n_kv_head=w.n_kv_head, head_dim=w.head_dim, theta=w.theta,
                    w_k=ws[1], w_v=ws[2])
    ep.run_proj(c.g_x.view(bf), ws[0], c.g_q, c.g_k, c.g_v, *c.g_b, c.g_pos, c.kc, c.vc,
                n_head=w.n_head, n_kv_head=w.n_kv_head, head_dim=w.head_dim, theta=w.theta,
                w_k=ws[1], w_v=ws[2], w_scale=c.g_scale)
    assert ep.status() == B.QKV_OK, ep.last_error()
    torch.cuda.synchronize()
    c.check("e4m3_wrapper")
    ep.close()
