"""GPU parity of the rotary variants -- interleaved (GPT-J) pairing and a
frequency scale -- against the oracle, for the fused kernel, the q/k-norm
variant and the unfused chain, plus the fused == unfused byte gate."""
import numpy as np
import pytest
import torch

from parity_helpers import Case, say, tensors_bitwise_equal
from qkv_bias_rope_amd import binding as B
from qkv_bias_rope_amd import workloads as wl

pytestmark = pytest.mark.gpu
IL = 1


@pytest.fixture(scope="module")
def handle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rc, h = B.qkv_epilogue_create(0, 4096)
    assert rc == 0, rc
    yield h
    B.qkv_epilogue_destroy(h)


def run(h, c, label, entry="run_ex"):
    say(f"[case] {label} style={c.style} scale={c.freq_scale} norm={c.norm} entry={entry}")
    c.run_oracle().upload()
    assert c.run_gpu(h, entry) == 0, B.qkv_epilogue_last_error(h)
    assert B.qkv_epilogue_status(h) == (B.QKV_ERR_POSITION_RANGE if c.o_bad else 0)
    c.download()
    return c.check(label=label)


@pytest.mark.parametrize("style,scale", [(IL, 1.0), (0, 0.25), (IL, 0.125)])
def test_prefill_full(handle, style, scale):
    run(handle, Case(wl.PREFILL_14B, style=style, freq_scale=scale), "prefill 4096")


@pytest.mark.parametrize("cd", [wl.CACHE_F16, wl.CACHE_F32])
def test_batched_full_interleaved(handle, cd):
    run(handle, Case(wl.BATCHED_DECODE_14B, cache_dtype=cd, style=IL), "batched 256 seq")
    torch.cuda.empty_cache()


@pytest.mark.parametrize("w", [wl.TINY_DECODE, wl.DECODE_7B, wl.DECODE_14B], ids=lambda w: w.name)
@pytest.mark.parametrize("form", ["separate", "concat"])
def test_decode_interleaved(handle, w, form):
    run(handle, Case(w, style=IL, form=form, freq_scale=0.5), f"{w.name} {form}")


@pytest.mark.parametrize("geom", [(14, 2, 64), (8, 8, 96), (5, 3, 8), (4, 2, 6), (3, 3, 2),
                                  (2, 1, 512), (7, 1, 18)])
@pytest.mark.parametrize("nt", [1, 37, 1100])
def test_geometries_interleaved(handle, geom, nt):
    nh, nkv, hd = geom
    w = wl.Workload(f"g{geom}", nh, nkv, hd, nt=nt, n_ctx=4096, n_slots=1, layers=1, seed=23,
                    cache_dtypes=(wl.CACHE_F16,))
    run(handle, Case(w, style=IL, pos=(np.arange(nt) * 7) % 4096), f"geometry {geom}")


def test_misaligned_interleaved(handle):
    w = wl.Workload("mis", 40, 8, 128, nt=9, n_ctx=4096, n_slots=1, layers=1, seed=31)
    run(handle, Case(w, misalign=1, style=IL, freq_scale=0.25, pos=np.arange(9) * 3), "misaligned")


@pytest.mark.parametrize("geom", [(40, 8, 128), (8, 8, 96), (4, 2, 6)])
def test_qk_norm_interleaved(handle, geom):
    nh, nkv, hd = geom
    w = wl.Workload(f"n{geom}", nh, nkv, hd, nt=300, n_ctx=4096, n_slots=1, layers=1, seed=25,
                    cache_dtypes=(wl.CACHE_F16,))
    run(handle, Case(w, norm=True, bias=False, style=IL, freq_scale=0.5,
                     pos=(np.arange(300) * 11) % 4096), f"qk-norm {geom}")


@pytest.mark.parametrize("style,scale", [(IL, 1.0), (0, 0.25), (IL, 0.25)])
@pytest.mark.parametrize("nt,geom", [(1, (40, 8, 128)), (1000, (40, 8, 128)), (19, (4, 2, 6))])
def test_unfused_matches_fused(handle, style, scale, nt, geom):
    nh, nkv, hd = geom
    w = wl.Workload(f"u{geom}", nh, nkv, hd, nt=nt, n_ctx=4096, n_slots=1, layers=1, seed=27,
                    cache_dtypes=(wl.CACHE_F16,))
    mk = lambda: Case(w, style=style, freq_scale=scale, pos=(np.arange(nt) * 5) % 4096)
    cu = mk()
    run(handle, cu, "unfused", entry="unfused")
    cf = mk().upload()
    assert cf.run_gpu(handle) == 0
    torch.cuda.synchronize()
    for n in ("q", "k", "v"):
        assert tensors_bitwise_equal(getattr(cu, "g_" + n).contiguous(), getattr(cf, "g_" + n).contiguous()), n
    assert tensors_bitwise_equal(cu.kc, cf.kc) and tensors_bitwise_equal(cu.vc, cf.vc)


def test_unknown_style_rejected(handle):
    c = Case(wl.TINY_DECODE).upload()
    a = c.args()
    a.rope_style = 2
    assert B.qkv_epilogue_run_ex(handle, a) == B.QKV_ERR_UNSUPPORTED
    assert B.qkv_epilogue_run_unfused(handle, a) == B.QKV_ERR_UNSUPPORTED
    a = c.args()
    a.freq_scale = -1.0
    assert B.qkv_epilogue_run_ex(handle, a) == B.QKV_ERR_INVALID_ARG
