"""GPU parity of the unfused chain (add_bias x3, rope x2, store x2 as seven
launches) against the CPU oracle, and the fusion gate: the fused kernel and the
unfused chain give byte-identical q/k/v sections and caches on the same inputs
(the page's probe compares the fused epilogue with the unfused chain byte for
byte on both pointer forms, f32 and f16 caches, 14B and 7B shapes)."""
import numpy as np
import pytest
import torch

from parity_helpers import Case, changed_rows, say, tensors_bitwise_equal
from qkv_bias_rope_amd import binding as B
from qkv_bias_rope_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def handle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rc, h = B.qkv_epilogue_create(0, 4096)
    assert rc == 0, rc
    yield h
    B.qkv_epilogue_destroy(h)


def run_both(h, make_case, label):
    """Run the oracle, the unfused chain and the fused kernel on identical
    inputs; check unfused vs oracle and fused vs unfused byte for byte."""
    say(f"[case] {label}")
    cu = make_case().run_oracle().upload()
    assert cu.run_gpu(h, "unfused") == 0, B.qkv_epilogue_last_error(h)
    st = B.qkv_epilogue_status(h)
    assert st == (B.QKV_ERR_POSITION_RANGE if cu.o_bad else 0)
    cu.download()
    cu.check(label=label + " unfused")
    cf = make_case().upload()
    assert cf.run_gpu(h, "run_ex") == 0, B.qkv_epilogue_last_error(h)
    assert B.qkv_epilogue_status(h) == (B.QKV_ERR_POSITION_RANGE if cu.o_bad else 0)
    torch.cuda.synchronize()
    for n in ("q", "k", "v"):
        a, b = getattr(cu, "g_" + n), getattr(cf, "g_" + n)
        assert tensors_bitwise_equal(a.contiguous(), b.contiguous()), f"{label}: fused {n} != unfused"
    assert tensors_bitwise_equal(cu.kc, cf.kc), f"{label}: K caches differ"
    assert tensors_bitwise_equal(cu.vc, cf.vc), f"{label}: V caches differ"


@pytest.mark.parametrize("form", ["separate", "concat"])
def test_tiny(handle, form):
    run_both(handle, lambda: Case(wl.TINY_DECODE, form=form), f"tiny {form}")


@pytest.mark.parametrize("w", [wl.DECODE_7B, wl.DECODE_14B], ids=lambda w: w.name)
@pytest.mark.parametrize("form", ["separate", "concat"])
@pytest.mark.parametrize("cd", [wl.CACHE_F16, wl.CACHE_F32])
def test_decode_shapes(handle, w, form, cd):
    for layer in (0, 1, w.layers - 1):
        run_both(handle, lambda: Case(w, layer=layer, form=form, cache_dtype=cd,
                                      pos=[(layer * 997 + 5) % w.n_ctx]),
                 f"{w.name} layer {layer} {form} cache={cd}")


@pytest.mark.parametrize("nt", [3, 37, 1000, 4096])
def test_prefill(handle, nt):
    run_both(handle, lambda: Case(wl.PREFILL_14B, nt=nt, pos=np.arange(nt) % 4096),
             f"prefill nt={nt}")


def test_prefill_concat_rows(handle):
    run_both(handle, lambda: Case(wl.PREFILL_14B, nt=77, form="concat", pos=np.arange(77) * 5),
             "prefill concat nt=77")


@pytest.mark.parametrize("cd", [wl.CACHE_F16, wl.CACHE_F32])
def test_batched_slots(handle, cd):
    w = wl.Workload("batched_mid", 40, 8, 128, nt=256, n_ctx=512, n_slots=256, layers=1, seed=4,
                    cache_dtypes=(cd,))
    run_both(handle, lambda: Case(w), f"batched 256 seq n_ctx=512 cache={cd}")


@pytest.mark.parametrize("geom", [(5, 3, 8), (4, 2, 6), (3, 3, 2), (2, 1, 512), (8, 8, 96)])
def test_geometries(handle, geom):
    nh, nkv, hd = geom
    w = wl.Workload(f"g{geom}", nh, nkv, hd, nt=19, n_ctx=97, n_slots=1, layers=1, seed=21,
                    cache_dtypes=(wl.CACHE_F16,))
    run_both(handle, lambda: Case(w, pos=np.arange(19) * 5), f"geometry {geom}")


def test_misaligned(handle):
    w = wl.Workload("mis", 40, 8, 128, nt=9, n_ctx=4096, n_slots=1, layers=1, seed=31)
    run_both(handle, lambda: Case(w, misalign=1, pos=np.arange(9) * 3), "misaligned")


def test_out_of_range(handle):
    w = wl.Workload("range", 40, 8, 128, nt=6, n_ctx=100, n_slots=1, layers=1, seed=41,
                    cache_dtypes=(wl.CACHE_F32,))
    run_both(handle, lambda: Case(w, pos=[0, 99, 100, -1, 50, 1 << 30]), "out of range")


def test_unfused_rejects_like_fused(handle):
    c = Case(wl.TINY_DECODE).upload()
    a = c.args()
    a.rope_style = 5
    assert B.qkv_epilogue_run_unfused(handle, a) == B.QKV_ERR_UNSUPPORTED
    a = c.args()
    a.vcache = a.kcache
    assert B.qkv_epilogue_run_unfused(handle, a) == B.QKV_ERR_ALIAS
    a = c.args()
    a.nt = 0
    assert B.qkv_epilogue_run_unfused(handle, a) == 0
    torch.cuda.synchronize()
    assert changed_rows(c.kc, c.cd).size == 0
