"""GPU parity of the q/k-norm variant (per-head RMS norm of q and k between
the bias add and the rope; biases optional, as in the Qwen3 attention) against
the oracle's qkv_norm_epilogue, same tolerances as the plain epilogue."""
import numpy as np
import pytest
import torch

from parity_helpers import Case, changed_rows, say
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


def run_norm(h, c, label):
    say(f"[case] qk-norm {label} nt={c.nt} bias={c.bias} cache={'f16' if c.cd else 'f32'}")
    c.run_oracle().upload()
    assert c.run_gpu(h) == 0, B.qkv_epilogue_last_error(h)
    assert B.qkv_epilogue_status(h) == (B.QKV_ERR_POSITION_RANGE if c.o_bad else 0)
    c.download()
    return c.check(label=f"qk-norm {label}")


@pytest.mark.parametrize("bias", [False, True])
def test_prefill_14b_full(handle, bias):
    run_norm(handle, Case(wl.PREFILL_14B, norm=True, bias=bias), "prefill 4096")


@pytest.mark.parametrize("bias", [False, True])
@pytest.mark.parametrize("form", ["separate", "concat"])
def test_decode_14b(handle, bias, form):
    w = wl.DECODE_14B
    for layer in (0, 7):
        run_norm(handle, Case(w, layer=layer, norm=True, bias=bias, form=form), f"decode layer {layer}")


@pytest.mark.parametrize("cd", [wl.CACHE_F16, wl.CACHE_F32])
def test_batched_256(handle, cd):
    w = wl.Workload("batched_norm", 40, 8, 128, nt=256, n_ctx=1024, n_slots=256, layers=1, seed=4,
                    cache_dtypes=(cd,))
    run_norm(handle, Case(w, norm=True, bias=False), "batched 256")


@pytest.mark.parametrize("nt", [2, 37, 1000])
def test_ragged(handle, nt):
    run_norm(handle, Case(wl.PREFILL_14B, nt=nt, norm=True, bias=False,
                          pos=(np.arange(nt) * 3) % 4096), f"ragged {nt}")


@pytest.mark.parametrize("geom", [(32, 8, 128), (14, 2, 64), (8, 8, 96), (5, 3, 8), (4, 2, 6),
                                  (3, 3, 2), (2, 1, 512), (7, 1, 18)])
@pytest.mark.parametrize("nt", [1, 19, 300])
def test_geometries(handle, geom, nt):
    nh, nkv, hd = geom
    w = wl.Workload(f"g{geom}", nh, nkv, hd, nt=nt, n_ctx=4096, n_slots=1, layers=1, seed=21,
                    cache_dtypes=(wl.CACHE_F16,))
    run_norm(handle, Case(w, norm=True, bias=(nt != 19), pos=(np.arange(nt) * 13) % 4096),
             f"geometry {geom}")


def test_misaligned_scalar_path(handle):
    w = wl.Workload("mis", 40, 8, 128, nt=9, n_ctx=4096, n_slots=1, layers=1, seed=31)
    run_norm(handle, Case(w, misalign=1, norm=True, pos=np.arange(9) * 3), "misaligned")


def test_out_of_range(handle):
    w = wl.Workload("range", 40, 8, 128, nt=6, n_ctx=100, n_slots=1, layers=1, seed=41,
                    cache_dtypes=(wl.CACHE_F32,))
    run_norm(handle, Case(w, norm=True, pos=[0, 99, 100, -1, 50, 1 << 30]), "out of range")


def test_invalid_requests(handle):
    c = Case(wl.TINY_DECODE, norm=True).upload()
    a = c.args()
    assert B.qkv_epilogue_run_qk_norm(handle, a, None, c.g_wk, 1e-6) == B.QKV_ERR_INVALID_ARG
    assert B.qkv_epilogue_run_qk_norm(handle, a, c.g_wq, c.g_wk, -1.0) == B.QKV_ERR_INVALID_ARG
    assert B.qkv_epilogue_run_qk_norm(handle, a, c.g_wq, c.g_wk, float("nan")) == \
        B.QKV_ERR_INVALID_ARG
    # a weight inside an output
    assert B.qkv_epilogue_run_qk_norm(handle, a, c.g_q, c.g_wk, 1e-6) == B.QKV_ERR_ALIAS
    # the plain entry still requires biases
    a.bq = None
    assert B.qkv_epilogue_run_ex(handle, a) == B.QKV_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert changed_rows(c.kc, c.cd).size == 0


@pytest.mark.parametrize("seed", range(24))
def test_random_shapes(handle, seed):
    """Seeded random launches of the q/k-norm variant: head dims 2-256, 1-16 q
    and 1-8 kv heads, 1-600 tokens at distinct positions, one sequence or
    three slots, either cache type, separate or concat sections, NeoX or
    interleaved pairing, biases or none."""
    rng = np.random.default_rng(3000 + seed)
    hd = int(rng.choice([2, 4, 8, 16, 18, 32, 64, 96, 128, 256]))
    nh, nkv = int(rng.integers(1, 17)), int(rng.integers(1, 9))
    nt = int(rng.choice([1, int(rng.integers(2, 40)), int(rng.integers(40, 600))]))
    n_slots = int(rng.choice([1, 3]))
    n_ctx = int(rng.integers(nt, nt + 200))
    cd = int(rng.choice([wl.CACHE_F32, wl.CACHE_F16]))
    w = wl.Workload(f"normrand{seed}", nh, nkv, hd, nt=nt, n_ctx=n_ctx, n_slots=n_slots, layers=1,
                    seed=90 + seed, cache_dtypes=(cd,))
    pos = rng.permutation(n_ctx)[:nt].astype(np.int32)
    slot = rng.integers(0, n_slots, nt).astype(np.int32) if n_slots > 1 else None
    c = Case(w, norm=True, bias=bool(rng.integers(0, 2)), pos=pos, slot=slot, n_ctx=n_ctx,
             n_slots=n_slots, form=str(rng.choice(["separate", "concat"])), style=int(rng.integers(0, 2)))
    run_norm(handle, c, f"rand {seed}: {nh}x{nkv}x{hd}")
