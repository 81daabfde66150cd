"""The benchmark's reference kernels (libqkv_probe.so) compute what they claim.

The floor and ceilings the benchmark reports are only meaningful if the probe
kernels really move the bytes: copy must copy, add must add one in place, and
the row pass must add the bias in place and store the k/v columns into the
addressed cache rows (f16 by round to nearest even), for every memory policy
and launch shape the benchmark sweeps.  Checked against torch on the device.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

P = pytest.importorskip("qkv_bias_rope_amd.probe")
DEV = "cuda:0"


@pytest.mark.parametrize("policy", (0, 1, 2, 3))
@pytest.mark.parametrize("vpt", (1, 2, 4, 8))
def test_copy_and_add(policy, vpt):
    n = 4 * (3 * 256 * vpt + 37)   # a ragged last workgroup
    src = torch.randn(n, device=DEV)
    dst = torch.full_like(src, -7.0)
    s = torch.cuda.current_stream()
    assert P.copy(dst, src, block=256, vpt=vpt, policy=policy, stream=s) == 0
    buf = src.clone()
    assert P.add(buf, block=128, vpt=vpt, policy=policy, stream=s) == 0
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    assert torch.equal(buf, src + 1.0)


def test_rejects_bad_arguments():
    x = torch.zeros(64, device=DEV)
    assert P.copy(x, x, block=100) == -1          # block not a multiple of 64
    assert P.add(x, vpt=3) == -1                  # no such instance
    assert P.add(x, policy=4) == -1               # no such policy
    assert P.empty(0, 64) == -1
    assert P.empty_args(0, 64) == -1
    assert P.empty_args(3, 100) == -1


def test_empty_kernels_launch():
    s = torch.cuda.current_stream()
    assert P.empty(14, 64, s) == 0
    assert P.empty_args(14, 64, s) == 0
    torch.cuda.synchronize()


@pytest.mark.parametrize("cache", (torch.float16, torch.float32))
@pytest.mark.parametrize("policy", (0, 1, 2, 3))
@pytest.mark.parametrize("tpb", (1, 2, 4))
def test_rows(cache, policy, tpb):
    rng = np.random.default_rng(5)
    nt, nqt, nkt, n_ctx, n_slots = 13, 96, 32, 50, 4
    width = nqt + 2 * nkt
    x0 = torch.from_numpy(rng.standard_normal((nt, width), dtype=np.float32)).to(DEV)
    b = torch.from_numpy(rng.standard_normal(width, dtype=np.float32)).to(DEV)
    slot = torch.from_numpy(rng.integers(0, n_slots, nt, dtype=np.int32)).to(DEV)
    # distinct (slot, pos) rows
    flat = rng.choice(n_slots * n_ctx, nt, replace=False)
    slot = torch.from_numpy((flat // n_ctx).astype(np.int32)).to(DEV)
    pos = torch.from_numpy((flat % n_ctx).astype(np.int32)).to(DEV)
    kc = torch.full((n_slots * n_ctx, nkt), 9.0, dtype=cache, device=DEV)
    vc = torch.full_like(kc, 9.0)
    x = x0.clone()
    assert P.rows(x, b, nqt, nkt, pos, slot, n_ctx, kc, vc, block=64, tpb=tpb, policy=policy,
                  stream=torch.cuda.current_stream()) == 0
    torch.cuda.synchronize()
    want = x0 + b
    assert torch.equal(x, want)
    rows = torch.from_numpy(flat.astype(np.int64)).to(DEV)
    assert torch.equal(kc[rows], want[:, nqt:nqt + nkt].to(cache))
    assert torch.equal(vc[rows], want[:, nqt + nkt:].to(cache))
    untouched = torch.ones(n_slots * n_ctx, dtype=torch.bool, device=DEV)
    untouched[rows] = False
    assert bool((kc[untouched] == 9.0).all()) and bool((vc[untouched] == 9.0).all())


@pytest.mark.parametrize("policy", (0, 1))
@pytest.mark.parametrize("vpt", (1, 2, 4, 8))
@pytest.mark.parametrize("block", (128, 256))
def test_read(policy, vpt, block):
    """Every wave's sum of the vectors it reads, exact with small integers
    (any summation order gives the same f32 value)."""
    rng = np.random.default_rng(vpt * 10 + policy)
    n16 = 3 * block * vpt + 37          # a ragged last workgroup
    src_np = rng.integers(-3, 4, 4 * n16).astype(np.float32)
    src = torch.from_numpy(src_np).to(DEV)
    n_out = P.read_out_numel(n16, block, vpt)
    out = torch.full((n_out,), -1.0, device=DEV)
    assert P.read(src, out, block=block, vpt=vpt, policy=policy,
                  stream=torch.cuda.current_stream()) == 0
    torch.cuda.synchronize()
    vec = src_np.reshape(n16, 4).sum(axis=1).astype(np.int64)
    groups = P.grid(n16, block, vpt)
    want = np.zeros(n_out, np.int64)
    for g in range(groups):
        for t in range(block):
            for j in range(vpt):
                k = g * block * vpt + j * block + t
                if k < n16:
                    want[g * (block // 64) + t // 64] += vec[k]
    assert np.array_equal(out.cpu().numpy().astype(np.int64), want)


def test_read_rejects_bad_arguments():
    x = torch.zeros(256, device=DEV)
    out = torch.zeros(64, device=DEV)
    assert P.read(x, out, policy=2) == -1        # loads have two policies only
    assert P.read(x, out, vpt=3) == -1
