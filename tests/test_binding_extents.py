"""The torch wrappers reject tensors too small for what the kernels address.

The C ABI takes bare pointers, so only the wrapper can compare extents.  Every
case here uses host tensors: a shape error must be raised before the device
check and before anything reaches the library.  A wrapper object is made
without a device handle (h = 0), so a check that let a case through would end
in the device TypeError, never in a launch.
"""
import pytest
import torch

from qkv_bias_rope_amd import binding as B

NH, NKV, HD, NT, NCTX = 4, 2, 8, 3, 16
NQT, NKT = NH * HD, NKV * HD


def _ep():
    ep = object.__new__(B.Epilogue)
    ep.h, ep.device, ep.n_ctx = 0, 0, NCTX
    return ep


def _good(n_slots=1, cache=torch.float16):
    f = torch.float32
    return dict(
        q=torch.zeros(NT, NQT, dtype=f), k=torch.zeros(NT, NKT, dtype=f),
        v=torch.zeros(NT, NKT, dtype=f), bq=torch.zeros(NQT, dtype=f),
        bk=torch.zeros(NKT, dtype=f), bv=torch.zeros(NKT, dtype=f),
        pos=torch.zeros(NT, dtype=torch.int32),
        kcache=torch.zeros(n_slots * NCTX, NKT, dtype=cache),
        vcache=torch.zeros(n_slots * NCTX, NKT, dtype=cache))


def _run(ep, t, **kw):
    ep.run(t["q"], t["k"], t["v"], t["bq"], t["bk"], t["bv"], t["pos"], t["kcache"], t["vcache"],
           n_head=NH, n_kv_head=NKV, head_dim=HD, **kw)


def test_good_shapes_reach_the_device_check():
    with pytest.raises(TypeError, match="cuda:0"):
        _run(_ep(), _good())


@pytest.mark.parametrize("name,bad", [
    ("q", torch.zeros(NT - 1, NQT)),
    ("q", torch.zeros(NT, NQT - 1)),
    ("q", torch.zeros(NT * NQT - 1)),
    ("k", torch.zeros(NT - 1, NKT)),
    ("v", torch.zeros(NT, NKT + 4)[:, :NKT - 4]),
    ("v", torch.zeros(NT * NKT)[::2]),
    ("bq", torch.zeros(NQT - 1)),
    ("bk", torch.zeros(NKT + 1)),
    ("bv", torch.zeros(2 * NKT)[::2]),
    ("kcache", torch.zeros(NCTX - 1, NKT, dtype=torch.float16)),
    ("vcache", torch.zeros(NCTX * NKT - 1, dtype=torch.float16)),
    ("kcache", torch.zeros(NKT, NCTX, dtype=torch.float16).t()),
])
def test_undersized_tensor_rejected(name, bad):
    t = _good()
    t[name] = bad
    with pytest.raises(ValueError, match=name):
        _run(_ep(), t)


def test_pos_sets_the_token_count():
    t = _good()
    t["pos"] = torch.zeros(NT + 1, dtype=torch.int32)
    with pytest.raises(ValueError, match="q"):
        _run(_ep(), t)


def test_slot_count_and_slot_cache_rows():
    t = _good()
    with pytest.raises(ValueError, match="slot"):
        _run(_ep(), t, slot=torch.zeros(NT - 1, dtype=torch.int32), n_slots=1)
    # three slots need 3*n_ctx rows; the handle's n_ctx applies when none is given
    with pytest.raises(ValueError, match="kcache"):
        _run(_ep(), t, slot=torch.zeros(NT, dtype=torch.int32), n_slots=3)
    t3 = _good(n_slots=3)
    with pytest.raises(TypeError, match="cuda:0"):
        _run(_ep(), t3, slot=torch.zeros(NT, dtype=torch.int32), n_slots=3)
    # a larger per-call n_ctx than the cache holds
    with pytest.raises(ValueError, match="kcache"):
        _run(_ep(), _good(), n_ctx=NCTX + 1)


def test_concat_views_pass():
    t = _good()
    buf = torch.zeros(NT, NQT + 2 * NKT)
    t["q"], t["k"], t["v"] = buf[:, :NQT], buf[:, NQT:NQT + NKT], buf[:, NQT + NKT:]
    with pytest.raises(TypeError, match="cuda:0"):
        _run(_ep(), t)


def _proj(ep, t, x, w, **kw):
    ep.run_proj(x, w, t["q"], t["k"], t["v"], t["bq"], t["bk"], t["bv"], t["pos"], t["kcache"],
                t["vcache"], n_head=NH, n_kv_head=NKV, head_dim=HD, **kw)


def test_proj_extents():
    hid = 32
    t = _good()
    x = torch.zeros(NT, hid, dtype=torch.bfloat16)
    w = torch.zeros(NQT + 2 * NKT, hid, dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="cuda:0"):
        _proj(_ep(), t, x, w)
    with pytest.raises(ValueError, match="x has"):
        _proj(_ep(), t, x[:NT - 1], w)
    with pytest.raises(ValueError, match="w has"):
        _proj(_ep(), t, x, w[:-1])
    wq, wk, wv = (torch.zeros(r, hid, dtype=torch.bfloat16) for r in (NQT, NKT, NKT))
    with pytest.raises(TypeError, match="cuda:0"):
        _proj(_ep(), t, x, wq, w_k=wk, w_v=wv)
    with pytest.raises(ValueError, match="w_k has"):
        _proj(_ep(), t, x, wq, w_k=wk[:-1], w_v=wv)
    t2 = dict(t)
    t2["q"] = torch.zeros(NT - 1, NQT)
    with pytest.raises(ValueError, match="q"):
        _proj(_ep(), t2, x, w)
    t3 = dict(t)
    t3["vcache"] = torch.zeros(NCTX - 1, NKT, dtype=torch.float16)
    with pytest.raises(ValueError, match="vcache"):
        _proj(_ep(), t3, x, w)
