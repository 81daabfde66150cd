"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports
every declared entry point, validates arguments as documented in
include/qkv_epilogue.h, plans the launch, and builds the same inverse-frequency
table as the oracle."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qkv_epilogue.h")

# QKV_HOST_LIB names a host-only build of the library's validation, planning
# and table code (qkv_host.cpp, built with the sanitizers by
# tests/test_sanitizers.py): the host cases below then run against it, and
# the checks of the product library's exports and links are skipped.
_HOST_LIB = os.environ.get("QKV_HOST_LIB")
if _HOST_LIB:
    import types
    from qkv_bias_rope_amd import abi as _abi
    _api = _abi.load_host(_HOST_LIB)
    B = types.SimpleNamespace(**{n: getattr(_abi, n) for n in dir(_abi) if not n.startswith("__")})
    for _n in _abi.HOST_EXPORTS:
        setattr(B, _n, getattr(_api, _n))
else:
    from qkv_bias_rope_amd import binding as B

product_only = pytest.mark.skipif(bool(_HOST_LIB), reason="checks the product library itself")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qkv_epilogue_[a-z_]+)\s*\(", src)))


@product_only
def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(B.EXPORTS), names
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (qkv_epilogue_\w+)", out))
    for n in names:
        assert n in exported, n
        assert hasattr(B.lib, n)


@product_only
def test_probe_library_exports_and_stands_apart():
    """The benchmark's reference kernels live in their own library: it exports
    its entry points, defines its launch stubs, and the epilogue library
    carries none of them."""
    from qkv_bias_rope_amd import probe as P
    out = subprocess.run(["nm", "-D", "--defined-only", P.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (qkv_probe_\w+)", out))
    assert exported == set(P.EXPORTS), exported
    und = subprocess.run(["nm", "-D", "--undefined-only", P.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    assert "device_stub" not in und
    epi = subprocess.run(["nm", "-D", B.LIB_PATH], capture_output=True, text=True).stdout
    assert "qkv_probe" not in epi


@product_only
def test_every_kernel_launch_stub_is_defined():
    """Every kernel the host code launches has its launch stub in the library:
    some device-code constructs in a kernel template make hipcc's host pass
    drop the stubs without a diagnostic, leaving undefined symbols that only
    fail when a launch is resolved."""
    out = subprocess.run(["nm", "-D", "--undefined-only", B.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    missing = [l for l in out.splitlines() if "device_stub" in l]
    assert not missing, missing[:5]


@product_only
def test_library_links_no_oracle():
    out = subprocess.run(["nm", "-D", B.LIB_PATH], capture_output=True, text=True).stdout
    assert "oracle" not in out
    ldd = subprocess.run(["ldd", B.LIB_PATH], capture_output=True, text=True).stdout
    assert "oracle" not in ldd


@pytest.mark.parametrize("theta", [1.0e6, 1.0e4, 5.0e5, 10000.0 * 1.5])
@pytest.mark.parametrize("hd", [2, 4, 6, 8, 64, 96, 128, 256, 512])
def test_inv_freq_table_matches_oracle(theta, hd):
    got = np.zeros(hd // 2, np.float32)
    assert B.qkv_epilogue_inv_freq(theta, hd, got.ctypes.data) == 0
    want = oracle.inv_freq(theta, hd)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("scale", [0.25, 1.0 / 3.0, 2.0, 1.0])
@pytest.mark.parametrize("hd", [4, 64, 128, 96])
def test_scaled_inv_freq_table_matches_oracle(scale, hd):
    got = np.zeros(hd // 2, np.float32)
    assert B.qkv_epilogue_inv_freq_scaled(1e6, scale, hd, got.ctypes.data) == 0
    want = oracle.inv_freq_scaled(1e6, scale, hd)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    assert B.qkv_epilogue_inv_freq_scaled(1e6, 0.0, hd, got.ctypes.data) == B.QKV_ERR_INVALID_ARG


def test_inv_freq_rejects_bad_input():
    buf = np.zeros(512, np.float32)
    for theta, hd in ((1e6, 3), (1e6, 0), (1e6, 514), (0.0, 4), (-1.0, 4), (float("inf"), 4),
                      (float("nan"), 4)):
        assert B.qkv_epilogue_inv_freq(theta, hd, buf.ctypes.data) == B.QKV_ERR_INVALID_ARG
    assert B.qkv_epilogue_inv_freq(1e6, 4, None) == B.QKV_ERR_INVALID_ARG


# Fake, well-separated device addresses: check_args/plan never dereference.
GB = 1 << 36


def base_args(nt=4, n_head=40, n_kv_head=8, hd=128, cache_dtype=1, **kw):
    nqt, nkt = n_head * hd, n_kv_head * hd
    a = B.make_args(q=1 * GB, k=2 * GB, v=3 * GB, bq=4 * GB, bk=5 * GB, bv=6 * GB,
                    pos=7 * GB, kcache=8 * GB, vcache=64 * GB, nt=nt, n_head=n_head,
                    n_kv_head=n_kv_head, head_dim=hd, theta=1e6, cache_dtype=cache_dtype,
                    n_ctx=4096)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def rc_of(a):
    rc, msg = B.qkv_epilogue_check_args(a)
    return rc, msg


def test_valid_args_ok():
    assert rc_of(base_args()) == (0, "")
    assert rc_of(base_args(rope_style=B.QKV_ROPE_INTERLEAVED)) == (0, "")
    assert rc_of(base_args(freq_scale=0.25)) == (0, "")
    assert rc_of(base_args(rope_style=B.QKV_ROPE_INTERLEAVED, head_dim=6, n_head=2, n_kv_head=1)) == (0, "")


@pytest.mark.parametrize("field", ["q", "k", "v", "bq", "bk", "bv", "pos", "kcache", "vcache"])
def test_null_pointer_rejected(field):
    a = base_args()
    setattr(a, field, None)
    rc, msg = rc_of(a)
    assert rc == B.QKV_ERR_INVALID_ARG and field in msg


def test_nt_zero_is_noop_even_with_nulls():
    a = base_args(nt=0)
    for f in ("q", "k", "v", "pos", "kcache"):
        setattr(a, f, None)
    assert rc_of(a)[0] == 0


@pytest.mark.parametrize("kw,code", [
    (dict(nt=-1), B.QKV_ERR_INVALID_ARG),
    (dict(n_head=0), B.QKV_ERR_INVALID_ARG),
    (dict(n_kv_head=0), B.QKV_ERR_INVALID_ARG),
    (dict(head_dim=127), B.QKV_ERR_INVALID_ARG),
    (dict(head_dim=0), B.QKV_ERR_INVALID_ARG),
    (dict(head_dim=514), B.QKV_ERR_INVALID_ARG),
    (dict(theta=0.0), B.QKV_ERR_INVALID_ARG),
    (dict(theta=-5.0), B.QKV_ERR_INVALID_ARG),
    (dict(theta=float("inf")), B.QKV_ERR_INVALID_ARG),
    (dict(theta=float("nan")), B.QKV_ERR_INVALID_ARG),
    (dict(cache_dtype=2), B.QKV_ERR_INVALID_ARG),
    (dict(rope_style=7), B.QKV_ERR_UNSUPPORTED),
    (dict(rope_style=-1), B.QKV_ERR_UNSUPPORTED),
    (dict(freq_scale=-0.5), B.QKV_ERR_INVALID_ARG),
    (dict(freq_scale=float("inf")), B.QKV_ERR_INVALID_ARG),
    (dict(freq_scale=float("nan")), B.QKV_ERR_INVALID_ARG),
    (dict(ld_q=5119), B.QKV_ERR_INVALID_ARG),
    (dict(ld_k=1000), B.QKV_ERR_INVALID_ARG),
    (dict(ld_v=-1), B.QKV_ERR_INVALID_ARG),
    (dict(n_ctx=-1), B.QKV_ERR_INVALID_ARG),
    (dict(n_slots=-2), B.QKV_ERR_INVALID_ARG),
    (dict(kcache=8 * GB + 1), B.QKV_ERR_INVALID_ARG),   # misaligned f16 cache
    (dict(q=1 * GB + 2), B.QKV_ERR_INVALID_ARG),        # misaligned f32
    (dict(pos=7 * GB + 2), B.QKV_ERR_INVALID_ARG),
])
def test_invalid_args(kw, code):
    a = base_args(**kw)
    rc, msg = rc_of(a)
    assert rc == code, (kw, rc, msg)
    assert msg


def test_cache_size_overflow_rejected():
    a = base_args(n_ctx=1 << 40, n_slots=1 << 30)
    assert rc_of(a)[0] == B.QKV_ERR_INVALID_ARG


def test_alias_checks():
    nqt, nkt = 5120, 1024
    # k overlapping the end of q
    a = base_args(nt=1)
    a.k = a.q + (nqt - 1) * 4
    assert rc_of(a)[0] == B.QKV_ERR_ALIAS
    # concat single row: q | k | v back to back is fine
    a = base_args(nt=1)
    a.k = a.q + nqt * 4
    a.v = a.q + (nqt + nkt) * 4
    assert rc_of(a) == (0, "")
    # concat rows with the concat stride: interleaved but disjoint
    ld = nqt + 2 * nkt
    a = base_args(nt=64, ld_q=ld, ld_k=ld, ld_v=ld)
    a.k = a.q + nqt * 4
    a.v = a.q + (nqt + nkt) * 4
    assert rc_of(a) == (0, "")
    # same, but dense strides: the rows of q run into k
    a = base_args(nt=64)
    a.k = a.q + nqt * 4
    a.v = a.q + (nqt + nkt) * 4
    assert rc_of(a)[0] == B.QKV_ERR_ALIAS
    # concat stride but v one element too early (overlaps k's last column)
    a = base_args(nt=8, ld_q=ld, ld_k=ld, ld_v=ld)
    a.k = a.q + nqt * 4
    a.v = a.q + (nqt + nkt - 1) * 4
    assert rc_of(a)[0] == B.QKV_ERR_ALIAS
    # v section's row t overlaps q's row t+1 when ld is too small for the sections
    a = base_args(nt=8, ld_q=ld, ld_k=ld, ld_v=ld)
    a.k = a.q + nqt * 4
    a.v = a.q + (nqt + nkt) * 4 + 4 * 4    # last 4 elements of v spill into the next row's q
    assert rc_of(a)[0] == B.QKV_ERR_ALIAS
    # kcache and vcache the same buffer
    a = base_args()
    a.vcache = a.kcache
    assert rc_of(a)[0] == B.QKV_ERR_ALIAS
    # the cache covering q
    a = base_args()
    a.kcache = a.q - 1024
    assert rc_of(a)[0] == B.QKV_ERR_ALIAS
    # a bias inside the output v
    a = base_args()
    a.bq = a.v
    assert rc_of(a)[0] == B.QKV_ERR_ALIAS
    # pos inside the K cache
    a = base_args()
    a.pos = a.kcache + 4096
    assert rc_of(a)[0] == B.QKV_ERR_ALIAS
    # read-only inputs may share memory with each other
    a = base_args()
    a.bk = a.bv
    assert rc_of(a) == (0, "")


def plan_of(a):
    rc, p = B.qkv_epilogue_plan(a)
    assert rc == 0
    return p


def test_plan_vector_path_and_units():
    p = plan_of(base_args(nt=4096))
    assert p.vec_width == 4
    assert p.units_per_token == (40 + 8) * 16 + 1024 // 8   # 896
    assert p.block % 64 == 0 and p.block <= 1024
    # the column blocks of a token cover its units
    assert p.col_blocks * p.block * p.units_per_thread >= 896
    assert (p.col_blocks - 1) * p.block * p.units_per_thread < 896
    assert p.grid == p.col_blocks * -(-4096 // p.tokens_per_block)
    p = plan_of(base_args(nt=256))
    assert p.vec_width == 4 and p.grid >= 256
    p = plan_of(base_args(nt=1))
    assert p.tokens_per_block == 1 and p.grid == p.col_blocks >= 4


def test_plan_scalar_path_for_misaligned_or_small_heads():
    a = base_args(nt=3)
    a.q = a.q + 4                       # 4-byte aligned only
    assert plan_of(a).vec_width == 1
    assert plan_of(base_args(nt=3, hd=6, n_head=2, n_kv_head=1)).vec_width == 1
    a = base_args(nt=3, ld_q=5124)      # stride keeps 16-byte rows
    assert plan_of(a).vec_width == 4
    a = base_args(nt=3, ld_q=5121)      # stride breaks 16-byte rows
    assert plan_of(a).vec_width == 1
    a = base_args(nt=3, cache_dtype=1)
    a.kcache = a.kcache + 2             # f16-aligned, not 8-byte aligned
    assert plan_of(a).vec_width == 1


def test_plan_lds_fits():
    for hd, nh, nkv in ((8, 1, 1), (512, 1, 1), (128, 40, 8), (64, 14, 2), (2, 1, 1)):
        p = plan_of(base_args(nt=100000, hd=hd, n_head=nh, n_kv_head=nkv))
        assert 0 < p.lds_bytes <= 64 * 1024


@product_only
def test_create_without_device_fails_loudly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    rc, h = B.qkv_epilogue_create(0, 4096)
    assert rc == B.QKV_ERR_HIP and h == 0
    rc, h = B.qkv_epilogue_create(0, 0)
    assert rc == B.QKV_ERR_INVALID_ARG
    assert B.qkv_epilogue_last_error(None) == "NULL handle"
    B.qkv_epilogue_destroy(None)   # no-op


def test_rows_too_wide_rejected():
    """The kernel decodes units with a reciprocal multiply exact below 2^22
    units per token: one more head past that is refused, one less is not."""
    # hd 128 on the vector path: 16 units per head, nkt/8 for v
    under = base_args(nt=1, n_head=(1 << 18) - 20)
    assert rc_of(under) == (0, "")
    rc, msg = rc_of(base_args(nt=1, n_head=1 << 18))
    assert rc == B.QKV_ERR_INVALID_ARG and "rows too wide" in msg
