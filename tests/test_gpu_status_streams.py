"""qkv_epilogue_status covers launches on every stream since the last status
call, not only the stream of the last launch.

A token with an out-of-range position is launched on one stream behind a few
large matrix products (so that it finishes late), then a valid launch goes to
another stream; status must still report the range error, and a second status
call must find the word cleared.  The same with nine streams, past the eight
the handle tracks one by one (status then waits for the device).
"""
import pytest
import torch

from parity_helpers import DEV, Case, say
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


def _busy(stream):
    """A few milliseconds of work ahead of the next launch on stream."""
    with torch.cuda.stream(stream):
        a = torch.randn(4096, 4096, device=DEV)
        for _ in range(4):
            a = a @ a
            a = a / a.abs().max()
    return a


def _launch(h, c, stream):
    rc = c.run_gpu(h, stream=stream)
    assert rc == 0, B.qkv_epilogue_last_error(h)


@pytest.mark.parametrize("n_streams", [2, 9])
def test_status_waits_for_every_stream(handle, n_streams):
    say(f"[case] status over {n_streams} streams")
    w = wl.TINY_DECODE
    streams = [torch.cuda.Stream() for _ in range(n_streams)]
    bad = Case(w, pos=[w.n_ctx + 3]).run_oracle().upload()
    assert bad.o_bad
    good = [Case(w, pos=[1 + i]).run_oracle().upload() for i in range(n_streams - 1)]
    torch.cuda.synchronize()
    keep = _busy(streams[0])
    _launch(handle, bad, streams[0])
    for c, s in zip(good, streams[1:]):
        _launch(handle, c, s)
    assert B.qkv_epilogue_status(handle) == B.QKV_ERR_POSITION_RANGE
    assert B.qkv_epilogue_status(handle) == B.QKV_OK
    del keep
    # the valid launches wrote their results
    for c in good:
        c.download()
        c.check(label="status streams")
