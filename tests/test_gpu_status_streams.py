"""qkv_epilogue_status covers launches on every stream since the last status
call, not only the stream of the last launch.

A token with an out-of-range position is launched on one stream behind a few
large matrix products (so that it finishes late), then valid launches go to
other streams; status must still report the range error, and a second status
call must find the word cleared.  Also after the streams of those launches
are destroyed, and for a range error that only a graph replay produces.
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


def test_status_after_the_streams_are_gone(handle):
    """Launches on streams the caller has destroyed (after synchronizing them)
    before calling status: status neither fails nor misses the error."""
    say("[case] status after the launch streams were destroyed")
    w = wl.TINY_DECODE
    bad = Case(w, pos=[w.n_ctx]).run_oracle().upload()
    good = Case(w, pos=[2]).run_oracle().upload()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    _launch(handle, bad, s1)
    _launch(handle, good, s2)
    s1.synchronize()
    s2.synchronize()
    del s1, s2
    import gc
    gc.collect()
    assert B.qkv_epilogue_status(handle) == B.QKV_ERR_POSITION_RANGE, B.qkv_epilogue_last_error(handle)
    assert B.qkv_epilogue_status(handle) == B.QKV_OK


def test_status_covers_graph_replays(handle):
    """A range error produced only by a replay of a captured graph (the
    captured launch itself is the library's only sight of it)."""
    say("[case] status after a graph replay")
    w = wl.TINY_DECODE
    c = Case(w, pos=[3]).run_oracle().upload()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        assert c.run_gpu(handle, stream=torch.cuda.current_stream()) == 0
    assert B.qkv_epilogue_status(handle) == B.QKV_OK
    # the captured launch reads pos from device memory: an out-of-range value
    # written there now is seen only by the replays
    c.g_pos.fill_(w.n_ctx + 1)
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        g.replay()
    assert B.qkv_epilogue_status(handle) == B.QKV_ERR_POSITION_RANGE
    assert B.qkv_epilogue_status(handle) == B.QKV_OK
