#!/usr/bin/env python3
"""Benchmark of the fused attention-input epilogue on one MI355X.

A step is one launch of the epilogue over one batch of synthetic input.  The
headline workload is the 14B-shape prefill: 4096 tokens at positions 0..4095,
40 query heads and 8 kv heads of 128, f32 q/k/v, f16 KV cache.  The value is
achieved HBM bandwidth in GB/s = algorithmic bytes per launch / mean launch
time, where the algorithmic bytes are

    per token : 2*(nqt + 2*nkt)*4   read and write back q, k, v
              + 2*nkt*cb            the K and V cache rows (cb = 2 for f16)
              + 4                   the position (+4 for a slot index)
    per launch: (nqt + 2*nkt)*4     the three biases

Input sets are rotated (each set has its own q/k/v and caches, together well
over the 256 MB last-level cache) so every launch reads its inputs from HBM.
Timing: HIP events on the launch stream around the timed launches.  Beside
that figure the line carries the p10/p50/p90 of single launches and the warm
figure (one input set reused).

Extra figures in the same line: the 256-sequence batched decode (f16 and f32
caches) in GB/s, decode microseconds per layer for the 7B and 14B decode steps
(stream loop and HIP-graph replay), the unfused seven-launch chain, the q/k-norm
variant, and the projection-fed epilogue (bf16 GEMM / GEMV with the epilogue in
its output stage) on the 14B prefill (TFLOP/s), the 14B one-token decode
(us per layer, GB/s of weight streaming) and a 48-layer decode step of it
(stream loop and HIP graph).  The CPU baseline is the oracle of
the unfused chain, single-threaded, timed on a bounded sample of the headline
workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "fused QKV epilogue achieved HBM GB/s (14B shape) + decode µs/layer"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algo_bytes(w, nt, cache_bytes, slot=False):
    per_tok = 2 * (w.nqt + 2 * w.nkt) * 4 + 2 * w.nkt * cache_bytes + 4 + (4 if slot else 0)
    return per_tok * nt + (w.nqt + 2 * w.nkt) * 4


def kernel_source_hash():
    """Hash of the fused kernel's sources (its file and the shared internals)."""
    h = hashlib.sha256()
    for f in ("qkv_epilogue.hip", "qkv_internal.h"):
        h.update(open(os.path.join(ROOT, "qkv_bias_rope_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def read_traffic(workload):
    """HBM traffic per launch from a committed rocprofv3 --pmc summary, if it
    was taken on the current kernel source (else None)."""
    p = os.path.join(ROOT, "profiles", f"pmc_qkv_epilogue_{workload}.txt")
    if not os.path.exists(p):
        return None
    vals = {}
    for line in open(p):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Sets:
    """R independent input sets of one workload on the device."""

    def __init__(self, w, R, cache_dtype, nt=None, share_cache=False, norm=False):
        import numpy as np
        import torch
        from qkv_bias_rope_amd import workloads as wl
        self.w = w
        self.nt = w.nt if nt is None else nt
        d = wl.draw_layer(w, 0, nt=self.nt)
        dev = "cuda:0"
        self.bq, self.bk, self.bv = (torch.from_numpy(d[n]).to(dev) for n in ("bq", "bk", "bv"))
        self.norm = norm
        if norm:   # the q/k-norm variant without biases (Qwen3-style attention)
            nw = wl.draw_norm_weights(w, 0)
            self.wq = torch.from_numpy(nw["wq"]).to(dev)
            self.wk = torch.from_numpy(nw["wk"]).to(dev)
            self.bq = self.bk = self.bv = None
        cdt = torch.float16 if cache_dtype == wl.CACHE_F16 else torch.float32
        rows = w.n_slots * w.n_ctx
        self.sets = []
        base = {n: torch.from_numpy(d[n]).to(dev) for n in ("q", "k", "v")}
        shared = None
        for r in range(R):
            s = {}
            for n in ("q", "k", "v"):
                s[n] = base[n].clone() if r else base[n]
            if w.pos_mode == "uniform":
                rng = np.random.default_rng(w.seed * 7919 + r)
                s["pos"] = torch.from_numpy(
                    rng.integers(0, w.n_ctx, size=self.nt, dtype=np.int32)).to(dev)
            else:
                s["pos"] = torch.from_numpy(d["pos"]).to(dev)
            s["slot"] = None if d["slot"] is None else torch.from_numpy(d["slot"]).to(dev)
            if share_cache and shared is not None:
                s["kc"], s["vc"] = shared
            else:
                s["kc"] = torch.empty((rows, w.nkt), dtype=cdt, device=dev)
                s["vc"] = torch.empty((rows, w.nkt), dtype=cdt, device=dev)
                shared = (s["kc"], s["vc"])
            self.sets.append(s)
        self.cache_dtype = cache_dtype

    def args(self, r, stream):
        from qkv_bias_rope_amd import binding as B
        s = self.sets[r % len(self.sets)]
        w = self.w
        return B.make_args(s["q"], s["k"], s["v"], self.bq, self.bk, self.bv, s["pos"], s["kc"],
                           s["vc"], n_head=w.n_head, n_kv_head=w.n_kv_head, head_dim=w.head_dim,
                           theta=w.theta, cache_dtype=self.cache_dtype, slot=s["slot"],
                           n_ctx=w.n_ctx, n_slots=w.n_slots, stream=stream, use_stream=True,
                           nt=self.nt)


def norm_runner(sets):
    """run_ex-shaped callable for the q/k-norm variant of a Sets."""
    from qkv_bias_rope_amd import binding as B
    from qkv_bias_rope_amd import workloads as wl
    return lambda h, a: B.qkv_epilogue_run_qk_norm(h, a, sets.wq, sets.wk, wl.QK_NORM_EPS)


def time_launches(h, arg_list, steps, warmup, stream, settle_s=0.3, fn=None):
    """Mean time per launch (ms) over `steps` launches cycling through
    arg_list, HIP events recorded on the launch stream.  Before the `warmup`
    untimed launches, the same launches run untimed for about settle_s
    seconds so the GPU clocks have ramped up when timing starts."""
    import torch
    from qkv_bias_rope_amd import binding as B
    run = fn or B.qkv_epilogue_run_ex
    t_end = time.perf_counter() + settle_s
    i = 0
    while time.perf_counter() < t_end:
        for _ in range(len(arg_list)):
            rc = run(h, arg_list[i % len(arg_list)])
            assert rc == 0, B.qkv_epilogue_last_error(h)
            i += 1
        torch.cuda.synchronize()
    for i in range(warmup):
        rc = run(h, arg_list[i % len(arg_list)])
        assert rc == 0, B.qkv_epilogue_last_error(h)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        run(h, arg_list[i % len(arg_list)])
    e1.record(stream)
    e1.synchronize()
    torch.cuda.synchronize()
    assert B.qkv_epilogue_status(h) == 0, B.qkv_epilogue_last_error(h)
    return e0.elapsed_time(e1) / steps


def launch_percentiles(h, arg_list, n, stream, fn=None):
    """p10 / p50 / p90 of single-launch durations (us): n launches cycling
    through arg_list, each bracketed by its own pair of events on the stream."""
    import torch
    from qkv_bias_rope_amd import binding as B
    run = fn or B.qkv_epilogue_run_ex
    pairs = []
    for i in range(n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        rc = run(h, arg_list[i % len(arg_list)])
        assert rc == 0, B.qkv_epilogue_last_error(h)
        e1.record(stream)
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in pairs)
    q = lambda f: us[min(len(us) - 1, int(f * (len(us) - 1) + 0.5))]
    return dict(p10=round(q(0.1), 3), p50=round(q(0.5), 3), p90=round(q(0.9), 3), launches=n)


def bench_bandwidth(h, w, cache_dtype, steps, warmup, stream, min_set_bytes=1.5e9, slot=False,
                    fn=None, norm=False, rope_style=0, freq_scale=0.0):
    from qkv_bias_rope_amd import workloads as wl
    cb = 2 if cache_dtype == wl.CACHE_F16 else 4
    nbytes = algo_bytes(w, w.nt, cb, slot=slot)
    if norm:   # no biases; the two [head_dim] norm weights instead
        nbytes += 2 * w.head_dim * 4 - (w.nqt + 2 * w.nkt) * 4
    per_set = w.nt * (w.nqt + 2 * w.nkt) * 4 * 2
    R = max(2, int(-(-min_set_bytes // per_set)))
    # big caches (batched decode) are shared by the sets: their rows are written
    # at random positions, so a shared cache gets no reuse anyway
    share = w.n_slots > 1
    sets = Sets(w, R, cache_dtype, share_cache=share, norm=norm)
    args = [sets.args(r, stream) for r in range(R)]
    for a in args:
        a.rope_style, a.freq_scale = rope_style, freq_scale
    if norm:
        fn = norm_runner(sets)
    ms = time_launches(h, args, steps, warmup, stream, fn=fn)
    return dict(ms=ms, bytes=nbytes, gbs=nbytes / (ms * 1e-3) / 1e9, sets=R), sets


def bench_decode(h, w, steps, warmup, stream, unfused=False):
    """One decode step = one fused launch per layer (or, with unfused=True, the
    seven-launch unfused chain per layer).  Returns microseconds per layer for a
    plain stream loop and for a HIP-graph replay of the whole step."""
    import torch
    from qkv_bias_rope_amd import binding as B
    from qkv_bias_rope_amd import workloads as wl
    layers = []
    for layer in range(w.layers):
        s = Sets(w, 1, w.cache_dtypes[0])
        if w.concat_even_layers and layer % 2 == 0:
            # one [nqt + 2*nkt] row holding the three sections
            buf = torch.cat([s.sets[0]["q"], s.sets[0]["k"], s.sets[0]["v"]], dim=1).contiguous()
            s.sets[0]["q"] = buf[:, :w.nqt]
            s.sets[0]["k"] = buf[:, w.nqt:w.nqt + w.nkt]
            s.sets[0]["v"] = buf[:, w.nqt + w.nkt:]
            s.buf = buf
        layers.append(s)
    args = [s.args(0, stream) for s in layers]
    run = B.qkv_epilogue_run_unfused if unfused else B.qkv_epilogue_run_ex
    n_loops = max(1, steps)
    # stream loop
    ms_step = time_launches(h, args, n_loops * w.layers, warmup * w.layers, stream,
                            fn=run) * w.layers
    cb = 2 if w.cache_dtypes[0] == wl.CACHE_F16 else 4
    res = dict(us_per_layer_stream=ms_step * 1e3 / w.layers,
               launches_per_layer=7 if unfused else 1,
               bytes_per_layer=algo_bytes(w, 1, cb), layers=w.layers)
    if w.layers == 1:
        # a one-kernel graph would time the graph launch, not the layer
        assert B.qkv_epilogue_status(h) == 0
        return res
    # graph replay of one step
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for a in args:
            a.stream = torch.cuda.current_stream().cuda_stream
            assert run(h, a) == 0
    t_end = time.perf_counter() + 0.2
    while time.perf_counter() < t_end:
        g.replay()
        torch.cuda.synchronize()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    cur = torch.cuda.current_stream()
    e0.record(cur)
    for _ in range(n_loops):
        g.replay()
    e1.record(cur)
    e1.synchronize()
    ms_graph = e0.elapsed_time(e1) / n_loops
    assert B.qkv_epilogue_status(h) == 0
    res["us_per_layer_graph"] = ms_graph * 1e3 / w.layers
    return res


PEAK_BF16_TFLOPS = 2500.0


class ProjSets:
    """Input sets of the projection-fed epilogue: bf16 activations and concat
    weights (bf16, or E4M3 codes with f32 row scales), f32 q/k/v outputs and
    the caches, R copies rotated so that the weights and activations come from
    HBM on every launch."""

    def __init__(self, w, hidden, R, cache_dtype, nt=None, wfmt="bf16"):
        import numpy as np
        import torch
        from qkv_bias_rope_amd import workloads as wl
        dev = "cuda:0"
        d = wl.draw_projection(w, hidden, nt=nt)
        self.w, self.hidden, self.cd = w, hidden, cache_dtype
        self.nt = int(d["pos"].size)
        cdt = torch.float16 if cache_dtype == wl.CACHE_F16 else torch.float32
        x = torch.from_numpy(d["x"].view(np.int16)).to(dev)
        self.wfmt = wfmt
        self.scale = None
        if wfmt == "e4m3":
            codes, scale = wl.draw_e4m3_weights(w.nqt + 2 * w.nkt, hidden, w.seed)
            wt = torch.from_numpy(codes).to(dev)
            self.scale = torch.from_numpy(scale).to(dev)
        else:
            wt = torch.from_numpy(d["w"].view(np.int16)).to(dev)
        self.b = [torch.from_numpy(d[n]).to(dev) for n in ("bq", "bk", "bv")]
        pos = torch.from_numpy(d["pos"]).to(dev)
        slot = None if d["slot"] is None else torch.from_numpy(d["slot"]).to(dev)
        rows = w.n_slots * w.n_ctx
        # one K/V cache pair shared by the sets (the 256-slot cache is 17 GB;
        # its rows land at random positions, so sharing gives no reuse)
        kc = torch.empty((rows, w.nkt), dtype=cdt, device=dev)
        vc = torch.empty((rows, w.nkt), dtype=cdt, device=dev)
        self.sets = []
        for r in range(R):
            self.sets.append(dict(
                x=x.clone() if r else x, w=wt.clone() if r else wt, pos=pos, slot=slot,
                q=torch.empty((self.nt, w.nqt), device=dev),
                k=torch.empty((self.nt, w.nkt), device=dev),
                v=torch.empty((self.nt, w.nkt), device=dev), kc=kc, vc=vc))

    def args(self, r, stream):
        from qkv_bias_rope_amd import binding as B
        s, w = self.sets[r % len(self.sets)], self.w
        epi = B.make_args(s["q"], s["k"], s["v"], *self.b, s["pos"], s["kc"], s["vc"],
                          n_head=w.n_head, n_kv_head=w.n_kv_head, head_dim=w.head_dim,
                          theta=w.theta, cache_dtype=self.cd, slot=s["slot"], n_ctx=w.n_ctx,
                          n_slots=w.n_slots, stream=stream, use_stream=True, nt=self.nt)
        if self.wfmt == "e4m3":
            return B.make_proj_args(s["x"], s["w"], self.hidden, epi, w_format=B.QKV_WEIGHT_E4M3,
                                    w_scale=self.scale)
        return B.make_proj_args(s["x"], s["w"], self.hidden, epi)


def proj_bytes(w, nt, hidden, cb, wfmt="bf16"):
    """Algorithmic HBM bytes of one projection-fed launch: x and W once (and
    the row scales of E4M3 weights), the q/k/v rows written, the K/V cache
    rows, positions and biases."""
    n = w.nqt + 2 * w.nkt
    wbytes = n * hidden + n * 4 if wfmt == "e4m3" else n * hidden * 2
    return (nt * hidden * 2 + wbytes + nt * n * 4 + 2 * nt * w.nkt * cb + nt * 4
            + n * 4)


def bench_proj(h, w, hidden, steps, warmup, stream, min_set_bytes=1.5e9, nt=None, wfmt="bf16"):
    """Projection-fed epilogue (one launch: GEMM/GEMV + epilogue)."""
    import torch
    from qkv_bias_rope_amd import binding as B
    from qkv_bias_rope_amd import workloads as wl
    cd = w.cache_dtypes[0]
    cb = 2 if cd == wl.CACHE_F16 else 4
    nt = w.nt if nt is None else nt
    n = w.nqt + 2 * w.nkt
    per_set = nt * hidden * 2 + n * hidden * (1 if wfmt == "e4m3" else 2) + nt * n * 4
    R = max(2, int(-(-min_set_bytes // per_set)))
    sets = ProjSets(w, hidden, R, cd, nt=nt, wfmt=wfmt)
    args = [sets.args(r, stream) for r in range(R)]
    ms = time_launches(h, args, steps, warmup, stream, fn=B.qkv_epilogue_run_proj)
    flops = 2.0 * nt * n * hidden
    nbytes = proj_bytes(w, nt, hidden, cb, wfmt)
    res = dict(us_per_launch=ms * 1e3, tflops=flops / (ms * 1e-3) / 1e12,
               gbs=nbytes / (ms * 1e-3) / 1e9, flops=flops, bytes=nbytes, sets=R)
    if wfmt == "e4m3":
        del sets
        torch.cuda.empty_cache()
        return res
    # reference: torch's bf16 matmul of the same shape (library GEMM, bf16 out,
    # no epilogue), event-timed per call over the same rotating input sets so
    # its operands come from HBM too; host overhead included
    xw = [(d["x"].view(torch.bfloat16), d["w"].view(torch.bfloat16).t()) for d in sets.sets]
    ys = [torch.empty(nt, n, dtype=torch.bfloat16, device=xw[0][0].device) for _ in xw]
    with torch.cuda.stream(stream):
        for i in range(max(5, len(xw))):
            torch.matmul(*xw[i % len(xw)], out=ys[i % len(xw)])
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        k = max(5, steps // 2)
        e0.record(stream)
        for i in range(k):
            torch.matmul(*xw[i % len(xw)], out=ys[i % len(xw)])
        e1.record(stream)
        e1.synchronize()
    res["library_bf16_matmul_call_us"] = e0.elapsed_time(e1) / k * 1e3
    del sets, xw, ys
    torch.cuda.empty_cache()
    return res


def bench_proj_decode(h, w, hidden, steps, warmup, stream, wfmt="bf16"):
    """A decode step of the projection-fed epilogue: one token, one launch per
    layer, every layer with its own weights (48 x 73 MB at 14B, so each step
    streams them from HBM).  Microseconds per layer for a stream loop and for a
    HIP-graph replay of the whole step."""
    import torch
    from qkv_bias_rope_amd import binding as B
    layers = [ProjSets(w, hidden, 1, w.cache_dtypes[0], nt=1, wfmt=wfmt) for _ in range(w.layers)]
    args = [ls.args(0, stream) for ls in layers]
    n_loops = max(1, steps)
    ms_step = time_launches(h, args, n_loops * w.layers, warmup * w.layers, stream,
                            fn=B.qkv_epilogue_run_proj) * w.layers
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for a in args:
            a.epi.stream = torch.cuda.current_stream().cuda_stream
            assert B.qkv_epilogue_run_proj(h, a) == 0
    for _ in range(max(1, warmup)):
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    cur = torch.cuda.current_stream()
    e0.record(cur)
    for _ in range(n_loops):
        g.replay()
    e1.record(cur)
    e1.synchronize()
    ms_graph = e0.elapsed_time(e1) / n_loops
    assert B.qkv_epilogue_status(h) == 0
    del layers, args, g
    torch.cuda.empty_cache()
    return dict(us_per_layer_stream=ms_step * 1e3 / w.layers,
                us_per_layer_graph=ms_graph * 1e3 / w.layers, layers=w.layers)


def cpu_baseline(w, cache_dtype, budget_s=10.0):
    """The oracle (single-threaded C, unfused chain) on the headline workload,
    repeated over whole launches until about budget_s seconds have passed."""
    import numpy as np
    import oracle
    from qkv_bias_rope_amd import workloads as wl
    d = wl.draw_layer(w, 0)
    cb = 2 if cache_dtype == wl.CACHE_F16 else 4
    n = 0
    t0 = time.perf_counter()
    while True:
        q, k, v = (d[x].copy() for x in ("q", "k", "v"))
        ts = time.perf_counter()
        oracle.qkv_epilogue(q.ravel(), k.ravel(), v.ravel(), d["bq"], d["bk"], d["bv"], d["pos"],
                            n_head=w.n_head, n_kv_head=w.n_kv_head, head_dim=w.head_dim,
                            theta=w.theta, n_ctx=w.n_ctx, cache_dtype=cache_dtype,
                            slot=d["slot"], n_slots=w.n_slots)
        n += 1
        if n == 1:
            spent = time.perf_counter() - ts
        else:
            spent += time.perf_counter() - ts
        if time.perf_counter() - t0 >= budget_s:
            break
    s_per = spent / n
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), cpu)
    except OSError:
        pass
    return dict(value=algo_bytes(w, w.nt, cb) / s_per / 1e9, unit="GB/s", cores=1, kind="oracle",
                sample=f"{n} full launch(es) of {w.name} ({w.nt} tokens, f16 cache) on 1 host "
                       f"thread, {s_per:.3f} s each", cpu=cpu)


def hbm_ceiling(steps, stream, nbytes=251703296, sets=8):
    """A practical HBM ceiling on the same box: torch's in-place add over
    buffers that move the headline launch's bytes (half read, half written),
    rotated over `sets` buffers so they come from HBM.  Event-timed per call."""
    import torch
    n = nbytes // 8                                   # float32 elements per buffer
    bufs = [torch.ones(n, dtype=torch.float32, device="cuda:0") for _ in range(sets)]
    with torch.cuda.stream(stream):
        for i in range(2 * sets):
            bufs[i % sets].add_(1.0)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            bufs[i % sets].add_(1.0)
        e1.record(stream)
        e1.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del bufs
    torch.cuda.empty_cache()
    return dict(us_per_call=round(ms * 1e3, 3), gbs=round(n * 8 / (ms * 1e-3) / 1e9, 1), bytes=n * 8)


def copy_calibration(steps):
    """A plain device copy of known size (for scaling FETCH_SIZE/WRITE_SIZE)."""
    import torch
    n = 256 * 1024 * 1024  # float32 elements = 1 GiB
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4,
                      "launches": steps}))


PROJ_SWEEP_TOKENS = (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096)


def proj_sweep(args):
    """The projection-fed epilogue over token counts, each launch event-timed
    with rotating input sets (weights from HBM on every launch)."""
    import torch
    from qkv_bias_rope_amd import binding as B
    from qkv_bias_rope_amd import workloads as wl
    rc, h = B.qkv_epilogue_create(0, 4096)
    assert rc == 0, rc
    stream = torch.cuda.Stream()
    w = wl.Workload("proj_sweep_14b", 40, 8, 128, nt=1, n_ctx=4096, n_slots=1, layers=1, seed=30)
    hidden = 5120
    with torch.cuda.stream(stream):
        for nt in PROJ_SWEEP_TOKENS:
            steps = args.steps if nt <= 512 else max(10, args.steps // 5)
            r = bench_proj(h, w, hidden, steps, args.warmup, stream, min_set_bytes=1.0e9, nt=nt)
            print(json.dumps({"proj_sweep_tokens": nt, "hidden": hidden,
                              "us_per_launch": round(r["us_per_launch"], 2),
                              "tflops": round(r["tflops"], 1), "gbs": round(r["gbs"], 1),
                              "library_bf16_matmul_call_us": round(r["library_bf16_matmul_call_us"], 2)}),
                  flush=True)
    B.qkv_epilogue_destroy(h)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-extra", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calib", action="store_true",
                    help="run only a 1 GiB device copy (counter calibration)")
    ap.add_argument("--proj-sweep", action="store_true",
                    help="run only the projection-fed epilogue at 1..4096 tokens (14B width, "
                         "hidden 5120), one JSON line per token count")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported (the epilogue "
              "needs no collective: each GPU would run the same kernels on its own share of the "
              "tokens, or of the heads with their biases and cache columns)", file=sys.stderr)
        sys.exit(2)

    import torch
    from qkv_bias_rope_amd import build as _b
    if not os.path.exists(_b.LIB):
        _b.build()
    from qkv_bias_rope_amd import binding as B
    from qkv_bias_rope_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calib:
        copy_calibration(args.steps)
        return
    if args.proj_sweep:
        proj_sweep(args)
        return

    rc, h = B.qkv_epilogue_create(0, 4096)
    assert rc == 0, rc
    # all work on one non-default stream (a HIP graph cannot capture the null stream)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        line = run_all(args, h, stream)
    B.qkv_epilogue_destroy(h)
    print(json.dumps(line), flush=True)


def run_all(args, h, stream):
    import torch
    from qkv_bias_rope_amd import binding as B
    from qkv_bias_rope_amd import workloads as wl

    w = wl.PREFILL_14B
    log(f"[bench] {w.name}: {args.warmup} warmup + {args.steps} timed launches")
    main_res, sets = bench_bandwidth(h, w, wl.CACHE_F16, args.steps, args.warmup, stream)
    log(f"[bench] {w.name}: {main_res['ms'] * 1e3:.2f} us/launch, {main_res['gbs']:.1f} GB/s")
    extra = {}
    if not args.no_extra:
        # the distribution of single launches over the same rotated sets, and
        # the warm figure: one input set reused (252 MB, partly resident in the
        # 256 MB last-level cache between launches)
        arg_list = [sets.args(r, stream) for r in range(len(sets.sets))]
        extra[w.name + "_per_launch_us"] = launch_percentiles(h, arg_list, 60, stream)
        warm_ms = time_launches(h, arg_list[:1], args.steps, args.warmup, stream)
        extra[w.name + "_warm"] = dict(us_per_launch=round(warm_ms * 1e3, 3),
                                       gbs=round(main_res["bytes"] / (warm_ms * 1e-3) / 1e9, 1))
        log(f"[bench]   per launch {extra[w.name + '_per_launch_us']}, warm "
            f"{extra[w.name + '_warm']}")
    del sets
    torch.cuda.empty_cache()
    if not args.no_extra:
        extra["hbm_ceiling_inplace_add"] = hbm_ceiling(args.steps, stream)
        log(f"[bench] HBM ceiling (in-place add of the same bytes): {extra['hbm_ceiling_inplace_add']}")

    if not args.no_extra:
        wb = wl.BATCHED_DECODE_14B
        for cd, tag in ((wl.CACHE_F16, "f16"), (wl.CACHE_F32, "f32")):
            log(f"[bench] {wb.name} {tag}")
            r, sets = bench_bandwidth(h, wb, cd, args.steps, args.warmup, stream,
                                      min_set_bytes=1.0e9, slot=True)
            del sets
            torch.cuda.empty_cache()
            extra[f"{wb.name}_{tag}"] = dict(
                gbs=round(r["gbs"], 1), us_per_launch=round(r["ms"] * 1e3, 3),
                bytes_per_launch=r["bytes"], frac_of_peak=round(r["gbs"] / PEAK_HBM_GBS, 4),
                input_sets=r["sets"])
            log(f"[bench]   {r['ms'] * 1e3:.2f} us/launch, {r['gbs']:.1f} GB/s")
        for wd in (wl.TINY_DECODE, wl.DECODE_7B, wl.DECODE_14B):
            log(f"[bench] {wd.name}")
            r = bench_decode(h, wd, max(10, args.steps // 10), max(2, args.warmup // 10), stream)
            extra[wd.name] = {k: (round(v, 3) if isinstance(v, float) else v) for k, v in r.items()}
            log(f"[bench]   {r['us_per_layer_stream']:.2f} us/layer (stream), "
                f"{r.get('us_per_layer_graph', float('nan')):.2f} us/layer (graph)")
            torch.cuda.empty_cache()
        # same-binary A/B of the fusion: the unfused seven-launch chain
        wd = wl.DECODE_14B
        log(f"[bench] {wd.name} unfused chain")
        r = bench_decode(h, wd, max(10, args.steps // 10), max(2, args.warmup // 10), stream,
                         unfused=True)
        extra[wd.name + "_unfused"] = {k: (round(v, 3) if isinstance(v, float) else v)
                                       for k, v in r.items()}
        log(f"[bench]   {r['us_per_layer_stream']:.2f} us/layer (stream), "
            f"{r['us_per_layer_graph']:.2f} us/layer (graph)")
        torch.cuda.empty_cache()
        log(f"[bench] {w.name} unfused chain")
        r, sets = bench_bandwidth(h, w, wl.CACHE_F16, max(20, args.steps // 4),
                                  max(2, args.warmup // 4), stream, fn=B.qkv_epilogue_run_unfused)
        del sets
        torch.cuda.empty_cache()
        extra[w.name + "_unfused"] = dict(gbs=round(r["gbs"], 1),
                                          us_per_launch_chain=round(r["ms"] * 1e3, 3),
                                          launches=7)
        log(f"[bench]   {r['ms'] * 1e3:.2f} us per 7-launch chain, {r['gbs']:.1f} GB/s")
        # the q/k-norm variant (no biases, per-head RMS norm before the rope)
        log(f"[bench] {w.name} q/k-norm variant")
        r, sets = bench_bandwidth(h, w, wl.CACHE_F16, max(20, args.steps // 2),
                                  max(2, args.warmup // 2), stream, norm=True)
        del sets
        torch.cuda.empty_cache()
        extra[w.name + "_qk_norm"] = dict(gbs=round(r["gbs"], 1), us_per_launch=round(r["ms"] * 1e3, 3),
                                          bytes_per_launch=r["bytes"],
                                          frac_of_peak=round(r["gbs"] / PEAK_HBM_GBS, 4))
        log(f"[bench]   {r['ms'] * 1e3:.2f} us/launch, {r['gbs']:.1f} GB/s")
        # the rope variants on the same workload: interleaved (GPT-J) pairing,
        # and NeoX with a frequency scale
        for tag, style, fs in (("interleaved", 1, 0.0), ("freq_scale_0.25", 0, 0.25)):
            log(f"[bench] {w.name} rope {tag}")
            r, sets = bench_bandwidth(h, w, wl.CACHE_F16, max(20, args.steps // 2),
                                      max(2, args.warmup // 2), stream, rope_style=style, freq_scale=fs)
            del sets
            torch.cuda.empty_cache()
            extra[w.name + "_rope_" + tag] = dict(gbs=round(r["gbs"], 1), us_per_launch=round(r["ms"] * 1e3, 3),
                                                  bytes_per_launch=r["bytes"],
                                                  frac_of_peak=round(r["gbs"] / PEAK_HBM_GBS, 4))
            log(f"[bench]   {r['ms'] * 1e3:.2f} us/launch, {r['gbs']:.1f} GB/s")
        # the projection feeding the epilogue, fused into one launch
        hid = wl.HIDDEN[w.name]
        log(f"[bench] {w.name} projection-fed epilogue (hidden {hid})")
        r = bench_proj(h, w, hid, max(20, args.steps // 2), max(2, args.warmup // 4), stream,
                       min_set_bytes=1.0e9)
        extra[w.name + "_proj"] = dict(
            us_per_launch=round(r["us_per_launch"], 2), tflops=round(r["tflops"], 1),
            frac_of_bf16_peak=round(r["tflops"] / PEAK_BF16_TFLOPS, 4), hidden=hid,
            library_bf16_matmul_call_us=round(r["library_bf16_matmul_call_us"], 2),
            input_sets=r["sets"])
        log(f"[bench]   {r['us_per_launch']:.1f} us/launch, {r['tflops']:.1f} TFLOP/s "
            f"(library bf16 matmul call {r['library_bf16_matmul_call_us']:.1f} us)")
        wd = wl.DECODE_14B
        hid = wl.HIDDEN[wd.name]
        log(f"[bench] {wd.name} projection-fed epilogue, one token (hidden {hid})")
        r = bench_proj(h, wd, hid, max(50, args.steps // 2), max(5, args.warmup // 2), stream,
                       min_set_bytes=1.5e9)
        extra[wd.name + "_proj"] = dict(
            us_per_layer=round(r["us_per_launch"], 2), gbs=round(r["gbs"], 1),
            frac_of_peak=round(r["gbs"] / PEAK_HBM_GBS, 4), bytes_per_layer=r["bytes"],
            hidden=hid, library_bf16_matmul_call_us=round(r["library_bf16_matmul_call_us"], 2),
            input_sets=r["sets"])
        log(f"[bench]   {r['us_per_launch']:.1f} us/layer, {r['gbs']:.1f} GB/s "
            f"(library bf16 matmul call {r['library_bf16_matmul_call_us']:.1f} us)")
        log(f"[bench] {wd.name} projection-fed epilogue, {wd.layers}-layer decode step")
        r = bench_proj_decode(h, wd, hid, max(5, args.steps // 20), 2, stream)
        extra[wd.name + "_proj_step"] = {k: (round(v, 3) if isinstance(v, float) else v)
                                         for k, v in r.items()}
        log(f"[bench]   {r['us_per_layer_stream']:.2f} us/layer (stream), "
            f"{r['us_per_layer_graph']:.2f} us/layer (graph)")
        # the same decode with E4M3 weights and row scales (half the weight bytes)
        log(f"[bench] {wd.name} projection-fed epilogue, one token, E4M3 weights")
        r = bench_proj(h, wd, hid, max(50, args.steps // 2), max(5, args.warmup // 2), stream,
                       min_set_bytes=1.5e9, wfmt="e4m3")
        extra[wd.name + "_proj_e4m3"] = dict(
            us_per_layer=round(r["us_per_launch"], 2), gbs=round(r["gbs"], 1),
            frac_of_peak=round(r["gbs"] / PEAK_HBM_GBS, 4), bytes_per_layer=r["bytes"],
            hidden=hid, input_sets=r["sets"])
        log(f"[bench]   {r['us_per_launch']:.1f} us/layer, {r['gbs']:.1f} GB/s")
        r = bench_proj_decode(h, wd, hid, max(5, args.steps // 20), 2, stream, wfmt="e4m3")
        extra[wd.name + "_proj_e4m3_step"] = {k: (round(v, 3) if isinstance(v, float) else v)
                                              for k, v in r.items()}
        log(f"[bench]   {r['us_per_layer_stream']:.2f} us/layer (stream), "
            f"{r['us_per_layer_graph']:.2f} us/layer (graph)")

    cpu = None
    if not args.no_cpu:
        log("[bench] CPU oracle baseline")
        cpu = cpu_baseline(w, wl.CACHE_F16)
        cpu["value"] = round(cpu["value"], 4)
        log(f"[bench]   {cpu['value']} GB/s")

    traffic = read_traffic(w.name)
    achieved = main_res["gbs"]
    line = {
        "metric": METRIC,
        "value": round(achieved, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,1) q/k/v, N(0,0.1) biases)",
        "config": {"workload": w.name, "n_head": w.n_head, "n_kv_head": w.n_kv_head,
                   "head_dim": w.head_dim, "tokens": w.nt, "positions": "0..4095",
                   "cache": "f16", "theta": w.theta, "input_sets_rotated": main_res["sets"],
                   "bytes_per_launch": main_res["bytes"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    return line


if __name__ == "__main__":
    main()
