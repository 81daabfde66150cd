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

Reference points measured in the same run with the probe library
(libqkv_probe.so, not part of the epilogue):
  * ceiling: the best bare in-place add and copy of the prefill launch's bytes
    over rotating buffers (swept over store policy and vectors per thread) --
    "frac_of_achievable" is the epilogue's rate over the better of the two --
    and the row pass of the prefill's own byte pattern (rows read and written
    back, the cache rows at the tokens' positions); "frac_of_fastest_bare_pass"
    is the epilogue's rate over the fastest of all three;
  * the 256-sequence decode (f16 and f32 caches) is timed on the GPU side: 256
    launches over 64 rotating input sets captured in one HIP graph and
    replayed, beside a bare row pass that moves the same bytes from the same
    sets into the same caches, and an empty kernel of the same launch shape;
  * the empty-kernel floor of each decode launch shape, beside the decode
    microseconds per layer (7B, 14B and the tiny decode; stream loop and
    HIP-graph replay of a whole step).
Also: the unfused seven-launch chain, the q/k-norm variant, the rope variants,
and the projection-fed epilogue (bf16 GEMM / GEMV with the epilogue in its
output stage) on the 14B prefill (TFLOP/s), the 14B one-token decode and a
48-layer decode step of it.  The CPU baseline is the oracle of the unfused
chain on the host cores, every configuration, one thread and a thread pool over
token chunks; the headline's pool figure is `cpu_baseline`.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu]
       python bench.py --batched-only | --copy-calib | --proj-sweep
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


def time_graph(launch, n_launch, replays, stream, warm_replays=2):
    """Microseconds per launch of `launch(i)` (i = 0..n_launch-1) captured
    into one HIP graph on `stream` and replayed `replays` times between two
    events on the same stream: the GPU-side rate of back-to-back launches,
    with no host issue in the timed region (each launch still waits for the
    previous one, as consecutive layers do)."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(n_launch):
            rc = launch(i)
            assert rc == 0, rc
    with torch.cuda.stream(stream):
        t_end = time.perf_counter() + 0.2
        while time.perf_counter() < t_end:
            g.replay()
            torch.cuda.synchronize()
        for _ in range(warm_replays):
            g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(replays):
            g.replay()
        e1.record(stream)
        e1.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (n_launch * replays)
    del g
    return us


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


def bench_batched(h, w, cache_dtype, stream, n_launch=256, replays=4, R=64):
    """The 256-sequence decode, GPU side: `n_launch` launches over R rotating
    input sets (~470 MB of q/k/v, beyond the 256 MB last-level cache; one
    shared cache pair, written at fresh random rows by every set) captured in
    a HIP graph and replayed.  Beside it, on the same sets, positions and
    caches: the probe library's row pass that moves the same bytes from
    concat [nt][nqt+2nkt] copies of the rows (the bare pass; best over tokens
    per workgroup and store policy, and at one token per workgroup like the
    epilogue), the epilogue itself on those concat rows, the in-place add of
    the q/k/v alone, and an empty kernel of the epilogue's launch shape."""
    import torch
    from qkv_bias_rope_amd import binding as B
    from qkv_bias_rope_amd import probe as P
    from qkv_bias_rope_amd import workloads as wl
    cb = 2 if cache_dtype == wl.CACHE_F16 else 4
    nbytes = algo_bytes(w, w.nt, cb, slot=True)
    sets = Sets(w, R, cache_dtype, share_cache=True)
    args = [sets.args(r, stream) for r in range(R)]
    run = B.qkv_epilogue_run_ex
    ep_us = time_graph(lambda i: run(h, args[i % R]), n_launch, replays, stream)
    loop_ms = time_launches(h, args, n_launch, 32, stream)
    assert B.qkv_epilogue_status(h) == 0, B.qkv_epilogue_last_error(h)
    rc, plan = B.qkv_epilogue_plan(args[0])
    assert rc == 0
    # the same bytes through the bare row pass: concat copies of the sets' rows
    xs = [torch.cat([st["q"], st["k"], st["v"]], dim=1).contiguous() for st in sets.sets]
    bcat = torch.cat([sets.bq, sets.bk, sets.bv]).contiguous()
    kc, vc = sets.sets[0]["kc"], sets.sets[0]["vc"]
    # the epilogue on that concat layout too (q|k|v sections of one row)
    cargs = []
    for r in range(R):
        x, st = xs[r], sets.sets[r]
        cargs.append(B.make_args(x[:, :w.nqt], x[:, w.nqt:w.nqt + w.nkt], x[:, w.nqt + w.nkt:], sets.bq,
                                 sets.bk, sets.bv, st["pos"], kc, vc, n_head=w.n_head,
                                 n_kv_head=w.n_kv_head, head_dim=w.head_dim, theta=w.theta,
                                 cache_dtype=cache_dtype, slot=st["slot"], n_ctx=w.n_ctx,
                                 n_slots=w.n_slots, stream=stream, use_stream=True))
    cat_us = time_graph(lambda i: run(h, cargs[i % R]), n_launch, replays, stream)
    assert B.qkv_epilogue_status(h) == 0, B.qkv_epilogue_last_error(h)
    rows = []
    for tpb in (1, 2, 4):
        for pol in (1, 2, 3):
            us = time_graph(lambda i, tpb=tpb, pol=pol: P.rows(
                xs[i % R], bcat, w.nqt, w.nkt, sets.sets[i % R]["pos"], sets.sets[i % R]["slot"],
                w.n_ctx, kc, vc, block=256, tpb=tpb, policy=pol, stream=stream), n_launch, replays, stream)
            rows.append(dict(tokens_per_workgroup=tpb, policy=pol, us=round(us, 3),
                             gbs=round(nbytes / us / 1e3, 1)))
    adds = []
    for pol in (1, 2, 3):
        us = time_graph(lambda i, pol=pol: P.add(xs[i % R], 256, 1, pol, stream), n_launch, replays,
                        stream)
        adds.append(dict(policy=pol, us=round(us, 3)))
    empty_us = time_graph(lambda i: P.empty(int(plan.grid), int(plan.block), stream), n_launch,
                          replays, stream)
    bare = _best(rows)
    bare1 = _best([r for r in rows if r["tokens_per_workgroup"] == 1])
    gbs = nbytes / ep_us / 1e3
    res = dict(us_per_launch=round(ep_us, 3), gbs=round(gbs, 1),
               frac_of_peak=round(gbs / PEAK_HBM_GBS, 4),
               bare_pass_us=bare["us"], bare_pass_gbs=bare["gbs"],
               frac_of_achievable=round(bare["us"] / ep_us, 4),
               bare_pass_one_token_per_workgroup_us=bare1["us"],
               concat_layout_us_per_launch=round(cat_us, 3),
               concat_layout_frac_of_bare_pass_one_token=round(bare1["us"] / cat_us, 4),
               inplace_add_qkv_only_us=_best(adds)["us"],
               empty_kernel_same_launch_us=round(empty_us, 3),
               stream_loop_us_per_launch=round(loop_ms * 1e3, 3),
               launch=dict(grid=int(plan.grid), block=int(plan.block)),
               bytes_per_launch=nbytes, input_sets=R, graph_launches=n_launch,
               graph_replays=replays, bare_pass_sweep=rows)
    del sets, args, xs, cargs
    torch.cuda.empty_cache()
    return res


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


def cpu_threads():
    """Host threads for the oracle's parallel leg: the cores this process may
    run on, capped by OMP_NUM_THREADS when set (the share of a shared host)."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            return next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")),
                        "unknown")
    except OSError:
        return "unknown"


def oracle_launch_s(w, d, cache_dtype, threads, budget_s):
    """Seconds per launch of the oracle's unfused chain on one launch's inputs
    (q/k/v copied fresh before each timed call), repeated for about budget_s.
    With threads > 1 the tokens are split into contiguous chunks, one oracle
    call each, run by a thread pool: the chain is unchanged (tokens are
    independent and ctypes releases the interpreter lock during the call)."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    nt = int(d["pos"].size)
    chunks = [(a, min(nt, a + -(-nt // threads))) for a in range(0, nt, -(-nt // threads))]

    def one(q, k, v, a, b):
        oracle.qkv_epilogue(q[a:b].ravel(), k[a:b].ravel(), v[a:b].ravel(), d["bq"], d["bk"],
                            d["bv"], d["pos"][a:b], n_head=w.n_head, n_kv_head=w.n_kv_head,
                            head_dim=w.head_dim, theta=w.theta, n_ctx=w.n_ctx,
                            cache_dtype=cache_dtype,
                            slot=None if d["slot"] is None else d["slot"][a:b],
                            n_slots=w.n_slots)

    pool = ThreadPoolExecutor(threads) if len(chunks) > 1 else None
    n, spent = 0, 0.0
    t_end = time.perf_counter() + budget_s
    while True:
        q, k, v = (d[x].copy() for x in ("q", "k", "v"))
        ts = time.perf_counter()
        if pool is None:
            one(q, k, v, 0, nt)
        else:
            list(pool.map(lambda c: one(q, k, v, *c), chunks))
        spent += time.perf_counter() - ts
        n += 1
        if time.perf_counter() >= t_end and n >= 3:
            break
    if pool is not None:
        pool.shutdown()
    return spent / n, n


def cpu_oracle_all(budget_s=3.0):
    """The oracle on the host cores, every configuration: one thread, and a
    thread pool over token chunks (batched launches only).  Microseconds per
    launch (per layer for the decode shapes) and GB/s by the same byte count
    as the GPU.  The 256-sequence decode keeps only the 256 written rows
    (the oracle returns the rows; no cache is allocated)."""
    from qkv_bias_rope_amd import workloads as wl
    nthr = cpu_threads()
    out = {"cpu": cpu_model(), "affinity_cores": len(os.sched_getaffinity(0)),
           "threads_parallel": nthr}
    for w in wl.ALL:
        for cd in w.cache_dtypes:
            cb = 2 if cd == wl.CACHE_F16 else 4
            nbytes = algo_bytes(w, w.nt, cb, slot=w.n_slots > 1)
            d = wl.draw_layer(w, 0)
            tag = w.name + ("" if len(w.cache_dtypes) == 1 else ("_f16" if cd == wl.CACHE_F16 else "_f32"))
            s1, n1 = oracle_launch_s(w, d, cd, 1, budget_s)
            r = dict(us_per_launch_1thread=round(s1 * 1e6, 2), gbs_1thread=round(nbytes / s1 / 1e9, 4),
                     launches_1thread=n1, bytes_per_launch=nbytes)
            if w.nt > 1:
                sn, nn = oracle_launch_s(w, d, cd, nthr, budget_s)
                r.update(us_per_launch_nthread=round(sn * 1e6, 2),
                         gbs_nthread=round(nbytes / sn / 1e9, 4), launches_nthread=nn)
            out[tag] = r
            log(f"[bench]   oracle {tag}: {r}")
    return out


def _best(results, key="us"):
    return min(results, key=lambda r: r[key])


def ceilings_prefill(steps, stream, nbytes=251703296, sets=8):
    """What a bare streaming pass achieves for the prefill launch's bytes on
    this device: the probe library's in-place add (half read, half written,
    like the epilogue's q/k/v) and copy, each over `sets` rotating buffers so
    every launch comes from HBM, swept over store policy and vectors per
    thread; event-timed over a stream loop like the headline."""
    import torch
    from qkv_bias_rope_amd import probe as P
    n = nbytes // 8 // 4 * 4                        # float32 elements per buffer
    bufs = [torch.ones(n, dtype=torch.float32, device="cuda:0") for _ in range(sets)]
    dsts = [torch.empty_like(b) for b in bufs]
    out = {"bytes": n * 8, "rotating_buffers": sets, "block": 256}
    k = max(20, min(steps, 100))
    for name in ("inplace_add", "copy"):
        res = []
        for pol in (1, 2, 3):
            for vpt in (1, 2):
                if name == "inplace_add":
                    fn = lambda i, pol=pol, vpt=vpt: P.add(bufs[i % sets], 256, vpt, pol, stream)
                else:
                    fn = lambda i, pol=pol, vpt=vpt: P.copy(dsts[i % sets], bufs[i % sets], 256, vpt,
                                                            pol, stream)
                with torch.cuda.stream(stream):
                    for i in range(2 * sets):
                        assert fn(i) == 0
                    torch.cuda.synchronize()
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    for i in range(k):
                        fn(i)
                    e1.record(stream)
                    e1.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / k
                res.append(dict(policy=pol, vpt=vpt, us=round(us, 3), gbs=round(n * 8 / us / 1e3, 1)))
        b = _best(res)
        out[name] = dict(best_us=b["us"], best_gbs=b["gbs"], best_policy=b["policy"],
                         best_vpt=b["vpt"], sweep=res)
    out["achievable_gbs"] = max(out["inplace_add"]["best_gbs"], out["copy"]["best_gbs"])
    del bufs, dsts
    torch.cuda.empty_cache()
    return out


def ceiling_prefill_rows(h, steps, stream, R=8):
    """The prefill's own byte pattern without its arithmetic: the probe
    library's row pass over concat [4096][nqt+2nkt] copies of the rows (read
    and written back in place, the bias read once, the k/v columns stored to
    the f16 cache rows at the tokens' positions), rotating R buffers, swept
    over tokens per workgroup and store policy; beside it the epilogue itself
    on the same concat rows.  Event-timed stream loops, as the headline."""
    import torch
    from qkv_bias_rope_amd import binding as B
    from qkv_bias_rope_amd import probe as P
    from qkv_bias_rope_amd import workloads as wl
    w = wl.PREFILL_14B
    nbytes = algo_bytes(w, w.nt, 2)
    sets = Sets(w, R, wl.CACHE_F16, share_cache=True)
    xs = [torch.cat([st["q"], st["k"], st["v"]], dim=1).contiguous() for st in sets.sets]
    for st in sets.sets:
        st["q"] = st["k"] = st["v"] = None
    torch.cuda.empty_cache()
    bcat = torch.cat([sets.bq, sets.bk, sets.bv]).contiguous()
    kc, vc = sets.sets[0]["kc"], sets.sets[0]["vc"]
    pos = sets.sets[0]["pos"]
    k = max(20, min(steps, 100))

    def loop(fn):
        with torch.cuda.stream(stream):
            for i in range(2 * R):
                assert fn(i) == 0
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(k):
                fn(i)
            e1.record(stream)
            e1.synchronize()
        return e0.elapsed_time(e1) * 1e3 / k

    res = []
    for tpb in (1, 2, 4):
        for pol in (1, 2, 3):
            us = loop(lambda i, tpb=tpb, pol=pol: P.rows(xs[i % R], bcat, w.nqt, w.nkt, pos, None, w.n_ctx,
                                                         kc, vc, block=256, tpb=tpb, policy=pol,
                                                         stream=stream))
            res.append(dict(tokens_per_workgroup=tpb, policy=pol, us=round(us, 3),
                            gbs=round(nbytes / us / 1e3, 1)))
    cargs = [B.make_args(x[:, :w.nqt], x[:, w.nqt:w.nqt + w.nkt], x[:, w.nqt + w.nkt:], sets.bq, sets.bk,
                         sets.bv, pos, kc, vc, n_head=w.n_head, n_kv_head=w.n_kv_head,
                         head_dim=w.head_dim, theta=w.theta, cache_dtype=wl.CACHE_F16, n_ctx=w.n_ctx,
                         stream=stream, use_stream=True) for x in xs]
    cat_us = loop(lambda i: B.qkv_epilogue_run_ex(h, cargs[i % R]))
    assert B.qkv_epilogue_status(h) == 0, B.qkv_epilogue_last_error(h)
    b = _best(res)
    del sets, xs, cargs
    torch.cuda.empty_cache()
    return dict(bytes=nbytes, rotating_buffers=R, block=256, best_us=b["us"], best_gbs=b["gbs"],
                best_tokens_per_workgroup=b["tokens_per_workgroup"], best_policy=b["policy"],
                epilogue_concat_layout_us=round(cat_us, 3),
                epilogue_concat_layout_frac_of_row_pass=round(b["us"] / cat_us, 4), sweep=res)


def ceiling_read(nbytes, steps, stream, min_set_bytes=1.5e9):
    """What a bare read of `nbytes` (a decode step's weight matrix) takes on
    this device: the probe library's read-only pass over rotating buffers (as
    many as the projection's own timing rotates, so every launch comes from
    HBM), swept over load policy and vectors per thread; event-timed over a
    stream loop."""
    import torch
    from qkv_bias_rope_amd import probe as P
    n = nbytes // 4 // 4 * 4
    sets = max(2, int(-(-min_set_bytes // (n * 4))))
    bufs = [torch.ones(n, dtype=torch.float32, device="cuda:0") for _ in range(sets)]
    out = torch.empty(P.read_out_numel(n // 4, 256, 1), dtype=torch.float32, device="cuda:0")
    k = max(50, min(steps, 200))
    res = []
    for pol in (0, 1):
        for vpt in (1, 2, 4, 8):
            fn = lambda i, pol=pol, vpt=vpt: P.read(bufs[i % sets], out, 256, vpt, pol, stream)
            with torch.cuda.stream(stream):
                for i in range(2 * sets):
                    assert fn(i) == 0
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for i in range(k):
                    fn(i)
                e1.record(stream)
                e1.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / k
            res.append(dict(policy=pol, vpt=vpt, us=round(us, 3), gbs=round(n * 4 / us / 1e3, 1)))
    b = _best(res)
    del bufs, out
    torch.cuda.empty_cache()
    return dict(bytes=n * 4, rotating_buffers=sets, block=256, best_us=b["us"], best_gbs=b["gbs"],
                best_policy=b["policy"], best_vpt=b["vpt"], sweep=res)


def floors(stream, shapes):
    """Per-launch floor of an empty kernel at the given (grid, block) launch
    shapes: back-to-back in a HIP-graph replay (GPU side) and in a stream
    loop issued from this process (host issue included)."""
    import torch
    from qkv_bias_rope_amd import probe as P
    out = {}
    for g_, b_ in shapes:
        gu = time_graph(lambda i: P.empty(g_, b_, stream), 256, 4, stream)
        with torch.cuda.stream(stream):
            for _ in range(64):
                P.empty(g_, b_, stream)
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(512):
                P.empty(g_, b_, stream)
            e1.record(stream)
            e1.synchronize()
        loop_us = e0.elapsed_time(e1) * 1e3 / 512
        # the same empty kernel taking 1280 bytes of arguments, as a launch of
        # the epilogue does: HIP's host path for a launch that carries them
        with torch.cuda.stream(stream):
            for _ in range(64):
                P.empty_args(g_, b_, stream)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(512):
                P.empty_args(g_, b_, stream)
            e1.record(stream)
            e1.synchronize()
        out[f"grid{g_}x{b_}"] = dict(graph_us=round(gu, 3), stream_loop_us=round(loop_us, 3),
                                     stream_loop_us_with_1280_byte_args=round(
                                         e0.elapsed_time(e1) * 1e3 / 512, 3))
    return out


def copy_calibration(steps):
    """Known traffic for scaling FETCH_SIZE / WRITE_SIZE: the probe library's
    copy of 1 GiB (1 GiB read, 1 GiB written) under the non-temporal policy,
    then under the write-through policy the epilogue's streaming stores use;
    `steps` launches each."""
    import torch
    from qkv_bias_rope_amd import probe as P
    n = 256 * 1024 * 1024  # float32 elements = 1 GiB
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    s = torch.cuda.current_stream()
    for pol in (1, 2):
        for _ in range(steps):
            assert P.copy(dst, src, 256, 1, pol, s) == 0
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_policy": pol, "bytes_read": n * 4, "bytes_written": n * 4,
                          "launches": steps}), flush=True)


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
    # each launch is a prompt of nt tokens at positions 0..nt-1 (distinct
    # cache rows, as in a real prefill)
    w = wl.Workload("proj_sweep_14b", 40, 8, 128, nt=1, n_ctx=4096, n_slots=1, layers=1, seed=30,
                    pos_mode="arange")
    hidden = 5120
    with torch.cuda.stream(stream):
        for nt in PROJ_SWEEP_TOKENS:
            steps = args.steps if nt <= 512 else max(10, args.steps // 5)
            r = bench_proj(h, w, hidden, steps, args.warmup, stream, min_set_bytes=1.0e9, nt=nt)
            r8 = bench_proj(h, w, hidden, steps, args.warmup, stream, min_set_bytes=1.0e9, nt=nt,
                            wfmt="e4m3")
            print(json.dumps({"proj_sweep_tokens": nt, "hidden": hidden,
                              "us_per_launch": round(r["us_per_launch"], 2),
                              "tflops": round(r["tflops"], 1), "gbs": round(r["gbs"], 1),
                              "library_bf16_matmul_call_us": round(r["library_bf16_matmul_call_us"], 2),
                              "e4m3_us_per_launch": round(r8["us_per_launch"], 2),
                              "e4m3_gbs": round(r8["gbs"], 1)}),
                  flush=True)
    B.qkv_epilogue_destroy(h)


def decode_loop_c(w, steps, warmup):
    """The decode step issued from C with no Python in the process
    (tests/c/decode_loop, built by __graft_entry__.build()): microseconds per
    layer of an event-timed stream loop and host microseconds per call.  None
    when the program is not built."""
    import subprocess
    exe = os.path.join(ROOT, "tests", "c", "decode_loop")
    if not os.path.exists(exe):
        log("[bench]   tests/c/decode_loop not built; skipped")
        return None
    r = subprocess.run([exe, str(w.n_head), str(w.n_kv_head), str(w.head_dim), str(w.layers), str(steps),
                        str(warmup)], capture_output=True, text=True, timeout=120)
    if r.returncode != 0:
        log(f"[bench]   decode_loop failed: {r.stderr.strip()}")
        return None
    return json.loads(r.stdout.strip().splitlines()[-1])


def decode_all(h, args, stream):
    """The one-token decode workloads (tiny, 7B, 14B) beside the empty kernel
    of each one's launch shape."""
    import torch
    from qkv_bias_rope_amd import workloads as wl
    out = {}
    fl = floors(stream, [(3, 64), (9, 64), (14, 64)])
    out["empty_kernel_floor"] = fl
    log(f"[bench] empty-kernel floor: {fl}")
    shape = {wl.TINY_DECODE.name: "grid3x64", wl.DECODE_7B.name: "grid9x64",
             wl.DECODE_14B.name: "grid14x64"}
    for wd in (wl.TINY_DECODE, wl.DECODE_7B, wl.DECODE_14B):
        log(f"[bench] {wd.name}")
        r = bench_decode(h, wd, max(10, args.steps // 10), max(2, args.warmup // 10), stream)
        r["empty_kernel_same_launch"] = fl[shape[wd.name]]
        if wd.layers > 1:
            # the same step issued from C (separate section buffers on every layer)
            c = decode_loop_c(wd, max(50, args.steps // 2), 5)
            if c is not None:
                r["us_per_layer_stream_from_c"] = round(c["us_per_layer"], 3)
                r["host_issue_us_per_call_from_c"] = round(c["host_issue_us_per_call"], 3)
        out[wd.name] = {k: (round(v, 3) if isinstance(v, float) else v) for k, v in r.items()}
        log(f"[bench]   {r['us_per_layer_stream']:.2f} us/layer (stream), "
            f"{r.get('us_per_layer_graph', float('nan')):.2f} us/layer (graph)")
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-extra", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calib", action="store_true",
                    help="run only a 1 GiB device copy (counter calibration)")
    ap.add_argument("--batched-only", action="store_true",
                    help="run only the 256-sequence decode (f16 and f32 caches), one JSON line")
    ap.add_argument("--decode-only", action="store_true",
                    help="run only the one-token decode workloads and the empty-kernel floor, "
                         "one JSON line")
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
    if args.decode_only:
        rc, h = B.qkv_epilogue_create(0, 4096)
        assert rc == 0, rc
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            out = decode_all(h, args, stream)
        B.qkv_epilogue_destroy(h)
        print(json.dumps(out), flush=True)
        return
    if args.batched_only:
        rc, h = B.qkv_epilogue_create(0, 4096)
        assert rc == 0, rc
        stream = torch.cuda.Stream()
        out = {}
        with torch.cuda.stream(stream):
            for cd, tag in ((wl.CACHE_F16, "f16"), (wl.CACHE_F32, "f32")):
                r = bench_batched(h, wl.BATCHED_DECODE_14B, cd, stream)
                out[f"{wl.BATCHED_DECODE_14B.name}_{tag}"] = r
                log(f"[bench] {tag}: {r['us_per_launch']} us/launch, bare pass {r['bare_pass_us']} us")
        B.qkv_epilogue_destroy(h)
        print(json.dumps(out), flush=True)
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
    ceil = None
    if not args.no_extra:
        log("[bench] ceilings: bare passes of the prefill launch's bytes")
        ceil = ceilings_prefill(args.steps, stream)
        extra["ceiling_prefill_14b_4096"] = ceil
        extra[w.name + "_frac_of_achievable"] = round(main_res["gbs"] / ceil["achievable_gbs"], 4)
        rp = ceiling_prefill_rows(h, args.steps, stream)
        ceil["row_pass"] = rp
        extra[w.name + "_frac_of_row_pass"] = round(rp["best_us"] / (main_res["ms"] * 1e3), 4)
        fastest = max(ceil["achievable_gbs"], rp["best_gbs"])
        extra[w.name + "_fastest_bare_pass_gbs"] = fastest
        extra[w.name + "_frac_of_fastest_bare_pass"] = round(main_res["gbs"] / fastest, 4)
        log(f"[bench]   row pass of the same byte pattern {rp['best_us']} us ({rp['best_gbs']} GB/s); "
            f"epilogue on concat rows {rp['epilogue_concat_layout_us']} us")
        log(f"[bench]   achievable {ceil['achievable_gbs']} GB/s (add {ceil['inplace_add']['best_gbs']}, "
            f"copy {ceil['copy']['best_gbs']}); epilogue at "
            f"{extra[w.name + '_frac_of_achievable']:.3f} of it")

    if not args.no_extra:
        wb = wl.BATCHED_DECODE_14B
        for cd, tag in ((wl.CACHE_F16, "f16"), (wl.CACHE_F32, "f32")):
            log(f"[bench] {wb.name} {tag} (HIP-graph replay)")
            r = bench_batched(h, wb, cd, stream)
            extra[f"{wb.name}_{tag}"] = r
            log(f"[bench]   {r['us_per_launch']:.3f} us/launch, {r['gbs']:.1f} GB/s; bare pass "
                f"{r['bare_pass_us']:.3f} us ({r['frac_of_achievable']:.3f} of achievable); empty "
                f"kernel {r['empty_kernel_same_launch_us']:.3f} us")
        extra.update(decode_all(h, args, stream))
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
        # the same launch with E4M3 weights (bf16 products on the matrix cores)
        log(f"[bench] {w.name} projection-fed epilogue, E4M3 weights")
        r = bench_proj(h, w, hid, max(20, args.steps // 2), max(2, args.warmup // 4), stream,
                       min_set_bytes=1.0e9, wfmt="e4m3")
        extra[w.name + "_proj_e4m3"] = dict(
            us_per_launch=round(r["us_per_launch"], 2), tflops=round(r["tflops"], 1),
            frac_of_bf16_peak=round(r["tflops"] / PEAK_BF16_TFLOPS, 4), hidden=hid, input_sets=r["sets"])
        log(f"[bench]   {r['us_per_launch']:.1f} us/launch, {r['tflops']:.1f} TFLOP/s")
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
        # the GEMV streams the weights once: a bare read of the same bytes
        cr = ceiling_read((wd.nqt + 2 * wd.nkt) * hid * 2, args.steps, stream)
        extra["ceiling_decode_14b_proj_weights_bf16"] = cr
        extra[wd.name + "_proj"]["bare_read_of_weights_us"] = cr["best_us"]
        extra[wd.name + "_proj"]["frac_of_bare_read"] = round(cr["best_us"] / r["us_per_launch"], 4)
        log(f"[bench]   bare read of the {cr['bytes']} weight bytes: {cr['best_us']} us "
            f"({cr['best_gbs']} GB/s)")
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
        cr = ceiling_read((wd.nqt + 2 * wd.nkt) * hid, args.steps, stream)
        extra["ceiling_decode_14b_proj_weights_e4m3"] = cr
        extra[wd.name + "_proj_e4m3"]["bare_read_of_weights_us"] = cr["best_us"]
        extra[wd.name + "_proj_e4m3"]["frac_of_bare_read"] = round(cr["best_us"] / r["us_per_launch"], 4)
        log(f"[bench]   bare read of the {cr['bytes']} weight bytes: {cr['best_us']} us")
        r = bench_proj_decode(h, wd, hid, max(5, args.steps // 20), 2, stream, wfmt="e4m3")
        extra[wd.name + "_proj_e4m3_step"] = {k: (round(v, 3) if isinstance(v, float) else v)
                                              for k, v in r.items()}
        log(f"[bench]   {r['us_per_layer_stream']:.2f} us/layer (stream), "
            f"{r['us_per_layer_graph']:.2f} us/layer (graph)")

    cpu = None
    if not args.no_cpu:
        log("[bench] CPU oracle on the host cores, every configuration")
        co = cpu_oracle_all()
        extra["cpu_oracle"] = co
        c4 = co[w.name]
        cpu = {"value": c4["gbs_nthread"], "unit": "GB/s", "cores": co["threads_parallel"],
               "kind": "oracle",
               "sample": (f"{c4['launches_nthread']} full launches of {w.name} ({w.nt} tokens, f16 "
                          f"cache), tokens split over {co['threads_parallel']} host threads; "
                          f"{c4['us_per_launch_nthread'] / 1e3:.1f} ms per launch"),
               "single_thread": {"value": c4["gbs_1thread"], "cores": 1,
                                 "ms_per_launch": round(c4["us_per_launch_1thread"] / 1e3, 2),
                                 "launches": c4["launches_1thread"]},
               "cpu": co["cpu"]}

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
