#!/usr/bin/env python3
"""Decode-step benchmark of int4-KV split-K attention on one MI355X.

Workload: the Llama-3.1-70B-shaped decode layer (batch 1, 64 query heads,
8 KV heads, head_dim 128, int4 group-64 K/V with fp16 scale and bias,
softmax scale 1/sqrt(128), split-K chunks of 512 rows) at Skv = 131072 by
default. One step is one pass of the whole path for one layer: quantise the
new token's K and V into the cache (n = 1 append at row Skv-1), then the
split-K partial kernel and the reduce, all on one stream. Steps rotate over a
pool of distinct layers (>= 640 MB, 2.5x the 256 MB last-level cache) so that
the cache is read from HBM, not from the Infinity Cache.

Inputs are seeded synthetic fp16 N(0,1) draws made on the GPU and quantised
by the library itself; they are resident in HBM before timing starts.

Output: one JSON line (rank 0) with value = effective HBM GB/s of the step
(algorithmic bytes: int4 codes + fp16 scale/bias of K and V, plus the
appended row), the per-kernel roofline of the partial kernel (HIP events
around each launch in a second timed pass of the same steps) and the CPU
oracle timed on the host as a reported baseline.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20
B, HQ, HKV, D, G = 1, 64, 8, 128, 64


TRAFFIC_FILES = {
    4: os.path.join(ROOT, "profiles", "sdpa_partial_llama_128k_traffic.txt"),
    8: os.path.join(ROOT, "profiles", "sdpa_partial_int8_llama_128k_traffic.txt"),  # absent until profiled
}


def measured_traffic(skv: int, chunk: int, kernel: str, bits: int = 4, step: str = "fused"):
    """HBM bytes per attention launch of the decode step from the committed
    counter summary, or None when this run is not the profiled configuration
    (the Llama layer at 131072 rows, chunk 512, kvq_decode_step with AUTO or
    MFMA) or the kernel sources changed since the counters were taken (their
    hash differs)."""
    if skv != 131072 or chunk != 512 or kernel not in ("auto", "mfma") or step != "fused":
        return None
    path = TRAFFIC_FILES[bits]
    try:
        kv = {}
        for line in open(path):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        root = os.path.dirname(path)
        h = hashlib.sha256()
        for rel in kv["source_files"].split():
            with open(os.path.join(root, "..", rel), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != kv["source_sha256"]:
            return None
        return int(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def layer_bytes(skv: int, bits: int = 4, hkv: int = HKV) -> int:
    return hkv * skv * (D * bits // 8 + 4 * (D // G)) * 2  # K and V: codes + fp16 scale + fp16 bias


def append_bytes(bits: int = 4, hkv: int = HKV) -> int:
    return 2 * B * hkv * D * 2 + 2 * B * hkv * (D * bits // 8 + 4 * (D // G))  # fp16 rows in, packed row out


def make_pool(kvq, torch, skv: int, pool_bytes: int, chunk: int, seed: int = 1234, bits: int = 4, hkv: int = HKV):
    """Distinct layers of the Llama-shaped cache (hkv KV heads, 8 query heads
    each) totalling at least pool_bytes, filled with seeded fp16 N(0,1) rows
    quantised by the library."""
    hq = 8 * hkv
    n_layers = max(2, math.ceil(pool_bytes / layer_bytes(skv, bits, hkv)))
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    pool = []
    for i in range(n_layers):
        gen.manual_seed(seed * 1000003 + skv * 131 + i)
        cache = kvq.QuantKVCache(B, hkv, D, skv, G, device=dev, bits=bits)
        # fill in slabs so the fp16 staging stays small
        slab = 16384
        for t0 in range(0, skv, slab):
            n = min(slab, skv - t0)
            k = torch.randn((B, hkv, n, D), generator=gen, device=dev, dtype=torch.float32).half()
            v = torch.randn((B, hkv, n, D), generator=gen, device=dev, dtype=torch.float32).half()
            kvq.quantize_kv_append(cache, t0, k, v)
        q = torch.randn((B, hq, D), generator=gen, device=dev, dtype=torch.float32).half()
        k_new = torch.randn((B, hkv, 1, D), generator=gen, device=dev, dtype=torch.float32).half()
        v_new = torch.randn((B, hkv, 1, D), generator=gen, device=dev, dtype=torch.float32).half()
        ws = kvq.partials_buffers(B, hq, D, skv, chunk, device=dev)
        out = torch.empty((B, hq, D), dtype=torch.float32, device=dev)
        qr = torch.empty((B, hq, D), dtype=torch.float32, device=dev)
        ws1 = kvq.decode_workspace(cache, hq, skv)
        pool.append(dict(cache=cache, q=q, k_new=k_new, v_new=v_new, ws=ws, ws1=ws1, out=out, qr=qr))
    torch.cuda.synchronize()
    return pool


def run_steps(kvq, torch, pool, skv, chunk, kernel, n, events=None, step="fused"):
    """n decode steps, each on a different layer of the pool: the current
    token's K/V row is quantised into row skv-1 and attention runs over skv
    rows. step "fused": kvq_decode_step (append inside the attention kernel,
    then the reduce); "unfused": append, partial and reduce as three calls;
    "rotated": the Hadamard-rotated cache through kvq_decode_step_rotated
    (query, appended rows and output rotated inside the attention kernel and
    the reduce: two launches); "rotated-unfused": the same step as five calls
    (rotate q, rotated append, partial with fp32 q, reduce, rotate back).
    events[i]: (start, stop) recorded in the attention kernel's own dispatch
    (not for "rotated")."""
    alpha = 1.0 / math.sqrt(D)
    stream = torch.cuda.current_stream()
    for i in range(n):
        L = pool[i % len(pool)]
        ev = events[i] if events is not None else None
        if step == "single":
            kvq.decode_step_single_launch(L["cache"], skv - 1, L["k_new"], L["v_new"], L["q"], alpha,
                                          workspace=L["ws1"], out=L["out"], stream=stream, events=ev)
            continue
        if step == "fused":
            kvq.decode_step(L["cache"], skv - 1, L["k_new"], L["v_new"], L["q"], alpha, chunk, out=L["out"],
                            workspace=L["ws"], kernel=kernel, stream=stream, events=ev)
            continue
        if step == "rotated":
            kvq.decode_step_rotated(L["cache"], skv - 1, L["k_new"], L["v_new"], L["q"], alpha, chunk, out=L["out"],
                                    workspace=L["ws"], kernel=kernel, stream=stream)
            continue
        q = L["q"]
        if step == "rotated-unfused":
            q = kvq.hadamard_rotate(L["q"], out=L["qr"], stream=stream)
            kvq.quantize_kv_append_rotated(L["cache"], skv - 1, L["k_new"], L["v_new"], stream=stream)
        else:
            kvq.quantize_kv_append(L["cache"], skv - 1, L["k_new"], L["v_new"], stream=stream)
        m, l, acc = L["ws"]
        if ev is not None:
            kvq.sdpa_int4_partial_timed(L["cache"], skv, q, alpha, chunk, m, l, acc, ev[0], ev[1],
                                        kernel=kernel, stream=stream)
        else:
            kvq.sdpa_int4_partial(L["cache"], skv, q, alpha, chunk, m, l, acc, kernel=kernel, stream=stream)
        kvq.sdpa_int4_reduce(m, l, acc, L["out"], stream=stream)
        if step == "rotated-unfused":
            kvq.hadamard_rotate(L["out"], out=L["out"], stream=stream)


def graph_step_ms(kvq, torch, pool, skv, chunk, kernel, step, reps=5):
    """Per-step time with the host out of the loop: one pass over the pool
    (every layer once, so the cache still streams from HBM) captured in a HIP
    graph, replayed `reps` times with events around each replay; median."""
    n = len(pool)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_steps(kvq, torch, pool, skv, chunk, kernel, n, step=step)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_steps(kvq, torch, pool, skv, chunk, kernel, n, step=step)
    g.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        per.append(a.elapsed_time(b) / n)
    del g
    return sorted(per)[len(per) // 2]


def time_config(kvq, torch, skv, chunk, kernel, steps, warmup, pool_bytes, step="fused", bits=4, hkv=HKV,
                repeats=0, graph=False):
    pool = make_pool(kvq, torch, skv, pool_bytes, chunk, bits=bits, hkv=hkv)
    run_steps(kvq, torch, pool, skv, chunk, kernel, warmup, step=step)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    run_steps(kvq, torch, pool, skv, chunk, kernel, steps, step=step)
    t1.record()
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / steps
    # second pass of the same steps with HIP events recorded in every
    # attention kernel's own dispatch: that kernel's execution time (the
    # rotated step has no timed entry point: its step time only)
    if step == "rotated":
        kern_ms = [float("nan")] * steps
    else:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        run_steps(kvq, torch, pool, skv, chunk, kernel, steps, events=evs, step=step)
        torch.cuda.synchronize()
        kern_ms = sorted(a.elapsed_time(b) for a, b in evs)
    res = dict(skv=skv, ms_per_step=ms_per_step, partial_ms_avg=sum(kern_ms) / len(kern_ms),  # nan: not timed
               partial_ms_p10=kern_ms[len(kern_ms) // 10], partial_ms_p90=kern_ms[(9 * len(kern_ms)) // 10],
               pool_layers=len(pool), pool_mb=len(pool) * layer_bytes(skv, bits, hkv) / 1e6)
    if graph:
        res.update(graph_ms_per_step=graph_step_ms(kvq, torch, pool, skv, chunk, kernel, step))
    if repeats:
        # the step time's spread: `repeats` runs of steps // repeats steps,
        # events around each run, per-step time of each run
        per_run = max(1, steps // repeats)
        runs = []
        for _ in range(repeats):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            run_steps(kvq, torch, pool, skv, chunk, kernel, per_run, step=step)
            b.record()
            torch.cuda.synchronize()
            runs.append(a.elapsed_time(b) / per_run)
        runs.sort()
        res.update(step_ms_median=runs[len(runs) // 2], step_ms_p10=runs[len(runs) // 10],
                   step_ms_p90=runs[(9 * len(runs)) // 10], step_repeats=repeats, step_per_repeat=per_run)
    last = pool[-1]
    del pool
    return res, last


def hbm_read_calibration(kvq, torch, gib: int = 1, reps: int = 20):
    """Achievable HBM read bandwidth on this GPU, the context of the spec
    fraction: the library's plain grid-stride read kernel (kvq_hbm_read)
    over `gib` GiB, which no cache level holds; median over `reps` calls,
    events around each."""
    x = torch.ones((gib << 28,), dtype=torch.int32, device="cuda")
    sink = torch.zeros((1,), dtype=torch.int32, device="cuda")
    for _ in range(3):
        kvq.hbm_read(x, sink)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        kvq.hbm_read(x, sink)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    ts.sort()
    nbytes = x.numel() * 4
    del x
    ms = ts[len(ts) // 2]
    return dict(kind="kvq_hbm_read (grid-stride 16-byte loads, 2048 x 256 threads) over %d GiB, median of %d calls"
                % (gib, reps), bytes=nbytes, ms=round(ms, 4), gbs=round(nbytes / (ms * 1e-3) / 1e9, 1))


def time_layer_loop(kvq, torch, layers, skv, chunk, kernel, steps, warmup):
    """The full-depth decode step: one decode step (fused append + attention
    + reduce) on each of `layers` distinct caches of the Llama layer, in
    order, on one stream; the caches stay resident in HBM. Returns ms per
    step (all layers) and the cache bytes."""
    pool = make_pool(kvq, torch, skv, layers * layer_bytes(skv), chunk, seed=4321)
    assert len(pool) == layers
    run_steps(kvq, torch, pool, skv, chunk, kernel, warmup * layers)
    torch.cuda.synchronize()
    per = []
    for _ in range(steps):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        run_steps(kvq, torch, pool, skv, chunk, kernel, layers)
        t1.record()
        torch.cuda.synchronize()
        per.append(t0.elapsed_time(t1))
    cache_bytes = sum(L["cache"].nbytes() for L in pool)
    del pool
    per.sort()
    return dict(ms_median=per[len(per) // 2], ms_p10=per[len(per) // 10], ms_p90=per[(9 * len(per)) // 10],
                ms_min=per[0], cache_bytes=cache_bytes)


APPEND_ROWS, APPEND_LEN, APPEND_CAP = 4096, 61440, 65536  # the outlier workload's bulk append


def time_bulk_append(kvq, torch, rotated: bool, reps: int = 40, n_inputs: int = 20, bits: int = 4):
    """Bulk append of the outlier workload's shape (4096 fp16 rows per KV head
    at row 61440 of a 65536-row cache), plain or Hadamard-rotated, over
    n_inputs distinct input sets (336 MB, more than the Infinity Cache).
    Returns the median time of one append call in ms (events around the call)."""
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(777)
    inputs = [(torch.randn((B, HKV, APPEND_ROWS, D), generator=gen, device=dev).half(),
               torch.randn((B, HKV, APPEND_ROWS, D), generator=gen, device=dev).half()) for _ in range(n_inputs)]
    cache = kvq.QuantKVCache(B, HKV, D, APPEND_CAP, G, device=dev, bits=bits)
    fn = kvq.quantize_kv_append_rotated if rotated else kvq.quantize_kv_append
    for i in range(5):
        fn(cache, APPEND_LEN, *inputs[i % n_inputs])
    torch.cuda.synchronize()
    # One call takes longer on the host than on the GPU, so events around
    # single calls would time the host; the calls are captured in a graph
    # (they enqueue one kernel each and no memset) and the replays timed.
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            for i in range(reps):
                fn(cache, APPEND_LEN, *inputs[i % n_inputs])
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) / reps)
    del graph, inputs, cache
    return sorted(per)[len(per) // 2]


MFMA_F16_PEAK_TFLOPS = 2500.0  # dense fp16 matrix-core peak


def prefill_flops(q_start: int, sq: int, hq: int = HQ) -> int:
    """Algorithmic flops of causal prefill attention: per query head and
    position i, q.k and p.v over its q_start + i + 1 rows, 2 * D flops each."""
    rows = sq * q_start + sq * (sq + 1) // 2
    return 2 * 2 * hq * D * rows


def time_prefill(kvq, torch, q_start: int, sq: int, reps: int = 5, bits: int = 4):
    """Prefill attention on the Llama layer: a cache of q_start + sq rows
    (seeded fp16 N(0,1), quantised by the library with `bits` per code), then
    kvq_sdpa_int4_prefill for the sq positions after q_start. Returns the
    median kernel time in ms (events around each call; one call runs for
    milliseconds)."""
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(99)
    S = q_start + sq
    cache = kvq.QuantKVCache(B, HKV, D, S, G, device=dev, bits=bits)
    for t0 in range(0, S, 16384):
        n = min(16384, S - t0)
        k = torch.randn((B, HKV, n, D), generator=gen, device=dev).half()
        v = torch.randn((B, HKV, n, D), generator=gen, device=dev).half()
        kvq.quantize_kv_append(cache, t0, k, v)
    q = torch.randn((B, HQ, sq, D), generator=gen, device=dev).half()
    out = torch.empty((B, HQ, sq, D), dtype=torch.float32, device=dev)
    alpha = 1.0 / math.sqrt(D)
    kvq.sdpa_int4_prefill(cache, q_start, q, alpha, out=out)
    torch.cuda.synchronize()
    per = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        kvq.sdpa_int4_prefill(cache, q_start, q, alpha, out=out)
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1))
    del cache, q, out
    return sorted(per)[len(per) // 2]


GEMMA_SKVS = (33, 423, 786, 950, 8192)  # the Gemma page's decode contexts and the 8K case
GEMMA_HQ, GEMMA_HKV, GEMMA_D = 32, 16, 256


def gemma_bytes(skv: int) -> int:
    return GEMMA_HKV * skv * (GEMMA_D // 2 + 4 * (GEMMA_D // G)) * 2  # int4 codes + fp16 scale/bias, K and V


def time_gemma_decode(kvq, torch, skv: int, steps: int, warmup: int, pool_bytes: int, max_layers: int = 64):
    """Decode steps (kvq_decode_step, AUTO) on the Gemma-style layer: batch 1,
    32 query heads on 16 KV heads, head_dim 256, softmax scale 1, Q and K
    rows at unit RMS times a per-channel gain ~U(0.5, 2) (one gain vector
    each), V ~N(0,1), all drawn on the GPU from a seed and quantised by the
    library; over a pool of distinct layers (>= pool_bytes, at most
    max_layers). Returns (us per step, pool layers)."""
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(31 * skv + 7)
    gq = torch.rand((GEMMA_D,), generator=gen, device=dev) * 1.5 + 0.5
    gk = torch.rand((GEMMA_D,), generator=gen, device=dev) * 1.5 + 0.5

    def rms_gain(x, gain):
        return x / x.pow(2).mean(dim=-1, keepdim=True).sqrt() * gain

    n_layers = max(2, min(max_layers, math.ceil(pool_bytes / gemma_bytes(skv))))
    pool = []
    for _ in range(n_layers):
        cache = kvq.QuantKVCache(B, GEMMA_HKV, GEMMA_D, skv, G, device=dev)
        k = rms_gain(torch.randn((B, GEMMA_HKV, skv, GEMMA_D), generator=gen, device=dev), gk).half()
        v = torch.randn((B, GEMMA_HKV, skv, GEMMA_D), generator=gen, device=dev).half()
        kvq.quantize_kv_append(cache, 0, k[:, :, :skv - 1].contiguous(), v[:, :, :skv - 1].contiguous())
        q = rms_gain(torch.randn((B, GEMMA_HQ, GEMMA_D), generator=gen, device=dev), gq).contiguous()
        kn, vn = k[:, :, skv - 1].contiguous(), v[:, :, skv - 1].contiguous()
        ws = kvq.partials_buffers(B, GEMMA_HQ, GEMMA_D, skv, 512, device=dev)
        out = torch.empty((B, GEMMA_HQ, GEMMA_D), dtype=torch.float32, device=dev)
        pool.append((cache, q, kn, vn, ws, out))
        del k, v
    def run(n, stream):
        for i in range(n):
            cache, q, kn, vn, ws, out = pool[i % len(pool)]
            kvq.decode_step(cache, skv - 1, kn, vn, q, 1.0, 512, out=out, workspace=ws, stream=stream)

    stream = torch.cuda.current_stream()
    run(warmup, stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    run(steps, stream)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    # the same steps with the host out of the loop: one pass over the pool
    # (every layer once) captured in a HIP graph, median of 5 replays
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        run(len(pool), side)
        with torch.cuda.graph(graph, stream=side):
            run(len(pool), side)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        graph.replay()
        b.record()
        torch.cuda.synchronize()
        per.append(a.elapsed_time(b) * 1e3 / len(pool))
    del graph, pool
    return us, n_layers, sorted(per)[len(per) // 2]


def time_outlier_append_decode(kvq, torch, steps: int, warmup: int, reps: int = 40):
    """The append + decode workload: 4096 new fp16 rows per KV head with
    outlier-heavy K (Student-t with 3 degrees of freedom, as Z / sqrt(chi2_3 / 3),
    and 4 channels per KV head scaled by 20, the same channels for every row;
    V ~N(0,1)) appended at row 61440 of a 65536-row Llama-layout cache, then
    decode steps over all 65536 rows. Returns (append us, decode us)."""
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(4096)

    def student_t(shape):
        z = torch.randn(shape, generator=gen, device=dev)
        chi2 = torch.randn((3,) + tuple(shape), generator=gen, device=dev).pow(2).sum(0)
        return z / (chi2 / 3).sqrt()

    chans = torch.stack([torch.randperm(D, generator=gen, device=dev)[:4] for _ in range(HKV)])
    boost = torch.ones((HKV, D), device=dev)
    boost[torch.arange(HKV, device=dev)[:, None], chans] = 20.0
    n_inputs = 8
    inputs = []
    for _ in range(n_inputs):
        k = (student_t((B, HKV, APPEND_ROWS, D)) * boost[None, :, None, :]).clamp(-60000, 60000).half()
        v = torch.randn((B, HKV, APPEND_ROWS, D), generator=gen, device=dev).half()
        inputs.append((k, v))
    cache = kvq.QuantKVCache(B, HKV, D, APPEND_CAP, G, device=dev)
    for t0 in range(0, APPEND_LEN, APPEND_ROWS):
        k, v = inputs[(t0 // APPEND_ROWS) % n_inputs]
        kvq.quantize_kv_append(cache, t0, k, v)
    torch.cuda.synchronize()
    # the append, captured in a graph (one kernel per call) and replayed
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for i in range(reps):
                kvq.quantize_kv_append(cache, APPEND_LEN, *inputs[i % n_inputs])
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) / reps)
    append_us = sorted(per)[len(per) // 2] * 1e3
    del graph
    # decode steps over the 65536 rows (the last row rewritten by each step)
    q = torch.randn((B, HQ, D), generator=gen, device=dev).half()
    kn, vn = inputs[0][0][:, :, 0].contiguous(), inputs[0][1][:, :, 0].contiguous()
    ws = kvq.partials_buffers(B, HQ, D, APPEND_CAP, 512, device=dev)
    out = torch.empty((B, HQ, D), dtype=torch.float32, device=dev)
    alpha = 1.0 / math.sqrt(D)
    for _ in range(warmup):
        kvq.decode_step(cache, APPEND_CAP - 1, kn, vn, q, alpha, 512, out=out, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        kvq.decode_step(cache, APPEND_CAP - 1, kn, vn, q, alpha, 512, out=out, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    decode_us = e0.elapsed_time(e1) * 1e3 / steps
    del inputs, cache
    return append_us, decode_us


def bulk_append_bytes(bits: int = 4) -> int:
    rows = B * HKV * APPEND_ROWS
    return 2 * rows * D * 2 + 2 * rows * (D * bits // 8 + 4 * (D // G))  # fp16 K and V in, packed rows out


def cpu_baseline(kvq, torch, entry, skv):
    """Time the float64 oracle on one full layer-call of the same workload."""
    import numpy as np

    import oracle

    cache = entry["cache"]
    oc = oracle.Cache(B, HKV, D, skv, G, bits=cache.bits)
    oc.k_q[...] = cache.k_q.cpu().numpy().view(np.uint32)
    oc.v_q[...] = cache.v_q.cpu().numpy().view(np.uint32)
    oc.k_scale[...] = cache.k_scale.cpu().numpy().view(np.uint16)
    oc.k_bias[...] = cache.k_bias.cpu().numpy().view(np.uint16)
    oc.v_scale[...] = cache.v_scale.cpu().numpy().view(np.uint16)
    oc.v_bias[...] = cache.v_bias.cpu().numpy().view(np.uint16)
    q = entry["q"].float().cpu().numpy()
    threads = oracle.default_threads()
    t = time.perf_counter()
    ref = oracle.sdpa(oc, skv, q, 1.0 / math.sqrt(D), nthreads=threads)
    dt = time.perf_counter() - t
    # the GPU output of this layer must agree with it (a sanity line, not the parity test)
    alpha = 1.0 / math.sqrt(D)
    out = kvq.sdpa_int4(cache, skv, entry["q"], alpha)
    torch.cuda.synchronize()
    err = float(np.abs(out.cpu().numpy() - ref).max())
    return dict(value=layer_bytes(skv, cache.bits) / dt / 1e9, unit="GB/s", cores=threads, kind="oracle",
                sample="one full layer-call (64 q-heads, Skv=%d) of the float64 oracle, %.2f s wall on %d threads "
                       "(at most %.0f thread-seconds of CPU work)" % (skv, dt, threads, dt * threads),
                seconds=dt, max_abs_err_vs_gpu=err)


def build_parser():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--skv", type=int, default=131072)
    ap.add_argument("--chunk", type=int, default=512)
    ap.add_argument("--pool-mb", type=int, default=int(2.5 * MALL_BYTES / 1e6))
    ap.add_argument("--kernel", choices=["auto", "valu", "mfma", "mfma-split", "mfma-wave"], default="auto")
    ap.add_argument("--sweep", default="1024,16384,65536",
                    help="extra Skv values timed with fewer steps (empty to skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip the measurements of the rows beyond the headline path (Hadamard-rotated cache, "
                         "8-bit cache, prefill)")
    ap.add_argument("--step", choices=["single", "fused", "unfused", "rotated", "rotated-unfused"], default="fused",
                    help="fused: kvq_decode_step (append inside the attention kernel, then the reduce); "
                         "unfused: append, partial and reduce as three calls")
    ap.add_argument("--layers", type=int, default=80,
                    help="layers of the full-depth decode step timed after the headline (0 skips it)")
    ap.add_argument("--bits", type=int, choices=[4, 8], default=4,
                    help="bits per cached code of the headline run (8: the 8-bit cache)")
    ap.add_argument("--repeats", type=int, default=10,
                    help="after the timed steps, time the same steps again as this many separate runs "
                         "(median / p10 / p90 of the per-step time; 0 skips)")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other workloads' timings (Gemma-style decode at 33..8192 rows, the outlier "
                         "append + 64K decode pair, the single-launch step)")
    ap.add_argument("--no-hbm-calibration", action="store_true",
                    help="skip the plain read of 1 GiB that gives the achievable HBM bandwidth")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="after timing, run one plain device copy of this many MB (a known-size reference "
                         "for hardware byte counters)")
    return ap


def main():
    args = build_parser().parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: there is no multi-GPU path here (the decode path would shard "
              "over KV heads or over sequence chunks). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import quantized_kv_cache_quantize_amd as kvq

    kvq.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    kernel = {"auto": kvq.KERNEL_AUTO, "valu": kvq.KERNEL_VALU, "mfma": kvq.KERNEL_MFMA,
              "mfma-split": kvq.KERNEL_MFMA_SPLIT, "mfma-wave": kvq.KERNEL_MFMA_WAVE}[args.kernel]
    pool_bytes = args.pool_mb * 1000 * 1000

    bits = args.bits
    main_res, last = time_config(kvq, torch, args.skv, args.chunk, kernel, args.steps, args.warmup, pool_bytes,
                                 step=args.step, bits=bits, repeats=args.repeats)
    sweep = []
    for s in [int(x) for x in args.sweep.split(",") if x.strip()]:
        r, _ = time_config(kvq, torch, s, args.chunk, kernel, max(20, args.steps // 2), args.warmup, pool_bytes,
                           step=args.step, bits=bits, graph=True)
        r["us_per_layer"] = r["ms_per_step"] * 1e3
        r["gbs"] = (layer_bytes(s, bits) + append_bytes(bits)) / (r["ms_per_step"] * 1e-3) / 1e9
        r["partial_gbs"] = layer_bytes(s, bits) / (r["partial_ms_avg"] * 1e-3) / 1e9
        sweep.append(r)

    depth = None
    if args.layers > 0:
        lp = time_layer_loop(kvq, torch, args.layers, args.skv, args.chunk, kernel, steps=10, warmup=2)
        step_b = args.layers * (layer_bytes(args.skv) + append_bytes())
        depth = {
            "workload": "%d distinct Llama-shaped layers at Skv %d resident in HBM (%.2f GB of int4 cache); one "
                        "decode step = kvq_decode_step on every layer in order, one stream" % (
                            args.layers, args.skv, lp["cache_bytes"] / 1e9),
            "layers": args.layers,
            "ms_per_step": round(lp["ms_median"], 4),
            "ms_p10": round(lp["ms_p10"], 4),
            "ms_p90": round(lp["ms_p90"], 4),
            "us_per_layer": round(lp["ms_median"] * 1e3 / args.layers, 3),
            "gbs": round(step_b / (lp["ms_median"] * 1e-3) / 1e9, 2),
            "frac_of_hbm_peak": round(step_b / (lp["ms_median"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "timing": "median of 10 steps, events around each step's %d x 2 launches" % args.layers,
        }
        # the one-GPU share of head sharding over 8 GPUs: one KV head and its 8 query heads
        sh, _ = time_config(kvq, torch, args.skv, args.chunk, kernel, max(20, args.steps // 2), args.warmup,
                            pool_bytes, step=args.step, hkv=1)
        sb = layer_bytes(args.skv, 4, 1)
        depth["shard_share"] = {
            "workload": "one GPU's share of the Llama layer split over 8 GPUs by KV head: Hkv 1, Hq 8, Skv %d "
                        "(%d bytes)" % (args.skv, sb),
            "us_per_layer": round(sh["ms_per_step"] * 1e3, 3),
            "gbs": round((sb + append_bytes(4, 1)) / (sh["ms_per_step"] * 1e-3) / 1e9, 2),
            "attention_us": round(sh["partial_ms_avg"] * 1e3, 3),
            "attention_gbs": round(sb / (sh["partial_ms_avg"] * 1e-3) / 1e9, 2),
        }

    if args.calib_copy_mb > 0:
        n = args.calib_copy_mb * 1000 * 1000 // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    next_rows = None
    if not args.no_next_rows:
        plain_ms = time_bulk_append(kvq, torch, False)
        rot_ms = time_bulk_append(kvq, torch, True)
        nb = bulk_append_bytes()
        s64 = 65536
        rot_res, _ = time_config(kvq, torch, s64, args.chunk, kernel, max(20, args.steps // 2), args.warmup,
                                 pool_bytes, step="rotated")
        rotu_res, _ = time_config(kvq, torch, s64, args.chunk, kernel, max(20, args.steps // 2), args.warmup,
                                  pool_bytes, step="rotated-unfused")
        next_rows = {"hadamard": {
            "workload": "outlier-workload shape: append 4096 fp16 rows per KV head (B1 Hkv8 D128 G64) at row "
                        "61440; rotated decode step at Skv 65536",
            "append_bytes": nb,
            "append_us": round(plain_ms * 1e3, 3),
            "append_rotated_us": round(rot_ms * 1e3, 3),
            "append_rotated_gbs": round(nb / (rot_ms * 1e-3) / 1e9, 2),
            "append_rotated_frac": round(nb / (rot_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "step_rotated_us_64k": round(rot_res["ms_per_step"] * 1e3, 3),
            "step_rotated_gbs_64k": round((layer_bytes(s64) + append_bytes()) / (rot_res["ms_per_step"] * 1e-3) / 1e9, 2),
            "step_rotated_unfused_us_64k": round(rotu_res["ms_per_step"] * 1e3, 3),
            "attention_rotated_unfused_us_64k": round(rotu_res["partial_ms_avg"] * 1e3, 3),
            "timing": "append: 40 calls captured in a HIP graph, median over 5 replays of the per-call time; "
                      "step: as the headline step, through kvq_decode_step_rotated (two launches), and as the "
                      "five separate calls",
        }}
        s8 = args.skv
        i8, _ = time_config(kvq, torch, s8, args.chunk, kvq.KERNEL_AUTO, max(20, args.steps // 2), args.warmup,
                            pool_bytes, step="fused", bits=8)
        i8_ms = time_bulk_append(kvq, torch, False, bits=8)
        nb8 = bulk_append_bytes(8)
        att8 = layer_bytes(s8, 8) / (i8["partial_ms_avg"] * 1e-3) / 1e9
        next_rows["int8"] = {
            "workload": "the headline layer (B1 Hq64 Hkv8 D128 G64, Skv %d) with 8-bit codes: decode step "
                        "(append inside the eight-wavefront matrix-core attention kernel, then the reduce); bulk "
                        "append of the outlier-workload shape" % s8,
            "layer_bytes": layer_bytes(s8, 8),
            "step_us": round(i8["ms_per_step"] * 1e3, 3),
            "step_gbs": round((layer_bytes(s8, 8) + append_bytes(8)) / (i8["ms_per_step"] * 1e-3) / 1e9, 2),
            "attention_us": round(i8["partial_ms_avg"] * 1e3, 3),
            "attention_gbs": round(att8, 2),
            "attention_frac": round(att8 / HBM_PEAK_GBS, 4),
            "attention_traffic": measured_traffic(s8, args.chunk, "auto", 8),
            "append_us": round(i8_ms * 1e3, 3),
            "append_gbs": round(nb8 / (i8_ms * 1e-3) / 1e9, 2),
            "timing": "step and attention as the headline; append as the hadamard row's",
        }
        pf = {}
        for name, qs, sq, pbits in (("chunk4096_at_61440", APPEND_LEN, APPEND_ROWS, 4), ("prompt4096", 0, 4096, 4),
                                    ("chunk4096_at_61440_int8", APPEND_LEN, APPEND_ROWS, 8)):
            ms = time_prefill(kvq, torch, qs, sq, bits=pbits)
            fl = prefill_flops(qs, sq)
            pf[name] = {
                "q_start": qs, "sq": sq, "bits": pbits, "ms": round(ms, 4),
                "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                "mfma_frac": round(fl / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
                "cache_gbs": round(layer_bytes(qs + sq, pbits) / (ms * 1e-3) / 1e9, 1),
            }
        next_rows["prefill"] = dict(
            workload="prefill-side attention on the Llama layer's quantised cache (Hq 64, Hkv 8, D 128, fp16 q, "
                     "causal): the outlier workload's 4096-row chunk at row 61440 (int4 and 8-bit codes), and a "
                     "4096-token prompt (int4)",
            roofline="mfma: algorithmic flops 4 * Hq * D * (rows each position sees), dense fp16 peak 2500 TFLOP/s",
            timing="median of 5 calls, events around each (one kernel of milliseconds)", **pf)

    workloads = None
    if not args.no_workloads:
        gem = []
        for gs in GEMMA_SKVS:
            us, nl, gus = time_gemma_decode(kvq, torch, gs, max(20, args.steps // 2), args.warmup, pool_bytes)
            gb = gemma_bytes(gs)
            gem.append({"skv": gs, "us_per_step": round(us, 3), "gbs": round(gb / (us * 1e-6) / 1e9, 2),
                        "frac_of_hbm_peak": round(gb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                        "graph_us_per_step": round(gus, 3),
                        "graph_gbs": round(gb / (gus * 1e-6) / 1e9, 2), "pool_layers": nl})
        app_us, dec_us = time_outlier_append_decode(kvq, torch, max(20, args.steps // 2), args.warmup)
        ab = bulk_append_bytes()
        db = layer_bytes(APPEND_CAP)
        single_res, _ = time_config(kvq, torch, args.skv, args.chunk, kernel, max(20, args.steps // 2), args.warmup,
                                    pool_bytes, step="single", bits=bits)
        sb = layer_bytes(args.skv, bits) + append_bytes(bits)
        workloads = {
            "gemma_decode": {
                "workload": "Gemma-style unscaled decode layer: B1 Hq32 Hkv16 D256, softmax scale 1, Q/K rows at "
                            "unit RMS x per-channel gain U(0.5,2), V N(0,1); kvq_decode_step (AUTO) at each "
                            "context (cache capacity: the context); bytes = int4 K+V codes "
                            "+ fp16 scale/bias (4608 B per row)",
                "timing": "events around max(20, steps/2) steps over a pool of distinct layers (<= 64; the "
                          "short contexts then sit in the 256 MB last-level cache: latency-bound); graph_*: one "
                          "pass over the pool captured in a HIP graph, median of 5 replays (no host issue time)",
                "points": gem},
            "outlier_append_decode": {
                "workload": "append of 4096 fp16 rows per KV head (Llama layout B1 Hkv8 D128 G64; K Student-t(3) "
                            "with 4 channels per KV head x20, V N(0,1)) at row 61440 of a 65536-row int4 cache, "
                            "then kvq_decode_step (AUTO, Hq 64) over all 65536 rows",
                "append_us": round(app_us, 3),
                "append_bytes": ab,
                "append_gbs": round(ab / (app_us * 1e-6) / 1e9, 2),
                "append_frac_of_hbm_peak": round(ab / (app_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "decode_us": round(dec_us, 3),
                "decode_gbs": round(db / (dec_us * 1e-6) / 1e9, 2),
                "decode_frac_of_hbm_peak": round(db / (dec_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "pair_us": round(app_us + dec_us, 3),
                "timing": "append: 40 calls on 8 input sets captured in a HIP graph, median of 5 replays; "
                          "decode: events around max(20, steps/2) steps on the one cache"},
            "single_launch_step": {
                "workload": "the headline layer and step through kvq_decode_step_single_launch (the split-K "
                            "merge inside the attention launch)",
                "us_per_layer": round(single_res["ms_per_step"] * 1e3, 3),
                "gbs": round(sb / (single_res["ms_per_step"] * 1e-3) / 1e9, 2),
                "frac_of_hbm_peak": round(sb / (single_res["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "kernel_us": round(single_res["partial_ms_avg"] * 1e3, 3)},
        }

    step_bytes = layer_bytes(args.skv, bits) + append_bytes(bits)
    ms = main_res["ms_per_step"]
    value = step_bytes / (ms * 1e-3) / 1e9
    achieved = layer_bytes(args.skv, bits) / (main_res["partial_ms_avg"] * 1e-3) / 1e9
    calib = None if args.no_hbm_calibration else hbm_read_calibration(kvq, torch)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(kvq, torch, last, args.skv)

    line = {
        "metric": "effective HBM GB/s (and us/layer) of int4-KV decode SDPA, Llama-70B layer",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "us_per_layer": round(ms * 1e3, 3),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "step_spread": None if "step_ms_median" not in main_res else {
            "us_median": round(main_res["step_ms_median"] * 1e3, 3),
            "us_p10": round(main_res["step_ms_p10"] * 1e3, 3),
            "us_p90": round(main_res["step_ms_p90"] * 1e3, 3),
            "runs": main_res["step_repeats"], "steps_per_run": main_res["step_per_repeat"]},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int%d codes + fp16 scale/bias, f32 math" % bits,
        "data": "synthetic (seeded fp16 N(0,1) K/V/Q drawn on the GPU, quantised by the library)",
        "config": {
            "workload": ("Llama-3.1-70B-shaped decode layer: B1 Hq64 Hkv8 D128, int%d G64 fp16 scale+bias, "
                         "alpha 1/sqrt(128); one decode step = quantise the token's K/V row into the cache + "
                         "split-K attention over 512-row chunks + reduce" % bits),
            "step": args.step,
            "skv": args.skv,
            "chunk": args.chunk,
            "kernel": args.kernel,
            "global_batch": B,
            "seq_len": args.skv,
            "parallelism": "single GPU",
            "pool_layers": main_res["pool_layers"],
            "pool_mb": round(main_res["pool_mb"], 1),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": ("sdpa_partial_mfma1_kernel<128, 2, false, 2, %d, 8> (the decode step's attention launch: "
                       "eight-wavefront workgroups, appends the row, one merged partial per workgroup)" % bits
                       if args.step == "fused" and args.kernel in ("auto", "mfma") else
                       "the attention launch of the step (also appends the row in the fused steps)"),
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(args.skv, args.chunk, args.kernel, bits, args.step),
            "bytes_per_launch": layer_bytes(args.skv, bits),
            "avg_launch_us": round(main_res["partial_ms_avg"] * 1e3, 3),
            "timing": "HIP events recorded in the kernel's own dispatch (hipExtLaunchKernel), averaged over the steps",
            "p10_launch_us": round(main_res["partial_ms_p10"] * 1e3, 3),
            "p90_launch_us": round(main_res["partial_ms_p90"] * 1e3, 3),
            "achievable": None if calib is None else dict(
                calib, frac=round(achieved / calib["gbs"], 4),
                note="the attention kernel's achieved bandwidth as a fraction of this GPU's plain read rate"),
        },
        "cpu_baseline": cpu,
        "sweep": [{"skv": r["skv"], "us_per_layer": round(r["us_per_layer"], 3), "gbs": round(r["gbs"], 2),
                   "us_per_layer_graph": round(r["graph_ms_per_step"] * 1e3, 3),
                   "partial_us": round(r["partial_ms_avg"] * 1e3, 3), "partial_gbs": round(r["partial_gbs"], 2)}
                  for r in sweep],
        "sweep_note": ("us_per_layer: steps issued one by one from Python; us_per_layer_graph: one pass over "
                       "the same pool captured in a HIP graph and replayed (the host out of the loop)"),
        "full_depth": depth,
        "workloads": workloads,
        "next_rows": next_rows,
        "context": "pages' Apple-Silicon fused-kernel latency on this shape: 1.6/2.7/5.7/9.9 ms at 1K/16K/64K/128K",
    }
    def no_nan(x):  # untimed figures (the rotated step's kernel) as null
        if isinstance(x, float) and math.isnan(x):
            return None
        if isinstance(x, dict):
            return {k: no_nan(v) for k, v in x.items()}
        if isinstance(x, list):
            return [no_nan(v) for v in x]
        return x

    print(json.dumps(no_nan(line)), flush=True)


if __name__ == "__main__":
    main()
