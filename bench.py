"""Throughput of the GDN state update on one MI355X, as one JSON line.

Primary line: batched decode -- 64 requests, 16 key / 32 value heads, 128 x 128
fp32 state tiles in a 256-slot pool, bf16 q/k/v -- one step = one
gdn_decode_step over the batch (slot resolution, normalisation, decay, delta
write, read-out, state store). The K timed steps rotate over 4 GDN layers, each
with its own pool of the workload; a layer's first step reads the source slots
and writes fresh destination slots, its later steps update those in place, and
between two of its steps the other layers stream 768 MiB, so its state comes
from HBM, not the 256 MB MALL. The K steps are recorded once as a HIP graph and
replayed, as the engine on the TokenSpeed pages records its decode loop.
`value` is algorithmic bytes per second over the K timed steps (inputs
resident in HBM); a decode-shaped tile copy on the same protocol is reported
beside it as the measured ceiling.

Also measured in the same run (the metric has two halves):
  * chunked prefill of one 8192-token bf16 sequence (same head shape), reported
    under "prefill" as tokens/s and algorithmic MFMA flops against the bf16
    dense peak;
  * the long/packed prefill (219K tokens in 17 sequences), one 1M-token
    prefill (the longest context of the pages' table), the multi-turn
    resume (16 x 800 tokens from 4 shared checkpoints, then 32 decode steps at
    B = 16), fp32-input prefill, speculative verify, state pack/unpack and
    recorded decode layer stacks, each under its own key;
  * the fp64 CPU oracle on a bounded sample of the decode workload
    ("cpu_baseline", rank 0, one GPU only).

Usage: python bench.py [--gpus 1] [--steps 100] [--warmup 10]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense fp32 MFMA, TFLOP/s
METRIC = "GDN decode state-update HBM GB/s (% peak); chunked prefill tokens/s (MFMA %)"


def decode_bytes_per_request(HK, HV, dk, dv, elem):
    """Algorithmic HBM bytes of one request-step: state tile in and out (fp32),
    q and k, v and o, g and beta (fp32), the two slot indices."""
    return 2 * HV * dk * dv * 4 + 2 * HK * dk * elem + 2 * HV * dv * elem + 8 * HV + 8


def verify_bytes_per_request(K, HK, HV, dk, dv, elem):
    """Algorithmic HBM bytes of verifying K draft tokens of one request with
    every draft state stored: the source tile read once, K tiles written, and
    per token q and k, v and o, g and beta; plus the source and K destination
    indices."""
    return HV * dk * dv * 4 * (1 + K) + K * (2 * HK * dk * elem + 2 * HV * dv * elem + 8 * HV) + 4 * (1 + K)


def prefill_flops_per_token(HV, dk, dv, C=64, G=2):
    """Algorithmic MFMA flops per token of the chunk form (full chunks): W, U',
    U, inter-chunk output, intra-chunk output, state advance, shared Grams."""
    return HV * (2 * C * dk + 4 * C * dv + 6 * dk * dv + 4 * C * dk // G)


def prefill_f32_flops_per_token_head(dk, dv, C=64, G=2):
    """Algorithmic flops per token and value head of the fp32 chunk form:
    K H, Q H and the state advance (6 dk dv), the triangular T R and P U
    (2 (C + 1) dv), the triangular Gram matrices shared by the G value heads
    of a key head (2 C dk / G) and the triangular solve (C^2 / 3)."""
    return 6 * dk * dv + 2 * (C + 1) * dv + 2 * C * dk / G + C * C / 3


def prefill_bytes_per_token(HK, HV, dk, dv, elem=2):
    return 2 * HK * dk * elem + 2 * HV * dv * elem + 8 * HV


def _src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "hybrid_linear_attention_02_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(profile_name, src_names, launches_bytes_key):
    """HBM traffic per launch from a committed rocprofv3 counter summary, or
    None when the summary is missing or was taken on a different kernel."""
    path = os.path.join(ROOT, "profiles", profile_name)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != _src_hash(*src_names):
        return None
    try:
        return float(vals[launches_bytes_key])
    except (KeyError, ValueError):
        return None


DECODE_LAYERS = 4   # GDN layers the timed decode steps rotate over (HBM-only protocol)


def _decode_layers(wl, layers):
    """`layers` GDN layers of the batched workload, each its own 256-slot pool
    (the same initial tiles and slot tables): sources hold checkpoints,
    destinations come off the free list."""
    import torch
    from hybrid_linear_attention_02_amd import gdn
    init = torch.from_numpy(np.ascontiguousarray(wl.pool)).cuda()
    pools = []
    dst = None
    for _ in range(layers):
        pool = gdn.gdn_state_pool_create(wl.num_slots, wl.HV, wl.dk, wl.dv, storage=init.clone())
        pool.alloc(wl.num_slots)
        keep = set(int(s) for s in wl.src)
        for s in range(wl.num_slots):
            if s not in keep:
                pool.release(s)
        d = pool.alloc(wl.B)
        pool.validate(list(wl.src), d)
        assert dst is None or d == dst
        dst = d
        pools.append(pool)
    return init, pools, dst


def bench_decode(steps, warmup, layers=DECODE_LAYERS):
    """Batched decode, HBM-only protocol (``value`` and the roofline).

    Every timed step is one gdn_decode_step of the batched workload (64
    requests, 16/32 heads, 128 x 128 fp32 tiles in a 256-slot pool, bf16
    inputs). The K steps rotate over `layers` GDN layers, each with its own
    pool: step s updates layer s % layers, whose first step reads the source
    checkpoints and writes fresh slots and whose later steps update those in
    place. Between two steps of a layer the other layers read and write
    3 x 256 MiB, so the 256 MB MALL holds none of that layer's 128 MiB of
    state: the steps stream HBM, as a decode step does in a model whose other
    layers run in between. The K steps are recorded once as a HIP graph (the
    engine on the pages records its decode loop) and replayed.

    Reported beside it: the same K steps on one layer (in place, whose 128
    MiB working set the MALL can hold: warm), eager launches, and single
    launches after a 1 GiB device write (cold)."""
    import torch
    from hybrid_linear_attention_02_amd import gdn
    from hybrid_linear_attention_02_amd.workloads import batched_decode

    wl = batched_decode(steps=max(steps, 1) + warmup)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    inputs = [(bf(t.q), bf(t.k), bf(t.v), dev(t.g), dev(t.beta)) for t in wl.steps]
    init, pools, dst = _decode_layers(wl, layers)
    src_t = torch.tensor(wl.src, dtype=torch.int32, device="cuda")
    dst_t = torch.tensor(dst, dtype=torch.int32, device="cuda")
    o = torch.empty((wl.B, wl.HV, wl.dv), dtype=torch.bfloat16, device="cuda")
    per_req = decode_bytes_per_request(wl.HK, wl.HV, wl.dk, wl.dv, 2)
    bytes_step = wl.B * per_req
    stream = torch.cuda.current_stream()

    def step(pool, i, first):
        q, k, v, g, b = inputs[i]
        gdn.gdn_decode_step(pool, q, k, v, g, b, o, src_t if first else dst_t, dst_t)

    def reset():
        for p in pools:
            p.storage.copy_(init)
        torch.cuda.synchronize()

    for i in range(warmup):
        step(pools[i % layers], steps + i, i < layers)
    torch.cuda.synchronize()

    def record(n_layers):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            for i in range(steps):
                step(pools[i % n_layers], i, i < n_layers)
        torch.cuda.synchronize()
        return graph

    def replay(graph):
        reset()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record(stream)
        graph.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1), time.perf_counter() - t0

    g_rot = record(layers)
    span_ms, wall = replay(g_rot)
    value = bytes_step * steps / (span_ms * 1e-3) / 1e9
    launch_ms = span_ms / steps               # average launch duration inside the replay
    achieved = bytes_step / (launch_ms * 1e-3) / 1e9
    del g_rot
    g_one = record(1)
    warm_ms, _ = replay(g_one)
    del g_one

    # eager launches on the rotating layers, each bracketed by its own events
    reset()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        step(pools[i % layers], i, i < layers)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    eager_ms = np.array([a.elapsed_time(b) for a, b in ev])
    eager_span = ev[0][0].elapsed_time(ev[-1][1])

    # cold-cache figure: each launch preceded by a 1 GiB write (outside the events)
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    cold = []
    for i in range(20):
        flush.fill_(float(i))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step(pools[0], i, False)
        b.record(stream)
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(b))
    del flush
    cold_gbs = bytes_step / (float(np.median(cold)) * 1e-3) / 1e9

    # decode-shaped copy on the same protocol: the library's tile gather
    # (gdn_state_pool_pack: one workgroup per 64 KiB tile, 128-bit
    # non-temporal loads and stores, as the decode kernel streams its tiles)
    # of the same 64 slots x 32 heads per step, rotating over the layers
    # into one buffer per layer: 128 MiB read + 128 MiB written per step
    bufs = [torch.empty((wl.B, wl.HV, wl.dk, wl.dv), dtype=torch.float32, device="cuda") for _ in range(layers)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g_copy = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_copy, stream=side):
        for i in range(steps):
            gdn.gdn_state_pool_pack(pools[i % layers], dst_t, bufs[i % layers])
    torch.cuda.synchronize()
    copy_ms, _ = replay(g_copy)
    copy_bytes = 2 * wl.B * wl.HV * wl.dk * wl.dv * 4
    copy_gbs = copy_bytes * steps / (copy_ms * 1e-3) / 1e9
    del g_copy, bufs
    traffic = _traffic("decode_counters_batched_b64_h32_128x128.txt", ["gdn_decode.hip"], "hbm_bytes_per_launch")
    for p in pools:
        p.close()
    return dict(
        value=value, ms_per_step=span_ms / steps, wall_s=wall, achieved=achieved, cold_gbs=cold_gbs,
        warm_gbs=bytes_step * steps / (warm_ms * 1e-3) / 1e9, tile_copy_gbs=copy_gbs, layers=layers,
        bytes_step=bytes_step, per_req=per_req, B=wl.B, HK=wl.HK, HV=wl.HV, dk=wl.dk, dv=wl.dv,
        launch_ms_mean=launch_ms, traffic=traffic,
        eager={"launch_us_mean": float(eager_ms.mean() * 1e3), "launch_us_median": float(np.median(eager_ms) * 1e3),
               "span_us_per_step": float(eager_span / steps * 1e3),
               "gbs_per_launch": bytes_step / (float(eager_ms.mean()) * 1e-3) / 1e9})


def bench_prefill(reps=20, warmup=3):
    """Chunked prefill of one 8192-token sequence from a zero state into slot 1.

    Three timings of the same call (repeats are idempotent: zero initial state,
    same destination):
      * steady state (``value``): `reps` calls issued back to back between two
        events, the host running ahead of the GPU as in a pipelined engine;
      * graph replay: the call recorded once as a HIP graph and replayed `reps`
        times (no host work inside the timed region; outputs checked equal to
        the eager call's);
      * latency: median of single calls, each synchronised, host marshalling
        and planning included.
    """
    import torch
    from hybrid_linear_attention_02_amd import gdn
    from hybrid_linear_attention_02_amd.workloads import chunked_prefill

    pw = chunked_prefill()
    tk = pw.tokens
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v, g, b = bf(tk.q), bf(tk.k), bf(tk.v), dev(tk.g), dev(tk.beta)
    T = int(pw.cu_seqlens[-1])
    o = torch.empty((T, pw.HV, pw.dv), dtype=torch.bfloat16, device="cuda")
    storage = torch.zeros((pw.num_slots, pw.HV, pw.dk, pw.dv), dtype=torch.float32, device="cuda")
    pool = gdn.gdn_state_pool_create(pw.num_slots, pw.HV, pw.dk, pw.dv, storage=storage)
    pool.alloc(pw.num_slots)
    cu = dev(pw.cu_seqlens)
    src = torch.tensor([-1], dtype=torch.int32, device="cuda")
    dst = torch.tensor([1], dtype=torch.int32, device="cuda")
    ws = None
    call = lambda: gdn.gdn_prefill_chunked(pool, q, k, v, g, b, o, cu, pw.cu_seqlens, src, dst, workspace=ws)
    for _ in range(warmup):
        ws = gdn.gdn_prefill_chunked(pool, q, k, v, g, b, o, cu, pw.cu_seqlens, src, dst, workspace=ws)
    torch.cuda.synchronize()
    o_ref = o.clone()
    s_ref = storage[1].clone()

    def span(fn, n):
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(n):
            fn()
        e.record()
        torch.cuda.synchronize()
        return a.elapsed_time(e) / n * 1e-3

    steady = span(call, reps)
    lat = []
    for _ in range(reps):
        lat.append(span(call, 1))
    latency = float(np.median(lat))

    # cold: a 1 GiB device write before each call evicts the inputs from the
    # MALL; the write is still running while the call is enqueued, so the
    # events bracket the kernels alone
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    cold = []
    for i in range(reps):
        flush.fill_(float(i))
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        call()
        e.record(stream)
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(e) * 1e-3)
    del flush
    cold_s = float(np.median(cold))

    graph_s = None
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    o.zero_()
    graph_s = span(graph.replay, reps)
    graph_ok = bool(torch.equal(o, o_ref) and torch.equal(storage[1], s_ref))

    flops = T * prefill_flops_per_token(pw.HV, pw.dk, pw.dv)
    tflops = flops / steady / 1e12
    pool.close()
    return {
        "workload": "chunked_prefill_bf16_t8192_hk16_hv32_128x128_c64",
        "value": T / steady, "unit": "tok/s", "ms": steady * 1e3, "dtype": "bf16",
        "graph_ms": graph_s * 1e3, "graph_matches_eager": graph_ok,
        "latency_ms": latency * 1e3, "cold_ms": cold_s * 1e3,
        "timing": "value: back-to-back calls (host overlapped); graph_ms: HIP-graph replay; "
                  "latency_ms: one synchronised call including host marshalling and planning; "
                  "cold_ms: median of single calls, each after a 1 GiB device write",
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / BF16_PEAK_TFLOPS,
                     "traffic": _traffic("prefill_t8192_counters.md", ["gdn_prefill.hip", "gdn_prefill_common.h", "gdn_abi.cpp"],
                                         "hbm_bytes_per_call"),
                     "scope": "whole gdn_prefill_chunked call (prep + intra-chunk + recurrence kernels)"},
        "algorithmic_gflop": flops / 1e9,
        "hbm_gbs_algorithmic": (T * prefill_bytes_per_token(pw.HK, pw.HV, pw.dk, pw.dv) + pw.HV * pw.dk * pw.dv * 4)
        / steady / 1e9,
    }


def bench_prefill_packed(reps=10, warmup=3):
    """Chunked prefill of the long/packed workload: one 50,000-token sequence
    plus 16 sequences of U[1K, 16K] tokens in one call, zero initial states,
    16/32 heads, 128 x 128 bf16. Many independent (sequence, head) chains fill
    more of the chip than the single 8192-token sequence. `warmup` untimed
    calls, then `reps` calls back to back between two events."""
    import torch
    from hybrid_linear_attention_02_amd import gdn
    from hybrid_linear_attention_02_amd.workloads import long_packed_prefill

    pw = long_packed_prefill()
    tk = pw.tokens
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v, g, b = bf(tk.q), bf(tk.k), bf(tk.v), dev(tk.g), dev(tk.beta)
    T = int(pw.cu_seqlens[-1])
    N = len(pw.cu_seqlens) - 1
    o = torch.empty((T, pw.HV, pw.dv), dtype=torch.bfloat16, device="cuda")
    pool = gdn.gdn_state_pool_create(pw.num_slots, pw.HV, pw.dk, pw.dv)
    pool.alloc(pw.num_slots)
    cu = dev(pw.cu_seqlens)
    src = torch.full((N,), -1, dtype=torch.int32, device="cuda")
    dst = torch.arange(1, N + 1, dtype=torch.int32, device="cuda")
    ws = gdn.gdn_prefill_chunked(pool, q, k, v, g, b, o, cu, pw.cu_seqlens, src, dst)
    for _ in range(warmup - 1):
        gdn.gdn_prefill_chunked(pool, q, k, v, g, b, o, cu, pw.cu_seqlens, src, dst, workspace=ws)
    torch.cuda.synchronize()
    a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        gdn.gdn_prefill_chunked(pool, q, k, v, g, b, o, cu, pw.cu_seqlens, src, dst, workspace=ws)
    e.record()
    torch.cuda.synchronize()
    t = a.elapsed_time(e) / reps * 1e-3
    tflops = T * prefill_flops_per_token(pw.HV, pw.dk, pw.dv) / t / 1e12
    pool.close()
    del ws, o, q, k, v
    return {"workload": f"long_packed_prefill_bf16_{N}seqs_t{T}_hk16_hv32_128x128", "tokens": T, "ms": round(t * 1e3, 3),
            "tok_per_s": round(T / t, 1), "tflops_algorithmic": round(tflops, 1),
            "frac_bf16_mfma": round(tflops / BF16_PEAK_TFLOPS, 4)}


def bench_resume(reps=20, warmup=3):
    """Multi-turn resume: 16 sequences of 800 bf16 tokens resume from 4 shared
    checkpoint slots into fresh slots (the checkpoints are only read), then
    32 decode steps at B = 16 in place on the fresh slots, 16/32 heads,
    128 x 128. The prefill is timed as `reps` calls back to back (each call
    reads the same checkpoints and rewrites the same fresh slots); the 32
    decode steps are recorded once as a HIP graph and replayed."""
    import torch
    from hybrid_linear_attention_02_amd import gdn
    from hybrid_linear_attention_02_amd.workloads import multiturn_resume

    pw, dec = multiturn_resume()
    tk = pw.tokens
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v, g, b = bf(tk.q), bf(tk.k), bf(tk.v), dev(tk.g), dev(tk.beta)
    T = int(pw.cu_seqlens[-1])
    N = len(pw.cu_seqlens) - 1
    storage = dev(pw.pool)
    pool = gdn.gdn_state_pool_create(pw.num_slots, pw.HV, pw.dk, pw.dv, storage=storage)
    ck = pool.alloc(4)
    for c in ck:
        for _ in range(4):
            pool.retain(c)
    src = [int(s) for s in pw.src]
    dst = [pool.cow(s) for s in src]
    pool.validate(src, dst)
    src_t = torch.tensor(src, dtype=torch.int32, device="cuda")
    dst_t = torch.tensor(dst, dtype=torch.int32, device="cuda")
    cu = dev(pw.cu_seqlens)
    o = torch.empty((T, pw.HV, pw.dv), dtype=torch.bfloat16, device="cuda")
    ws = gdn.gdn_prefill_chunked(pool, q, k, v, g, b, o, cu, pw.cu_seqlens, src_t, dst_t)
    for _ in range(warmup - 1):
        gdn.gdn_prefill_chunked(pool, q, k, v, g, b, o, cu, pw.cu_seqlens, src_t, dst_t, workspace=ws)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        gdn.gdn_prefill_chunked(pool, q, k, v, g, b, o, cu, pw.cu_seqlens, src_t, dst_t, workspace=ws)
    e.record(stream)
    torch.cuda.synchronize()
    t_pre = a.elapsed_time(e) / reps * 1e-3
    flops = T * prefill_flops_per_token(pw.HV, pw.dk, pw.dv)
    state_bytes = pw.HV * pw.dk * pw.dv * 4
    pre_bytes = T * prefill_bytes_per_token(pw.HK, pw.HV, pw.dk, pw.dv) + 2 * N * state_bytes

    # decode: 32 steps in place on the fresh slots, recorded once
    inputs = [(bf(t.q), bf(t.k), bf(t.v), dev(t.g), dev(t.beta)) for t in dec]
    od = torch.empty((N, pw.HV, pw.dv), dtype=torch.bfloat16, device="cuda")
    for i in range(min(warmup, len(inputs))):
        gdn.gdn_decode_step(pool, *inputs[i], od, dst_t, dst_t)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for inp in inputs:
            gdn.gdn_decode_step(pool, *inp, od, dst_t, dst_t)
    torch.cuda.synchronize()
    a.record(stream)
    graph.replay()
    e.record(stream)
    torch.cuda.synchronize()
    t_dec = a.elapsed_time(e) / len(inputs) * 1e-3
    dec_bytes = N * decode_bytes_per_request(pw.HK, pw.HV, pw.dk, pw.dv, 2)
    del graph
    pool.close()
    del ws, o, q, k, v, storage
    return {"workload": f"multiturn_resume_bf16_{N}x{T // N}_from_4_checkpoints_then_{len(inputs)}_decode_steps_b{N}",
            "prefill_ms": round(t_pre * 1e3, 4), "prefill_tok_per_s": round(T / t_pre, 1),
            "prefill_tflops_algorithmic": round(flops / t_pre / 1e12, 1),
            "prefill_frac_bf16_mfma": round(flops / t_pre / 1e12 / BF16_PEAK_TFLOPS, 4),
            "prefill_gbs_algorithmic": round(pre_bytes / t_pre / 1e9, 1),
            "decode_us_per_step": round(t_dec * 1e6, 2), "decode_bytes_per_step": dec_bytes,
            "decode_gbs": round(dec_bytes / t_dec / 1e9, 1),
            "decode_frac_hbm": round(dec_bytes / t_dec / 1e9 / HBM_PEAK_GBS, 4),
            "timing": "prefill: back-to-back calls between two events; decode: HIP-graph replay of the 32 steps",
            "note": "the 16 fresh slots (32 MiB of state) stay in the 256 MB MALL between decode steps"}


def bench_prefill_long_context(tokens=1 << 20, reps=3):
    """Chunked prefill of one 1,048,576-token sequence at the batched head
    shape (16/32 heads, 128 x 128, bf16), the longest context of the pages'
    long-context table; inputs drawn on the device from a seeded generator
    (q, k, v ~ N(0, 1), g = -U(0.01, 0.5), beta = sigmoid(N(0, 1))), zero
    initial state. One untimed call, then `reps` calls back to back."""
    import torch
    from hybrid_linear_attention_02_amd import gdn

    HK, HV, DK, DV = 16, 32, 128, 128
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20)
    q = torch.randn((tokens, HK, DK), generator=gen, device="cuda", dtype=torch.bfloat16)
    k = torch.randn((tokens, HK, DK), generator=gen, device="cuda", dtype=torch.bfloat16)
    v = torch.randn((tokens, HV, DV), generator=gen, device="cuda", dtype=torch.bfloat16)
    g = -(0.01 + 0.49 * torch.rand((tokens, HV), generator=gen, device="cuda"))
    b = torch.sigmoid(torch.randn((tokens, HV), generator=gen, device="cuda"))
    o = torch.empty((tokens, HV, DV), dtype=torch.bfloat16, device="cuda")
    pool = gdn.gdn_state_pool_create(2, HV, DK, DV)
    pool.alloc(2)
    cu_host = np.asarray([0, tokens], np.int32)
    cu = torch.from_numpy(cu_host).cuda()
    src = torch.tensor([-1], dtype=torch.int32, device="cuda")
    dst = torch.tensor([1], dtype=torch.int32, device="cuda")
    ws = gdn.gdn_prefill_chunked(pool, q, k, v, g, b, o, cu, cu_host, src, dst)
    torch.cuda.synchronize()
    a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        gdn.gdn_prefill_chunked(pool, q, k, v, g, b, o, cu, cu_host, src, dst, workspace=ws)
    e.record()
    torch.cuda.synchronize()
    t = a.elapsed_time(e) / reps * 1e-3
    tflops = tokens * prefill_flops_per_token(HV, DK, DV) / t / 1e12
    pool.close()
    del q, k, v, g, b, o, ws
    torch.cuda.empty_cache()
    return {"workload": f"long_context_prefill_bf16_t{tokens}_hk16_hv32_128x128", "tokens": tokens,
            "ms": round(t * 1e3, 3), "tok_per_s": round(tokens / t, 1), "tflops_algorithmic": round(tflops, 1),
            "frac_bf16_mfma": round(tflops / BF16_PEAK_TFLOPS, 4),
            "data": "synthetic, drawn on the device from a seeded generator"}


def bench_prefill_f32(reps=5):
    """Prefill with float32 inputs at 16/32 heads, 128 x 128: one 8192-token
    sequence, and 16 sequences of 800 tokens from zero states. The chunk form
    runs with every product on the fp32 MFMA. Flops are the chunk form's
    algorithmic count per token and value head: 6 dk dv (K H, Q H and the
    state advance), 2 (C + 1) dv (the triangular T R and P U), 2 C dk / G (the
    triangular Gram matrices, shared by the G value heads of a key head) and
    C^2 / 3 (the triangular solve), C = 64; against the dense fp32 MFMA peak."""
    import torch
    from hybrid_linear_attention_02_amd import gdn
    from hybrid_linear_attention_02_amd.workloads import F32, prefill_workload

    flops_per_tok = prefill_f32_flops_per_token_head(128, 128)
    out = {}
    for name, lengths in (("one_seq_t8192", [8192]), ("packed_16x800", [800] * 16)):
        pw = prefill_workload(name, seed=2, lengths=lengths, HK=16, HV=32, dk=128, dv=128, dtype=F32,
                              num_slots=2 * len(lengths))
        tk = pw.tokens
        d = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
        q, k, v, g, b = d(tk.q), d(tk.k), d(tk.v), d(tk.g), d(tk.beta)
        o = torch.empty_like(v)
        pool = gdn.gdn_state_pool_create(pw.num_slots, 32, 128, 128)
        pool.alloc(pw.num_slots)
        N = len(lengths)
        src = torch.full((N,), -1, dtype=torch.int32, device="cuda")
        dst = torch.arange(N, 2 * N, dtype=torch.int32, device="cuda")
        cu = d(pw.cu_seqlens)
        ws = gdn.gdn_prefill_chunked(pool, q, k, v, g, b, o, cu, pw.cu_seqlens, src, dst)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            gdn.gdn_prefill_chunked(pool, q, k, v, g, b, o, cu, pw.cu_seqlens, src, dst, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / reps * 1e-3
        T = int(pw.cu_seqlens[-1])
        tflops = flops_per_tok * 32 * T / t / 1e12
        out[name] = {"ms": round(t * 1e3, 3), "tok_per_s": round(T / t, 1),
                     "tflops_fp32": round(tflops, 2), "frac_fp32_mfma": round(tflops / FP32_MFMA_PEAK_TFLOPS, 4)}
        pool.close()
    out["bound"] = "mfma (fp32 16x16x4; the chunk recurrence is sequential per (sequence, head, 16 columns))"
    out["traffic_one_seq_t8192"] = _traffic("prefill_f32_t8192_counters.md",
                                            ["gdn_prefill.hip", "gdn_prefill_common.h", "gdn_prefill_f32.hip",
                                             "gdn_abi.cpp"], "hbm_bytes_per_call")
    out["flops_per_token_head"] = flops_per_tok
    return out


def bench_verify(reps=48, warmup=8, layers=4):
    """Speculative-decode verification: 64 requests x 4 draft tokens at the
    16/32-head 128 x 128 bf16 shape, every draft state stored (one launch).

    HBM-only protocol: launches rotate over `layers` GDN layers, each with
    its own 320-slot pool; between two launches of a layer the others read
    3 x 128 MiB of sources and write 3 x 512 MiB, so the 256 MB MALL holds
    none of a layer's sources when it runs. Launches are idempotent (sources
    are only read), so they run back to back between two events. Reported
    beside it: the same launches on one layer (warm: its 128 MiB of sources
    can stay in the MALL), and a copy of the same traffic shape (torch's
    broadcast copy of the source tiles to the 4 destinations) on the same
    rotation."""
    import torch
    from hybrid_linear_attention_02_amd import gdn
    from hybrid_linear_attention_02_amd.workloads import spec_verify

    wl = spec_verify()
    B, K = wl.B, wl.K
    tk = wl.tokens
    shp = lambda x: np.ascontiguousarray(x.reshape((B, K) + x.shape[1:]))
    bf = lambda x: torch.from_numpy(shp(x).view(np.int16)).view(torch.bfloat16).cuda()
    dv_ = lambda x: torch.from_numpy(shp(x)).cuda()
    q, k, v, g, b = bf(tk.q), bf(tk.k), bf(tk.v), dv_(tk.g), dv_(tk.beta)
    init = torch.from_numpy(wl.pool).cuda()
    pools = [gdn.gdn_state_pool_create(wl.num_slots, wl.HV, wl.dk, wl.dv, storage=init.clone())
             for _ in range(layers)]
    src = torch.tensor(wl.src, dtype=torch.int32, device="cuda")
    free = np.setdiff1d(np.arange(wl.num_slots), wl.src)[:B * K]
    dst = torch.tensor(free.reshape(B, K), dtype=torch.int32, device="cuda")
    o = torch.empty_like(v)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, n_layers):
        for i in range(warmup):
            fn(i % n_layers)
        torch.cuda.synchronize()
        e0.record()
        for i in range(reps):
            fn(i % n_layers)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    call = lambda i: gdn.gdn_decode_verify(pools[i], q, k, v, g, b, o, src, dst)
    t = timed(call, layers)
    t_warm = timed(call, 1)
    per_req = verify_bytes_per_request(K, wl.HK, wl.HV, wl.dk, wl.dv, 2)
    gbs = B * per_req / t / 1e9
    for pl in pools:
        pl.close()
    del pools
    # a copy of the same shape on the same rotation: each layer's 64 source
    # tiles (128 MiB) read once and written to K destinations each
    tiles = [init[src.long()].contiguous() for _ in range(layers)]
    outs = [torch.empty((K,) + tuple(tiles[0].shape), dtype=torch.float32, device="cuda") for _ in range(layers)]
    copy = lambda i: outs[i].copy_(tiles[i].unsqueeze(0).expand_as(outs[i]))
    tc = timed(copy, layers)
    copy_gbs = (1 + K) * tiles[0].numel() * 4 / tc / 1e9
    del outs, tiles
    return {"workload": "spec_verify_bf16_b64_k4_hk16_hv32_128x128", "value": B * K / t, "unit": "draft tok/s",
            "us_per_launch": t * 1e6, "gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
            "bytes_per_launch": B * per_req, "layers_rotated": layers,
            "warm_one_layer_us": t_warm * 1e6, "warm_one_layer_gbs": B * per_req / t_warm / 1e9,
            "verify_shaped_copy_gbs": copy_gbs, "vs_verify_shaped_copy": gbs / copy_gbs,
            "copy_protocol": f"the {B} source tiles x {wl.HV} heads read once and written to {K} destinations each "
                             f"(torch broadcast copy), rotating over {layers} copies",
            "vs_decode_steps": "one launch reads each source tile once for 4 tokens; 4 decode steps would move "
                               f"{4 * B * decode_bytes_per_request(wl.HK, wl.HV, wl.dk, wl.dv, 2) / 1e6:.0f} MB "
                               f"against {B * per_req / 1e6:.0f} MB"}


def bench_transfer(reps=20):
    """State hand-over: pack the 64 batched-decode requests' slots (all 32
    heads, 128 x 128 fp32: 134 MB) into one buffer, then unpack it into other
    slots; GB/s counts bytes read plus bytes written."""
    import torch
    from hybrid_linear_attention_02_amd import gdn
    from hybrid_linear_attention_02_amd.workloads import batched_decode

    wl = batched_decode(steps=1)
    storage = torch.from_numpy(wl.pool).cuda()
    pool = gdn.gdn_state_pool_create(wl.num_slots, wl.HV, wl.dk, wl.dv, storage=storage)
    src = torch.tensor(wl.src, dtype=torch.int32, device="cuda")
    dst = torch.tensor(np.setdiff1d(np.arange(wl.num_slots), wl.src)[:wl.B], dtype=torch.int32, device="cuda")
    buf = torch.empty((wl.B, wl.HV, wl.dk, wl.dv), dtype=torch.float32, device="cuda")
    nbytes = buf.numel() * 4

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    tp = timed(lambda: gdn.gdn_state_pool_pack(pool, src, buf))
    tu = timed(lambda: gdn.gdn_state_pool_unpack(pool, dst, buf))
    pool.close()
    return {"workload": "pack/unpack of 64 slots x 32 heads x 128x128 fp32", "bytes_each_way": nbytes,
            "pack_us": tp * 1e6, "pack_gbs": 2 * nbytes / tp / 1e9,
            "unpack_us": tu * 1e6, "unpack_gbs": 2 * nbytes / tu / 1e9}


def bench_graph(reps=200, warmup=20):
    """Launch overhead of a whole decode step: the same decode launches made
    one by one through the Python binding ("binding", what a Python-driven
    scheduler pays per launch), through the C ABI with prebuilt argument
    structs ("eager"), and replayed as one recorded graph. Rates are wall-clock
    over `reps` back-to-back steps, host launch cost included.
      tiny_chain: the tiny fp32 workload's 8 sequential tokens (1 request,
        2 value heads, 16 x 16), slot 1 -> 2 then in place; also as one
        verify launch over the 8 known tokens (Python binding call included);
      stack_b{B}: one token through 32 GDN layers (own storages, in place) at
        16/32 heads, 128 x 128 bf16, for B = 1 and 8 requests."""
    import ctypes
    import time
    import torch
    from hybrid_linear_attention_02_amd import gdn
    from hybrid_linear_attention_02_amd.workloads import BF16, decode_workload, tiny_decode

    lib = gdn.load_library()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def dev(x, dt):
        if dt == BF16:
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()

    def run(pool, entries, storages):
        keep = []
        args = [gdn.decode_args(*e, err_flag=err) for e in entries]
        graph = gdn.DecodeGraph(pool, args, storages=storages, keep=entries)
        handle = ctypes.c_void_p(pool.handle)
        eager_pools, pool_objs = [], []
        for t in (storages or [None] * len(entries)):
            if t is None:
                eager_pools.append(handle)
                pool_objs.append(pool)
            else:
                p = gdn.gdn_state_pool_create(pool.num_slots, pool.num_v_heads, pool.dk, pool.dv, storage=t)
                p.alloc(pool.num_slots)
                keep.append(p)
                eager_pools.append(ctypes.c_void_p(p.handle))
                pool_objs.append(p)
        refs = [ctypes.byref(a) for a in args]

        def binding():
            for p, e in zip(pool_objs, entries):
                gdn.gdn_decode_step(p, *e, err_flag=err)

        def eager():
            for h, a in zip(eager_pools, refs):
                if lib.gdn_decode_step(h, a, sp) != 0:
                    raise RuntimeError(gdn.gdn_last_error())

        gh = ctypes.c_void_p(graph.handle)

        def replay():
            if lib.gdn_decode_graph_launch(gh, sp) != 0:
                raise RuntimeError(gdn.gdn_last_error())

        out = {}
        for name, fn in (("binding", binding), ("eager", eager), ("graph", replay)):
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(reps):
                fn()
            torch.cuda.synchronize()
            out[name] = (time.perf_counter() - t0) / reps
        n, f = graph.poll()
        assert n == warmup + reps and f == 0, (n, f)
        assert int(err.item()) == 0
        graph.close()
        for p in keep:
            p.close()
        return out

    res = {}
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    # tiny chain
    wl = tiny_decode(steps=8)
    storage = torch.from_numpy(wl.pool.copy()).cuda()
    pool = gdn.gdn_state_pool_create(wl.num_slots, wl.HV, wl.dk, wl.dv, storage=storage)
    pool.alloc(wl.num_slots)
    t1, t2, t22 = [torch.tensor([x], dtype=torch.int32, device="cuda") for x in (1, 2, 2)]
    entries = []
    for i, tk in enumerate(wl.steps):
        q, k, v = dev(tk.q, wl.dtype), dev(tk.k, wl.dtype), dev(tk.v, wl.dtype)
        entries.append((q, k, v, dev(tk.g, None), dev(tk.beta, None), torch.empty_like(v),
                        t1 if i == 0 else t22, t2 if i == 0 else t22))
    r = run(pool, entries, None)
    # the same 8 known tokens as one verify launch (slot 1 -> the state after
    # every token kept in slot 2, i.e. in place after the first): the chain
    # then runs inside one kernel with the state in registers
    cat = lambda i: torch.stack([e[i][0] for e in entries])[None]
    vq, vk, vv, vg, vb = (cat(i) for i in range(5))
    vo = torch.empty_like(vv)
    vsrc = torch.tensor([1], dtype=torch.int32, device="cuda")
    vdst = torch.tensor([[-1] * 7 + [2]], dtype=torch.int32, device="cuda")
    fused = lambda: gdn.gdn_decode_verify(pool, vq, vk, vv, vg, vb, vo, vsrc, vdst)
    for _ in range(warmup):
        fused()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        fused()
    torch.cuda.synchronize()
    t_fused = (time.perf_counter() - t0) / reps
    res["tiny_chain_8_tokens"] = {"binding_us_per_token": r["binding"] / 8 * 1e6,
                                  "eager_us_per_token": r["eager"] / 8 * 1e6,
                                  "graph_us_per_token": r["graph"] / 8 * 1e6,
                                  "one_verify_launch_us_per_token": t_fused / 8 * 1e6,
                                  "speedup": r["eager"] / r["graph"],
                                  "speedup_vs_binding": r["binding"] / r["graph"]}
    pool.close()
    # layer stacks
    L = 32
    for B in (1, 8):
        wl = decode_workload(f"stack_b{B}", seed=60 + B, B=B, HK=16, HV=32, dk=128, dv=128, dtype=BF16,
                             num_slots=B, pool_sigma=0.05, steps=1)
        tk = wl.steps[0]
        pool = gdn.gdn_state_pool_create(B, 32, 128, 128)
        pool.alloc(B)
        slots = torch.arange(B, dtype=torch.int32, device="cuda")
        q, k, v = dev(tk.q, BF16), dev(tk.k, BF16), dev(tk.v, BF16)
        g, beta = dev(tk.g, None), dev(tk.beta, None)
        storages = [torch.from_numpy(wl.pool).cuda() for _ in range(L)]
        entries = [(q, k, v, g, beta, torch.empty_like(v), slots, slots) for _ in range(L)]
        r = run(pool, entries, storages)
        res[f"stack_b{B}_32_layers"] = {"binding_us_per_step": r["binding"] * 1e6,
                                        "eager_us_per_step": r["eager"] * 1e6, "graph_us_per_step": r["graph"] * 1e6,
                                        "graph_us_per_layer": r["graph"] / L * 1e6,
                                        "speedup": r["eager"] / r["graph"],
                                        "speedup_vs_binding": r["binding"] / r["graph"]}
        pool.close()
        del storages
    return {k: {kk: round(vv, 3) for kk, vv in v.items()} for k, v in res.items()}


def _oracle_worker(args):
    os.environ["OMP_NUM_THREADS"] = "1"
    (pool_part, src, dst, steps_part, scale, repeats) = args
    from oracle import bf16_bits_to_f64, decode_step
    t0 = time.perf_counter()
    for _ in range(repeats):
        p = pool_part
        for i, (q, k, v, g, b) in enumerate(steps_part):
            s = src if i == 0 else dst
            _, p, _ = decode_step(p, s, dst, bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), g, b,
                                  scale, 1e-6)
    return time.perf_counter() - t0


def _oracle_prefill_worker(args):
    os.environ["OMP_NUM_THREADS"] = "1"
    (q, k, v, g, b, dk, dv, scale) = args
    from oracle import bf16_bits_to_f64, recurrent_sequence
    t0 = time.perf_counter()
    recurrent_sequence(np.zeros((v.shape[1], dk, dv)), bf16_bits_to_f64(q), bf16_bits_to_f64(k),
                       bf16_bits_to_f64(v), g, b, scale, 1e-6)
    return time.perf_counter() - t0


def cpu_baseline_prefill(tokens=8192):
    """The fp64 oracle's token loop on the first `tokens` tokens of the
    8192-token prefill workload, all 32 value heads, one process per key head
    (at most the host's cores, 16 at most)."""
    from concurrent.futures import ProcessPoolExecutor
    from hybrid_linear_attention_02_amd.workloads import chunked_prefill

    pw = chunked_prefill()
    tk = pw.tokens
    cores = max(1, min(len(os.sched_getaffinity(0)), 16, pw.HK))
    G = pw.HV // pw.HK
    jobs = []
    for js in np.array_split(np.arange(pw.HK), cores):
        hv = np.concatenate([np.arange(j * G, (j + 1) * G) for j in js])
        jobs.append((tk.q[:tokens, js], tk.k[:tokens, js], tk.v[:tokens, hv], tk.g[:tokens, hv],
                     tk.beta[:tokens, hv], pw.dk, pw.dv, pw.dk ** -0.5))
    t0 = time.perf_counter()
    with ProcessPoolExecutor(max_workers=cores) as ex:
        per = list(ex.map(_oracle_prefill_worker, jobs))
    wall = time.perf_counter() - t0
    flop = tokens * pw.HV * 7 * pw.dk * pw.dv
    return {"value": tokens / wall, "unit": "tok/s", "cores": cores, "kind": "oracle",
            "sample": f"first {tokens} tokens of the 8192-token workload, all {pw.HV} value heads; fp64 token "
                      f"loop, one process per key head group ({cores} processes); wall {wall:.1f} s",
            "per_core_tok_s": float(np.mean([tokens * len(j[2][0]) / pw.HV / t for j, t in zip(jobs, per)])),
            "fp64_gflops": flop / wall / 1e9}


def cpu_baseline(per_req_bytes, repeats=8):
    """The fp64 oracle (as it stands) on the whole batched-decode workload --
    64 requests x 100 steps, run `repeats` times back to back so the timed CPU
    work lasts some seconds -- one process per host core (at most 16), each
    owning a contiguous block of requests and a private copy of their slots."""
    from concurrent.futures import ProcessPoolExecutor
    from hybrid_linear_attention_02_amd.workloads import batched_decode

    wl = batched_decode(steps=100)
    cores = max(1, min(len(os.sched_getaffinity(0)), 16, wl.B))
    groups = np.array_split(np.arange(wl.B), cores)
    jobs = []
    for rows in groups:
        src = wl.src[rows]
        npool = np.concatenate([wl.pool[src], np.zeros_like(wl.pool[src])])
        lsrc = np.arange(len(rows))
        ldst = np.arange(len(rows), 2 * len(rows))
        steps_part = [(t.q[rows], t.k[rows], t.v[rows], t.g[rows], t.beta[rows]) for t in wl.steps]
        jobs.append((npool, lsrc, ldst, steps_part, wl.dk ** -0.5, repeats))
    t0 = time.perf_counter()
    with ProcessPoolExecutor(max_workers=cores) as ex:
        per = list(ex.map(_oracle_worker, jobs))
    wall = time.perf_counter() - t0
    req_steps = wl.B * len(wl.steps) * repeats
    per_core = float(np.mean([len(rows) * len(wl.steps) * repeats / t for rows, t in zip(groups, per)]))
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": req_steps * per_req_bytes / wall / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"whole batched-decode workload (64 requests x 100 steps, 16/32 heads, 128x128) run "
                      f"{repeats} times; fp64 token loop in {cores} processes on {cpu_model or 'host CPU'}; "
                      f"{req_steps / wall:.1f} request-steps/s, wall {wall:.1f} s",
            "request_steps_per_s": req_steps / wall, "wall_s": wall,
            "per_core_request_steps_per_s": per_core,
            "fp64_gflops": req_steps * wl.HV * 7 * wl.dk * wl.dv / wall / 1e9}


def achievable():
    """Measured denominators next to the nominal peaks: a 1 GiB device copy
    (bytes read + written per second) and a bf16 8192^3 GEMM (torch.matmul)."""
    import torch
    n = 1 << 28
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    c = torch.empty_like(a)
    x = torch.randn(8192, 8192, dtype=torch.bfloat16, device="cuda")
    y = torch.randn(8192, 8192, dtype=torch.bfloat16, device="cuda")

    def best(fn, reps=10):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return min(ts)

    tc = best(lambda: c.copy_(a))
    tf = best(lambda: c.fill_(1.5))
    tg = best(lambda: torch.matmul(x, y))
    copy_gbs = 2 * n * 4 / tc / 1e9
    fill_gbs = n * 4 / tf / 1e9
    gemm = 2 * 8192 ** 3 / tg / 1e12
    del a, c, x, y
    return {"copy_gbs": round(copy_gbs, 1), "copy_frac_of_peak": round(copy_gbs / HBM_PEAK_GBS, 4),
            "fill_gbs": round(fill_gbs, 1), "fill_frac_of_peak": round(fill_gbs / HBM_PEAK_GBS, 4),
            "gemm_bf16_tflops": round(gemm, 1), "gemm_frac_of_peak": round(gemm / BF16_PEAK_TFLOPS, 4),
            "protocol": "best of 10: 1 GiB float32 device copy (bytes read + written); 1 GiB device fill "
                        "(bytes written); torch.matmul of two 8192x8192 bf16 matrices"}


def run_counters(launches=5, copy_mib=128):
    """Short run for hardware-counter passes (rocprofv3 --pmc FETCH_SIZE, then
    WRITE_SIZE): `launches` eager batched-decode steps, then one plain device
    copy of `copy_mib` MiB whose counter readings calibrate the decode ones
    (bytes actually moved / bytes the counter reports)."""
    import torch
    from hybrid_linear_attention_02_amd import gdn
    from hybrid_linear_attention_02_amd.workloads import batched_decode

    wl = batched_decode(steps=launches)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    inputs = [(bf(t.q), bf(t.k), bf(t.v), dev(t.g), dev(t.beta)) for t in wl.steps]
    storage = dev(wl.pool)
    pool = gdn.gdn_state_pool_create(wl.num_slots, wl.HV, wl.dk, wl.dv, storage=storage)
    pool.alloc(wl.num_slots)
    keep = set(int(s) for s in wl.src)
    for s in range(wl.num_slots):
        if s not in keep:
            pool.release(s)
    dst = pool.alloc(wl.B)
    src_t = torch.tensor(wl.src, dtype=torch.int32, device="cuda")
    dst_t = torch.tensor(dst, dtype=torch.int32, device="cuda")
    o = torch.empty((wl.B, wl.HV, wl.dv), dtype=torch.bfloat16, device="cuda")
    for i in range(launches):
        q, k, v, g, b = inputs[i]
        gdn.gdn_decode_step(pool, q, k, v, g, b, o, src_t if i == 0 else dst_t, dst_t)
    torch.cuda.synchronize()
    n = copy_mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    c = torch.empty_like(a)
    c.copy_(a)
    torch.cuda.synchronize()
    pool.close()
    del a, c
    # two calls of the 8192-token prefill (the second one is the one to read)
    from hybrid_linear_attention_02_amd.workloads import chunked_prefill
    pw = chunked_prefill()
    tk = pw.tokens
    pq, pk, pv, pg, pb = bf(tk.q), bf(tk.k), bf(tk.v), dev(tk.g), dev(tk.beta)
    T = int(pw.cu_seqlens[-1])
    po = torch.empty((T, pw.HV, pw.dv), dtype=torch.bfloat16, device="cuda")
    pst = torch.zeros((pw.num_slots, pw.HV, pw.dk, pw.dv), dtype=torch.float32, device="cuda")
    ppool = gdn.gdn_state_pool_create(pw.num_slots, pw.HV, pw.dk, pw.dv, storage=pst)
    ppool.alloc(pw.num_slots)
    pcu = dev(pw.cu_seqlens)
    psrc = torch.tensor([-1], dtype=torch.int32, device="cuda")
    pdst = torch.tensor([1], dtype=torch.int32, device="cuda")
    ws = None
    for _ in range(2):
        ws = gdn.gdn_prefill_chunked(ppool, pq, pk, pv, pg, pb, po, pcu, pw.cu_seqlens, psrc, pdst, workspace=ws)
    torch.cuda.synchronize()
    ppool.close()
    del ws, po
    # two calls of the fp32-input 8192-token prefill (the second one is read)
    from hybrid_linear_attention_02_amd.workloads import F32, prefill_workload
    fw = prefill_workload("one_seq_t8192", seed=2, lengths=[8192], HK=16, HV=32, dk=128, dv=128, dtype=F32,
                          num_slots=2)
    ft = fw.tokens
    fq, fk, fv, fg, fb = dev(ft.q), dev(ft.k), dev(ft.v), dev(ft.g), dev(ft.beta)
    fo = torch.empty_like(fv)
    fpool = gdn.gdn_state_pool_create(2, 32, 128, 128)
    fpool.alloc(2)
    fcu = dev(fw.cu_seqlens)
    ws = None
    for _ in range(2):
        ws = gdn.gdn_prefill_chunked(fpool, fq, fk, fv, fg, fb, fo, fcu, fw.cu_seqlens, psrc, pdst, workspace=ws)
    torch.cuda.synchronize()
    fpool.close()
    print(json.dumps({"decode_launches": launches,
                      "decode_algorithmic_bytes_per_launch": wl.B * decode_bytes_per_request(wl.HK, wl.HV, wl.dk, wl.dv, 2),
                      "copy_bytes_each_way": n * 4,
                      "decode_kernel_source_sha256_16": _src_hash("gdn_decode.hip")}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--counters", action="store_true",
                    help="short decode + calibration-copy run for rocprofv3 counter passes; prints no bench line")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the GDN state update shards over heads and requests with no "
              "exchange, so there is no multi-GPU step to time here. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    # The CPU baseline forks its worker processes before this process touches
    # the GPU.
    if args.counters:
        run_counters()
        return
    cpu = None if args.no_cpu_baseline else cpu_baseline(decode_bytes_per_request(16, 32, 128, 128, 2))
    cpu_pre = None if (args.no_cpu_baseline or args.no_prefill) else cpu_baseline_prefill()
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    from hybrid_linear_attention_02_amd import gdn
    gdn.load_library()

    d = bench_decode(args.steps, args.warmup)
    pre = None if args.no_prefill else bench_prefill()
    if pre is not None and not args.no_cpu_baseline:
        pre["cpu_baseline"] = cpu_pre
    pre32 = None if args.no_prefill else bench_prefill_f32()
    packed = None if args.no_prefill else bench_prefill_packed()
    resume = None if args.no_prefill else bench_resume()
    long_ctx = None if args.no_prefill else bench_prefill_long_context()
    ver = bench_verify()
    xfer = bench_transfer()
    grf = bench_graph()
    ach = achievable()
    line = {
        "metric": METRIC,
        "value": round(d["value"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(d["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "batched_decode_bf16_b64_hk16_hv32_128x128_pool256",
            "requests": d["B"], "k_heads": d["HK"], "v_heads": d["HV"], "dk": d["dk"], "dv": d["dv"],
            "io_dtype": "bf16", "state_dtype": "f32", "pool_slots": 256,
            "bytes_per_step": d["bytes_step"], "layers_rotated": d["layers"],
        },
        "hbm_frac": round(d["value"] / HBM_PEAK_GBS, 4),
        "roofline": {
            "bound": "hbm", "achieved": round(d["achieved"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(d["achieved"] / HBM_PEAK_GBS, 4), "traffic": d["traffic"],
            "kernel": "gdn_decode_kernel<128,128,128,bf16> (whole tiles)", "launch_us_mean": round(d["launch_ms_mean"] * 1e3, 2),
            "timing": f"HIP-graph replay of the K timed steps rotating over {d['layers']} layers' pools "
                      "(HBM-only: the MALL holds none of a layer's state between its steps); "
                      "achieved = bytes per launch / (replay span / K)",
            "vs_tile_copy": round(d["achieved"] / d["tile_copy_gbs"], 4),
        },
        "decode_shaped_copy": {"value": round(d["tile_copy_gbs"], 1), "unit": "GB/s",
                               "frac": round(d["tile_copy_gbs"] / HBM_PEAK_GBS, 4),
                               "protocol": "gdn_state_pool_pack of the same 64 slots x 32 heads per step (one "
                                           "workgroup per 64 KiB tile, read then written), K steps rotating over "
                                           "the same layers, one HIP-graph replay"},
        "warm_one_layer": {"value": round(d["warm_gbs"], 1), "unit": "GB/s", "frac": round(d["warm_gbs"] / HBM_PEAK_GBS, 4),
                           "protocol": "the K steps on one layer in place (128 MiB working set, which the 256 MB "
                                       "MALL can hold), one HIP-graph replay"},
        "eager": {k: round(v, 2) for k, v in d["eager"].items()},
        "cold_cache": {"value": round(d["cold_gbs"], 1), "unit": "GB/s", "frac": round(d["cold_gbs"] / HBM_PEAK_GBS, 4),
                       "protocol": "median of 20 single launches, each after a 1 GiB device write"},
        "cpu_baseline": cpu,
        "achievable": ach,
        "verify": ver,
        "transfer": xfer,
        "decode_graph": grf,
        "prefill": pre,
        "prefill_packed": packed,
        "resume": resume,
        "prefill_long_context": long_ctx,
        "prefill_f32": pre32,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
