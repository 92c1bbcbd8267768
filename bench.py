#!/usr/bin/env python3
"""Benchmark of the BlockRank hot path on one MI355X.

A step is one pass of the whole path over one synthetic prompt batch: block-sparse prefill
attention (br_attn_fwd), attention-mass document scores (br_doc_scores) and the per-prompt
ranking (br_sort_docs), inputs resident in HBM before timing starts.

Prints ONE JSON line.  `value` is allowed-pair TFLOP/s of the whole step, counting
4 * d * Hq FLOPs per allowed (query, key) pair with the blog's closed-form pair count
(diagonal blocks whole); the exact causal count is reported beside it.  `roofline` covers the
attention kernel (the dominant one), timed with HIP events recorded on the launch stream
around the kernel itself.  `cpu_baseline` times the fp64 CPU oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "block-sparse prefill TFLOP/s (allowed pairs) + prompts/s at N=100,500; % MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E

TRAFFIC_SUMMARY = {  # rocprofv3 counter summaries of the attention kernel, per workload
    "long": os.path.join(ROOT, "profiles", "attn_fwd_long_N500_traffic.md"),
}
# the attention kernel and the planner whose schedule decides which K/V reads hit L2
ATTN_SOURCES = [os.path.join(ROOT, "block_sparse_attention_segment_amd", "csrc", f) for f in ("attn_fwd.hip", "plan.cpp")]


def attn_source_digest():
    h = hashlib.sha256()
    for path in ATTN_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]

WORKLOAD_NAMES = {
    "tiny": "tiny: 1 head, d=64, p=32, N=4 x l=64, q=32 (L=320), |S|=4",
    "worked": "worked: p=32, q=32, N=100 x l=128 (L=12864), 32 Q / 8 KV heads, d=128, |S|=8, B=1",
    "long": "long: p=64, q=32, N=500 x l=200 (L=100096), 32 Q / 8 KV heads, d=128, |S|=8, B=1",
    "ragged": "ragged: p=48, q=24, N=200, l~U{32..256}, 32 Q / 8 KV heads, d=128, |S|=8, B=1",
    "batched": "batched: B=16 x (p=32, q=32, N=100, l~U{64..192}), 32 Q / 8 KV heads, d=128, |S|=8",
}


def pair_counts(w):
    """Allowed pairs per the blog's closed form (diagonal blocks whole) and the causal count."""
    blk = exact = 0
    for (p, lens, q) in w.prompts:
        D = sum(lens)
        b = p * p + sum(l * l + p * l for l in lens) + q * (p + q + D)
        blk += b
        exact += b - sum(n * (n - 1) // 2 for n in [p, q] + list(lens))
    return blk, exact


def measured_traffic(config):
    """HBM bytes per attention launch from the committed counter summary, or None when there is
    none for this workload or the kernel or planner source changed since the counters were taken."""
    path = TRAFFIC_SUMMARY.get(config)
    if not path or not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(("|", "#", "`")):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != attn_source_digest() or "bytes_per_launch" not in fields:
        return None
    return float(fields["bytes_per_launch"])


ATTN_ROWS_PER_TILE = 128   # (token, head) rows of one attention work item
ATTN_KEY_TILE = 64         # keys per LDS tile of the attention kernel


def tile_efficiency(w, dims):
    """(token, head, key) triples the attention kernel's MFMA tiles visit: key tiles per work item
    (from the host plan) x rows per item x keys per tile, over all KV heads."""
    import block_sparse_attention_segment_amd as br
    items, _ = br.attn_plan_items(dims, w.segment_offsets, w.seg_ptr)
    return float(items[:, 7].astype(np.int64).sum()) * ATTN_ROWS_PER_TILE * ATTN_KEY_TILE * dims.num_kv_heads


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence (hip_runtime_api.h)


class HipEvents:
    """Raw hipEvent_t handles (libamdhip64) so the library can record them on its launch stream."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            # timing-only events: no system-scope fence (cache writeback) when they are recorded
            rc = self.hip.hipEventCreateWithFlags(ctypes.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE)
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
            self.ev.append(e.value)

    def elapsed_ms(self, a, b):
        out = ctypes.c_float()
        self.hip.hipEventSynchronize(ctypes.c_void_p(self.ev[b]))
        rc = self.hip.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(self.ev[a]), ctypes.c_void_p(self.ev[b]))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(out.value)

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def measure(config, seed, steps, warmup, log):
    import torch

    import block_sparse_attention_segment_amd as br
    import workloads

    t0 = time.time()
    w = workloads.make(config, seed)
    log(f"[bench] generated {config} (T={w.total_tokens}) in {time.time() - t0:.1f}s")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    Q, K, V, Q_S = dev(w.Q), dev(w.K), dev(w.V), dev(w.Q_S)
    T, Hq, d = Q.shape
    Hkv = K.shape[1]
    dims = br.make_dims(w.num_prompts, Hq, Hkv, d, T)
    out = torch.empty_like(Q)
    scores = torch.empty(w.num_docs, dtype=torch.float32, device="cuda")
    order = torch.empty(w.num_docs, dtype=torch.int32, device="cuda")
    ws = torch.empty(br.rank_workspace_bytes(dims, w.segment_offsets, w.seg_ptr, w.n_signal, w.doc_offsets, w.doc_ptr),
                     dtype=torch.uint8, device="cuda")
    ev = HipEvents(2 * steps)
    stream = torch.cuda.current_stream()

    def step(kernel_events=None):
        # attention (+ split-key merge), readout and rank in one library call (br_rank_prompts)
        br.rank_step(Q, K, V, Q_S, w.segment_offsets, w.seg_ptr, w.doc_offsets, w.doc_ptr, out=out, scores=scores,
                     order=order, workspace=ws, stream=stream, kernel_events=kernel_events)

    # Measured first (they also bring the GPU to its working clocks before the timed steps): the
    # attention alone (br_attn_fwd, nothing else on the GPU), for comparison with its duration
    # inside a step, ...
    attn_ws = torch.empty(br.attn_workspace_bytes(dims, w.segment_offsets, w.seg_ptr), dtype=torch.uint8,
                          device="cuda")
    # A GPU that has been idle runs its first milliseconds of work measurably slower (about 15% at
    # this size): bring it to its working clocks with half a second of the attention first.
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < 0.5:
        for _ in range(4):
            br.attn_fwd(Q, K, V, w.segment_offsets, w.seg_ptr, out=out, workspace=attn_ws, stream=stream)
        torch.cuda.synchronize()
    for i in range(steps):
        br.attn_fwd(Q, K, V, w.segment_offsets, w.seg_ptr, out=out, workspace=attn_ws, stream=stream,
                    kernel_events=(ev.ev[2 * i], ev.ev[2 * i + 1]))
    torch.cuda.synchronize()
    kern_iso = [ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(steps)]
    del attn_ws
    # ... and the readout alone (br_doc_scores: partials, row statistics, scores), between torch
    # events on the same stream.
    sc_ws = torch.empty(br.doc_scores_workspace_bytes(dims, w.n_signal, w.doc_offsets, w.doc_ptr), dtype=torch.uint8,
                        device="cuda")
    for _ in range(max(1, warmup // 2)):
        br.doc_scores(Q_S, K, w.doc_offsets, w.doc_ptr, scores=scores, workspace=sc_ws, stream=stream)
    torch.cuda.synchronize()
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r0.record(stream)
    for _ in range(steps):
        br.doc_scores(Q_S, K, w.doc_offsets, w.doc_ptr, scores=scores, workspace=sc_ws, stream=stream)
    r1.record(stream)
    torch.cuda.synchronize()
    readout_ms = r0.elapsed_time(r1) / steps
    del sc_ws
    doc_tokens = int(sum(sum(lens) for (_, lens, _) in w.prompts))
    readout_bytes = float(doc_tokens * Hkv * d * 2 + Q_S.numel() * 2 + w.num_docs * 4)
    # The readout measurement leaves the GPU mostly idle, and a GPU that has been idle runs its
    # first milliseconds slower: a quarter second of steps brings it back to its working clocks
    # before the warm-up steps (without it, 20 timed steps at 100K tokens measured 0.70 ms per
    # step after 5 warm-up steps and 0.65-0.67 ms after 25).
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < 0.25:
        for _ in range(4):
            step()
        torch.cuda.synchronize()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] {config}: {warmup} warm-up steps done")
    # Timed region: K back-to-back steps between two events, with nothing else recorded (an event
    # between two kernels costs the stream a few microseconds).
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = e0.elapsed_time(e1) / steps
    # Kernel region: K more back-to-back steps, the attention kernel's own duration per step from
    # events the library records around it on its launch stream; the step takes the same path as
    # in the timed region (the readout on the side stream for large batches), so this is the
    # kernel's duration inside a step.
    torch.cuda.synchronize()
    for i in range(steps):
        step(kernel_events=(ev.ev[2 * i], ev.ev[2 * i + 1]))
    torch.cuda.synchronize()
    kern = [ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(steps)]
    ev.close()
    # Per-step latency distribution (one step at a time, each between two events).
    lat = []
    for _ in range(steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        b.synchronize()
        lat.append(a.elapsed_time(b))
    cold = cold_plan_latency(w, Q, K, V, Q_S, stream, log)
    peak_mb = torch.cuda.max_memory_allocated() / 2**20
    log(f"[bench] {config}: {steps} timed steps, {ms_step:.4f} ms/step, attention kernel {np.mean(kern):.4f} ms "
        f"in the step, {np.mean(kern_iso):.4f} ms alone; readout {readout_ms:.4f} ms")
    blk, exact = pair_counts(w)
    flop_blk = 4.0 * d * Hq * blk
    flop_exact = 4.0 * d * Hq * exact
    kernel_s = float(np.mean(kern)) / 1e3
    bytes_alg = float(T) * (2 * Hq + 2 * Hkv) * d * 2
    return dict(w=w, ms_step=ms_step, wall_s=wall, kernel_ms=float(np.mean(kern)), kernel_ms_p50=float(np.median(kern)),
                kernel_ms_isolated=float(np.mean(kern_iso)), readout_ms=readout_ms, readout_bytes=readout_bytes,
                cold=cold,
                flop_blk=flop_blk, flop_exact=flop_exact, pairs_blk=blk, pairs_exact=exact, bytes_alg=bytes_alg,
                kernel_s=kernel_s, lat_p50=float(np.percentile(lat, 50)), lat_p95=float(np.percentile(lat, 95)),
                peak_mb=peak_mb, visited_pairs=tile_efficiency(w, dims))


def cold_plan_latency(w, Q, K, V, Q_S, stream, log, n_tables=5, rounds=2):
    """Single-step host-to-completion latency of br_rank_prompts when its plan is not cached: the
    batch's first prompt with one token moved between its first two documents, in n_tables (more
    than the library's four cached plans) variants visited in turn, so every call builds,
    schedules and uploads a fresh plan; beside it, the same latency with the original table (a
    cached plan)."""
    import torch

    import block_sparse_attention_segment_amd as br
    import workloads
    p0, lens0, q0 = w.prompts[0]
    if len(lens0) < 2 or min(lens0[0], lens0[1]) <= n_tables:
        return None
    tables = []
    for i in range(1, n_tables + 1):
        prompts = [(p0, [lens0[0] - i, lens0[1] + i] + list(lens0[2:]), q0)] + list(w.prompts[1:])
        tables.append(workloads.segment_tables(prompts))
    T, Hq, d = Q.shape
    dims = br.make_dims(w.num_prompts, Hq, K.shape[1], d, T)
    need = max(br.rank_workspace_bytes(dims, seg, sp, w.n_signal, do, dp) for (seg, sp, do, dp) in tables)
    need = max(need, br.rank_workspace_bytes(dims, w.segment_offsets, w.seg_ptr, w.n_signal, w.doc_offsets, w.doc_ptr))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(Q)
    scores = torch.empty(w.num_docs, dtype=torch.float32, device="cuda")
    order = torch.empty(w.num_docs, dtype=torch.int32, device="cuda")

    def one(seg, sp, do, dp):
        torch.cuda.synchronize()
        t = time.perf_counter()
        br.rank_step(Q, K, V, Q_S, seg, sp, do, dp, out=out, scores=scores, order=order, workspace=ws, stream=stream)
        stream.synchronize()
        return (time.perf_counter() - t) * 1e3

    cold = [one(*tables[i % n_tables]) for i in range(rounds * n_tables)]
    warm = [one(w.segment_offsets, w.seg_ptr, w.doc_offsets, w.doc_ptr) for _ in range(rounds * n_tables + 1)][1:]
    log(f"[bench] single-step latency: fresh plan {np.median(cold):.3f} ms, cached plan {np.median(warm):.3f} ms")
    return dict(fresh_plan_ms_p50=round(float(np.median(cold)), 4), cached_plan_ms_p50=round(float(np.median(warm)), 4),
                calls=len(cold))


def measure_query_only(w, n_queries, q_len, steps, warmup, seed, log):
    """Query-only attention over a cached corpus: the corpus is the prompt's instruction and
    documents (its K/V already prefilled), scored against n_queries new queries of q_len tokens.
    Times whole br_query_attn_fwd calls (plan copy, attention, merge) between events."""
    import torch

    import block_sparse_attention_segment_amd as br
    import workloads

    offs = [int(x) for x in w.segment_offsets]
    corpus = offs[-2]
    Hq, d = w.Q.shape[1], w.Q.shape[2]
    Hkv = w.K.shape[1]
    rng = np.random.default_rng(seed + 1000)
    nq = n_queries * q_len
    bf = lambda a: workloads.f32_to_bf16_bits(a.astype(np.float32))
    Kq, Vq = bf(rng.standard_normal((nq, Hkv, d))), bf(rng.standard_normal((nq, Hkv, d)))
    Qq = bf(rng.standard_normal((nq, Hq, d)))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    K = torch.cat([dev(w.K[:corpus]), dev(Kq)]).contiguous()
    V = torch.cat([dev(w.V[:corpus]), dev(Vq)]).contiguous()
    Q = dev(Qq)
    qo = np.arange(n_queries + 1, dtype=np.int64) * q_len + corpus
    dims = br.make_dims(n_queries, Hq, Hkv, d, corpus + nq)
    ws = torch.empty(br.query_attn_workspace_bytes(dims, corpus, qo), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(Q)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        br.query_attn(Q, K, V, corpus, qo, out=out, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        br.query_attn(Q, K, V, corpus, qo, out=out, workspace=ws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    pairs = n_queries * (q_len * corpus + q_len * (q_len + 1) // 2)
    flop = 4.0 * d * Hq * pairs
    alg_bytes = float(corpus) * Hkv * d * 2 * 2 + float(nq) * (2 * Hq + 2 * Hkv) * d * 2
    log(f"[bench] query-only: {n_queries} x {q_len} tokens over a {corpus}-token corpus, {ms:.4f} ms/call")
    return {"workload": f"{n_queries} queries x {q_len} tokens over the long prompt's cached corpus "
                        f"(instruction + 500 documents, {corpus} tokens), {Hq} Q / {Hkv} KV heads, d={d}",
            "bound": "mfma",  # each corpus K/V byte serves every query: ~2000 FLOP/B, far above the ridge
            "ms": round(ms, 5), "tflops_allowed_pairs": round(flop / (ms / 1e3) / 1e12, 3),
            "mfma_peak_frac": round(flop / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "algorithmic_gbps": round(alg_bytes / (ms / 1e3) / 1e9, 1),
            "hbm_roofline_frac": round(alg_bytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBPS, 4)}


def measure_routed(w, top_b, steps, warmup, log):
    """Top-B routed attention on the prompt: the readout ranks the documents, the top_b stay.
    Times br_attn_routed_fwd calls (plan copy, attention, merge) between events; the ranking
    and the device-to-host copy of the kept list are outside the timed calls."""
    import torch

    import block_sparse_attention_segment_amd as br

    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    Q, K, V, Q_S = dev(w.Q), dev(w.K), dev(w.V), dev(w.Q_S)
    scores = br.doc_scores(Q_S, K, w.doc_offsets, w.doc_ptr)
    keep = br.sort_docs(scores, w.doc_ptr)[:top_b].cpu().numpy().astype(np.int64)
    kp = [0, top_b]
    Hq, d = w.Q.shape[1], w.Q.shape[2]
    dims = br.make_dims(1, Hq, w.K.shape[1], d, w.total_tokens)
    ws = torch.empty(br.attn_routed_workspace_bytes(dims, w.segment_offsets, w.seg_ptr, kp, keep), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(Q)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        br.attn_routed(Q, K, V, w.segment_offsets, w.seg_ptr, kp, keep, out=out, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        br.attn_routed(Q, K, V, w.segment_offsets, w.seg_ptr, kp, keep, out=out, workspace=ws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # allowed pairs of the routed prompt: drop the other documents and count as for a prompt
    offs = [int(x) for x in w.segment_offsets]
    p, q = offs[1] - offs[0], offs[-1] - offs[-2]
    lens = [offs[k + 2] - offs[k + 1] for k in sorted(int(x) for x in keep)]
    pairs = p * p + sum(l * l + p * l for l in lens) + q * (p + q + sum(lens))
    flop = 4.0 * d * Hq * pairs
    log(f"[bench] routed top-{top_b}: {ms:.4f} ms/call")
    return {"workload": f"top-{top_b} routing of the long prompt's {w.num_docs} documents by its own readout "
                        f"(kept documents' rows, instruction and query rows computed)",
            "ms": round(ms, 5), "allowed_pairs_closed_form": int(pairs),
            "tflops_allowed_pairs": round(flop / (ms / 1e3) / 1e12, 3),
            "mfma_peak_frac": round(flop / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def measure_rope(w, steps, warmup, log):
    """Rotary embedding of the prompt's Q and K at BlockRank's permutation-invariant positions
    (out of place).  HBM-bound: every element is read once and written once."""
    import torch

    import block_sparse_attention_segment_amd as br

    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    Q, K = dev(w.Q), dev(w.K)
    Qo, Ko = torch.empty_like(Q), torch.empty_like(K)
    Hq, d = w.Q.shape[1], w.Q.shape[2]
    Hkv = w.K.shape[1]
    dims = br.make_dims(w.num_prompts, Hq, Hkv, d, w.total_tokens)
    ws = torch.empty(br.rope_workspace_bytes(dims, w.seg_ptr), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    call = lambda: br.rope(Q, K, w.segment_offsets, w.seg_ptr, 10000.0, Q_out=Qo, K_out=Ko, workspace=ws,
                           stream=stream)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    alg = 2.0 * w.total_tokens * (Hq + Hkv) * d * 2
    gbps = alg / (ms / 1e3) / 1e9
    log(f"[bench] rope Q+K: {ms:.4f} ms/call, {gbps:.0f} GB/s")
    # Rotation followed by attention, two ways: the separate pass over Q and K then br_attn_fwd,
    # or K rotated alone and Q rotated inside the attention kernel (br_attn_fwd_rope).
    V = dev(w.V)
    out = torch.empty_like(Q)
    attn_ws = torch.empty(br.attn_workspace_bytes(dims, w.segment_offsets, w.seg_ptr), dtype=torch.uint8, device="cuda")
    fused_ws = torch.empty(br.attn_fwd_rope_workspace_bytes(dims, w.segment_offsets, w.seg_ptr), dtype=torch.uint8,
                           device="cuda")

    def separate():
        call()
        br.attn_fwd(Qo, Ko, V, w.segment_offsets, w.seg_ptr, out=out, workspace=attn_ws, stream=stream)

    def fused():
        br.rope(None, K, w.segment_offsets, w.seg_ptr, 10000.0, K_out=Ko, workspace=ws, stream=stream)
        br.attn_fwd_rope(Q, Ko, V, w.segment_offsets, w.seg_ptr, 10000.0, out=out, workspace=fused_ws, stream=stream)

    times = {}
    for name, fn in (("separate", separate), ("fused", fused), ("separate2", separate), ("fused2", fused)):
        for _ in range(max(1, warmup)):
            fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        times.setdefault(name.rstrip("2"), []).append(e0.elapsed_time(e1) / steps)
    sep, fus = min(times["separate"]), min(times["fused"])
    log(f"[bench] rope + attention: separate {sep:.4f} ms, Q rotated inside the attention kernel {fus:.4f} ms")
    return {"workload": f"RoPE of the long prompt's Q and K ({w.total_tokens} tokens, {Hq} Q / {Hkv} KV heads, d={d}) "
                        f"at permutation-invariant positions, out of place",
            "bound": "hbm", "ms": round(ms, 5), "bytes_per_call": alg, "achieved_gbps": round(gbps, 1),
            "hbm_roofline_frac": round(gbps / PEAK_HBM_GBPS, 4),
            "with_attention": {"separate_rope_then_attention_ms": round(sep, 5),
                               "k_rope_then_attention_rotating_q_ms": round(fus, 5),
                               "note": "best of two interleaved runs of K calls each"}}


def measure_backward(w, steps, warmup, log):
    """Training side of the long prompt: the attention backward for an upstream dO (with the
    forward's O and lse), and the auxiliary-loss chain readout -> InfoNCE -> readout backward
    (adding into the attention's dK).  Inputs resident in HBM; the forward is outside the timed
    region."""
    import torch

    import block_sparse_attention_segment_amd as br
    import workloads

    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    Q, K, V, Q_S = dev(w.Q), dev(w.K), dev(w.V), dev(w.Q_S)
    T, Hq, d = Q.shape
    Hkv = K.shape[1]
    rng = np.random.default_rng(7)
    dO = dev(workloads.f32_to_bf16_bits(rng.standard_normal((T, Hq, d), dtype=np.float32)))
    O, lse = br.attn_fwd(Q, K, V, w.segment_offsets, w.seg_ptr, lse=True)
    dims = br.make_dims(w.num_prompts, Hq, Hkv, d, T)
    ws = torch.empty(br.attn_bwd_workspace_bytes(dims, w.segment_offsets, w.seg_ptr), dtype=torch.uint8, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    dQ, dK, dV = torch.empty((T, Hq, d), **f32), torch.empty((T, Hkv, d), **f32), torch.empty((T, Hkv, d), **f32)
    gold = np.zeros(w.num_prompts, dtype=np.int32)
    scores = torch.empty(w.num_docs, **f32)
    loss, ds = torch.empty(w.num_prompts, **f32), torch.empty(w.num_docs, **f32)
    dQs = torch.empty(tuple(w.Q_S.shape), **f32)
    ws_s = torch.empty(br.doc_scores_workspace_bytes(dims, w.n_signal, w.doc_offsets, w.doc_ptr), dtype=torch.uint8,
                       device="cuda")
    ws_r = torch.empty(br.doc_scores_bwd_workspace_bytes(dims, w.n_signal, w.doc_offsets, w.doc_ptr), dtype=torch.uint8,
                       device="cuda")
    ws_i = torch.empty(1 << 12, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def attn_bwd():
        br.attn_bwd(Q, K, V, O, dO, lse, w.segment_offsets, w.seg_ptr, dQ=dQ, dK=dK, dV=dV, workspace=ws, stream=stream)

    def aux_chain():
        br.doc_scores(Q_S, K, w.doc_offsets, w.doc_ptr, scores=scores, workspace=ws_s, stream=stream)
        br.infonce(scores, w.doc_ptr, gold, loss=loss, dscores=ds, workspace=ws_i, stream=stream)
        br.doc_scores_bwd(Q_S, K, w.doc_offsets, w.doc_ptr, ds, dQ_S=dQs, dK=dK, accumulate=True, workspace=ws_r,
                          stream=stream)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms_attn = timed(attn_bwd)
    ms_aux = timed(aux_chain)
    blk, _ = pair_counts(w)
    flop = 10.0 * d * Hq * blk   # recomputed S, dP, dV, dQ, dK: five products of 2 d FLOPs per pair
    io_bytes = float(T) * (3 * Hq * d * 2 + 2 * Hkv * d * 2 + Hq * 4 + Hq * d * 4 + 2 * Hkv * d * 4)
    log(f"[bench] attention backward {ms_attn:.4f} ms, loss chain {ms_aux:.4f} ms")
    return {"workload": f"long prompt backward: attention dQ/dK/dV for a random upstream dO; readout -> InfoNCE "
                        f"(tau 0.05) -> readout backward adding into dK",
            "attn_bwd_ms": round(ms_attn, 5),
            "attn_bwd_tflops_allowed_pairs": round(flop / (ms_attn / 1e3) / 1e12, 3),
            "attn_bwd_mfma_peak_frac": round(flop / (ms_attn / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "attn_bwd_io_bytes": io_bytes,
            "attn_bwd_io_gbps": round(io_bytes / (ms_attn / 1e3) / 1e9, 1),
            "aux_loss_chain_ms": round(ms_aux, 5)}


def cpu_baseline(w, n_docs_sample, log):
    """Time the fp64 oracle on a bounded sample of the same prompt and scale to the whole step."""
    import oracle.oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    so, sp = w.segment_offsets, w.seg_ptr
    offs = so[sp[0]:sp[1]]
    N = len(offs) - 3
    k = min(n_docs_sample, N)
    inst = np.arange(int(offs[0]), int(offs[1]))
    docs = np.arange(int(offs[1]), int(offs[1 + k]))
    query = np.arange(int(offs[-2]), int(offs[-1]))
    timings = {}
    for name, rows in (("instruction", inst), ("docs", docs), ("query", query)):
        t = time.perf_counter()
        if len(rows):
            orc.attn_rows(w.Q, w.K, w.V, so, sp, rows=rows)
        timings[name] = time.perf_counter() - t
    t = time.perf_counter()
    s, _ = orc.doc_scores(w.Q_S, w.K, w.doc_offsets, w.doc_ptr)
    timings["scores"] = time.perf_counter() - t
    t = time.perf_counter()
    orc.rank(s, w.doc_ptr)
    timings["rank"] = time.perf_counter() - t
    est = timings["instruction"] + timings["docs"] * (N / k) + timings["query"] + timings["scores"] + timings["rank"]
    log(f"[bench] cpu oracle sample: {json.dumps({a: round(b, 3) for a, b in timings.items()})}, "
        f"estimated full step {est:.1f}s")
    return dict(est_s=est, threads=threads, k=k, N=N, sampled_s=sum(timings.values()))


def cpu_model():
    """The host CPU's model name as lscpu reports it (from /proc/cpuinfo when lscpu is absent)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except Exception:  # pragma: no cover
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return platform.processor() or platform.machine()


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="long", choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--secondary", default="worked,batched,ragged",
                    help="extra configs timed in the same run, comma-separated ('' for none)")
    ap.add_argument("--query-only", type=int, default=1,
                    help="also time query-only attention over the long prompt's cached corpus, top-256 routed "
                         "attention, RoPE of Q and K, and the backward (0 to skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-docs", type=int, default=200, help="documents in the CPU oracle's timed sample")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    log = lambda m: print(m, file=sys.stderr, flush=True)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path shards with no "
              "cross-GPU traffic for document rows, but no multi-GPU run is implemented", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_mib:
        # Calibration for HBM byte counters: each launch reads and writes exactly copy_mib MiB.
        n = args.copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": args.steps}), flush=True)
        return

    r = measure(args.config, args.seed, args.steps, args.warmup, log)
    w = r["w"]
    step_s = r["ms_step"] / 1e3
    value = r["flop_blk"] / step_s / 1e12
    attn_tflops_blk = r["flop_blk"] / r["kernel_s"] / 1e12
    achieved_gbps = r["bytes_alg"] / r["kernel_s"] / 1e9
    iso_s = r["kernel_ms_isolated"] / 1e3
    traffic = measured_traffic(args.config)
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[args.config], "seed": args.seed, "global_batch": w.num_prompts,
                   "seq_len": w.total_tokens, "parallelism": "single-gpu"},
        "prompts_per_s": round(w.num_prompts / step_s, 2),
        "step_ms_p50": round(r["lat_p50"], 5),
        "step_ms_p95": round(r["lat_p95"], 5),
        "peak_device_mb": round(r["peak_mb"], 1),
        "tile_efficiency_exact": round(r["pairs_exact"] * w.num_q_heads / r["visited_pairs"], 4),
        "tflops_exact_pairs": round(r["flop_exact"] / step_s / 1e12, 3),
        "mfma_peak_frac_step": round(value / PEAK_BF16_TFLOPS, 4),
        "allowed_pairs": {"closed_form": r["pairs_blk"], "exact_causal": r["pairs_exact"]},
        "attention_kernel": {"ms": round(r["kernel_ms"], 5), "ms_p50": round(r["kernel_ms_p50"], 5),
                             "timing": "inside the timed steps (same launch path, readout alongside)",
                             "ms_isolated": round(r["kernel_ms_isolated"], 5),
                             "tflops_closed_form_pairs": round(attn_tflops_blk, 3),
                             "mfma_peak_frac": round(attn_tflops_blk / PEAK_BF16_TFLOPS, 4),
                             "mfma_peak_frac_isolated": round(r["flop_blk"] / iso_s / 1e12 / PEAK_BF16_TFLOPS, 4)},
        "roofline": {"bound": "hbm", "achieved": round(achieved_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved_gbps / PEAK_HBM_GBPS, 4), "traffic": traffic,
                     "kernel": "attn_fwd_kernel", "bytes_per_launch": r["bytes_alg"],
                     "timing": "kernel duration inside the timed steps",
                     "frac_isolated": round(r["bytes_alg"] / iso_s / 1e9 / PEAK_HBM_GBPS, 4),
                     "traffic_gbps": None if traffic is None else round(traffic / r["kernel_s"] / 1e9, 1)},
        "readout": {"kernels": "br_doc_scores (partials, row statistics, scores)", "ms": round(r["readout_ms"], 5),
                    "algorithmic_bytes": r["readout_bytes"],
                    "hbm_gbps": round(r["readout_bytes"] / r["readout_ms"] / 1e6, 1),
                    "hbm_roofline_frac": round(r["readout_bytes"] / r["readout_ms"] / 1e6 / PEAK_HBM_GBPS, 4)},
        "single_step_latency": r["cold"],
    }
    for name in [s for s in args.secondary.split(",") if s and s != args.config]:
        if name not in WORKLOAD_NAMES:
            raise SystemExit(f"unknown secondary config {name!r}")
        r2 = measure(name, args.seed, args.steps, args.warmup, log)
        s2 = r2["ms_step"] / 1e3
        entry = {"workload": WORKLOAD_NAMES[name], "ms_per_step": round(r2["ms_step"], 5),
                 "prompts_per_s": round(r2["w"].num_prompts / s2, 2),
                 "tflops_closed_form_pairs": round(r2["flop_blk"] / s2 / 1e12, 3),
                 "attention_kernel_ms": round(r2["kernel_ms"], 5),
                 "attention_kernel_ms_isolated": round(r2["kernel_ms_isolated"], 5),
                 "readout_hbm_gbps": round(r2["readout_bytes"] / r2["readout_ms"] / 1e6, 1),
                 "single_step_latency": r2["cold"]}
        # the first extra config keeps the key "secondary"; the others are keyed by name
        line["secondary" if "secondary" not in line else name] = entry
    if args.query_only and args.config == "long":
        line["query_only"] = measure_query_only(w, 16, 32, args.steps, args.warmup, args.seed, log)
        line["routed"] = measure_routed(w, 256, args.steps, args.warmup, log)
        line["rope"] = measure_rope(w, args.steps, args.warmup, log)
        line["backward"] = measure_backward(w, args.steps, args.warmup, log)
    if not args.no_cpu_baseline:
        runs = [cpu_baseline(w, args.cpu_docs, log) for _ in range(3)]
        cb = sorted(runs, key=lambda x: x["est_s"])[1]  # the median of three runs
        run_list = ", ".join(f"{x['est_s']:.1f}" for x in runs)
        line["cpu_baseline"] = {
            "value": round(r["flop_blk"] / cb["est_s"] / 1e12, 6), "unit": "TFLOP/s", "cores": cb["threads"],
            "kind": "oracle",
            "sample": (f"fp64 NumPy oracle on instruction rows, {cb['k']} of {cb['N']} documents' rows and all "
                       f"query rows, plus the full readout and rank ({cb['sampled_s']:.1f}s measured); time "
                       f"scaled to all {cb['N']} documents ({cb['est_s']:.1f}s per step, the median of 3 runs: "
                       f"{run_list}s); host "
                       f"{cpu_model()}, os.cpu_count()={os.cpu_count()}"),
        }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
