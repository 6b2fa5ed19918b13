#!/usr/bin/env python3
"""Benchmark of the hybrid compressed-attention hot path on one MI355X.

The timed step is one decode step of a CSA + HCA layer pair at 1M context
(8 sequences of 2^20 raw tokens, one query each at position L-1, 64 heads x
128, window 128, HISA B=128 m=64 k=2048 on a 16 x 128 indexer over 262,143
CSA entries, 8,192 HCA entries):

  CSA: one launch compresses the window the new token completes, refreshes
       the HISA block mean holding that entry and writes the visible count
       -> HISA (block scores, block top-m, token scores in the chosen
       blocks, token top-k) -> sparse attention
  HCA: the same launch for the completed 128-token window (no block means)
       -> dense attention

Every step is one run of a native decode plan (hattn_decode_plan_run): one
host call enqueues 6 kernels on the current stream, the HCA branch's work
riding in the CSA branch's launches (a shared launch for both caches'
maintenance and HISA's block scores, a shared attention launch, a shared
merge launch), so the branches overlap on
the GPU with no cross-stream synchronisation.  (The same step as two HIP
graphs on two streams joined every step is reported beside it: torch's graph
replays and stream joins cost more host time than the GPU needs.)
Caches are replicated R times (R plans) and steps rotate through them, so
the working set (about 70 MB a step) is not served by the 256 MB last-level
cache.  Inputs are seeded synthetic tensors drawn on the device.

Per-kernel durations come from the library's event timer (events recorded on
the launch stream around every kernel) over a second, eager pass of the same
steps.  Extras: HCA dense decode at batch 32 (timed as graphs of four
consecutive steps, one per cache replica), the CSA prefill chunk (1,024
queries of a 32K sequence), the 128K indexer chunk (flat and HISA),
compression of 1M-token sequences.  The CPU baseline is the fp64
oracle on a bounded sample of the same decode step.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
MiB = 1 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------
# Algorithmic traffic / work models (what the method must move or compute).
# ----------------------------------------------------------------------------

def attn_bytes(n_keys, H=64, d=128):
    """One query: every key row (K|V bf16) once, q in, fp32 out and lse."""
    return n_keys * 2 * d * 2 + H * d * 2 + H * d * 4 + H * 4


def attn_flops(n_keys, H=64, d=128):
    return 4.0 * H * d * n_keys


def hisa_stage1_bytes(nb, d_i=128, h_i=16):
    return nb * d_i * 4 + h_i * d_i * 2 + h_i * 4 + nb * 4


def hisa_stage2_bytes(ncand, d_i=128, h_i=16):
    return ncand * d_i * 2 + h_i * d_i * 2 + h_i * 4 + ncand * 4


# ----------------------------------------------------------------------------

def timed_graphs(graphs, steps, warmup):
    import torch

    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps  # ms per step


def capture(fn, reps, stream=None):
    """One graph per replica.  Graphs that will replay concurrently must be
    captured on different streams: the binding keys its scratch workspaces by
    stream, so they then own separate workspaces."""
    import torch

    graphs = []
    for r in reps:
        fn(r)  # eager warm-up on the current stream (workspaces, LDS limits)
    torch.cuda.synchronize()
    for r in reps:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            fn(r)
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def capture_chain(fn, reps):
    """One graph holding one step per replica, in order: replaying it runs
    len(reps) steps, so the graph's own launch cost is shared by them."""
    import torch

    for r in reps:
        fn(r)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for r in reps:
            fn(r)
    torch.cuda.synchronize()
    return g


def kernel_times(fn, reps, steps):
    """Eager pass with the library's event timer: {kernel: avg ms}."""
    import torch
    from compressed_attention_amd import ops

    for r in reps:
        fn(r)
    torch.cuda.synchronize()
    ops.timer_enable(True)
    for i in range(steps):
        fn(reps[i % len(reps)])
    tot = ops.timer_collect()
    ops.timer_enable(False)
    return {k: (v[0] / v[1], v[1] // steps) for k, v in tot.items()}


def step_distribution(run_step, n):
    """Per-step GPU time (us) of n consecutive steps: an event before each
    step on the current stream (the same stream the steps are launched on),
    so step i's time is the gap between its event and the next.  Returns
    median / p10 / p90 / mean over the n steps."""
    import numpy as np
    import torch

    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    for i in range(n):
        evs[i].record()
        run_step(i)
    evs[n].record()
    torch.cuda.synchronize()
    us = np.array([evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(n)])
    return dict(n=n, median=float(np.median(us)), p10=float(np.percentile(us, 10)),
                p90=float(np.percentile(us, 90)), mean=float(us.mean()))


RING = 128


def keep_rings(t, L):
    """Replaces the raw K|V and logits of both layers by rings of their
    newest RING rows (row r at slot r % RING), as a decode loop keeps them:
    the full prefix only builds the caches."""
    import torch

    for n in ("csa_raw_kv", "hca_raw_kv", "csa_z", "hca_z"):
        full = t[n]
        ring = torch.empty((full.shape[0], RING) + tuple(full.shape[2:]), dtype=full.dtype, device=full.device)
        rows = torch.arange(L - RING, L, device=full.device)
        ring[:, rows % RING] = full[:, rows]
        t[n] = ring
        del full
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def flat_decode_step(args, t, caches, k):
    """The same decode step with the flat indexer in place of HISA (scores
    every one of the 262,143 visible entries of each query), as one graph
    per cache replica; returns ms per step."""
    from compressed_attention_amd import ops

    L = 1 << 20

    def step(c):
        nv = ops.decode_append(t["csa_raw_kv"], t["csa_z"], t["csa_b"], 8, 4, t["q_pos"], c["ckv"], L=L)
        idx = ops.index_topk(t["q_i"], c["k_i"], t["w_i"], nv, k)
        o1 = ops.sparse_attn(t["csa_q"], c["ckv"], idx, t["csa_raw_kv"], t["q_pos"], 128, L=L)
        nvh = ops.decode_append(t["hca_raw_kv"], t["hca_z"], t["hca_b"], 128, 128, t["q_pos"], c["hkv"], L=L)
        o2 = ops.dense_compressed_attn(t["hca_q"], c["hkv"], nvh, t["hca_raw_kv"], t["q_pos"], 128, L=L)
        return o1, o2

    graphs = capture(step, caches)
    ms = timed_graphs(graphs, max(10, args.steps), 3)
    del graphs
    return ms


# ----------------------------------------------------------------------------
# main workload: hybrid layer pair decode at 1M
# ----------------------------------------------------------------------------

def hybrid_pair(args):
    import torch
    from compressed_attention_amd import ops, synth

    dev = "cuda:0"
    bt, L, k = 8, 1 << 20, args.k
    N, Nh, B, m = 262143, 8192, 128, 64
    t0 = time.time()
    W = synth.hybrid_pair_decode(0, device=dev, bt=bt, L=L, N_csa=N)
    t = W.tensors
    ckv = ops.compress(t["csa_raw_kv"], t["csa_z"], t["csa_b"], 8, 4)
    hkv = ops.compress(t["hca_raw_kv"], t["hca_z"], t["hca_b"], 128, 128)
    reps = ops.hisa_pool(t["k_i"], B)
    torch.cuda.synchronize()
    assert ckv.shape[1] == N and hkv.shape[1] == Nh
    nb = reps.shape[1]
    keep_rings(t, L)
    R = args.replicas
    caches = [dict(ckv=ckv, hkv=hkv, k_i=t["k_i"], reps=reps)]
    for _ in range(R - 1):
        caches.append(dict(ckv=ckv.clone(), hkv=hkv.clone(), k_i=t["k_i"].clone(), reps=reps.clone()))
    torch.cuda.synchronize()
    log(f"[bench] hybrid pair inputs + {R} cache replicas ready in {time.time() - t0:.1f}s")

    def csa_select(c):
        # compressed entry + block mean + visible count of the new token, one launch
        nv = ops.decode_append(t["csa_raw_kv"], t["csa_z"], t["csa_b"], 8, 4, t["q_pos"], c["ckv"], c["k_i"],
                               c["reps"], B, L=L)
        return ops.hisa_topk(t["q_i"], c["k_i"], t["w_i"], nv, c["reps"], B, m, k)

    def csa_attend(c, idx):
        return ops.sparse_attn(t["csa_q"], c["ckv"], idx, t["csa_raw_kv"], t["q_pos"], 128, L=L)

    def csa_step(c):
        return csa_attend(c, csa_select(c))

    def hca_step(c):
        nvh = ops.decode_append(t["hca_raw_kv"], t["hca_z"], t["hca_b"], 128, 128, t["q_pos"], c["hkv"], L=L)
        return ops.dense_compressed_attn(t["hca_q"], c["hkv"], nvh, t["hca_raw_kv"], t["q_pos"], 128, L=L)

    def step(c):  # eager, one stream
        return csa_step(c), hca_step(c)

    # The two branches' inputs are independent.  Each step is one native
    # plan run (hattn_decode_plan_run): one host call, 6 kernels on the
    # current stream with the HCA work inside the CSA launches.  One plan per
    # cache replica.
    plans = [ops.DecodePlan(q_pos=t["q_pos"], csa_raw_kv=t["csa_raw_kv"], csa_logits=t["csa_z"],
                            csa_pos_bias=t["csa_b"], csa_ckv=c["ckv"], k_i=c["k_i"], reps=c["reps"], q_i=t["q_i"],
                            w_i=t["w_i"], csa_q=t["csa_q"], hca_raw_kv=t["hca_raw_kv"], hca_logits=t["hca_z"],
                            hca_pos_bias=t["hca_b"], hca_ckv=c["hkv"], hca_q=t["hca_q"], B=B, m=m, k=k, L=L)
             for c in caches]

    def replay(i):
        plans[i % R].run()

    for i in range(args.warmup):
        replay(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        replay(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    dist = step_distribution(replay, max(30, args.steps))

    # The same step as one launch: each plan's graph of its 6 kernels
    # (hattn_decode_plan_run_graph; the first call per plan captures it).
    def replay_graph(i):
        plans[i % R].run_graph()

    for i in range(max(args.warmup, R)):
        replay_graph(i)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        replay_graph(i)
    e1.record()
    torch.cuda.synchronize()
    native_graph_ms = e0.elapsed_time(e1) / args.steps
    native_graph_dist = step_distribution(replay_graph, max(30, args.steps))

    # The same plan steps replayed from one HIP graph holding one step per
    # cache replica (a decode loop captured once): kernel boundaries inside a
    # graph cost less than stream launches, and one replay enqueues R steps.
    chain = capture_chain(lambda p_: p_.run(), plans)
    reps_graph = max(1, args.steps // R)
    graph_plan_ms = timed_graphs([chain], reps_graph, max(1, args.warmup // R)) / R
    graph_dist = step_distribution(lambda i: chain.replay(), max(30, args.steps // R))
    graph_dist = {kk: (v / R if kk != "n" else v) for kk, v in graph_dist.items()}
    del chain

    # For comparison: the same step as two HIP graphs (one per branch) on two
    # streams joined every step; torch's graph replays and stream joins cost
    # more host time than the GPU needs for the step.
    side = torch.cuda.Stream()
    g_csa = capture(csa_step, caches, stream=torch.cuda.Stream())
    g_hca = capture(hca_step, caches, stream=torch.cuda.Stream())
    main = torch.cuda.current_stream()

    def graph_replay(i):
        side.wait_stream(main)
        with torch.cuda.stream(side):
            g_hca[i % R].replay()
        g_csa[i % R].replay()
        main.wait_stream(side)

    for i in range(args.warmup):
        graph_replay(i)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        graph_replay(i)
    e1.record()
    torch.cuda.synchronize()
    graph_ms = e0.elapsed_time(e1) / args.steps
    del g_csa, g_hca
    kt = kernel_times(lambda p_: p_.run(), plans, args.steps)  # the timed path
    kt_calls = kernel_times(step, caches, args.steps)  # the same step through the separate calls
    o1, o2 = step(caches[0])
    torch.cuda.synchronize()
    assert torch.isfinite(o1).all() and torch.isfinite(o2).all()

    # per-kernel algorithmic bytes for this step (one launch each)
    win = 128
    kb = {
        "attn_pair_mfma": bt * (attn_bytes(Nh + win) + attn_bytes(k + win)),  # HCA dense + CSA sparse, one launch
        "attn_pair_fused": bt * (attn_bytes(Nh + win) + attn_bytes(k + win)),  # the same, token select fused in
        "score_stage1_mfma": bt * hisa_stage1_bytes(nb),
        "score_stage2_mfma": bt * hisa_stage2_bytes(m * B),
        "stage2_fused": bt * hisa_stage2_bytes(m * B),
    }
    step_bytes = sum(kb.values())
    flat_ms = flat_decode_step(args, t, caches, k) if args.flat_compare else None
    info = dict(ms=ms, graph_ms=graph_ms, kernels=kt, kernels_calls=kt_calls, kernel_bytes=kb, step_bytes=step_bytes,
                bt=bt, N=N, Nh=Nh, k=k, L=L, dist=dist, flat_ms=flat_ms, graph_plan_ms=graph_plan_ms,
                graph_dist=graph_dist, native_graph_ms=native_graph_ms, native_graph_dist=native_graph_dist)
    for p_ in plans:
        p_.close()
    return info


# ----------------------------------------------------------------------------
# extras
# ----------------------------------------------------------------------------

def hca_decode_b32(args):
    import torch
    from compressed_attention_amd import ops, synth

    dev = "cuda:0"
    bt, L, Nh = 32, 1 << 20, 8192
    W = synth.hca_decode(0, device=dev, bt=bt, L=L)
    t = W.tensors
    # compression of 32 x 1M tokens (HCA, disjoint 128)
    hkv = ops.compress(t["raw_kv"], t["z"], t["b"], 128, 128)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        ops.compress(t["raw_kv"], t["z"], t["b"], 128, 128, out=hkv)
    e1.record()
    torch.cuda.synchronize()
    comp_ms = e0.elapsed_time(e1) / 3
    comp_bytes = bt * (L * 512 + L * 4 + Nh * 512)
    nvh = ops.visible_count(t["q_pos"], 128, 128, Nh)
    reps = [hkv] + [hkv.clone() for _ in range(3)]

    def step(c):
        return ops.dense_compressed_attn(t["q"], c, nvh, t["raw_kv"], t["q_pos"], 128)

    # the replicas' steps back to back in one graph (len(reps) steps a replay)
    g = capture_chain(step, reps)
    ms = timed_graphs([g], max(1, args.steps // len(reps)), max(1, args.warmup // len(reps))) / len(reps)
    kt = kernel_times(step, reps, args.steps)
    byt = bt * attn_bytes(Nh + 128)
    del g
    return dict(ms=ms, kernels=kt, step_bytes=byt, compress_ms=comp_ms, compress_bytes=comp_bytes, bt=bt)


def csa2_decode(args):
    """CSA2 decode step at 1M context: 8 sequences, a group of 2 layers
    sharing one cache compressed at rate 2 (w = 4, s = 2: 524,287 entries)
    and one flat top-512 selection (16 x 128 indexer over the compressed
    indexer keys), each layer's 64 heads attending to the selection plus its
    128-token window (the two layers as 128 MFMA heads).  The step compresses
    the entry the new token completes (K|V and indexer key together), counts
    the visible entries, selects and attends; replayed as graphs."""
    import numpy as np
    import torch
    from compressed_attention_amd import ops, synth

    dev = "cuda:0"
    bt, L, G, H, d, DI, k, w, s = 8, 1 << 20, 2, 64, 128, 128, 512, 4, 2
    N = (L - w) // s + 1
    names = synth.tensor_seeds(11, ["raw", "raw_ki", "z", "b", "q", "q_i", "w_i"])
    raw = synth.normal((bt, L, 2 * d), names["raw"], dtype=torch.bfloat16, device=dev)
    raw_ki = synth.normal((bt, L, DI), names["raw_ki"], dtype=torch.bfloat16, device=dev)
    z = synth.normal((bt, L), names["z"], device=dev)
    b = synth.tiled_bias(2, w, names["b"]).to(dev)
    q = synth.normal((bt, 1, G * H, d), names["q"], dtype=torch.bfloat16, device=dev)
    q_i = synth.normal((bt, 1, 16, DI), names["q_i"], dtype=torch.bfloat16, device=dev)
    w_i = synth.uniform((bt, 1, 16), names["w_i"], device=dev)
    q_pos = torch.full((bt, 1), L - 1, dtype=torch.int32, device=dev)
    ckv, k_i = ops.compress_with_index(raw, raw_ki, z, b, w, s)
    torch.cuda.synchronize()

    def step(_):
        ops.compress_with_index(raw, raw_ki, z, b, w, s, N - 1, N, out=ckv, out_i=k_i)
        nv = ops.visible_count(q_pos, w, s, N)
        idx = ops.index_topk(q_i, k_i, w_i, nv, k)
        return ops.sparse_attn(q, ckv, idx, raw, q_pos, 128)

    graphs = capture(step, [None])
    ms = timed_graphs(graphs, max(10, args.steps), 3)
    kt = kernel_times(step, [None], max(10, args.steps // 2))
    del graphs

    # The same step with HISA in place of the flat indexer (B = 128, m = 16:
    # 2,048 candidates for the top-512, the pages' m*B = 4k); the step also
    # refreshes the mean of the block holding the new entry.  After the
    # entry and its indexer key are compressed, one decode-append launch
    # gives the visible count and that block mean (it writes the K|V entry
    # again, the same 4-row merge).
    B, m = 128, 16
    reps = ops.hisa_pool(k_i, B)

    def step_hisa(_):
        ops.compress_with_index(raw, raw_ki, z, b, w, s, N - 1, N, out=ckv, out_i=k_i)
        nv = ops.decode_append(raw, z, b, w, s, q_pos, ckv, k_i=k_i, reps=reps, B=B)
        idx = ops.hisa_topk(q_i, k_i, w_i, nv, reps, B, m, k)
        return ops.sparse_attn(q, ckv, idx, raw, q_pos, 128), idx

    graphs = capture(lambda c: step_hisa(c)[0], [None])
    ms_h = timed_graphs(graphs, max(10, args.steps), 3)
    kt_h = kernel_times(lambda c: step_hisa(c)[0], [None], max(10, args.steps // 2))
    del graphs
    nv = ops.visible_count(q_pos, w, s, N)
    i_flat = ops.index_topk(q_i, k_i, w_i, nv, k).cpu().numpy()
    i_hisa = step_hisa(None)[1].cpu().numpy()
    iou = float(np.mean([len(np.intersect1d(i_flat[r, 0], i_hisa[r, 0])) /
                         len(np.union1d(i_flat[r, 0], i_hisa[r, 0])) for r in range(bt)]))
    return dict(ms=ms, kernels=kt, bt=bt, layers=G, N=N, ms_hisa=ms_h, kernels_hisa=kt_h, iou=iou)


def csa_prefill(args):
    """CSA prefill chunk: 1,024 query tokens at the end of a 32K sequence
    (H=64, d=128; 8,191 entries; 16 x 64 indexer; k=512 + window 128).  The
    step is compress (whole sequence) -> visible counts -> flat top-k ->
    sparse attention, replayed as one graph."""
    import torch
    from compressed_attention_amd import ops, synth

    dev = "cuda:0"
    W = synth.csa_prefill_chunk(0, device=dev)
    t = W.tensors
    N, nq, k = 8191, 1024, 512
    ckv = ops.compress(t["raw_kv"], t["z"], t["b"], 8, 4)

    def step(_):
        ops.compress(t["raw_kv"], t["z"], t["b"], 8, 4, out=ckv)
        nv = ops.visible_count(t["q_pos"], 8, 4, N)
        idx = ops.index_topk(t["q_i"], t["k_i"], t["w_i"], nv, k)
        return ops.sparse_attn(t["q"], ckv, idx, t["raw_kv"], t["q_pos"], 128), nv

    graphs = capture(step, [None])
    ms = timed_graphs(graphs, max(10, args.steps // 2), 3)
    kt = kernel_times(step, [None], max(10, args.steps // 2))
    _, nv = step(None)
    torch.cuda.synchronize()
    nvh = nv.cpu().numpy()[0].astype(float)
    idx_flops = 2.0 * 16 * 64 * float(nvh.sum())
    attn_flops = 4.0 * 64 * 128 * nq * (k + 128)
    del graphs
    return dict(ms=ms, kernels=kt, idx_flops=idx_flops, attn_flops=attn_flops, nq=nq,
                compress_bytes=32768 * 512 + 32768 * 4 + N * 512)


def tiny_layer(args):
    """The tiny fp32 hybrid layer (64 queries at 4K; the parity workload),
    timed for information: both branches (compression, visible counts, flat
    top-64, sparse attention; compression, dense attention), one graph."""
    from compressed_attention_amd import ops, synth

    dev = "cuda:0"
    w = synth.tiny_hybrid_layer(0, device=dev)
    t, P = w.tensors, w.params

    def step(_):
        ckv = ops.compress(t["raw_kv"], t["z"], t["b_csa"], 8, 4)
        nv = ops.visible_count(t["q_pos"], 8, 4, ckv.shape[1])
        idx = ops.index_topk(t["q_i"], t["k_i"], t["w_i"], nv, P["k"])
        o1 = ops.sparse_attn(t["q"], ckv, idx, t["raw_kv"], t["q_pos"], P["window"])
        hkv = ops.compress(t["raw_kv"], t["z"], t["b_hca"], 128, 128)
        nvh = ops.visible_count(t["q_pos"], 128, 128, hkv.shape[1])
        o2 = ops.dense_compressed_attn(t["q"], hkv, nvh, t["raw_kv"], t["q_pos"], P["window"])
        return o1, o2

    graphs = capture(step, [None])
    ms = timed_graphs(graphs, 30, 3)
    del graphs
    return dict(ms=ms, nq=P["nq"])


def indexer_128k(args):
    import numpy as np
    import torch
    from compressed_attention_amd import ops, synth

    dev = "cuda:0"
    W = synth.indexer_128k(0, device=dev)
    t = W.tensors
    N, nq, k, B, m = 131072, 1024, 2048, 128, 64
    pos = torch.arange(N - nq, N, dtype=torch.int32, device=dev).reshape(1, nq)
    nv = ops.visible_count(pos, 1, 1, N)
    reps = ops.hisa_pool(t["k_i"], B)

    def flat(_):
        return ops.index_topk(t["q_i"], t["k_i"], t["w_i"], nv, k)

    def hisa(_):
        r = ops.hisa_pool(t["k_i"], B, out=reps)
        return ops.hisa_topk(t["q_i"], t["k_i"], t["w_i"], nv, r, B, m, k)

    # block-sparse baseline at the same attention budget: k / B whole blocks
    def block_sparse(_):
        r = ops.hisa_pool(t["k_i"], B, out=reps)
        return ops.block_sparse_topk(t["q_i"], t["k_i"], t["w_i"], nv, r, B, k // B)

    out = {}
    for name, fn in (("flat", flat), ("hisa", hisa), ("block_sparse", block_sparse)):
        graphs = capture(fn, [None])
        ms = timed_graphs(graphs, max(5, args.steps // 5), 2)
        kt = kernel_times(fn, [None], max(5, args.steps // 5))
        out[name] = dict(ms=ms, kernels=kt)
        del graphs
    i_f = flat(None).cpu().numpy()[0]
    i_h = hisa(None).cpu().numpy()[0]
    i_b = block_sparse(None).cpu().numpy()[0]
    ious, ious_b, rec_f, rec_h, rec_b = [], [], [], [], []
    needles = set(t["needles"].tolist())
    nvh = nv.cpu().numpy()[0]
    for q in range(nq):
        a, b = set(i_f[q][i_f[q] >= 0].tolist()), set(i_h[q][i_h[q] >= 0].tolist())
        c = set(i_b[q][i_b[q] >= 0].tolist())
        ious.append(len(a & b) / max(1, len(a | b)))
        ious_b.append(len(a & c) / max(1, len(a | c)))
        vis = {x for x in needles if x < nvh[q]}
        if vis:
            rec_f.append(len(vis & a) / len(vis))
            rec_h.append(len(vis & b) / len(vis))
            rec_b.append(len(vis & c) / len(vis))
    flops = 2.0 * 16 * 128 * float(nvh.sum())
    # HISA's own work: every candidate block of each query (stage 1) and the
    # visible tokens of its m chosen blocks (stage 2, at most m * B)
    nbq = (nvh.astype(float) + B - 1) // B
    hisa_flops = 2.0 * 16 * 128 * float((nbq + np.minimum(m * B, nvh)).sum())
    out.update(hisa_flops=hisa_flops)
    out.update(iou_mean=float(sum(ious) / len(ious)), iou_min=float(min(ious)),
               needle_recall_flat=float(sum(rec_f) / len(rec_f)), needle_recall_hisa=float(sum(rec_h) / len(rec_h)),
               iou_block_sparse=float(sum(ious_b) / len(ious_b)),
               needle_recall_block_sparse=float(sum(rec_b) / len(rec_b)),
               flat_flops=flops)
    return out


# ----------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on a bounded sample of the same decode step
# ----------------------------------------------------------------------------

def host_cpu_info():
    """nproc (this process's CPU affinity), the CPU model and the BLAS pool."""
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        nproc = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = 1
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        pass
    return nproc, model, blas


def _oracle_decode_rate(k, seconds):
    """Decode queries/s of the fp64 oracle on one 2^20-token sequence per
    query (both layers), for about `seconds` of host time."""
    import numpy as np
    import torch

    import oracle
    from compressed_attention_amd import synth

    N, Nh, B, m, W = 262143, 8192, 128, 64, 128
    # One sequence's caches, drawn on the host (values do not affect timing).
    ckv = synth.normal((N, 256), 901, dtype=torch.bfloat16).double().numpy()
    hkv = synth.normal((Nh, 256), 902, dtype=torch.bfloat16).double().numpy()
    k_i = synth.normal((N, 128), 903, dtype=torch.bfloat16).double().numpy()
    tail = synth.normal((256, 256), 904, dtype=torch.bfloat16).double().numpy()  # last raw rows
    z = synth.normal((256,), 905).double().numpy()
    b8 = synth.tiled_bias(4, 8, 906).double().numpy()
    b128 = synth.tiled_bias(128, 128, 907).double().numpy()
    reps = oracle.hisa_pool(k_i, B)  # the static block-mean cache, kept outside the timing
    p_local = 255  # the query is the last of the 256 tail rows (position L-1)
    done, el = 0, 0.0
    while True:
        q = synth.normal((1, 64, 128), 1000 + done, dtype=torch.bfloat16).double().numpy()
        qh = synth.normal((1, 64, 128), 2000 + done, dtype=torch.bfloat16).double().numpy()
        q_i = synth.normal((1, 16, 128), 3000 + done, dtype=torch.bfloat16).double().numpy()
        w_i = synth.uniform((1, 16), 4000 + done).double().numpy()
        s = time.perf_counter()
        ckv[N - 1] = oracle.compress(tail[-8:], z[-8:], b8, 8, 4)[0]
        hkv[Nh - 1] = oracle.compress(tail[-128:], z[-128:], b128, 128, 128)[0]
        reps[-1] = oracle.hisa_pool(k_i[(N // B) * B:], B)[0]
        idx, _ = oracle.hisa_topk(q_i, k_i, w_i, np.array([N]), B, m, k, reps=reps)
        oracle.sparse_attention(q, ckv, idx, tail, np.array([p_local]), W, 1 / math.sqrt(128))
        oracle.dense_compressed_attention(qh, hkv, np.array([Nh]), tail, np.array([p_local]), W, 1 / math.sqrt(128))
        done += 1
        el += time.perf_counter() - s
        if el >= seconds or done >= 2000:
            break
    return done, el


def _median_s(fn, reps=3):
    import numpy as np

    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts))


def cpu_configs():
    """The fp64 oracle on the host for the other configurations, in the GPU's
    units, each bounded to a few seconds: the tiny layer in full (median of
    3); the CSA prefill chunk with its compression in full and the indexer
    and attention on 64 of its 1,024 queries; HCA decode: one query's
    attention, and the compression of 1/16 of a 2^20-token sequence; the 128K
    indexer chunk: pooling in full, flat and HISA selection on 16 of its
    1,024 queries.  Sampled parts are scaled to the whole and say so."""
    import numpy as np
    import torch

    import oracle
    from compressed_attention_amd import synth

    f = lambda x: x.double().numpy()  # noqa: E731
    out = {}
    # tiny hybrid layer (fp32), whole layer
    t, P = (lambda w: (w.tensors, w.params))(synth.tiny_hybrid_layer(0))
    raw, z, pos = f(t["raw_kv"][0]), f(t["z"][0]), t["q_pos"][0].numpy()

    def tiny():
        ckv = oracle.compress(raw, z, f(t["b_csa"]), 8, 4)
        nv = np.array([oracle.n_visible(int(p), 8, 4, ckv.shape[0]) for p in pos])
        idx = oracle.flat_topk(f(t["q_i"][0]), f(t["k_i"][0]), f(t["w_i"][0]), nv, P["k"])
        oracle.sparse_attention(f(t["q"][0]), ckv, idx, raw, pos, 128, 1 / 8)
        hkv = oracle.compress(raw, z, f(t["b_hca"]), 128, 128)
        nvh = np.array([oracle.n_visible(int(p), 128, 128, hkv.shape[0]) for p in pos])
        oracle.dense_compressed_attention(f(t["q"][0]), hkv, nvh, raw, pos, 128, 1 / 8)

    out["tiny_layer_fp32"] = dict(ms=round(_median_s(tiny) * 1e3, 2), sample="whole layer, median of 3")
    # CSA prefill chunk
    t = synth.csa_prefill_chunk(0).tensors
    raw, z, b = f(t["raw_kv"][0]), f(t["z"][0]), f(t["b"])
    t0 = time.perf_counter()
    ckv = oracle.compress(raw, z, b, 8, 4)
    comp_s = time.perf_counter() - t0
    rows = np.arange(0, 1024, 16)
    pos = t["q_pos"][0].numpy()[rows]
    nv = np.array([oracle.n_visible(int(p), 8, 4, ckv.shape[0]) for p in pos])
    t0 = time.perf_counter()
    idx = oracle.flat_topk(f(t["q_i"][0, rows]), f(t["k_i"][0]), f(t["w_i"][0, rows]), nv, 512)
    idx_s = (time.perf_counter() - t0) * 1024 / len(rows)
    t0 = time.perf_counter()
    oracle.sparse_attention(f(t["q"][0, rows]), ckv, idx, raw, pos, 128, 1 / math.sqrt(128))
    attn_s = (time.perf_counter() - t0) * 1024 / len(rows)
    chunk_s = comp_s + idx_s + attn_s
    out["csa_prefill_32k_chunk1024"] = dict(
        ms=round(chunk_s * 1e3, 1), tokens_per_s=round(1024 / chunk_s, 1),
        stage_ms=dict(compress=round(comp_s * 1e3, 1), index=round(idx_s * 1e3, 1), attention=round(attn_s * 1e3, 1)),
        sample="compression in full; indexer and attention on 64 of the 1,024 queries, scaled by 16")
    del t, raw, ckv
    # HCA decode: one query's attention over 8,192 entries + window; the
    # compression of a sequence from 1/16 of it
    hkv = synth.normal((8192, 256), 911, dtype=torch.bfloat16).double().numpy()
    tail = synth.normal((128, 256), 912, dtype=torch.bfloat16).double().numpy()
    q = synth.normal((1, 64, 128), 913, dtype=torch.bfloat16).double().numpy()
    att_s = _median_s(lambda: oracle.dense_compressed_attention(q, hkv, [8192], tail, np.array([127]), 128,
                                                               1 / math.sqrt(128)))
    seg = synth.normal((65536, 256), 914, dtype=torch.bfloat16).double().numpy()
    zs = synth.normal((65536,), 915).double().numpy()
    bs = synth.tiled_bias(128, 128, 916).double().numpy()
    t0 = time.perf_counter()
    oracle.compress(seg, zs, bs, 128, 128)
    comp_s = (time.perf_counter() - t0) * 16
    out["hca_decode"] = dict(
        queries_per_s=round(1 / att_s, 1), compress_1M_tokens_s=round(comp_s, 2),
        sample="one query's attention (median of 3); compression of 65,536 tokens scaled by 16 to one sequence")
    del hkv, seg
    # 128K indexer chunk
    t = synth.indexer_128k(0).tensors
    k_i = f(t["k_i"][0])
    rows = np.arange(0, 1024, 64)
    nv = t["entry_pos"][0].numpy()[rows] + 1
    q_i, w_i = f(t["q_i"][0, rows]), f(t["w_i"][0, rows])
    t0 = time.perf_counter()
    reps = oracle.hisa_pool(k_i, 128)
    pool_s = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.flat_topk(q_i, k_i, w_i, nv, 2048)
    flat_s = (time.perf_counter() - t0) * 1024 / len(rows)
    t0 = time.perf_counter()
    oracle.hisa_topk(q_i, k_i, w_i, nv, 128, 64, 2048, reps=reps)
    hisa_s = (time.perf_counter() - t0) * 1024 / len(rows) + pool_s
    out["indexer_128k"] = dict(
        flat_ms=round(flat_s * 1e3, 1), hisa_ms=round(hisa_s * 1e3, 1), hisa_pool_ms=round(pool_s * 1e3, 1),
        sample="pooling in full; flat and HISA selection on 16 of the 1,024 queries, scaled by 64")
    return out


def cpu_baseline(args, k):
    """The oracle timed twice on the host: with the BLAS pool as the process
    starts it (all of the host share) and limited to one thread."""
    nproc, model, blas = host_cpu_info()
    half = max(1.0, args.cpu_seconds / 2)
    done, el = _oracle_decode_rate(k, half)
    one = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            d1, e1 = _oracle_decode_rate(k, half)
        one = d1 / e1
    except Exception as exc:  # pragma: no cover
        log(f"[bench] one-thread oracle run skipped: {exc}")
    return dict(value=done / el, unit="decode queries/s", cores=int(blas), kind="oracle",
                value_1core=one, nproc=nproc, cpu_model=model, blas_threads=int(blas),
                sample=f"{done} decode queries of one 2^20-token sequence each (both layers, k={k}), "
                       f"{el:.1f} s of host time with {blas} BLAS threads, then the same with 1 thread; "
                       f"block means precomputed as in the GPU step")


# ----------------------------------------------------------------------------
# counter probe: the decode step as timed (its dominant kernel is the paired
# attention launch), plus a plain copy of known size that calibrates the
# counters
# ----------------------------------------------------------------------------

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_pair_decode_1M_b8_traffic.txt")
ATTN_SOURCES = ["compressed_attention_amd/csrc/attention.hip", "compressed_attention_amd/csrc/common.h",
                "compressed_attention_amd/csrc/internal.h"]
COPY_BYTES = 256 * MiB


def attn_sources_sha():
    import hashlib

    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def probe_decode_plan(args):
    """Runs the layer-pair decode step (the native plan, 8 sequences at 1M)
    ``args.steps`` times over rotating cache replicas, then copies a 256 MiB
    buffer 3 times.  Run under rocprofv3 --pmc."""
    import torch
    from compressed_attention_amd import ops, synth

    dev = "cuda:0"
    bt, L, N, B, m = 8, 1 << 20, 262143, 128, 64
    W = synth.hybrid_pair_decode(0, device=dev, bt=bt, L=L, N_csa=N)
    t = dict(W.tensors)
    ckv = ops.compress(t["csa_raw_kv"], t["csa_z"], t["csa_b"], 8, 4)
    hkv = ops.compress(t["hca_raw_kv"], t["hca_z"], t["hca_b"], 128, 128)
    reps = ops.hisa_pool(t["k_i"], B)
    keep_rings(t, L)
    plans = []
    for r in range(args.replicas):
        c = (ckv, hkv, reps) if r == 0 else (ckv.clone(), hkv.clone(), reps.clone())
        plans.append(ops.DecodePlan(q_pos=t["q_pos"], csa_raw_kv=t["csa_raw_kv"], csa_logits=t["csa_z"],
                                    csa_pos_bias=t["csa_b"], csa_ckv=c[0], k_i=t["k_i"], reps=c[2], q_i=t["q_i"],
                                    w_i=t["w_i"], csa_q=t["csa_q"], hca_raw_kv=t["hca_raw_kv"], hca_logits=t["hca_z"],
                                    hca_pos_bias=t["hca_b"], hca_ckv=c[1], hca_q=t["hca_q"], B=B, m=m, k=args.k,
                                    L=L))
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev).normal_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    log(f"[probe] sources {attn_sources_sha()}: {args.steps} decode steps, then 3 copies of {COPY_BYTES} B")
    for i in range(args.steps):
        plans[i % len(plans)].run()
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)  # one elementwise kernel: reads and writes COPY_BYTES
    torch.cuda.synchronize()
    for p_ in plans:
        p_.close()
    log("[probe] done")


def probe_indexer_128k(args):
    """Runs the 128K flat indexer chunk (1,024 queries, 16 x 128, k = 2,048)
    and then the HISA indexer on it, ``args.steps`` times each.  Run under
    rocprofv3 --pmc for the score kernels' MFMA and VALU counters."""
    import torch
    from compressed_attention_amd import ops, synth

    dev = "cuda:0"
    W = synth.indexer_128k(0, device=dev)
    t = W.tensors
    N, nq, k, B, m = 131072, 1024, 2048, 128, 64
    pos = torch.arange(N - nq, N, dtype=torch.int32, device=dev).reshape(1, nq)
    nv = ops.visible_count(pos, 1, 1, N)
    reps = ops.hisa_pool(t["k_i"], B)
    torch.cuda.synchronize()
    log(f"[probe] {args.steps} flat indexer chunks, then {args.steps} HISA chunks")
    for _ in range(args.steps):
        ops.index_topk(t["q_i"], t["k_i"], t["w_i"], nv, k)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        ops.hisa_topk(t["q_i"], t["k_i"], t["w_i"], nv, reps, B, m, k)
    torch.cuda.synchronize()
    log("[probe] done")


def probe_hca_b32(args):
    """Compresses 32 sequences of 1M tokens (HCA, w = s = 128) once, runs
    ``args.steps`` HCA dense decode steps at batch 32 over rotating cache
    replicas, then copies a 256 MiB buffer 3 times.  Run under rocprofv3
    --pmc for the compression and attention kernels' HBM traffic."""
    import torch
    from compressed_attention_amd import ops, synth

    dev = "cuda:0"
    bt, L, Nh = 32, 1 << 20, 8192
    W = synth.hca_decode(0, device=dev, bt=bt, L=L)
    t = W.tensors
    hkv = ops.compress(t["raw_kv"], t["z"], t["b"], 128, 128)
    nvh = ops.visible_count(t["q_pos"], 128, 128, Nh)
    reps = [hkv] + [hkv.clone() for _ in range(3)]
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev).normal_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    log(f"[probe] sources {attn_sources_sha()}: {args.steps} HCA decode steps at batch 32, "
        f"then 3 copies of {COPY_BYTES} B")
    for i in range(args.steps):
        ops.dense_compressed_attn(t["q"], reps[i % len(reps)], nvh, t["raw_kv"], t["q_pos"], 128)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log("[probe] done")


def load_traffic(kernel):
    """Calibrated HBM bytes per launch of the dominant kernel (its timer
    name), from the committed counter summary; None when it is missing,
    covers another kernel, or was taken on other sources than the ones
    here."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as fh:
            for line in fh:
                if ":" in line and not line.startswith(("#", " ")):
                    a, b = line.split(":", 1)
                    kv[a.strip()] = b.strip()
        if kv.get("sources_sha256_16") != attn_sources_sha() or kv.get("timer_name") != kernel:
            return None
        return float(kv["fetch_bytes_per_launch"]) + float(kv["write_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None

# ----------------------------------------------------------------------------

def roofline_entry(kern_ms, nbytes):
    gbs = nbytes / (kern_ms * 1e-3) / 1e9
    return gbs


def measured_copy_GBps(nbytes: int = 1 << 30, reps: int = 10) -> dict:
    """HBM bandwidth (read + written bytes per second) of two plain streams
    that each read and write nbytes: the runtime's device-to-device copy
    (copy_) and one elementwise kernel (neg on bf16).  The faster one is the
    measured reference reported beside the 8 TB/s spec peak."""
    import torch

    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda:0").normal_()
    dst = torch.empty_like(src)
    runs = {"copy_": lambda: dst.copy_(src), "neg_bf16": lambda: torch.neg(src, out=dst)}
    res = {}
    for name, fn in runs.items():
        for _ in range(2):
            fn()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        res[name] = round(2.0 * nbytes * reps / (t0.elapsed_time(t1) * 1e-3) / 1e9, 1)
    del src, dst
    torch.cuda.empty_cache()
    return {"best": max(res.values()), "streams": res}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--k", type=int, default=2048, choices=[512, 2048])
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flat-compare", dest="flat_compare", action="store_false",
                    help="skip timing the decode step with the flat indexer in place of HISA")
    ap.add_argument("--probe", choices=["decode_plan", "indexer_128k", "hca_b32"], default=None,
                    help="run only the decode step and a calibration copy, only the 128K indexer chunk, or "
                         "only the batch-32 HCA compression and decode with a calibration copy "
                         "(for rocprofv3 --pmc)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(decode batches shard by sequence with no communication).", file=sys.stderr)
        sys.exit(2)

    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    from compressed_attention_amd import _lib

    _lib.lib()  # fail loudly if the HIP library is missing
    if args.probe == "decode_plan":
        probe_decode_plan(args)
        return
    if args.probe == "indexer_128k":
        probe_indexer_128k(args)
        return
    if args.probe == "hca_b32":
        probe_hca_b32(args)
        return

    main_k = args.k
    res = hybrid_pair(args)
    log(f"[bench] hybrid pair k={main_k}: {res['ms'] * 1e3:.1f} us/step (two HIP graphs: {res['graph_ms'] * 1e3:.1f})")
    extras = {}
    if not args.no_extras:
        a2 = argparse.Namespace(**vars(args))
        a2.k = 512 if main_k == 2048 else 2048
        r2 = hybrid_pair(a2)
        extras[f"hybrid_pair_k{a2.k}"] = dict(us_per_step=r2["ms"] * 1e3, queries_per_s=r2["bt"] / (r2["ms"] * 1e-3),
                                             step_us=r2["dist"],
                                             flat_indexer_step_us=None if r2["flat_ms"] is None else r2["flat_ms"] * 1e3,
                                             step_GBps=r2["step_bytes"] / (r2["ms"] * 1e-3) / 1e9,
                                             hbm_frac=r2["step_bytes"] / (r2["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS)
        torch.cuda.empty_cache()
        h = hca_decode_b32(args)
        dk = h["kernels"].get("attn_dense_mfma", (float("nan"), 1))[0]
        extras["hca_decode_b32"] = dict(
            us_per_step=h["ms"] * 1e3, queries_per_s=h["bt"] / (h["ms"] * 1e-3),
            step_MiB=h["step_bytes"] / MiB, step_GBps=h["step_bytes"] / (h["ms"] * 1e-3) / 1e9,
            hbm_frac_step=h["step_bytes"] / (h["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
            attn_kernel_us=dk * 1e3, hbm_frac_attn_kernel=h["step_bytes"] / (dk * 1e-3) / 1e9 / HBM_PEAK_GBS,
            kernels_us={kk: v[0] * 1e3 for kk, v in h["kernels"].items()})
        extras["compress_1M_hca_b32"] = dict(ms=h["compress_ms"], GBps=h["compress_bytes"] / (h["compress_ms"] * 1e-3) / 1e9,
                                             hbm_frac=h["compress_bytes"] / (h["compress_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS)
        torch.cuda.empty_cache()
        c2 = csa2_decode(args)
        extras["csa2_decode_1M_b8_2layers"] = dict(
            us_per_step=c2["ms"] * 1e3, layer_queries_per_s=c2["bt"] * c2["layers"] / (c2["ms"] * 1e-3),
            entries=c2["N"], kernels_us={kk: v[0] * 1e3 for kk, v in c2["kernels"].items()},
            hisa_us_per_step=c2["ms_hisa"] * 1e3,
            hisa_layer_queries_per_s=c2["bt"] * c2["layers"] / (c2["ms_hisa"] * 1e-3),
            hisa_kernels_us={kk: v[0] * 1e3 for kk, v in c2["kernels_hisa"].items()},
            hisa_vs_flat_iou_mean=c2["iou"],
            note="rate-2 cache (w=4, s=2), flat top-512 over the compressed indexer keys, 2 layers as 128 heads; "
                 "hisa_*: the same step with HISA (B=128, m=16) selecting the top-512")
        torch.cuda.empty_cache()
        tl = tiny_layer(args)
        extras["tiny_layer_fp32"] = dict(ms=tl["ms"], queries_per_s=tl["nq"] / (tl["ms"] * 1e-3),
                                         note="parity workload (64 queries, both branches, fp32), one graph "
                                              "replay; for information")
        cp = csa_prefill(args)
        ck = {kk: v[0] for kk, v in cp["kernels"].items()}
        sk = ck.get("score_flat_mfma", float("nan"))
        ak = ck.get("attn_sparse_mfma", float("nan"))
        extras["csa_prefill_32k_chunk1024"] = dict(
            ms=cp["ms"], tokens_per_s=cp["nq"] / (cp["ms"] * 1e-3),
            step_TFLOPs=(cp["idx_flops"] + cp["attn_flops"]) / (cp["ms"] * 1e-3) / 1e12,
            step_mfma_frac=(cp["idx_flops"] + cp["attn_flops"]) / (cp["ms"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            index_score_mfma_frac=cp["idx_flops"] / (sk * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            sparse_attn_mfma_frac=cp["attn_flops"] / (ak * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            kernels_us={kk: v * 1e3 for kk, v in ck.items()})
        torch.cuda.empty_cache()
        ix = indexer_128k(args)
        # the pass that scores every visible key: the collecting pass of the
        # fused path (its sample pass is extra work, not counted)
        fkern = ix["flat"]["kernels"]
        fk = fkern.get("score_flat_collect", fkern.get("score_flat_mfma", (float("nan"), 1)))[0]
        extras["indexer_128k"] = dict(
            flat_ms=ix["flat"]["ms"], hisa_ms=ix["hisa"]["ms"], hisa_speedup=ix["flat"]["ms"] / ix["hisa"]["ms"],
            flat_score_kernel_ms=fk, flat_score_TFLOPs=ix["flat_flops"] / (fk * 1e-3) / 1e12,
            flat_score_mfma_frac=ix["flat_flops"] / (fk * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            flat_total_mfma_frac=ix["flat_flops"] / (ix["flat"]["ms"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            hisa_TFLOPs=ix["hisa_flops"] / (ix["hisa"]["ms"] * 1e-3) / 1e12,
            hisa_mfma_frac=ix["hisa_flops"] / (ix["hisa"]["ms"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            hisa_vs_flat_iou_mean=ix["iou_mean"], hisa_vs_flat_iou_min=ix["iou_min"],
            block_sparse_ms=ix["block_sparse"]["ms"], block_sparse_blocks=16,
            block_sparse_vs_flat_iou_mean=ix["iou_block_sparse"],
            needle_recall_block_sparse=ix["needle_recall_block_sparse"],
            block_sparse_kernels_ms={kk: v[0] for kk, v in ix["block_sparse"]["kernels"].items()},
            needle_recall_flat=ix["needle_recall_flat"], needle_recall_hisa=ix["needle_recall_hisa"],
            flat_kernels_ms={kk: v[0] for kk, v in ix["flat"]["kernels"].items()},
            hisa_kernels_ms={kk: v[0] for kk, v in ix["hisa"]["kernels"].items()},
            pages_context="HISA about 2x (32K) / 4x (128K) faster than the flat indexer, hardware not stated")
        torch.cuda.empty_cache()

    ms = res["ms"]
    kt = res["kernels"]
    # dominant kernel of the step: the modelled kernel with the largest time
    # per step (kernel times come from the sequential eager pass)
    dom = max((kk for kk in kt if kk in res["kernel_bytes"]), key=lambda kk: kt[kk][0] * kt[kk][1])
    dom_ms = kt[dom][0]
    dom_bytes = res["kernel_bytes"].get(dom)
    traffic = load_traffic(dom)
    roof = dict(bound="hbm", achieved=None, peak=HBM_PEAK_GBS, unit="GB/s", frac=None,
                traffic=None if traffic is None else round(traffic), kernel=dom, kernel_us=dom_ms * 1e3)
    if dom_bytes:
        a = dom_bytes / (dom_ms * 1e-3) / 1e9
        roof.update(achieved=round(a, 1), frac=round(a / HBM_PEAK_GBS, 4), algorithmic_bytes=dom_bytes)
    copy = measured_copy_GBps()
    copy_gbps = copy["best"]
    roof["measured_copy_GBps"] = copy_gbps
    roof["measured_copy_streams_GBps"] = copy["streams"]
    if dom_bytes:
        roof["frac_of_measured_copy"] = round(roof["achieved"] / copy_gbps, 4)
    line = {
        "metric": "decode queries/s at 1M context (CSA+HCA hybrid layer pair, HISA top-k)",
        "value": round(res["bt"] / (ms * 1e-3), 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded device draws; N(0,1) K/V/q, logits N(0,1), bias N(0,0.1))",
        "config": {"workload": "hybrid_pair_decode_1M", "batch": res["bt"], "context": res["L"], "heads": 64,
                   "head_dim": 128, "window": 128, "csa_entries": res["N"], "hca_entries": res["Nh"],
                   "indexer": "16x128", "hisa_B": 128, "hisa_m": 64, "k": res["k"], "cache_replicas": args.replicas,
                   "raw_rows_kept": 128,
                   "launch": "native decode plan (one host call, 6 kernels per step)"},
        "step_us": {kk: round(v, 2) for kk, v in res["dist"].items() if kk != "n"} | {"n": res["dist"]["n"]},
        "step_us_one_launch": {"timed": round(res["native_graph_ms"] * 1e3, 2),
                               **{kk: round(v, 2) for kk, v in res["native_graph_dist"].items()}},
        "step_us_plan_graph": round(res["graph_plan_ms"] * 1e3, 2),
        "step_us_plan_graph_dist": {kk: round(v, 2) for kk, v in res["graph_dist"].items()},
        "flat_indexer_step_us": None if res["flat_ms"] is None else round(res["flat_ms"] * 1e3, 1),
        "step_GBps": round(res["step_bytes"] / (ms * 1e-3) / 1e9, 1),
        "step_hbm_frac": round(res["step_bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": roof,
        "kernels_us": {kk: round(v[0] * 1e3, 2) for kk, v in kt.items()},
        "kernels_us_separate_calls": {kk: round(v[0] * 1e3, 2) for kk, v in res["kernels_calls"].items()},
        "step_us_two_graphs": round(res["graph_ms"] * 1e3, 1),
        "extras": extras,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args, main_k)
        line["cpu_baseline"]["other_configs"] = cpu_configs()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
