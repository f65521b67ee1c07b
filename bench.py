#!/usr/bin/env python3
"""Benchmark of the indexer-selected sparse-attention hot path on one MI355X.

Headline (``value``): decode steps/s at 1,048,320-token context, batch 4,
12 sparse-attention layers run in sequence, one qsa_decode_layer call per
layer (pooled-key scan with per-chunk candidate lists; then per (query,
kv head, split) the exact top-512 blocks, sparse attention over the 2,048
selected tokens and the log-sum-exp merge). One step = all 12 layers for
the 4 sequences, captured once in a HIP graph and replayed, scheduled as
two micro-batches (sequences 0-1 and 2-3) that each go through the layers
in order on a stream of their own (pipeline.decode_step_streams): one
micro-batch's latency-bound attention tail overlaps the other's
bandwidth-bound scan; the outputs are checked bit-identical to the batch-4
calls. The same step on one stream (batch-4 calls) and as separate calls
(qsa_index_topk, qsa_sparse_decode, qsa_lse_merge) is timed the same way
and reported beside it. Inputs (K, V, raw and pooled
indexer keys, queries) are seeded, synthetic and resident in HBM before the
timed region.

Also reported: HBM GB/s of the step (algorithmic bytes), the prefill chunk
(4096 queries after a 60,000-token history, 8192-token history tiles, and
1024-token tiles) in query tokens/s, the roofline of the dominant kernel
(the pooled-key scan with its candidate lists, qsa_index_lists) with its launch duration
timed by HIP events on the launch stream, and the CPU oracle timed on the host on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse-attn decode steps/s + HBM GB/s at 1M ctx; prefill query tok/s"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0

DECODE = dict(name="decode L=1048320 B=4 12 layers, 16 q heads / 2 kv heads, head_dim 256, top-512 of 4-token blocks",
              config_id=3, ctx=1048320, batch=4, layers=12)
SMALL_DECODES = (dict(name="decode L=8192 B=1 1 layer", config_id=1, ctx=8192, layers=1),
                 dict(name="decode L=131072 B=1 12 layers run in sequence", config_id=2, ctx=131072, layers=12))
MLA = dict(name="shared-latent variant: 64 q heads over one 576-wide bf16 latent row per token (V = first 512), "
                "token indexer 4 heads x 64-d ReLU-weighted, top-2048 tokens, context 131072",
           config_id=5, ctx=131072, batch=8, chunk=2048, tiles=(131072, 32768))
PREFILL = dict(name="prefill 4096 queries after a 60000-token history, 8192-token tiles", config_id=4,
               history=60000, chunk=4096, tiles=(8192, 1024))


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def fill(t, seed, stream):
    from qsa_inputs.gpu import fill_normal_bf16
    fill_normal_bf16(t, seed, stream)


def build_decode(pkg, pipeline, qi, torch):
    """Device-resident inputs of the 1M-context decode workload."""
    L, B, NL = DECODE["ctx"], DECODE["batch"], DECODE["layers"]
    seed = qi.config_seed(DECODE["config_id"])
    dev = "cuda"
    layers = []
    t0 = time.time()
    for l in range(NL):
        raw = torch.empty(B, L, 128, dtype=torch.bfloat16, device=dev)
        k = torch.empty(B, L, 2, 256, dtype=torch.bfloat16, device=dev)
        v = torch.empty(B, L, 2, 256, dtype=torch.bfloat16, device=dev)
        q = torch.empty(B, 16, 256, dtype=torch.bfloat16, device=dev)
        q_idx = torch.empty(B, 1, 128, dtype=torch.bfloat16, device=dev)
        for s in range(B):
            fill(raw[s], seed, qi.stream_id(l, s, "raw_key"))
            fill(k[s], seed, qi.stream_id(l, s, "k"))
            fill(v[s], seed, qi.stream_id(l, s, "v"))
            fill(q[s], seed, qi.stream_id(l, s, "q"))
            fill(q_idx[s], seed, qi.stream_id(l, s, "q_idx"))
        pooled = torch.empty(B, L // 4, 128, dtype=torch.bfloat16, device=dev)
        layers.append(dict(raw=raw, k=k, v=v, q=q, q_idx=q_idx, pooled=pooled, kv=pkg.make_kv(k, v)))
        torch.cuda.synchronize()
        log(f"decode inputs: layer {l + 1}/{NL} filled ({time.time() - t0:.1f} s)")
    # pooling happens when a block completes (append time), not per step
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for lay in layers:
        pkg.qsa_pool_keys(lay["raw"], lay["pooled"], block=4)
    ev1.record()
    torch.cuda.synchronize()
    pool_ms = ev0.elapsed_time(ev1)
    q_ctx = torch.full((B,), L, dtype=torch.int32, device=dev)
    q_seq = torch.arange(B, dtype=torch.int32, device=dev)
    return layers, q_ctx, q_seq, pool_ms


def time_graph(torch, fn, steps, warmup):
    """Capture fn in a graph, replay warmup + steps times; ms per replay."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # eager run once (also checks the calls)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall, g


def replay_median(torch, g, steps):
    """Median and mean ms of `steps` replays of graph g, each between its own
    pair of HIP events (a separate pass from the one-pair headline timing)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in evs:
        e0.record()
        g.replay()
        e1.record()
    torch.cuda.synchronize()
    t = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    return t[len(t) // 2], sum(t) / len(t)


def time_launches(torch, fn, reps):
    """Average duration of one call of fn (HIP events on the current stream)."""
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def run_decode(pkg, pipeline, bm, qi, torch, steps, warmup):
    layers, q_ctx, q_seq, pool_ms = build_decode(pkg, pipeline, qi, torch)
    L, B = DECODE["ctx"], DECODE["batch"]
    bufs = [pipeline.decode_buffers(pkg.SEL_A, pkg.ATTN_A, B, L) for _ in layers]

    def step(fused):
        for lay, bf in zip(layers, bufs):
            pipeline.decode_layer(pkg.SEL_A, pkg.ATTN_A, q_ctx, L, lay["q_idx"], lay["pooled"], lay["q"], lay["kv"],
                                  bf, q_seq=q_seq, fused=fused)

    # headline: one qsa_decode_layer call per layer
    ms, wall, graph = time_graph(torch, lambda: step(True), steps, warmup)
    ms_med, ms_mean_each = replay_median(torch, graph, steps)
    del graph
    for bf in bufs:  # every bounded merge wait of the timed replays ended in time
        pkg.check_decode_layer_error(bf.layer_ws)
    # the same step as separate calls (index_topk, sparse_decode, lse_merge)
    ms_sep, _, graph = time_graph(torch, lambda: step(False), max(10, steps // 2), warmup)
    del graph
    unit_bytes = bm.decode_unit_bytes(L)
    step_bytes = unit_bytes * B * len(layers)
    # per-kernel durations, each timed alone over every layer (HIP events, launch stream)
    b0, lay0 = bufs[0], layers[0]
    reps = max(10, steps)

    def lists_only():  # as the headline runs it: no score buffer
        for lay, bf in zip(layers, bufs):
            pkg.qsa_index_lists(pkg.SEL_A, q_ctx, L, lay["q_idx"], lay["pooled"], None, bf.itk_ws, q_seq=q_seq)

    def scan_select_only():
        for lay, bf in zip(layers, bufs):
            pkg.qsa_index_topk(pkg.SEL_A, q_ctx, L, lay["q_idx"], lay["pooled"], bf.scores, bf.sel, bf.n_sel,
                               bf.itk_ws, q_seq=q_seq)

    lists_ms = time_launches(torch, lists_only, reps) / len(layers)
    scan_ms = time_launches(torch, scan_select_only, reps) / len(layers)
    # the step with the cache write in front of each layer: the token at
    # position L - 1 (its K/V rows, raw key, and the pooled key of the block
    # it completes), as a decode step does before the layer reads the cache
    seed = qi.config_seed(DECODE["config_id"])
    k_new = torch.empty(B, 2, 256, dtype=torch.bfloat16, device="cuda")
    v_new = torch.empty_like(k_new)
    raw_new = torch.empty(B, 128, dtype=torch.bfloat16, device="cuda")
    fill(k_new, seed, qi.stream_id(99, 0, "k"))
    fill(v_new, seed, qi.stream_id(99, 0, "v"))
    fill(raw_new, seed, qi.stream_id(99, 0, "raw_key"))
    q_pos = q_ctx - 1

    def step_append():
        for lay, bf in zip(layers, bufs):
            pkg.qsa_kv_append(pkg.SEL_A, pkg.ATTN_A, q_pos, k_new, lay["kv"], v_new=v_new, raw_new=raw_new,
                              raw_keys=lay["raw"], pooled=lay["pooled"], q_seq=q_seq)
            pipeline.decode_layer(pkg.SEL_A, pkg.ATTN_A, q_ctx, L, lay["q_idx"], lay["pooled"], lay["q"], lay["kv"],
                                  bf, q_seq=q_seq, fused=True)

    ms_app, _, graph = time_graph(torch, step_append, max(10, steps // 2), warmup)
    del graph
    # layer 0 with its K/V rows in pinned host memory, read zero-copy over the
    # host link (pooled keys, queries and outputs stay in device memory)
    lay0, b0 = layers[0], bufs[0]
    k_host = torch.empty(lay0["k"].shape, dtype=torch.bfloat16, pin_memory=True)
    v_host = torch.empty(lay0["v"].shape, dtype=torch.bfloat16, pin_memory=True)
    k_host.copy_(lay0["k"])
    v_host.copy_(lay0["v"])
    torch.cuda.synchronize()
    kv_host = pkg.make_kv(k_host, v_host)

    def layer_host():
        pipeline.decode_layer(pkg.SEL_A, pkg.ATTN_A, q_ctx, L, lay0["q_idx"], lay0["pooled"], lay0["q"], kv_host,
                              b0, q_seq=q_seq, fused=True)

    def layer_dev():
        pipeline.decode_layer(pkg.SEL_A, pkg.ATTN_A, q_ctx, L, lay0["q_idx"], lay0["pooled"], lay0["q"], lay0["kv"],
                              b0, q_seq=q_seq, fused=True)

    ms_host, _, graph = time_graph(torch, layer_host, max(10, steps // 2), warmup)
    del graph
    ms_dev1, _, graph = time_graph(torch, layer_dev, max(10, steps // 2), warmup)
    del graph
    rcache = run_row_cache(pkg, pipeline, qi, torch, lay0, kv_host, q_ctx, q_seq, L, B, b0.n_split)
    del kv_host, k_host, v_host
    # the same step with FP8 pooled keys (128 E4M3 codes + an fp32 scale per
    # block, quantized from each layer's bf16 pooled keys; K/V rows stay bf16)
    for lay in layers:
        lay["pooled_fp8"] = pkg.fp8_keys_empty(B, L // 4, 128)
        pkg.qsa_quantize_keys(lay["pooled"], lay["pooled_fp8"])
    torch.cuda.synchronize()

    def step_fp8():
        for lay, bf in zip(layers, bufs):
            pipeline.decode_layer(pkg.SEL_A_FP8, pkg.ATTN_A, q_ctx, L, lay["q_idx"], lay["pooled_fp8"], lay["q"],
                                  lay["kv"], bf, q_seq=q_seq, fused=True)

    def lists_fp8():
        for lay, bf in zip(layers, bufs):
            pkg.qsa_index_lists(pkg.SEL_A_FP8, q_ctx, L, lay["q_idx"], lay["pooled_fp8"], bf.scores, bf.itk_ws,
                                q_seq=q_seq)

    ms_fp8, _, graph = time_graph(torch, step_fp8, steps, warmup)
    del graph
    for bf in bufs:
        pkg.check_decode_layer_error(bf.layer_ws)
    lists_fp8_ms = time_launches(torch, lists_fp8, reps) / len(layers)
    for lay in layers:
        del lay["pooled_fp8"]
    # the headline schedule: two micro-batches (sequences 0-1 and 2-3), each
    # through its 12 layers in order on a stream of its own
    micro = pipeline.micro_batches(pkg.SEL_A, pkg.ATTN_A, q_ctx, q_seq, L, len(layers), 2, n_split=bufs[0].n_split,
                                   keep_scores=False)
    side = [torch.cuda.Stream()]
    lay_args = [(lay["q_idx"], lay["pooled"], lay["q"], lay["kv"]) for lay in layers]

    def step_two_streams():
        pipeline.decode_step_streams(pkg.SEL_A, pkg.ATTN_A, L, lay_args, micro, side)

    ms_two, wall_two, graph = time_graph(torch, step_two_streams, steps, warmup)
    ms_two_med, ms_two_mean_each = replay_median(torch, graph, steps)
    del graph
    for mb in micro:
        for bf in mb.bufs:
            pkg.check_decode_layer_error(bf.layer_ws)
    step(True)  # the batch-4 step again (the FP8 leg above reused its buffers)
    torch.cuda.synchronize()
    for l, bf in enumerate(bufs):  # the same step as the batch-4 calls, bit for bit
        for name in ("sel", "o", "o_bf16", "lse"):
            got = torch.cat([getattr(mb.bufs[l], name) for mb in micro])
            if not torch.equal(got, getattr(bf, name)):
                raise RuntimeError(f"two-stream step: layer {l} {name} differs from the batch-4 step")
    del micro
    scan_launch_bytes = B * (bm.scan_bytes(L) + 128 * 2)
    scan_fp8_bytes = B * (bm.scan_bytes_fp8(L) + 128 * 2)
    return dict(ms=ms, ms_med=ms_med, ms_mean_each=ms_mean_each, ms_sep=ms_sep, ms_app=ms_app, ms_host=ms_host, ms_dev1=ms_dev1, wall=wall, step_bytes=step_bytes,
                unit_bytes=unit_bytes, pool_ms=pool_ms, n_split=bufs[0].n_split, lists_ms=lists_ms, scan_ms=scan_ms,
                scan_launch_bytes=scan_launch_bytes, lists_gbs=scan_launch_bytes / (lists_ms * 1e-3) / 1e9,
                ms_fp8=ms_fp8, step_bytes_fp8=bm.decode_unit_bytes_fp8(L) * B * len(layers),
                lists_fp8_ms=lists_fp8_ms, lists_fp8_gbs=scan_fp8_bytes / (lists_fp8_ms * 1e-3) / 1e9,
                ms_two=ms_two, ms_two_med=ms_two_med, ms_two_mean_each=ms_two_mean_each, wall_two=wall_two,
                rcache=rcache, layers=layers, bufs=bufs)


def run_small_decode(pkg, pipeline, bm, qi, torch, cfg, steps, warmup):
    """A batch-1 decode workload (8,192 tokens and 1 layer, or 131,072 tokens
    and 12 layers run in sequence): one qsa_decode_layer call per layer,
    the step captured in a graph. These steps take tens of microseconds, so
    they are replayed at least 500 times."""
    L, NL = cfg["ctx"], cfg["layers"]
    seed = qi.config_seed(cfg["config_id"])
    layers = []
    for l in range(NL):
        raw = torch.empty(1, L, 128, dtype=torch.bfloat16, device="cuda")
        k = torch.empty(1, L, 2, 256, dtype=torch.bfloat16, device="cuda")
        v = torch.empty(1, L, 2, 256, dtype=torch.bfloat16, device="cuda")
        q = torch.empty(1, 16, 256, dtype=torch.bfloat16, device="cuda")
        q_idx = torch.empty(1, 1, 128, dtype=torch.bfloat16, device="cuda")
        for t, kind in ((raw, "raw_key"), (k, "k"), (v, "v"), (q, "q"), (q_idx, "q_idx")):
            fill(t[0], seed, qi.stream_id(l, 0, kind))
        pooled = torch.empty(1, L // 4, 128, dtype=torch.bfloat16, device="cuda")
        pkg.qsa_pool_keys(raw, pooled, block=4)
        layers.append(dict(q=q, q_idx=q_idx, pooled=pooled, kv=pkg.make_kv(k, v), k=k, v=v))
    q_ctx = torch.full((1,), L, dtype=torch.int32, device="cuda")
    q_seq = torch.zeros(1, dtype=torch.int32, device="cuda")
    bufs = [pipeline.decode_buffers(pkg.SEL_A, pkg.ATTN_A, 1, L) for _ in layers]

    def step():
        for lay, bf in zip(layers, bufs):
            pipeline.decode_layer(pkg.SEL_A, pkg.ATTN_A, q_ctx, L, lay["q_idx"], lay["pooled"], lay["q"], lay["kv"],
                                  bf, q_seq=q_seq, fused=True)

    reps = max(500, steps)
    ms, _, graph = time_graph(torch, step, reps, max(20, warmup))
    med, _ = replay_median(torch, graph, reps)
    del graph
    for bf in bufs:
        pkg.check_decode_layer_error(bf.layer_ws)
    step_bytes = bm.decode_unit_bytes(L) * NL
    out = dict(workload=cfg["name"], ctx=L, batch=1, layers=NL, n_split=bufs[0].n_split, replays=reps,
               ms_per_step=round(ms, 5), ms_per_step_median=round(med, 5), steps_s=round(1e3 / ms, 1),
               step_bytes=step_bytes, hbm_gbs=round(step_bytes / (ms * 1e-3) / 1e9, 1),
               hbm_frac=round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
    log(f"{cfg['name']}: {ms * 1e3:.1f} us/step")
    return out


ROW_CACHE_SLOTS = 65536  # 128 MiB per layer: about 8 steps of batch-4 rows
PAGES_CACHE_SLOTS = 12144  # the per-layer slot count the pages' cache used
LARGE_CACHE_SLOTS = 262144  # 512 MiB per layer (6 GiB for 12 layers)


def run_row_cache(pkg, pipeline, qi, torch, lay0, kv_host, q_ctx, q_seq, L, B, n_split, warm=16, timed=32, reps=3):
    """The attention of one layer over K/V rows in pinned host memory, without
    and with the HBM row cache, over consecutive decode steps whose
    selections come from AR(1)-correlated indexer queries (plus the
    repeated-selection and random-selection extremes). Per step: the cache
    step (the row each sequence just stored is dropped), the plan and the
    cached attention; the partial-result merge is the same for both paths and
    left out of both. Then the whole layer over the same steps (scan and
    selection from each step's indexer query, attention, merge): the one-call
    layer over host-resident rows against the separate calls with the cache."""
    import numpy as np
    T = warm + timed
    seed = qi.config_seed(DECODE["config_id"])
    rho = correlated_rho("correlated_overlap_decode.txt")
    qb = np.stack([qi.ar1_normal_bf16(seed, qi.stream_id(0, s, "q_idx", salt=2), T, 128, rho) for s in range(B)])
    q_all = torch.from_numpy(qb.view(np.int16)).to("cuda").view(torch.bfloat16)
    scores = torch.empty(B, L // 4, dtype=torch.float32, device="cuda")
    ws = pkg.index_topk_workspace(pkg.SEL_A, B, L)
    sel_corr = torch.empty(T, B, 512, dtype=torch.int32, device="cuda")
    n_sel = torch.empty(T, B, dtype=torch.int32, device="cuda")
    for t in range(T):
        pkg.qsa_index_topk(pkg.SEL_A, q_ctx, L, q_all[:, t:t + 1].contiguous(), lay0["pooled"], scores, sel_corr[t],
                           n_sel[t], ws, q_seq=q_seq)
    torch.cuda.synchronize()
    sc = sel_corr.cpu().numpy()
    overlap = float(np.mean([np.intersect1d(sc[t, b], sc[t - 1, b]).size / 512
                             for t in range(1, T) for b in range(B)]))
    rng = np.random.default_rng(seed)
    rnd = np.stack([np.stack([np.sort(rng.choice(L // 4, 512, replace=False)) for _ in range(B)])
                    for _ in range(T)]).astype(np.int32)
    sel_rnd = torch.from_numpy(rnd).cuda()
    sel_same = sel_corr[:1].expand(T, B, 512).contiguous()
    o = torch.empty(n_split, B, 16, 256, device="cuda")
    lse = torch.empty(n_split, B, 16, device="cuda")
    plan = torch.empty(B, pkg.qsa_decode_cached_plan_bytes(pkg.SEL_A, B) // (4 * B), dtype=torch.int32, device="cuda")
    stored = (q_ctx - 1).contiguous()

    def one(sel_t, ns_t, cache, n_slots, kv=kv_host):
        if cache is None:
            pkg.qsa_sparse_decode(pkg.SEL_A, pkg.ATTN_A, q_ctx, L, lay0["q"], kv, sel_t, ns_t, n_split, o, lse,
                                  q_seq=q_seq)
        else:
            pkg.qsa_row_cache_step(pkg.ATTN_A, cache, n_slots, stored, kv_host, row_seq=q_seq)
            pkg.qsa_sparse_decode_cached(pkg.SEL_A, pkg.ATTN_A, q_ctx, L, lay0["q"], kv_host, sel_t, ns_t, n_split,
                                         o, lse, cache, n_slots, plan, q_seq=q_seq)

    def regime(sel, n_slots=None, kv=kv_host):
        cache = pkg.row_cache_empty(pkg.ATTN_A, n_slots) if n_slots else None

        def warm_part():
            if cache is not None:
                cache.zero_()
            for t in range(warm):
                one(sel[t], n_sel[t], cache, n_slots, kv)

        def timed_part():
            for t in range(warm, T):
                one(sel[t], n_sel[t], cache, n_slots, kv)

        warm_part()
        timed_part()
        torch.cuda.synchronize()
        ga, gb = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(ga):
            warm_part()
        with torch.cuda.graph(gb):
            timed_part()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        tot = 0.0
        for _ in range(reps):
            ga.replay()
            e0.record()
            gb.replay()
            e1.record()
            torch.cuda.synchronize()
            tot += e0.elapsed_time(e1)
        out = dict(ms=round(tot / reps / timed, 4))
        if cache is not None:  # the same steps again, eagerly, counting the hits of the timed ones
            hits = 0
            cache.zero_()
            for t in range(T):
                one(sel[t], n_sel[t], cache, n_slots)
                if t >= warm:
                    hits += int((plan[:, :2048] < 0).sum().item())
            out["hit_rate"] = round(hits / (timed * B * 2048), 4)
            out["host_link_mb_per_step"] = round((1 - out["hit_rate"]) * B * 2048 * 2048 / 1e6, 2)
        del ga, gb
        return out

    res = {
        "all_rows_from_host": regime(sel_corr),
        "cached_correlated": regime(sel_corr, ROW_CACHE_SLOTS),
        "cached_correlated_pages_size": regime(sel_corr, PAGES_CACHE_SLOTS),
        "cached_correlated_large": regime(sel_corr, LARGE_CACHE_SLOTS),
        "cached_same_selection": regime(sel_same, ROW_CACHE_SLOTS),
        "cached_random_selection": regime(sel_rnd, ROW_CACHE_SLOTS),
        "all_rows_from_host_random": regime(sel_rnd),
        "all_rows_in_hbm": regime(sel_corr, kv=lay0["kv"]),
    }
    # the whole layer per step, from the step's indexer query
    q_steps = [q_all[:, t:t + 1].contiguous() for t in range(T)]
    lbuf = pipeline.decode_buffers(pkg.SEL_A, pkg.ATTN_A, B, L, n_split=n_split)
    ws = pkg.index_topk_workspace(pkg.SEL_A, B, L)
    sel_l = torch.empty(B, 512, dtype=torch.int32, device="cuda")
    nsel_l = torch.empty(B, dtype=torch.int32, device="cuda")
    o_fin = torch.empty(B, 16, 256, device="cuda")
    ob_fin = torch.empty(B, 16, 256, dtype=torch.bfloat16, device="cuda")
    lse_fin = torch.empty(B, 16, device="cuda")

    def layer_steps(cache, n_slots, ts):
        for t in ts:
            if cache is None:
                pipeline.decode_layer(pkg.SEL_A, pkg.ATTN_A, q_ctx, L, q_steps[t], lay0["pooled"], lay0["q"],
                                      kv_host, lbuf, q_seq=q_seq, fused=True)
                continue
            pkg.qsa_index_topk(pkg.SEL_A, q_ctx, L, q_steps[t], lay0["pooled"], scores, sel_l, nsel_l, ws,
                               q_seq=q_seq)
            pkg.qsa_row_cache_step(pkg.ATTN_A, cache, n_slots, stored, kv_host, row_seq=q_seq)
            pkg.qsa_sparse_decode_cached(pkg.SEL_A, pkg.ATTN_A, q_ctx, L, lay0["q"], kv_host, sel_l, nsel_l,
                                         n_split, o, lse, cache, n_slots, plan, q_seq=q_seq)
            pkg.qsa_lse_merge(o, lse, o_out=o_fin, o_out_bf16=ob_fin, lse_out=lse_fin)

    def layer_regime(n_slots):
        cache = pkg.row_cache_empty(pkg.ATTN_A, n_slots) if n_slots else None

        def warm_part():
            if cache is not None:
                cache.zero_()
            layer_steps(cache, n_slots, range(warm))

        warm_part()
        layer_steps(cache, n_slots, range(warm, T))
        torch.cuda.synchronize()
        ga, gb = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(ga):
            warm_part()
        with torch.cuda.graph(gb):
            layer_steps(cache, n_slots, range(warm, T))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        tot = 0.0
        for _ in range(reps):
            ga.replay()
            e0.record()
            gb.replay()
            e1.record()
            torch.cuda.synchronize()
            tot += e0.elapsed_time(e1)
        del ga, gb
        return round(tot / reps / timed, 4)

    layer = {"one_call_layer_all_rows_from_host": layer_regime(None),
             "separate_calls_with_cache": layer_regime(ROW_CACHE_SLOTS),
             "separate_calls_with_large_cache": layer_regime(LARGE_CACHE_SLOTS)}
    # the cached layer's output equals that of the same calls without the
    # cache, bit for bit (last step)
    pkg.qsa_index_topk(pkg.SEL_A, q_ctx, L, q_steps[T - 1], lay0["pooled"], scores, sel_l, nsel_l, ws, q_seq=q_seq)
    pkg.qsa_sparse_decode(pkg.SEL_A, pkg.ATTN_A, q_ctx, L, lay0["q"], kv_host, sel_l, nsel_l, n_split, o, lse,
                          q_seq=q_seq)
    pkg.qsa_lse_merge(o, lse, o_out=o_fin, o_out_bf16=ob_fin, lse_out=lse_fin)
    torch.cuda.synchronize()
    ref_o = o_fin.clone()
    cache = pkg.row_cache_empty(pkg.ATTN_A, ROW_CACHE_SLOTS)
    layer_steps(cache, ROW_CACHE_SLOTS, range(T))
    torch.cuda.synchronize()
    if not torch.equal(o_fin, ref_o):
        raise RuntimeError("row cache: cached layer output differs from the one-call layer's")
    del cache
    # the cached attention's outputs are those of the uncached one, bit for bit
    cache = pkg.row_cache_empty(pkg.ATTN_A, PAGES_CACHE_SLOTS)
    for t in range(3):
        one(sel_corr[t], n_sel[t], None, None)
        ref = (o.clone(), lse.clone())
        one(sel_corr[t], n_sel[t], cache, PAGES_CACHE_SLOTS)
        torch.cuda.synchronize()
        if not (torch.equal(o, ref[0]) and torch.equal(lse, ref[1])):
            raise RuntimeError("row cache: cached attention differs from the uncached one")
    del cache
    log("row cache: " + ", ".join(f"{k} {v['ms']:.4f} ms" + (f" (hits {v['hit_rate']:.3f})" if "hit_rate" in v else "")
                                  for k, v in res.items()) + f"; selection overlap {overlap:.3f}; layer {layer}")
    return dict(overlap_prev_step=round(overlap, 4), n_slots=ROW_CACHE_SLOTS, layer_ms=layer,
                cache_mib_per_layer=round(pkg.qsa_row_cache_bytes(pkg.ATTN_A, ROW_CACHE_SLOTS) / 2**20, 1),
                pages_n_slots=PAGES_CACHE_SLOTS, n_split=n_split, regimes=res)


def run_prefill(pkg, pipeline, bm, qi, torch, steps, warmup):
    H, C = PREFILL["history"], PREFILL["chunk"]
    ctx_max = H + C
    seed = qi.config_seed(PREFILL["config_id"])
    dev = "cuda"
    raw = torch.empty(1, ctx_max, 128, dtype=torch.bfloat16, device=dev)
    k = torch.empty(1, ctx_max, 2, 256, dtype=torch.bfloat16, device=dev)
    v = torch.empty(1, ctx_max, 2, 256, dtype=torch.bfloat16, device=dev)
    q = torch.empty(C, 16, 256, dtype=torch.bfloat16, device=dev)
    q_idx = torch.empty(C, 1, 128, dtype=torch.bfloat16, device=dev)
    fill(raw, seed, qi.stream_id(0, 0, "raw_key"))
    fill(k, seed, qi.stream_id(0, 0, "k"))
    fill(v, seed, qi.stream_id(0, 0, "v"))
    fill(q, seed, qi.stream_id(0, 0, "q"))
    fill(q_idx, seed, qi.stream_id(0, 0, "q_idx"))
    pooled = torch.empty(1, ctx_max // 4, 128, dtype=torch.bfloat16, device=dev)
    pkg.qsa_pool_keys(raw, pooled, block=4)
    kv = pkg.make_kv(k, v)
    ctxs = list(range(H + 1, H + C + 1))
    q_ctx = torch.tensor(ctxs, dtype=torch.int32, device=dev)
    flops = bm.prefill_flops(ctxs)
    out = {}
    for tile in PREFILL["tiles"]:
        bufs = pipeline.prefill_buffers(pkg.SEL_A, pkg.ATTN_A, C, ctx_max, tile)

        def chunk():
            pipeline.prefill_chunk(pkg.SEL_A, pkg.ATTN_A, q_ctx, ctx_max, q_idx, pooled, q, kv, bufs)

        ms, wall, g = time_graph(torch, chunk, max(10, steps // 5), max(2, warmup))
        out[tile] = dict(ms=ms, tok_s=C / (ms * 1e-3), tflops=flops["total"] / (ms * 1e-3) / 1e12)
        if tile == PREFILL["tiles"][0]:
            r = max(10, steps // 10)
            t_sc = time_launches(torch, lambda: pkg.qsa_index_scores(pkg.SEL_A, q_ctx, ctx_max, q_idx, pooled,
                                                                     bufs.scores), r)
            t_tk = time_launches(torch, lambda: pkg.qsa_topk_blocks(pkg.SEL_A, q_ctx, ctx_max, bufs.scores, bufs.sel,
                                                                    bufs.n_sel, bufs.ws), r)

            def tiles_only():
                for t, (a0, a1) in enumerate(bufs.tiles):
                    pkg.qsa_sparse_prefill(pkg.SEL_A, pkg.ATTN_A, q_ctx, ctx_max, q, kv, bufs.sel, bufs.n_sel, a0, a1,
                                           bufs.o_tiles[t], bufs.lse_tiles[t])

            t_at = time_launches(torch, tiles_only, r)
            t_mg = time_launches(torch, lambda: pkg.qsa_lse_merge(bufs.o_tiles, bufs.lse_tiles, o_out=bufs.o,
                                                                  o_out_bf16=bufs.o_bf16, lse_out=bufs.lse), r)

            def tiles_running():
                last = len(bufs.tiles) - 1
                for t, (a0, a1) in enumerate(bufs.tiles):
                    pkg.qsa_sparse_prefill_merge(pkg.SEL_A, pkg.ATTN_A, q_ctx, ctx_max, q, kv, bufs.sel, bufs.n_sel,
                                                 a0, a1, t == 0, t == last, bufs.o, bufs.lse, o_out_bf16=bufs.o_bf16)

            t_rm = time_launches(torch, tiles_running, r)
            out["breakdown_us"] = {"scores": round(t_sc * 1e3, 1), "topk": round(t_tk * 1e3, 1),
                                   "attend_all_tiles": round(t_at * 1e3, 1), "merge": round(t_mg * 1e3, 1),
                                   "attend_all_tiles_running_merge": round(t_rm * 1e3, 1)}
            out["attend_tflops"] = round(flops["attention"] / (t_at * 1e-3) / 1e12, 1)
        del g, bufs
        log(f"prefill tile {tile}: {ms:.3f} ms/chunk")
    # the same chunk with correlated indexer queries: AR(1) over positions,
    # neighbouring top-512 selections overlapping about 0.72 as the pages
    # measured (the correlation comes from tests/golden/correlated_overlap.txt)
    import numpy as np
    rho = correlated_rho()
    qc_np = qi.ar1_normal_bf16(seed, qi.stream_id(0, 0, "q_idx", salt=1), C, 128, rho)
    q_idx_c = torch.from_numpy(qc_np.view(np.int16)).view(torch.bfloat16).reshape(C, 1, 128).to(dev)
    tile = PREFILL["tiles"][0]
    bufs = pipeline.prefill_buffers(pkg.SEL_A, pkg.ATTN_A, C, ctx_max, tile)

    def chunk_c():
        pipeline.prefill_chunk(pkg.SEL_A, pkg.ATTN_A, q_ctx, ctx_max, q_idx_c, pooled, q, kv, bufs)

    ms_c, _, g = time_graph(torch, chunk_c, max(10, steps // 5), max(2, warmup))
    del g

    def tiles_c():
        for t, (a0, a1) in enumerate(bufs.tiles):
            pkg.qsa_sparse_prefill(pkg.SEL_A, pkg.ATTN_A, q_ctx, ctx_max, q, kv, bufs.sel, bufs.n_sel, a0, a1,
                                   bufs.o_tiles[t], bufs.lse_tiles[t])

    t_at_c = time_launches(torch, tiles_c, max(10, steps // 10))
    sel = bufs.sel.cpu().numpy()
    ov = [np.intersect1d(sel[i], sel[i - 1]).size / 512 for i in range(1, C)]
    out["correlated"] = dict(workload=f"the same chunk with AR(1) indexer queries over positions (rho {rho})",
                             ms_per_chunk=round(ms_c, 4), tok_s=round(C / (ms_c * 1e-3), 1),
                             tflops=round(flops["total"] / (ms_c * 1e-3) / 1e12, 2),
                             attend_all_tiles_us=round(t_at_c * 1e3, 1),
                             attend_tflops=round(flops["attention"] / (t_at_c * 1e-3) / 1e12, 1),
                             mean_selection_overlap=round(float(np.mean(ov)), 4))
    log(f"prefill correlated: {ms_c:.3f} ms/chunk, overlap {np.mean(ov):.3f}")
    del bufs
    return out, flops


def correlated_rho(name: str = "correlated_overlap.txt") -> float:
    """The AR(1) correlation of a correlated-selection workload (prefill:
    correlated_overlap.txt; the 1M-token decode: correlated_overlap_decode.txt)."""
    path = os.path.join(ROOT, "tests", "golden", name)
    with open(path) as f:
        for line in f:
            if line.startswith("rho "):
                return float(line.split()[1])
    raise RuntimeError(f"no rho in {path}")


def run_mla(pkg, pipeline, bm, qi, torch, steps, warmup):
    """Config 5: batch-8 decode at context 131,072 (indexer scores over every
    earlier token, top-2048, attention, merge) and a prefill chunk of 2048
    queries at positions 129,024..131,071 of one sequence."""
    import numpy as np
    L, B, C = MLA["ctx"], MLA["batch"], MLA["chunk"]
    seed = qi.config_seed(MLA["config_id"])
    dev = "cuda"
    bf16 = dict(dtype=torch.bfloat16, device=dev)
    out = {}
    lat = torch.empty(B, L, 1, 576, **bf16)
    keys = torch.empty(B, L, 64, **bf16)
    q = torch.empty(B, 64, 576, **bf16)
    q_idx = torch.empty(B, 4, 64, **bf16)
    for s in range(B):
        for t, kind in ((lat, "latent"), (keys, "raw_key"), (q, "q"), (q_idx, "q_idx")):
            fill(t[s], seed, qi.stream_id(0, s, kind))
    w = torch.tensor(np.stack([qi.uniform_f32(seed, qi.stream_id(0, s, "w_idx"), 4) for s in range(B)]), device=dev)
    kv = pkg.make_kv(lat, lat)
    q_ctx = torch.full((B,), L, dtype=torch.int32, device=dev)
    q_seq = torch.arange(B, dtype=torch.int32, device=dev)
    bufs = pipeline.decode_buffers(pkg.SEL_B, pkg.ATTN_B, B, L)

    def dstep_sep():
        pipeline.decode_layer(pkg.SEL_B, pkg.ATTN_B, q_ctx, L, q_idx, keys, q, kv, bufs, q_seq=q_seq, w_idx=w)

    ms_sep, _, g = time_graph(torch, dstep_sep, max(10, steps // 2), warmup)
    del g
    ref = [x.clone() for x in (bufs.sel, bufs.n_sel, bufs.o, bufs.o_bf16, bufs.lse)]
    for x in (bufs.sel, bufs.o, bufs.o_bf16, bufs.lse):
        x.zero_()

    # the step as one qsa_decode_layer_latent call (the headline when its
    # results are the separate calls' bit for bit)
    def dstep():
        pipeline.decode_layer(pkg.SEL_B, pkg.ATTN_B, q_ctx, L, q_idx, keys, q, kv, bufs, q_seq=q_seq, w_idx=w,
                              fused=True)

    ms, _, g = time_graph(torch, dstep, max(10, steps // 2), warmup)
    del g
    same = all(bool(torch.equal(a, b)) for a, b in zip(ref, (bufs.sel, bufs.n_sel, bufs.o, bufs.o_bf16, bufs.lse)))
    if not same:
        raise RuntimeError("shared-latent decode: the one-call layer's results differ from the separate calls'")
    reps = max(10, steps // 5)
    t_sc = time_launches(torch, lambda: pkg.qsa_index_scores(pkg.SEL_B, q_ctx, L, q_idx, keys, bufs.scores,
                                                             q_seq=q_seq, w_idx=w), reps)
    t_tk = time_launches(torch, lambda: pkg.qsa_topk_blocks(pkg.SEL_B, q_ctx, L, bufs.scores, bufs.sel, bufs.n_sel,
                                                            bufs.ws), reps)
    t_at = time_launches(torch, lambda: pkg.qsa_sparse_decode(pkg.SEL_B, pkg.ATTN_B, q_ctx, L, q, kv, bufs.sel,
                                                              bufs.n_sel, bufs.n_split, bufs.o_part, bufs.lse_part,
                                                              q_seq=q_seq), reps)
    step_bytes = B * bm.mla_decode_unit_bytes(L)
    out["decode"] = dict(workload=f"decode batch {B}, context {L}, one layer", steps_s=round(1e3 / ms, 1),
                         ms_per_step=round(ms, 5), hbm_gbs=round(step_bytes / (ms * 1e-3) / 1e9, 1),
                         step_bytes=step_bytes, n_split=bufs.n_split, schedule="one qsa_decode_layer_latent call",
                         separate_calls=dict(ms_per_step=round(ms_sep, 5), steps_s=round(1e3 / ms_sep, 1),
                                             hbm_gbs=round(step_bytes / (ms_sep * 1e-3) / 1e9, 1),
                                             breakdown_us={"scores": round(t_sc * 1e3, 2),
                                                           "topk": round(t_tk * 1e3, 2),
                                                           "attend": round(t_at * 1e3, 2)}))
    log(f"mla decode: {ms:.4f} ms/step one call, {ms_sep:.4f} separate calls")
    # the same step over FP8 sparse-MLA rows (656 bytes per token)
    rows8 = torch.empty(B, L, 656, dtype=torch.uint8, device=dev)
    pkg.qsa_quantize_latent(lat, rows8)
    kv8 = pkg.make_kv(rows8)

    def dstep8():
        pipeline.decode_layer(pkg.SEL_B, pkg.ATTN_B, q_ctx, L, q_idx, keys, q, kv8, bufs, q_seq=q_seq, w_idx=w)

    ms8, _, g = time_graph(torch, dstep8, max(10, steps // 2), warmup)
    del g
    t_at8 = time_launches(torch, lambda: pkg.qsa_sparse_decode(pkg.SEL_B, pkg.ATTN_B, q_ctx, L, q, kv8, bufs.sel,
                                                               bufs.n_sel, bufs.n_split, bufs.o_part, bufs.lse_part,
                                                               q_seq=q_seq), reps)
    step_bytes8 = B * bm.mla_decode_unit_bytes_fp8_rows(L)
    out["decode"]["fp8_rows"] = dict(ms_per_step=round(ms8, 5), steps_s=round(1e3 / ms8, 1), step_bytes=step_bytes8,
                                     hbm_gbs=round(step_bytes8 / (ms8 * 1e-3) / 1e9, 1),
                                     attend_us=round(t_at8 * 1e3, 2))
    # and with FP8 token keys too (68 + 656 bytes of cache per token)
    keys8 = pkg.fp8_keys_empty(B, L, 64)
    pkg.qsa_quantize_keys(keys, keys8)
    bufs8 = pipeline.decode_buffers(pkg.SEL_B_FP8, pkg.ATTN_B, B, L)

    def dstep88():
        pipeline.decode_layer(pkg.SEL_B_FP8, pkg.ATTN_B, q_ctx, L, q_idx, keys8, q, kv8, bufs8, q_seq=q_seq, w_idx=w)

    ms88, _, g = time_graph(torch, dstep88, max(10, steps // 2), warmup)
    del g
    t_sc8 = time_launches(torch, lambda: pkg.qsa_index_scores(pkg.SEL_B_FP8, q_ctx, L, q_idx, keys8, bufs8.scores,
                                                              q_seq=q_seq, w_idx=w), reps)
    step_bytes88 = B * bm.mla_decode_unit_bytes_fp8(L)
    out["decode"]["fp8_keys_and_rows"] = dict(ms_per_step=round(ms88, 5), steps_s=round(1e3 / ms88, 1),
                                              step_bytes=step_bytes88,
                                              hbm_gbs=round(step_bytes88 / (ms88 * 1e-3) / 1e9, 1),
                                              scores_us=round(t_sc8 * 1e3, 2))
    del lat, keys, q, q_idx, kv, bufs, rows8, kv8, keys8, bufs8
    torch.cuda.empty_cache()
    # prefill chunk: queries at positions L - C .. L - 1 of one sequence
    lat = torch.empty(1, L, 1, 576, **bf16)
    keys = torch.empty(1, L, 64, **bf16)
    q = torch.empty(C, 64, 576, **bf16)
    q_idx = torch.empty(C, 4, 64, **bf16)
    for t, kind in ((lat, "latent"), (keys, "raw_key"), (q, "q"), (q_idx, "q_idx")):
        fill(t, seed, qi.stream_id(1, 0, kind))
    w = torch.tensor(qi.uniform_f32(seed, qi.stream_id(1, 0, "w_idx"), C * 4).reshape(C, 4), device=dev)
    kv = pkg.make_kv(lat, lat)
    ctxs = list(range(L - C + 1, L + 1))
    q_ctx = torch.tensor(ctxs, dtype=torch.int32, device=dev)
    flops = bm.mla_prefill_flops(ctxs)
    pre = {}
    for tile in MLA["tiles"]:
        pb = pipeline.prefill_buffers(pkg.SEL_B, pkg.ATTN_B, C, L, tile)

        def chunk():
            pipeline.prefill_chunk(pkg.SEL_B, pkg.ATTN_B, q_ctx, L, q_idx, keys, q, kv, pb, w_idx=w)

        ms_p, _, g = time_graph(torch, chunk, max(10, steps // 10), max(2, warmup // 2))
        del g
        pre[tile] = dict(ms=ms_p, tok_s=C / (ms_p * 1e-3), tflops=flops["total"] / (ms_p * 1e-3) / 1e12)
        if tile == MLA["tiles"][0]:
            r = max(10, steps // 20)
            t_sc = time_launches(torch, lambda: pkg.qsa_index_scores(pkg.SEL_B, q_ctx, L, q_idx, keys, pb.scores,
                                                                     w_idx=w), r)
            t_tk = time_launches(torch, lambda: pkg.qsa_topk_blocks(pkg.SEL_B, q_ctx, L, pb.scores, pb.sel, pb.n_sel,
                                                                    pb.ws), r)
            t_sel = time_launches(torch, lambda: pkg.qsa_index_topk_prefill(pkg.SEL_B, q_ctx, L, q_idx, w, keys,
                                                                            pb.scores, pb.sel, pb.n_sel, pb.sel_ws), r)
            a0, a1 = pb.tiles[0]
            t_at = time_launches(torch, lambda: pkg.qsa_sparse_prefill(pkg.SEL_B, pkg.ATTN_B, q_ctx, L, q, kv, pb.sel,
                                                                       pb.n_sel, a0, a1, pb.o_tiles[0],
                                                                       pb.lse_tiles[0]), r)
            att_tflops = flops["attention"] / (t_at * 1e-3) / 1e12
            pre["breakdown_us"] = {"select": round(t_sel * 1e3, 1), "attend": round(t_at * 1e3, 1),
                                   "separate_calls": {"scores": round(t_sc * 1e3, 1), "topk": round(t_tk * 1e3, 1)}}
            pre["attend_tflops"] = round(att_tflops, 1)
        if tile == MLA["tiles"][0]:  # the same chunk over FP8 sparse-MLA rows
            rows8 = torch.empty(1, L, 656, dtype=torch.uint8, device=dev)
            pkg.qsa_quantize_latent(lat, rows8)
            kv8 = pkg.make_kv(rows8)

            def chunk8():
                pipeline.prefill_chunk(pkg.SEL_B, pkg.ATTN_B, q_ctx, L, q_idx, keys, q, kv8, pb, w_idx=w)

            ms8, _, g = time_graph(torch, chunk8, max(10, steps // 10), max(2, warmup // 2))
            del g
            a0, a1 = pb.tiles[0]
            t_at8 = time_launches(torch, lambda: pkg.qsa_sparse_prefill(pkg.SEL_B, pkg.ATTN_B, q_ctx, L, q, kv8, pb.sel,
                                                                        pb.n_sel, a0, a1, pb.o_tiles[0],
                                                                        pb.lse_tiles[0]), r)
            pre["fp8_rows"] = dict(ms_per_chunk=round(ms8, 4), tok_s=round(C / (ms8 * 1e-3), 1),
                                   tflops=round(flops["total"] / (ms8 * 1e-3) / 1e12, 2),
                                   attend_us=round(t_at8 * 1e3, 1),
                                   attend_tflops=round(flops["attention"] / (t_at8 * 1e-3) / 1e12, 1))
            del rows8, kv8
        del pb
        torch.cuda.empty_cache()
        log(f"mla prefill tile {tile}: {ms_p:.3f} ms/chunk")
    t0 = MLA["tiles"][0]
    out["prefill"] = dict(workload=f"prefill {C} queries at context {L - C + 1}..{L}, one sequence",
                          tok_s=round(pre[t0]["tok_s"], 1), ms_per_chunk=round(pre[t0]["ms"], 4),
                          tflops=round(pre[t0]["tflops"], 2), mfma_frac=round(pre[t0]["tflops"] / BF16_PEAK_TFLOPS, 4),
                          useful_gflop=round(flops["total"] / 1e9, 1), history_tile=t0,
                          attend_tflops=pre["attend_tflops"],
                          attend_mfma_frac=round(pre["attend_tflops"] / BF16_PEAK_TFLOPS, 4),
                          attend_counters=counter_mfma("attend_b_t"),
                          select_gemm_counters=counter_mfma("scores_gemm_b<false, true>"),
                          breakdown_us=pre["breakdown_us"], fp8_rows=pre["fp8_rows"],
                          **{f"tile_{t}": {"tok_s": round(pre[t]["tok_s"], 1), "ms_per_chunk": round(pre[t]["ms"], 4)}
                             for t in MLA["tiles"][1:]})
    return out


COUNTERS = os.path.join(ROOT, "profiles", "hbm_counters_decode_1M_b4_prefill_tile_mla.txt")


def counter_traffic(kernel: str, groups: str):
    """HBM bytes per launch (read + written) of `kernel` with `groups`
    work-groups from the committed rocprofv3 counter summary, or None if the
    kernel sources changed since those counters were taken (or none exist)."""
    from indexer_selected_sparse_pooled_amd.profile_kernels import source_digest
    if not os.path.exists(COUNTERS):
        return None
    lines = open(COUNTERS).read().splitlines()
    digest = [l.split(":", 1)[1].strip() for l in lines if l.startswith("source digest:")]
    if not digest or digest[0] != source_digest():
        return None
    for l in lines:  # the kernel name fills the first 40 columns (it may contain spaces)
        f = l[40:].split()
        if len(f) == 6 and l[:40].strip() == kernel and f[0] == groups:
            return int(f[4]) + int(f[5])
    return None


MFMA_COUNTERS = os.path.join(ROOT, "profiles", "mfma_lds_counters_prefill_4096q_tile_mla_2048q_131k.txt")


def counter_mfma(kernel: str):
    """Counter-measured MFMA busy % (AMD's MfmaUtil) and executed / useful
    MFMA work of `kernel` from the committed rocprofv3 summary, or None if
    the kernel sources changed since (or no summary exists)."""
    from indexer_selected_sparse_pooled_amd.profile_kernels import source_digest
    if not os.path.exists(MFMA_COUNTERS):
        return None
    text = open(MFMA_COUNTERS).read()
    digest = re.findall(r"^source digest: (\S+)", text, re.M)
    if not digest or digest[0] != source_digest():
        return None
    m = re.search(r"^" + re.escape(kernel) + r" \[.*?\n(.*?)(?=^\S|\Z)", text, re.M | re.S)
    if not m:
        return None
    busy = re.search(r"MFMA busy ([0-9.]+) %", m.group(1))
    ratio = re.search(r"executed / useful = ([0-9.]+)", m.group(1))
    out = {}
    if busy:
        out["mfma_busy_pct"] = float(busy.group(1))
    if ratio:
        out["executed_over_useful"] = float(ratio.group(1))
    return out or None


# ---------------------------------------------------------------- oracle --
# The CPU oracle (oracle/qsa_oracle.py, float64 numpy, as it stands) timed on
# the host cores: units of each workload (one query in one layer, which is
# how the oracle computes) run in a pool of single-threaded worker processes,
# one per core, each for a fixed time after building its inputs; throughput
# is units per second of wall time over the pool, scaled to the metric's unit.

ORACLE_UNITS = {
    1: ("steps/s", 1, "one decode step: scan of 2,048 pooled keys, top-512, attention over 2,048 tokens"),
    2: ("steps/s", 12, "one of the 12 layers of a step: scan of 32,768 pooled keys, top-512, attention over "
                       "2,048 tokens"),
    3: ("steps/s", 48, "one (layer, sequence) unit of the step: scan of 262,080 pooled keys, top-512, attention "
                       "over 2,048 tokens"),
    4: ("tok/s", 1, "one query of the chunk: scores of its 15,000..16,023 blocks, top-512, attention tile by tile "
                    "(8,192-token tiles) and the log-sum-exp merge"),
    "5a": ("tok/s", 1, "one query of the chunk: ReLU-weighted scores of its 129,025..131,072 tokens, top-2048, "
                       "attention of 64 heads over 2,048 latent rows"),
    "5b": ("steps/s", 8, "one query of the batch-8 step: scores of 131,072 tokens, top-2048, attention of 64 heads "
                         "over 2,048 latent rows"),
}


def _gen_rows(qi, seed, stream, toks, width):
    """Rows `toks` of a [tokens][width] bf16 tensor filled by the generator."""
    import numpy as np
    idx = (np.asarray(toks, dtype=np.int64)[:, None] * width + np.arange(width)[None, :]).reshape(-1)
    return qi.normal_bf16(seed, stream, 0, index=idx.astype(np.uint64)).reshape(len(toks), width)


def _one_thread():
    """Limit this worker's numeric libraries to one thread (numpy and the
    oracle are imported first, so their thread pools exist to be limited)."""
    import numpy  # noqa: F401

    from oracle import qsa_oracle  # noqa: F401
    from threadpoolctl import threadpool_limits
    return threadpool_limits(limits=1)


def _pool_slice(task):
    """Pool blocks [b0, b1) of the 1M-token decode workload's layer 0,
    sequence 0 into the shared pooled-key array (input preparation)."""
    shm_name, nb, b0, b1 = task
    from multiprocessing import shared_memory

    import numpy as np

    import qsa_inputs as qi
    from oracle import qsa_oracle as orc
    keep = _one_thread()
    seed = qi.config_seed(DECODE["config_id"])
    raw = qi.normal_bf16(seed, qi.stream_id(0, 0, "raw_key"), 4 * b0 * 128, 4 * (b1 - b0) * 128)
    shm = shared_memory.SharedMemory(name=shm_name)
    pooled = np.ndarray((nb, 128), dtype=np.uint16, buffer=shm.buf)
    pooled[b0:b1] = orc.pool_keys(raw.reshape(-1, 128), 4)
    del pooled, keep
    shm.close()
    return b1 - b0


def _oracle_worker(task):
    """One worker's share of an oracle measurement: build the inputs of its
    units (not timed), then run units for `budget` seconds on one thread.
    Returns (units, seconds, setup_seconds)."""
    cfg, worker, n_workers, budget, shm_name = task
    keep = _one_thread()
    import numpy as np

    import qsa_inputs as qi
    from oracle import qsa_oracle as orc
    t_setup = time.perf_counter()
    units = []  # callables, run round-robin
    max_units = 8  # distinct units a worker prepares (queries spread over the chunk)
    shm = None

    def gen(seed, stream, n):
        return qi.normal_bf16(seed, stream, 0, n)

    if cfg in (1, 2, 3):
        L = {1: 8192, 2: 131072, 3: DECODE["ctx"]}[cfg]
        seed = qi.config_seed(cfg)
        layer, seq = {1: (0, 0), 2: (worker % 12, 0), 3: (0, 0)}[cfg]
        S = lambda kind: qi.stream_id(layer, seq, kind)
        if cfg == 3:  # pooled in parallel beforehand (_pool_slice), shared by the workers
            from multiprocessing import shared_memory
            shm = shared_memory.SharedMemory(name=shm_name)
            pooled = np.ndarray((L // 4, 128), dtype=np.uint16, buffer=shm.buf)
        else:
            pooled = orc.pool_keys(gen(seed, S("raw_key"), L * 128).reshape(L, 128), 4)
        q_idx = gen(seed, S("q_idx"), 128)
        q = gen(seed, S("q"), 16 * 256).reshape(16, 256)
        # the selection does not change between repetitions: the K/V rows it
        # reads are generated once, by index
        toks0 = orc.selected_tokens(orc.select_blocks(orc.index_scores(q_idx, pooled, L // 4), L, 4, 512), L, 4)
        kr = _gen_rows(qi, seed, S("k"), toks0, 512).reshape(-1, 2, 256)
        vr = _gen_rows(qi, seed, S("v"), toks0, 512).reshape(-1, 2, 256)
        row_of = {int(t): r for r, t in enumerate(toks0)}

        def unit():
            sc = orc.index_scores(q_idx, pooled, L // 4)
            toks = orc.selected_tokens(orc.select_blocks(sc, L, 4, 512), L, 4)
            orc.attend(q, kr, vr, np.array([row_of[int(t)] for t in toks]), 1.0 / 16)

        units.append(unit)
    elif cfg == 4:
        H, C = PREFILL["history"], PREFILL["chunk"]
        n = H + C
        seed = qi.config_seed(4)
        S = lambda kind: qi.stream_id(0, 0, kind)
        pooled = orc.pool_keys(gen(seed, S("raw_key"), n * 128).reshape(n, 128), 4)
        k = gen(seed, S("k"), n * 512).reshape(n, 2, 256)
        v = gen(seed, S("v"), n * 512).reshape(n, 2, 256)
        for i in list(range(worker, C, n_workers))[::max(1, C // n_workers // max_units)][:max_units]:
            ctx = H + i + 1
            q_idx = qi.normal_bf16(seed, S("q_idx"), i * 128, 128)
            q = qi.normal_bf16(seed, S("q"), i * 4096, 4096).reshape(16, 256)

            def unit(ctx=ctx, q_idx=q_idx, q=q):
                sc = orc.index_scores(q_idx, pooled, ctx // 4)
                toks = orc.selected_tokens(orc.select_blocks(sc, ctx, 4, 512), ctx, 4)
                orc.prefill_query_tiled(q, k, v, toks, n, PREFILL["tiles"][0], 1.0 / 16)

            units.append(unit)
    else:
        L, C = MLA["ctx"], MLA["chunk"]
        seed = qi.config_seed(5)
        prefill = cfg == "5a"
        layer, seq = (1, 0) if prefill else (0, worker % MLA["batch"])
        S = lambda kind: qi.stream_id(layer, seq, kind)
        keys = gen(seed, S("raw_key"), L * 64).reshape(L, 64)
        qs = list(range(worker, C, n_workers))[::max(1, C // n_workers // max_units)][:max_units] if prefill else [0]
        w_all = qi.uniform_f32(seed, S("w_idx"), (C if prefill else 1) * 4).reshape(-1, 4)
        for i in qs:
            ctx = L - C + i + 1 if prefill else L
            q_idx = qi.normal_bf16(seed, S("q_idx"), i * 256, 256).reshape(4, 64)
            q = qi.normal_bf16(seed, S("q"), i * 64 * 576, 64 * 576).reshape(64, 576)
            w = w_all[i]
            toks0 = orc.selected_tokens(orc.select_blocks(orc.index_scores_relu(q_idx, w, keys, ctx), ctx, 1, 2048),
                                        ctx, 1)
            lat = _gen_rows(qi, seed, S("latent"), toks0, 576)[:, None, :]
            row_of = {int(t): r for r, t in enumerate(toks0)}

            def unit(ctx=ctx, q_idx=q_idx, q=q, w=w, lat=lat, row_of=row_of):
                sc = orc.index_scores_relu(q_idx, w, keys, ctx)
                toks = orc.selected_tokens(orc.select_blocks(sc, ctx, 1, 2048), ctx, 1)
                orc.attend(q, lat, lat, np.array([row_of[int(t)] for t in toks]), 1.0 / 24, dv=512)

            units.append(unit)
    setup = time.perf_counter() - t_setup
    done = 0
    t0 = time.perf_counter()
    while done < 1 or time.perf_counter() - t0 < budget:
        units[done % len(units)]()
        done += 1
    dt = time.perf_counter() - t0
    if shm is not None:
        del pooled, units
        shm.close()
    del keep
    return done, dt, setup


def cpu_baselines(budget=4.0, budget_headline=10.0):
    """The oracle on every workload, timed over the host cores (see above).
    Returns {config: dict(value, unit, cores, ...)}; config 3 is the
    headline's baseline."""
    import multiprocessing as mp
    from multiprocessing import shared_memory
    n_workers = max(1, min(16, os.cpu_count() or 1))
    ctx = mp.get_context("spawn")  # fresh interpreters: the workers never touch the GPU
    out = {}
    nb = DECODE["ctx"] // 4
    shm = shared_memory.SharedMemory(create=True, size=nb * 128 * 2)
    try:
        with ctx.Pool(n_workers) as pool:
            t0 = time.perf_counter()
            cuts = [nb * w // n_workers // 4 * 4 for w in range(n_workers)] + [nb]
            pool.map(_pool_slice, [(shm.name, nb, cuts[w], cuts[w + 1]) for w in range(n_workers)])
            log(f"oracle inputs: 262,080 pooled keys in {time.perf_counter() - t0:.1f} s")
            for cfg, (unit, per_metric, what) in ORACLE_UNITS.items():
                b = budget_headline if cfg == 3 else budget
                t0 = time.perf_counter()
                res = pool.map(_oracle_worker, [(cfg, w, n_workers, b, shm.name) for w in range(n_workers)])
                wall = time.perf_counter() - t0
                out[cfg] = _oracle_summary(res, n_workers, unit, per_metric, what, wall)
                log(f"oracle config {cfg}: {out[cfg]['value']:.4g} {unit} on {n_workers} cores "
                    f"({wall:.1f} s)")
    finally:
        shm.close()
        shm.unlink()
    return out


def _oracle_summary(res, n_workers, unit, per_metric, what, wall):
    """Pool throughput (units per second of the longest worker's timed
    span) and the one-core figure (units per second of summed worker time),
    both scaled to the metric's unit."""
    units = sum(r[0] for r in res)
    secs = max(r[1] for r in res)
    setup = max(r[2] for r in res)
    per_unit = sum(r[1] for r in res) / units  # seconds of one core per unit
    value = units / secs / per_metric
    return dict(value=round(value, 6), unit=unit, cores=n_workers, kind="oracle",
                sample=(f"{what}; {units} units over {n_workers} single-threaded worker processes, "
                        f"{secs:.1f} s each after {setup:.1f} s of input generation (not timed); "
                        f"{per_unit * 1e3:.1f} ms of one core per unit; one {unit.split('/')[0][:-1]} is "
                        f"{per_metric} unit(s)"),
                value_1core=round(1.0 / per_unit / per_metric, 6), wall_s=round(wall, 1))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}). "
              "The decode step would shard by sequence and layer, one GPU per shard; run with --gpus 1.",
              file=sys.stderr)
        return 2

    import torch

    import indexer_selected_sparse_pooled_amd as pkg
    import qsa_inputs as qi
    from indexer_selected_sparse_pooled_amd import bytemodel as bm
    from indexer_selected_sparse_pooled_amd import pipeline

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    pkg.qsa.lib()  # fails loudly if libqsa.so is missing
    torch.cuda.set_device(0)

    t_all = time.time()
    dec = run_decode(pkg, pipeline, bm, qi, torch, args.steps, args.warmup)
    log(f"decode: {dec['ms']:.4f} ms/step (separate calls {dec['ms_sep']:.4f}), "
        f"scan {dec['lists_ms'] * 1e3:.1f} us/launch")
    del dec["layers"], dec["bufs"]
    torch.cuda.empty_cache()
    small = [run_small_decode(pkg, pipeline, bm, qi, torch, c, args.steps, args.warmup) for c in SMALL_DECODES]
    torch.cuda.empty_cache()
    pre, pflops = run_prefill(pkg, pipeline, bm, qi, torch, args.steps, args.warmup)
    torch.cuda.empty_cache()
    mla = run_mla(pkg, pipeline, bm, qi, torch, args.steps, args.warmup)
    torch.cuda.empty_cache()

    cpu_all = cpu_baselines()
    cpu = cpu_all[3]
    cpu_model = None
    try:
        for line_ in open("/proc/cpuinfo"):
            if line_.startswith("model name"):
                cpu_model = line_.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass

    steps_s = 1e3 / dec["ms_two"]
    hbm_gbs = dec["step_bytes"] / (dec["ms_two"] * 1e-3) / 1e9
    t8 = pre[8192]
    line = {
        "metric": METRIC,
        "value": round(steps_s, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_two"], 5),
        "ms_per_step_replays": {"median": round(dec["ms_two_med"], 5), "mean": round(dec["ms_two_mean_each"], 5),
                                "how": "the same graph replayed `steps` times, each between its own pair of events"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded SplitMix64 inverse-CDF N(0,1) bf16, device-resident",
        "config": {"workload": DECODE["name"], "ctx": DECODE["ctx"], "batch": DECODE["batch"],
                   "layers": DECODE["layers"], "n_split": dec["n_split"], "graph": True,
                   "schedule": "two micro-batches (sequences 0-1, 2-3), each through its 12 layers in order "
                               "(one qsa_decode_layer call per layer, no score buffer) on its own stream; outputs "
                               "bit-identical to the batch-4 calls"},
        "hbm_gbs": round(hbm_gbs, 1),
        "hbm_frac": round(hbm_gbs / HBM_PEAK_GBS, 4),
        "step_bytes": dec["step_bytes"],
        "separate_calls_ms_per_step": round(dec["ms_sep"], 5),
        "with_kv_append_ms_per_step": round(dec["ms_app"], 5),
        "one_stream": {"workload": "the same step on one stream: one qsa_decode_layer call per layer over all 4 "
                                   "sequences",
                       "ms_per_step": round(dec["ms"], 5), "steps_s": round(1e3 / dec["ms"], 1),
                       "ms_per_step_replays_median": round(dec["ms_med"], 5),
                       "hbm_gbs": round(dec["step_bytes"] / (dec["ms"] * 1e-3) / 1e9, 1),
                       "hbm_frac": round(dec["step_bytes"] / (dec["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "fp8_keys": {"workload": "the same step with FP8 pooled keys (128 E4M3 codes + an fp32 scale = 132 B per "
                                 "block); K/V rows bf16",
                     "ms_per_step": round(dec["ms_fp8"], 5), "steps_s": round(1e3 / dec["ms_fp8"], 1),
                     "step_bytes": dec["step_bytes_fp8"],
                     "hbm_gbs": round(dec["step_bytes_fp8"] / (dec["ms_fp8"] * 1e-3) / 1e9, 1),
                     "scan_us_per_launch": round(dec["lists_fp8_ms"] * 1e3, 2),
                     "scan_gbs": round(dec["lists_fp8_gbs"], 1)},
        "host_resident_kv": {"workload": "one layer of the step (batch 4, 1,048,320 tokens) with K/V rows in pinned "
                                         "host memory read zero-copy; pooled keys in device memory",
                             "ms_per_layer": round(dec["ms_host"], 4),
                             "ms_per_layer_device_kv": round(dec["ms_dev1"], 4),
                             "kv_bytes_per_layer": 4 * 2048 * 2 * 2 * 256 * 2,
                             "kv_gbs": round(4 * 2048 * 2 * 2 * 256 * 2 / (dec["ms_host"] * 1e-3) / 1e9, 1),
                             "row_cache": dict(workload="the layer's attention over those host-resident K/V rows "
                                                        "over 32 consecutive decode steps (after 16 warm-up steps) "
                                                        "whose selections come from AR(1)-correlated indexer queries"
                                                        " (rho from tests/golden/correlated_overlap_decode.txt), "
                                                        "without and with the HBM row cache; ms per step",
                                               **dec["rcache"])},
        "breakdown_us_per_layer": {"scan_lists": round(dec["lists_ms"] * 1e3, 2),
                                   "select_attend_merge": round(dec["ms"] * 1e3 / DECODE["layers"]
                                                                - dec["lists_ms"] * 1e3, 2),
                                   "separate_scan_select": round(dec["scan_ms"] * 1e3, 2)},
        "pool_ms_all_layers": round(dec["pool_ms"], 3),
        "prefill": {"workload": PREFILL["name"], "tok_s": round(t8["tok_s"], 1), "ms_per_chunk": round(t8["ms"], 4),
                    "tflops": round(t8["tflops"], 2), "mfma_frac": round(t8["tflops"] / BF16_PEAK_TFLOPS, 5),
                    "useful_gflop": round(pflops["total"] / 1e9, 2),
                    "breakdown_us": pre["breakdown_us"], "attend_tflops": pre["attend_tflops"],
                    "attend_counters": counter_mfma("attend_a"), "scores_gemm_counters": counter_mfma("scores_gemm_a"),
                    "tile_1024": {"tok_s": round(pre[1024]["tok_s"], 1), "ms_per_chunk": round(pre[1024]["ms"], 4)},
                    "correlated": pre["correlated"], "oracle_tok_s": cpu_all[4]["value"]},
        "mla": dict(mla, decode=dict(mla["decode"], oracle_steps_s=cpu_all["5b"]["value"]),
                    prefill=dict(mla["prefill"], oracle_tok_s=cpu_all["5a"]["value"])),
        "decode_batch1": {f"config_{c['config_id']}": dict(r, oracle_steps_s=cpu_all[c["config_id"]]["value"])
                          for c, r in zip(SMALL_DECODES, small)},
        "roofline": {"kernel": "index_lists_a (pooled-key scan + per-chunk candidate lists, first launch of "
                               "qsa_decode_layer, no score buffer as in the headline)", "bound": "hbm",
                     "achieved": round(dec["lists_gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dec["lists_gbs"] / HBM_PEAK_GBS, 4),
                     "traffic": counter_traffic("index_lists_a<2, false>", "2048"),
                     "bytes_per_launch": dec["scan_launch_bytes"], "us_per_launch": round(dec["lists_ms"] * 1e3, 3)},
        "cpu_baseline": {**{k: cpu[k] for k in ("value", "unit", "cores", "kind", "sample", "value_1core")},
                         "cpu_model": cpu_model,
                         "other_workloads": {str(c): {k: v for k, v in r.items() if k != "kind"}
                                             for c, r in cpu_all.items() if c != 3}},
        "wall_s": round(time.time() - t_all, 1),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
