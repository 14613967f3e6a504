#!/usr/bin/env python3
"""Benchmark of the CSA decode step on one MI355X.

Workload (batch-4 long-context decode): 4 sequences of 1,048,576 raw tokens,
r = 4 gated pooling -> 262,144 compressed entries per sequence, fp8 (E4M3)
compressed cache with one fp32 scale per 64-entry page, 64 query heads of dim
128 over one KV head, 4 indexer heads of dim 64, Top-1024, a 128-token
window, and one indexer pass whose Top-K is reused by a group of 4 layers that
each keep their own compressed K/V. A step is one csa_index_topk over the 4
queries plus 4 csa_attend calls (one per layer). Inputs are seeded synthetic
data resident in HBM before timing; steps rotate over 8 identical cache
replicas so the 256 MB last-level cache cannot hold a step's working set.

The timed steps are HIP graph replays (a graph holds one step on every
replica, as a model's decode iteration holds several layer groups). Prints
one JSON line: decode tokens/s, the indexer scan kernel's achieved HBM
bandwidth against the 8 TB/s peak (HIP events around every scan launch of an
eager pass over the same steps) and against a plain streaming read of the same
size on the same GPU, and the CPU oracle's throughput on a bounded sample of
the same step.
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

METRIC = "CSA decode tokens/s/GPU at 1M ctx + achieved HBM GB/s vs peak; prefill MFMA util"
HBM_PEAK_GBPS = 8000.0

# the workload
BATCH, CONTEXT, RATIO, TOPK, WINDOW, HEADS, IDX_HEADS, LAYERS = 4, 1 << 20, 4, 1024, 128, 64, 4, 4
POOL_BLOCKS = 2048   # candidate pool of the hierarchical indexer: 2,048 blocks of 8 entries


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU-oracle sample budget")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle leg")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one 512 MiB device copy after timing (reference kernel for HBM counters)")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill-chunk MFMA-utilisation leg")
    ap.add_argument("--prefill-only", action="store_true", help="only run the prefill-chunk leg (same as --only prefill)")
    ap.add_argument("--only", choices=["c1", "c2", "c5", "prefill", "hca"],
                    help="run only this leg and print its record (profiling one workload at a time)")
    ap.add_argument("--no-hca", action="store_true", help="skip the heavily-compressed-attention leg")
    ap.add_argument("--no-hier", action="store_true", help="skip the hierarchical-indexer (pool / Reindex) leg")
    ap.add_argument("--no-swa-fp8", action="store_true", help="skip the fp8 window-ring decode leg")
    ap.add_argument("--no-fp4", action="store_true", help="skip the fp4 main-KV decode leg")
    ap.add_argument("--no-c1", action="store_true", help="skip the batch-1 4,096-token fp32 decode leg")
    ap.add_argument("--no-c2", action="store_true", help="skip the batch-32 65,536-token bf16 decode leg")
    ap.add_argument("--no-c5", action="store_true", help="skip the 64-request ragged serving leg")
    return ap.parse_args()


MFMA_BF16_PEAK_TFLOPS = 2500.0
PF_PRIOR, PF_CHUNK, PF_K = 131072, 2048, 1024


def build_prefill(seed, dev):
    """The prefill-chunk workload on `dev`: a bf16 cache holding the
    131,072-token context (pages in a seeded permuted order), the chunk's raw
    rows, queries and outputs, and chunk_step(stream), which compresses the
    chunk, indexes and attends all of its 2,048 tokens."""
    import torch
    from compressed_sparse_attention_csa_amd import synth as Sy
    from compressed_sparse_attention_csa_amd.cache import CacheSpec, CsaCache

    total = PF_PRIOR + PF_CHUNK
    pages = (total // RATIO + 63) // 64
    spec = CacheSpec(ratio=RATIO, q_heads=HEADS, idx_heads=IDX_HEADS, window=WINDOW, ring_rows=WINDOW + PF_CHUNK,
                     n_layers=1, max_seqs=1, max_pages_per_seq=pages, pool_pages=pages, kv_dtype="bf16",
                     act_dtype="bf16", max_queries=PF_CHUNK, max_k=PF_K)
    bt = torch.tensor(Sy.permutation(seed, pages, salt=5), dtype=torch.int32).view(1, pages).to(dev)
    c = CsaCache(spec, dev, block_table=bt)
    P = Sy.proj_matrix(seed, 128, 64, device=dev)
    rows = lambda kind, r0, n: Sy.normal_rows(seed, Sy.stream_id(kind, 0, 0), r0, n, 128, dev, torch.bfloat16)
    c.compress(0, [0], [PF_PRIOR], rows(Sy.KIND_K, 0, PF_PRIOR), rows(Sy.KIND_V, 0, PF_PRIOR), rows(Sy.KIND_Z, 0, PF_PRIOR), P)
    ck, cv, cz = rows(Sy.KIND_K, PF_PRIOR, PF_CHUNK), rows(Sy.KIND_V, PF_PRIOR, PF_CHUNK), rows(Sy.KIND_Z, PF_PRIOR, PF_CHUNK)
    qi = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_QI, 0, 1), 0, PF_CHUNK * IDX_HEADS, 64, dev, torch.bfloat16).view(PF_CHUNK, IDX_HEADS, 64)
    w = Sy.uniform_rows(seed, Sy.stream_id(Sy.KIND_W, 0, 1), 0, PF_CHUNK, IDX_HEADS, dev)
    q = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_Q, 0, 1), 0, PF_CHUNK * HEADS, 128, dev, torch.bfloat16).view(PF_CHUNK, HEADS, 128)
    T = torch.empty((PF_CHUNK, PF_K), dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    q_seq, q_pos = [0] * PF_CHUNK, list(range(PF_PRIOR, total))
    scale = 1.0 / math.sqrt(128)
    def chunk_step(stream):
        c.compress(0, [0], [PF_CHUNK], ck, cv, cz, P, stream=stream)
        c.index_topk(q_seq, q_pos, qi, w, PF_K, T, stream=stream)
        c.attend(0, q_seq, q_pos, q, T, PF_K, scale, out, stream=stream)
    return dict(cache=c, qi=qi, w=w, q=q, T=T, out=out, q_seq=q_seq, q_pos=q_pos, scale=scale, chunk_step=chunk_step)


def prefill_leg(seed, dev, steps=5):
    """Prefill chunk: 2,048 new tokens appended to a 131,072-token context (bf16,
    r = 4, Top-1024 per query token, W = 128, 64 heads). One step = compress the
    chunk, index (MFMA score GEMM + exact select) and attend all 2,048 tokens.
    Reports MFMA utilisation of the index score GEMM (the pass that scores every
    visible entry) and of the attention kernel, each timed by HIP events that
    its launch stamps (the last of the steps)."""
    import torch
    from compressed_sparse_attention_csa_amd import accounting as A
    from compressed_sparse_attention_csa_amd import binding as B

    W_ = build_prefill(seed, dev)
    c, qi, w, T, q_seq, q_pos, chunk_step = (W_[k] for k in ("cache", "qi", "w", "T", "q_seq", "q_pos", "chunk_step"))

    # warm-up, then the step captured once and replayed: host-side argument
    # marshalling stays out of the timed region
    B.csa_seq_set_len(c.handle, 0, 0, PF_PRIOR)
    chunk_step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    B.csa_seq_set_len(c.handle, 0, 0, PF_PRIOR)
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cap):
        chunk_step(torch.cuda.current_stream())
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    chunk_ms = e0.elapsed_time(e1) / steps
    # kernel timing: eager steps, each score-GEMM and attention launch stamps its own events
    B.csa_profile_begin(c.handle, B.PROFILE_INDEX | B.PROFILE_ATTEND)
    for _ in range(steps):
        B.csa_seq_set_len(c.handle, 0, 0, PF_PRIOR)
        chunk_step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    scan_ms, n = B.csa_profile_end(c.handle, B.PROFILE_INDEX)
    att_kernel_ms, n_att = B.csa_profile_end(c.handle, B.PROFILE_ATTEND)
    # the chunk's Full-layer index with and without its per-query candidate pool
    # (2,048 blocks of 8 entries), the cache holding the chunk
    pool = torch.empty((PF_CHUNK, POOL_BLOCKS), dtype=torch.int32, device=dev)
    idx_us = graph_us([lambda st: B.csa_index_topk(c.handle, q_seq, q_pos, qi, w, PF_K, T, st)], steps)
    pool_us = graph_us([lambda st: B.csa_index_topk_pool(c.handle, q_seq, q_pos, qi, w, PF_K, T, POOL_BLOCKS, pool, st)],
                       steps)
    flags = c.read_errors()
    if flags & ~B.ERR_FALLBACK:
        raise RuntimeError(f"prefill leg raised device error flags {flags}")
    idx_flops = A.index_flops(A.prefill_visible_scores(PF_PRIOR, PF_CHUNK, RATIO), IDX_HEADS, 64)
    att_flops = A.attend_flops(PF_CHUNK, HEADS, PF_K + WINDOW, 128)
    att_ms = att_kernel_ms / max(n_att, 1)
    res = {"workload": "prefill chunk: 2,048 tokens on a 131,072-token context, bf16, r=4, Top-1024, W=128, 64 heads",
           "ms_per_chunk": round(chunk_ms, 4), "tokens_per_s": round(PF_CHUNK / (chunk_ms * 1e-3), 1),
           "index_gemm": {"tflops": round(idx_flops / (scan_ms / max(n, 1) * 1e-3) / 1e12, 1),
                          "util": round(idx_flops / (scan_ms / max(n, 1) * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                          "us": round(scan_ms / max(n, 1) * 1e3, 2), "gflop": round(idx_flops / 1e9, 2)},
           "attend": {"tflops": round(att_flops / (att_ms * 1e-3) / 1e12, 1),
                      "util": round(att_flops / (att_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                      "us": round(att_ms * 1e3, 2), "gflop": round(att_flops / 1e9, 2)},
           "index_us": round(idx_us, 2), "index_with_pool_us": round(pool_us, 2),
           "peak_tflops": MFMA_BF16_PEAK_TFLOPS}
    c.close()
    return res


HCA_RATIO, HCA_REPLICAS = 128, 32


def build_hca(seed, dev):
    """The HCA workload's cache on `dev`: batch 4, each sequence's 1,048,576
    raw rows (layer stream 7) compressed at r = 128 into fp8 pages in a seeded
    permuted order, no indexer. Returns (cache, spec, block table)."""
    import torch
    from compressed_sparse_attention_csa_amd import synth as Sy
    from compressed_sparse_attention_csa_amd.cache import CacheSpec, CsaCache

    pages = CONTEXT // HCA_RATIO // 64
    spec = CacheSpec(ratio=HCA_RATIO, q_heads=HEADS, idx_heads=0, window=WINDOW, ring_rows=max(WINDOW, HCA_RATIO),
                     n_layers=1, max_seqs=BATCH, max_pages_per_seq=pages, pool_pages=BATCH * pages,
                     kv_dtype="fp8", act_dtype="bf16", max_queries=BATCH, max_k=1)
    bt = torch.tensor(Sy.permutation(seed, BATCH * pages, salt=7), dtype=torch.int32).view(BATCH, pages).to(dev)
    base = CsaCache(spec, dev, block_table=bt)
    chunk = 1 << 18
    for b in range(BATCH):
        for r0 in range(0, CONTEXT, chunk):
            rows = [Sy.normal_rows(seed, Sy.stream_id(kind, 7, b), r0, chunk, 128, dev, torch.bfloat16)
                    for kind in (Sy.KIND_K, Sy.KIND_V, Sy.KIND_Z)]
            base.compress(0, [b], [chunk], *rows)
    return base, spec, bt


def hca_q(seed, dev):
    """The HCA leg's batch of queries (64 heads, bf16)."""
    import torch
    from compressed_sparse_attention_csa_amd import synth as Sy
    return Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_Q, 7), 0, BATCH * HEADS, 128, dev, torch.bfloat16).view(BATCH, HEADS, 128)


def hca_leg(seed, dev, steps=50):
    """Heavily compressed attention layer at the same 1M-token batch-4 decode:
    r = 128 gives 8,192 fp8 entries per sequence, every one attended (no
    indexer) together with the 128-token window, 64 heads. Timed over graph
    replays rotating across 32 cache replicas (more than the last-level cache
    holds); the attention kernel's own time from launch-stamped events."""
    import torch
    from compressed_sparse_attention_csa_amd import accounting as A
    from compressed_sparse_attention_csa_amd import binding as B
    from compressed_sparse_attention_csa_amd.cache import CsaCache

    entries = CONTEXT // HCA_RATIO
    base, spec, bt = build_hca(seed, dev)
    caches = [base]
    for _ in range(1, HCA_REPLICAS):
        c = CsaCache(spec, dev, block_table=bt)
        for src, dst in ((base.kbar, c.kbar), (base.vbar, c.vbar), (base.kbar_scale, c.kbar_scale),
                         (base.vbar_scale, c.vbar_scale), (base.ring_k, c.ring_k), (base.ring_v, c.ring_v)):
            for s_, d_ in zip(src, dst):
                d_.copy_(s_)
        for b in range(BATCH):
            B.csa_seq_set_len(c.handle, 0, b, CONTEXT)
        caches.append(c)
    q = hca_q(seed, dev)
    out = torch.empty_like(q)
    q_seq, q_pos = list(range(BATCH)), [CONTEXT - 1] * BATCH
    scale = 1.0 / math.sqrt(128)
    torch.cuda.synchronize()
    us = graph_us([lambda s, c=c: B.csa_attend_dense(c.handle, 0, q_seq, q_pos, q, scale, out, s) for c in caches], steps)
    for c in caches:
        B.csa_profile_begin(c.handle, B.PROFILE_ATTEND)
    for i in range(len(caches)):
        B.csa_attend_dense(caches[i].handle, 0, q_seq, q_pos, q, scale, out, torch.cuda.current_stream())
    torch.cuda.synchronize()
    k_ms, k_n = 0.0, 0
    for c in caches:
        ms, n = B.csa_profile_end(c.handle, B.PROFILE_ATTEND)
        k_ms += ms
        k_n += n
    flags = max(c.read_errors() for c in caches)
    if flags:
        raise RuntimeError(f"HCA leg raised device error flags {flags}")
    nbytes = BATCH * A.attend_bytes(entries, WINDOW, 128, HEADS, "fp8", "bf16")
    kern_us = k_ms * 1e3 / max(k_n, 1)
    for c in caches:
        c.close()
    return {"workload": "HCA decode layer: batch 4, 1,048,576 tokens, r=128 (8,192 fp8 entries, all attended), "
                        "W=128, 64 heads", "us_per_call": round(us, 3), "tokens_per_s": round(BATCH / (us * 1e-6), 1),
            "attend_kernel_us": round(kern_us, 3), "bytes": nbytes,
            "hbm_gbps": round(nbytes / (kern_us * 1e-6) / 1e9, 1)}


def graph_us(calls, steps, warmup=3):
    """Mean microseconds per call when one HIP graph holding every callable
    once, in order, is replayed `steps` times (each callable enqueues on the
    stream it gets; the callables are the replicas of one step)."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        for fn in calls:
            fn(torch.cuda.current_stream())
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e6 / (steps * len(calls))


def kernel_us(caches, kind, fn, reps):
    """Mean duration of the score (kind 1) or attention (kind 2) kernel over
    eager calls fn(i), from events the launches themselves stamp."""
    import torch
    from compressed_sparse_attention_csa_amd import binding as B
    for c in caches:
        B.csa_profile_begin(c.handle, kind)
    for i in range(reps):
        fn(i)
    torch.cuda.synchronize()
    ms, n = 0.0, 0
    for c in caches:
        m, k = B.csa_profile_end(c.handle, kind)
        ms += m
        n += k
    return ms * 1e3 / max(n, 1)


def hier_leg(caches, qi, w, steps, seed):
    """Hierarchical sparse indexer on the headline caches: the Full layer's
    Top-K with its 2,048-block candidate pool, and a Reindex layer's Top-K
    inside that pool with its own indexer query (16,384 of 262,144 entries)."""
    import torch
    from compressed_sparse_attention_csa_amd import accounting as A
    from compressed_sparse_attention_csa_amd import binding as B
    from compressed_sparse_attention_csa_amd import synth as Sy
    dev = qi.device
    q_seq, q_pos = list(range(BATCH)), [CONTEXT - 1] * BATCH
    nb = POOL_BLOCKS
    topk = [torch.empty((BATCH, TOPK), dtype=torch.int32, device=dev) for _ in caches]
    pools = [torch.empty((BATCH, nb), dtype=torch.int32, device=dev) for _ in caches]
    t2 = [torch.empty((BATCH, TOPK), dtype=torch.int32, device=dev) for _ in caches]
    qi2 = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_QI, 1), 0, BATCH * IDX_HEADS, 64, dev, torch.bfloat16).view(BATCH, IDX_HEADS, 64)
    w2 = Sy.uniform_rows(seed, Sy.stream_id(Sy.KIND_W, 1), 0, BATCH, IDX_HEADS, dev)
    full = [lambda s, c=c, r=r: B.csa_index_topk(c.handle, q_seq, q_pos, qi, w, TOPK, topk[r], s)
            for r, c in enumerate(caches)]
    full_pool = [lambda s, c=c, r=r: B.csa_index_topk_pool(c.handle, q_seq, q_pos, qi, w, TOPK, topk[r], nb, pools[r], s)
                 for r, c in enumerate(caches)]
    reindex = [lambda s, c=c, r=r: B.csa_index_reindex(c.handle, q_seq, q_pos, qi2, w2, nb, pools[r], TOPK, t2[r], s)
               for r, c in enumerate(caches)]
    us_full = graph_us(full, steps)
    us_pool = graph_us(full_pool, steps)      # also leaves every replica's pool in place
    us_re = graph_us(reindex, steps)
    stream = torch.cuda.current_stream()
    rescan_us = kernel_us(caches, B.PROFILE_INDEX, lambda i: reindex[i % len(caches)](stream), steps)
    flags = max(c.read_errors() for c in caches)
    if flags & ~B.ERR_FALLBACK:
        raise RuntimeError(f"hierarchical leg raised device error flags {flags}")
    pool_entries = nb * 8
    nbytes = BATCH * A.reindex_bytes(pool_entries, nb, 64, "fp8")
    return {"workload": f"batch 4, 1,048,576 tokens (262,144 fp8 entries), Top-1024; pool of {nb} blocks x 8 entries "
                        f"({pool_entries} candidates)",
            "full_index_us": round(us_full, 3), "full_index_with_pool_us": round(us_pool, 3),
            "reindex_us": round(us_re, 3), "reindex_score_kernel_us": round(rescan_us, 3),
            "reindex_score_bytes": nbytes, "reindex_score_gbps": round(nbytes / (rescan_us * 1e-6) / 1e9, 1),
            "fallback_flag": bool(flags & B.ERR_FALLBACK)}


def variant_leg(seed, dev, replicas, qi, w, qs, steps, kv="fp8", swa=""):
    """The headline decode step on caches of another storage format (the
    window ring as E4M3 with one scale per row, or FP4 main K/V): same
    workload, same graph timing."""
    import torch
    from compressed_sparse_attention_csa_amd import accounting as A
    from compressed_sparse_attention_csa_amd import binding as B
    caches = build_cache(seed, replicas, dev, swa=swa, kv=kv)
    q_seq, q_pos = list(range(BATCH)), [CONTEXT - 1] * BATCH
    topk = [torch.empty((BATCH, TOPK), dtype=torch.int32, device=dev) for _ in caches]
    outs = [torch.empty((BATCH, HEADS, 128), dtype=torch.bfloat16, device=dev) for _ in range(LAYERS)]
    scale = 1.0 / math.sqrt(128)

    def make(r):
        c = caches[r]

        def fn(s):
            B.csa_index_topk(c.handle, q_seq, q_pos, qi, w, TOPK, topk[r], s)
            for l in range(LAYERS):
                B.csa_attend(c.handle, l, q_seq, q_pos, qs[l], topk[r], TOPK, scale, outs[l], s)
        return fn
    us = graph_us([make(r) for r in range(len(caches))], steps)
    stream = torch.cuda.current_stream()

    def attend_only(i):
        c = caches[i % len(caches)]
        for l in range(LAYERS):
            B.csa_attend(c.handle, l, q_seq, q_pos, qs[l], topk[i % len(caches)], TOPK, scale, outs[l], stream)
    att_us = kernel_us(caches, B.PROFILE_ATTEND, attend_only, steps // 4 + 1)
    flags = max(c.read_errors() for c in caches)
    if flags:
        raise RuntimeError(f"{kv}/{swa or 'bf16'} leg raised device error flags {flags}")
    for c in caches:
        c.close()
    sb = A.decode_step_bytes(BATCH, CONTEXT // RATIO, 128, 64, HEADS, IDX_HEADS, TOPK, WINDOW, LAYERS, kv, "bf16",
                             swa or "bf16")
    what = {"fp8": "fp8 pages (fp32 scale per page)", "fp4": "fp4 entries (E2M1, E4M3 scale per 16 channels)"}[kv]
    return {"workload": f"the headline decode step, main K/V as {what}, window ring {swa or 'bf16'}",
            "ms_per_step": round(us * 1e-3, 5), "tokens_per_s": round(BATCH / (us * 1e-6), 1),
            "attend_kernel_us": round(att_us, 3), "step_bytes": sb}


C1_CONTEXT, C1_HEADS, C1_K = 4096, 16, 64
C2_BATCH, C2_CONTEXT, C2_K = 32, 1 << 16, 512
C5_REQUESTS, C5_MIN, C5_MAX, C5_K = 64, 4096, 262144, 512


def timed_decode(caches, q_seq, q_pos, qi, w, qs, k, steps, compress=None):
    """A decode step - optionally compress(cache, stream) first, then one
    csa_index_topk and one csa_attend per query tensor in qs (the layers that
    share the Top-K) - timed as graph replays over the replicas (one graph
    holds a step on each). Returns (us per step, score-kernel us, attention-kernel
    us), the kernel times from launch-stamped events over eager steps without
    the compress."""
    import torch
    from compressed_sparse_attention_csa_amd import binding as B
    dev = qi.device
    topk = [torch.empty((len(q_seq), k), dtype=torch.int32, device=dev) for _ in caches]
    outs = [torch.empty_like(q) for q in qs]
    scale = 1.0 / math.sqrt(128)

    def index_attend(r, s_):
        c = caches[r]
        B.csa_index_topk(c.handle, q_seq, q_pos, qi, w, k, topk[r], s_)
        for l, q in enumerate(qs):
            B.csa_attend(c.handle, l, q_seq, q_pos, q, topk[r], k, scale, outs[l], s_)

    def make(r):
        def fn(s_):
            if compress is not None:
                compress(caches[r], s_)
            index_attend(r, s_)
        return fn
    us = graph_us([make(r) for r in range(len(caches))], steps)
    stream = torch.cuda.current_stream()
    for c in caches:
        B.csa_profile_begin(c.handle, B.PROFILE_INDEX | B.PROFILE_ATTEND)
    for i in range(max(len(caches), steps // 4)):
        index_attend(i % len(caches), stream)
    torch.cuda.synchronize()
    sms, sn, ams, an = 0.0, 0, 0.0, 0
    for c in caches:
        m, n = B.csa_profile_end(c.handle, B.PROFILE_INDEX)
        sms, sn = sms + m, sn + n
        m, n = B.csa_profile_end(c.handle, B.PROFILE_ATTEND)
        ams, an = ams + m, an + n
    flags = max(c.read_errors() for c in caches)
    if flags:
        raise RuntimeError(f"device error flags {flags}")
    return us, sms * 1e3 / max(sn, 1), ams * 1e3 / max(an, 1)


def decode_record(workload, us, scan_us, att_us, nbytes, n_tokens, extra=None):
    rec = {"workload": workload, "us_per_step": round(us, 3), "tokens_per_s": round(n_tokens / (us * 1e-6), 1),
           "step_bytes": nbytes, "hbm_gbps": round(nbytes / (us * 1e-6) / 1e9, 1),
           "frac_of_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
           "score_kernel_us": round(scan_us, 3), "attend_kernel_us": round(att_us, 3)}
    rec.update(extra or {})
    return rec


def c1_leg(seed, dev, replicas, steps):
    """Single decode step, batch 1, 4,096-token fp32 context: r = 4 (1,024
    entries), 16 query heads, 4 indexer heads, Top-64, W = 128. Launch-latency
    bound: reports microseconds per step."""
    import torch
    from compressed_sparse_attention_csa_amd import accounting as A
    from compressed_sparse_attention_csa_amd import synth as Sy
    from compressed_sparse_attention_csa_amd.cache import CacheSpec, CsaCache
    pages = C1_CONTEXT // RATIO // 64
    spec = CacheSpec(ratio=RATIO, q_heads=C1_HEADS, idx_heads=IDX_HEADS, window=WINDOW, ring_rows=WINDOW, n_layers=1,
                     max_seqs=1, max_pages_per_seq=pages, pool_pages=pages, kv_dtype="f32", act_dtype="f32",
                     max_queries=1, max_k=C1_K)
    bt = torch.tensor(Sy.permutation(seed, pages, salt=1), dtype=torch.int32).view(1, pages).to(dev)
    base = CsaCache(spec, dev, block_table=bt)
    rows = [Sy.normal_rows(seed, Sy.stream_id(kind, 0, 0), 0, C1_CONTEXT, 128, dev, torch.float32)
            for kind in (Sy.KIND_K, Sy.KIND_V, Sy.KIND_Z)]
    base.compress(0, [0], [C1_CONTEXT], *rows, Sy.proj_matrix(seed, 128, 64, device=dev))
    caches = [base] + [base.clone() for _ in range(replicas - 1)]
    qi = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_QI), 0, IDX_HEADS, 64, dev, torch.float32).view(1, IDX_HEADS, 64)
    w = Sy.uniform_rows(seed, Sy.stream_id(Sy.KIND_W), 0, 1, IDX_HEADS, dev)
    q = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_Q), 0, C1_HEADS, 128, dev, torch.float32).view(1, C1_HEADS, 128)
    us, sus, aus = timed_decode(caches, [0], [C1_CONTEXT - 1], qi, w, [q], C1_K, steps)
    nbytes = A.decode_step_bytes(1, C1_CONTEXT // RATIO, 128, 64, C1_HEADS, IDX_HEADS, C1_K, WINDOW, 1, "f32", "f32")
    for c in caches:
        c.close()
    return decode_record("decode, batch 1, 4,096-token fp32 context, r=4, Top-64, W=128, 16 heads", us, sus, aus,
                         nbytes, 1, {"bound": "launch latency", "replicas": replicas})


def c2_leg(seed, dev, replicas, steps):
    """Batched decode: 32 sequences of 65,536 bf16 tokens (16,384 entries
    each), 64 query heads, Top-512, W = 128, one layer. HBM bound: 70 % of the
    8 TB/s peak is the target."""
    import torch
    from compressed_sparse_attention_csa_amd import accounting as A
    from compressed_sparse_attention_csa_amd import synth as Sy
    from compressed_sparse_attention_csa_amd.cache import CacheSpec, CsaCache
    pages = C2_CONTEXT // RATIO // 64
    spec = CacheSpec(ratio=RATIO, q_heads=HEADS, idx_heads=IDX_HEADS, window=WINDOW, ring_rows=WINDOW, n_layers=1,
                     max_seqs=C2_BATCH, max_pages_per_seq=pages, pool_pages=C2_BATCH * pages, kv_dtype="bf16",
                     act_dtype="bf16", max_queries=C2_BATCH, max_k=C2_K)
    bt = torch.tensor(Sy.permutation(seed, C2_BATCH * pages, salt=9), dtype=torch.int32).view(C2_BATCH, pages).to(dev)
    base = CsaCache(spec, dev, block_table=bt)
    P = Sy.proj_matrix(seed, 128, 64, device=dev)
    for b in range(C2_BATCH):
        rows = [Sy.normal_rows(seed, Sy.stream_id(kind, 0, b), 0, C2_CONTEXT, 128, dev, torch.bfloat16)
                for kind in (Sy.KIND_K, Sy.KIND_V, Sy.KIND_Z)]
        base.compress(0, [b], [C2_CONTEXT], *rows, P)
    caches = [base] + [base.clone() for _ in range(replicas - 1)]
    B_ = C2_BATCH
    qi = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_QI), 0, B_ * IDX_HEADS, 64, dev, torch.bfloat16).view(B_, IDX_HEADS, 64)
    w = Sy.uniform_rows(seed, Sy.stream_id(Sy.KIND_W), 0, B_, IDX_HEADS, dev)
    q = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_Q), 0, B_ * HEADS, 128, dev, torch.bfloat16).view(B_, HEADS, 128)
    us, sus, aus = timed_decode(caches, list(range(B_)), [C2_CONTEXT - 1] * B_, qi, w, [q], C2_K, steps)
    nbytes = A.decode_step_bytes(B_, C2_CONTEXT // RATIO, 128, 64, HEADS, IDX_HEADS, C2_K, WINDOW, 1, "bf16", "bf16")
    for c in caches:
        c.close()
    return decode_record("decode, batch 32, 65,536-token bf16 contexts, r=4, Top-512, W=128, 64 heads", us, sus, aus,
                         nbytes, B_, {"target_us": round(nbytes / (0.7 * HBM_PEAK_GBPS * 1e9) * 1e6, 2),
                                      "replicas": replicas})


def c5_leg(seed, dev, replicas, steps):
    """Mixed serving step: 64 requests with contexts drawn log-uniform from 4K
    to 256K tokens in one paged fp8 pool (64-entry pages in a shuffled order).
    A step appends one token to every request (csa_compress: closes a block for
    about a quarter of them, fp8 page re-encode), then indexes (Top-512) and
    attends (W = 128, 64 heads). Bytes are exact for the drawn lengths."""
    import torch
    from compressed_sparse_attention_csa_amd import accounting as A
    from compressed_sparse_attention_csa_amd import binding as B
    from compressed_sparse_attention_csa_amd import synth as Sy
    from compressed_sparse_attention_csa_amd.cache import CacheSpec, CsaCache
    n = C5_REQUESTS
    lens = Sy.log_uniform_lengths(seed, n, C5_MIN, C5_MAX)
    pages = [((L + 1) // RATIO + 63) // 64 for L in lens]
    pool = sum(pages)
    perm = Sy.permutation(seed, pool, salt=13)
    bt = torch.full((n, max(pages)), -1, dtype=torch.int32)
    off = 0
    for b, p in enumerate(pages):
        bt[b, :p] = torch.tensor(perm[off:off + p], dtype=torch.int32)
        off += p
    spec = CacheSpec(ratio=RATIO, q_heads=HEADS, idx_heads=IDX_HEADS, window=WINDOW, ring_rows=WINDOW, n_layers=1,
                     max_seqs=n, max_pages_per_seq=max(pages), pool_pages=pool, kv_dtype="fp8", act_dtype="bf16",
                     max_queries=n, max_k=C5_K)
    base = CsaCache(spec, dev, block_table=bt.to(dev))
    P = Sy.proj_matrix(seed, 128, 64, device=dev)
    for b, L in enumerate(lens):
        rows = [Sy.normal_rows(seed, Sy.stream_id(kind, 0, b), 0, L, 128, dev, torch.bfloat16)
                for kind in (Sy.KIND_K, Sy.KIND_V, Sy.KIND_Z)]
        base.compress(0, [b], [L], *rows, P)
    caches = [base] + [base.clone() for _ in range(replicas - 1)]
    ids = list(range(n))
    new = [torch.cat([Sy.normal_rows(seed, Sy.stream_id(kind, 0, b), lens[b], 1, 128, dev, torch.bfloat16)
                      for b in ids]) for kind in (Sy.KIND_K, Sy.KIND_V, Sy.KIND_Z)]
    qi = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_QI), 0, n * IDX_HEADS, 64, dev, torch.bfloat16).view(n, IDX_HEADS, 64)
    w = Sy.uniform_rows(seed, Sy.stream_id(Sy.KIND_W), 0, n, IDX_HEADS, dev)
    q = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_Q), 0, n * HEADS, 128, dev, torch.bfloat16).view(n, HEADS, 128)

    # the graph replays the same append (token L of every request): writes the
    # same bytes each time, so every replay is a full serving step
    def compress(c, s_):
        B.csa_compress(c.handle, 0, ids, [1] * n, new[0], new[1], new[2], P, s_)
    us, sus, aus = timed_decode(caches, ids, lens, qi, w, [q], C5_K, steps, compress=compress)
    ents = [(L + 1) // RATIO for L in lens]
    cb = sum(A.compress_bytes(L, 1, RATIO, 128, 64, "fp8", "bf16", WINDOW) for L in lens)
    nbytes = cb + A.decode_step_bytes(n, ents, 128, 64, HEADS, IDX_HEADS, C5_K, WINDOW, 1, "fp8", "bf16")
    for c in caches:
        c.close()
    return decode_record("serving step: 64 requests, contexts log-uniform 4K-256K tokens (one paged fp8 pool), "
                         "append 1 token each (compress) + index Top-512 + attend W=128, 64 heads", us, sus, aus,
                         nbytes, n, {"compress_bytes": cb, "context_tokens": int(sum(lens)),
                                     "closing_blocks": int(sum((L + 1) % RATIO == 0 for L in lens)),
                                     "replicas": replicas})


def build_cache(seed, replicas, dev, swa="", kv="fp8"):
    import torch
    from compressed_sparse_attention_csa_amd import binding as B
    from compressed_sparse_attention_csa_amd import synth as Sy
    from compressed_sparse_attention_csa_amd.cache import CacheSpec, CsaCache

    entries = CONTEXT // RATIO
    pages = entries // 64
    spec = CacheSpec(ratio=RATIO, q_heads=HEADS, idx_heads=IDX_HEADS, window=WINDOW, ring_rows=WINDOW,
                     n_layers=LAYERS, max_seqs=BATCH, max_pages_per_seq=pages, pool_pages=BATCH * pages,
                     kv_dtype=kv, act_dtype="bf16", swa_dtype=swa, max_queries=BATCH, max_k=TOPK)
    perm = torch.tensor(Sy.permutation(seed, BATCH * pages, salt=3), dtype=torch.int32)
    bt = perm.view(BATCH, pages).to(dev)
    base = CsaCache(spec, dev, block_table=bt)
    P = Sy.proj_matrix(seed, 128, 64, device=dev)
    chunk = 1 << 18
    for layer in range(LAYERS):
        for b in range(BATCH):
            for r0 in range(0, CONTEXT, chunk):
                K = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_K, layer, b), r0, chunk, 128, dev, torch.bfloat16)
                V = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_V, layer, b), r0, chunk, 128, dev, torch.bfloat16)
                Z = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_Z, layer, b), r0, chunk, 128, dev, torch.bfloat16)
                base.compress(layer, [b], [chunk], K, V, Z, P if layer == 0 else None)
    torch.cuda.synchronize()
    flags = base.read_errors()
    if flags:
        raise RuntimeError(f"cache build raised device error flags {flags}")
    caches = [base]
    for _ in range(1, replicas):
        c = CsaCache(spec, dev, block_table=bt)
        for src, dst in ((base.kbar, c.kbar), (base.vbar, c.vbar), (base.kbar_scale, c.kbar_scale),
                         (base.vbar_scale, c.vbar_scale), (base.ring_k, c.ring_k), (base.ring_v, c.ring_v),
                         (base.ring_k_scale, c.ring_k_scale), (base.ring_v_scale, c.ring_v_scale),
                         (base.kbar_stage, c.kbar_stage), (base.vbar_stage, c.vbar_stage),
                         (base.kbar_gscale, c.kbar_gscale), (base.vbar_gscale, c.vbar_gscale),
                         (base.block_stage, c.block_stage)):
            for s_, d_ in zip(src, dst):
                d_.copy_(s_)
        c.kidx.copy_(base.kidx)
        c.kidx_scale.copy_(base.kidx_scale)
        c.kidx_stage.copy_(base.kidx_stage)
        for layer in range(LAYERS):
            for b in range(BATCH):
                B.csa_seq_set_len(c.handle, layer, b, CONTEXT)
        caches.append(c)
    torch.cuda.synchronize()
    return caches


def scan_bytes_per_launch():
    from compressed_sparse_attention_csa_amd import accounting as A
    per_q = A.index_scan_bytes(CONTEXT // RATIO, 64, "fp8") + IDX_HEADS * 64 * 2 + IDX_HEADS * 4
    return BATCH * per_q


def attend_bytes_per_launch():
    from compressed_sparse_attention_csa_amd import accounting as A
    return BATCH * A.attend_bytes(TOPK, WINDOW, 128, HEADS, "fp8", "bf16")


def step_bytes():
    from compressed_sparse_attention_csa_amd import accounting as A
    return A.decode_step_bytes(BATCH, CONTEXT // RATIO, 128, 64, HEADS, IDX_HEADS, TOPK, WINDOW, LAYERS, "fp8", "bf16")


def traffic_from_profiles(record="index_scan_1m_decode_traffic.json", source="index.hip"):
    """(HBM bytes per launch, scope) from a committed counter record, if it was
    taken on the current source of its kernel; else (None, None)."""
    path = os.path.join(ROOT, "profiles", record)
    src = os.path.join(ROOT, "compressed_sparse_attention_csa_amd", "csrc", source)
    try:
        with open(path) as f:
            rec = json.load(f)
        with open(src, "rb") as f:
            h = hashlib.sha256(f.read()).hexdigest()
        if rec.get("source_sha256") != h:
            return None, None
        return rec.get("bytes_per_launch"), rec.get("scope")
    except (OSError, ValueError):
        return None, None


def cpu_baseline(seed, budget_s, dev):
    """The oracle, as it stands, on the headline step's own seeded inputs:
    sequence 0's indexer keys and layer K/V come from the same seeded raw rows
    the GPU cache is built from (generated on the device by the same
    counter-based generator, then compressed and stored by the oracle in
    float64), and its query inputs are the step's. One oracle decode_step
    (indexer scores over 262,144 fp8 keys, Top-1024, 4 layer attends of 64
    heads over 1,024 gathered entries + 128 window rows) is repeated for
    `budget_s` seconds. Preparing the oracle's cache is not timed. Layers 1-3
    hold only the entries the step selects (the only ones it reads)."""
    import numpy as np
    import threadpoolctl
    import torch
    from compressed_sparse_attention_csa_amd import synth as Sy
    from oracle import csa_oracle as O

    def rows(kind, layer, r0, n):
        x = Sy.normal_rows(seed, Sy.stream_id(kind, layer, 0), r0, n, 128, dev, torch.bfloat16)
        return x.float().cpu().double().numpy()

    E, t = CONTEXT // RATIO, CONTEXT - 1
    P = Sy.proj_matrix(seed, 128, 64).double().numpy()
    kb = np.empty((E, 128))
    vb = np.empty((E, 128))
    ki = np.empty((E, 64))
    step = 1 << 18
    t_prep = time.perf_counter()
    for r0 in range(0, CONTEXT, step):
        a, b, c = O.compress(rows(Sy.KIND_K, 0, r0, step), rows(Sy.KIND_V, 0, r0, step),
                             rows(Sy.KIND_Z, 0, r0, step), RATIO, P)
        kb[r0 // RATIO:(r0 + step) // RATIO], vb[r0 // RATIO:(r0 + step) // RATIO] = a, b
        ki[r0 // RATIO:(r0 + step) // RATIO] = c
    kis = O.store(ki, "fp8")[0]
    qi = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_QI), 0, BATCH * IDX_HEADS, 64, dev,
                        torch.bfloat16).float().cpu().double().numpy()[:IDX_HEADS]
    w = Sy.uniform_rows(seed, Sy.stream_id(Sy.KIND_W), 0, BATCH, IDX_HEADS, dev).cpu().double().numpy()[0]
    T = O.topk(O.index_scores(qi, w, kis), TOPK)
    layers = []
    for layer in range(LAYERS):
        q = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_Q, layer), 0, BATCH * HEADS, 128, dev,
                           torch.bfloat16).float().cpu().double().numpy()[:HEADS]
        if layer == 0:
            kbl, vbl = O.store(kb, "fp8")[0], O.store(vb, "fp8")[0]
        else:
            # only the pages holding selected entries (a page's scale is its
            # amax, so each is compressed and stored whole)
            kbl, vbl = np.zeros((E, 128)), np.zeros((E, 128))
            sel = np.unique(T // 64)
            for r0 in range(0, CONTEXT, step):
                ps = sel[(sel >= r0 // (64 * RATIO)) & (sel < (r0 + step) // (64 * RATIO))]
                if not len(ps):
                    continue
                idx = torch.from_numpy((ps[:, None] * 64 * RATIO - r0 + np.arange(64 * RATIO)).reshape(-1)).to(dev)
                K, V, Z = (Sy.normal_rows(seed, Sy.stream_id(kind, layer, 0), r0, step, 128, dev, torch.bfloat16)
                           .index_select(0, idx).float().cpu().double().numpy()
                           for kind in (Sy.KIND_K, Sy.KIND_V, Sy.KIND_Z))
                a, b, _ = O.compress(K, V, Z, RATIO)
                ents = (ps[:, None] * 64 + np.arange(64)).reshape(-1)
                kbl[ents], vbl[ents] = O.store(a, "fp8")[0], O.store(b, "fp8")[0]
        rawk, rawv = np.zeros((CONTEXT, 128)), np.zeros((CONTEXT, 128))
        rawk[t - WINDOW + 1:] = rows(Sy.KIND_K, layer, t - WINDOW + 1, WINDOW)
        rawv[t - WINDOW + 1:] = rows(Sy.KIND_V, layer, t - WINDOW + 1, WINDOW)
        layers.append(dict(q=q, W=WINDOW, scale=1 / math.sqrt(128), kbar=kbl, vbar=vbl, rawk=rawk, rawv=rawv))
    prep_s = time.perf_counter() - t_prep
    n, t0 = 0, time.perf_counter()
    while True:
        To, _ = O.decode_step(qi, w, kis, RATIO, TOPK, t, layers)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s and n >= 3:
            break
    assert np.array_equal(To, T)
    threads = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] + [1])
    return {"value": round(n / el, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{n} repetitions of sequence 0's decode step on the workload's own seeded inputs "
                      f"(oracle decode_step: scores over {E:,} fp8 indexer keys, Top-{TOPK}, {LAYERS} attends of "
                      f"{HEADS} heads over {TOPK}+{WINDOW} keys) in {el:.1f} s, float64 NumPy; cores = BLAS "
                      f"threads; preparing the oracle's cache took {prep_s:.1f} s (not timed)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested); the library has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from compressed_sparse_attention_csa_amd import binding as B
    from compressed_sparse_attention_csa_amd import synth as Sy

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B.lib()
    only = "prefill" if args.prefill_only else args.only
    if only:
        legs = {"c1": lambda: c1_leg(args.seed, dev, args.replicas, args.steps),
                "c2": lambda: c2_leg(args.seed, dev, args.replicas, args.steps),
                "c5": lambda: c5_leg(args.seed, dev, args.replicas, args.steps),
                "prefill": lambda: prefill_leg(args.seed, dev),
                "hca": lambda: hca_leg(args.seed, dev)}
        print(json.dumps(legs[only]()), flush=True)
        return
    t_build = time.time()
    caches = build_cache(args.seed, args.replicas, dev)
    print(f"[bench] cache built: {len(caches)} replicas in {time.time() - t_build:.1f} s", file=sys.stderr, flush=True)

    # per-step inputs, resident in HBM
    q_seq = list(range(BATCH))
    q_pos = [CONTEXT - 1] * BATCH
    qi = Sy.normal_rows(args.seed, Sy.stream_id(Sy.KIND_QI), 0, BATCH * IDX_HEADS, 64, dev, torch.bfloat16).view(BATCH, IDX_HEADS, 64)
    w = Sy.uniform_rows(args.seed, Sy.stream_id(Sy.KIND_W), 0, BATCH, IDX_HEADS, dev)
    qs = [Sy.normal_rows(args.seed, Sy.stream_id(Sy.KIND_Q, l), 0, BATCH * HEADS, 128, dev, torch.bfloat16).view(BATCH, HEADS, 128)
          for l in range(LAYERS)]
    topk = [torch.empty((BATCH, TOPK), dtype=torch.int32, device=dev) for _ in caches]
    outs = [torch.empty((BATCH, HEADS, 128), dtype=torch.bfloat16, device=dev) for _ in range(LAYERS)]
    scale = 1.0 / math.sqrt(128)
    def step(i):
        c = caches[i % len(caches)]
        T = topk[i % len(caches)]
        stream = torch.cuda.current_stream()
        B.csa_index_topk(c.handle, q_seq, q_pos, qi, w, TOPK, T, stream)
        for l in range(LAYERS):
            B.csa_attend(c.handle, l, q_seq, q_pos, qs[l], T, TOPK, scale, outs[l], stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # The step's kernels are launched by HIP graph replay, so host-side launch
    # cost does not enter the timed region. One graph holds a step on every
    # replica, in the way a model's decode iteration captures several layer
    # groups in one graph; single-step graphs per replica cover a remainder.
    def enqueue(r, s_):
        c = caches[r]
        B.csa_index_topk(c.handle, q_seq, q_pos, qi, w, TOPK, topk[r], s_)
        for l in range(LAYERS):
            B.csa_attend(c.handle, l, q_seq, q_pos, qs[l], topk[r], TOPK, scale, outs[l], s_)
    cap = torch.cuda.Stream()
    g_all = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_all, stream=cap):
        for r in range(len(caches)):
            enqueue(r, torch.cuda.current_stream())
    graphs = []
    for r in range(len(caches)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            enqueue(r, torch.cuda.current_stream())
        graphs.append(g)

    def run_steps(n):
        for _ in range(n // len(caches)):
            g_all.replay()
        for i in range(n % len(caches)):
            graphs[i].replay()
    run_steps(args.warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(args.steps)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # kernel timing: eager steps, a HIP event pair stamped by every scan and
    # every attention launch
    for c in caches:
        B.csa_profile_begin(c.handle, B.PROFILE_INDEX | B.PROFILE_ATTEND)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    scan_ms, launches, att_ms, att_launches = 0.0, 0, 0.0, 0
    for c in caches:
        ms, n = B.csa_profile_end(c.handle, B.PROFILE_INDEX)
        scan_ms += ms
        launches += n
        ms, n = B.csa_profile_end(c.handle, B.PROFILE_ATTEND)
        att_ms += ms
        att_launches += n
    flags = max(c.read_errors() for c in caches)
    if flags:
        raise RuntimeError(f"device error flags {flags}")

    if args.calib_copy:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = BATCH * args.steps / elapsed
    scan_avg_ms = scan_ms / max(1, launches)
    sb = scan_bytes_per_launch()
    achieved = sb / (scan_avg_ms * 1e-3) / 1e9
    traffic, traffic_scope = traffic_from_profiles()
    att_avg_ms = att_ms / max(1, att_launches)
    ab = attend_bytes_per_launch()
    att_achieved = ab / (att_avg_ms * 1e-3) / 1e9
    att_traffic, att_scope = traffic_from_profiles("attend_decode_1m_traffic.json", "attend.hip")
    # the same number of bytes read by a plain 16-byte non-temporal streaming
    # kernel over 8 rotating buffers: what one launch of this size gets here
    ref_bufs = [torch.empty(sb, dtype=torch.uint8, device=dev) for _ in range(8)]
    B.csa_debug_stream_read(ref_bufs, sb, 8)
    ref_us = B.csa_debug_stream_read(ref_bufs, sb, 80)
    del ref_bufs
    ref_gbps = sb / (ref_us * 1e-6) / 1e9
    scan_rec = {"bound": "hbm", "kernel": "idx_scan (indexer scores over the fp8 indexer-key pages)",
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic, "traffic_scope": traffic_scope,
                "bytes_per_launch": sb, "avg_launch_us": round(scan_avg_ms * 1e3, 3), "launches": launches,
                "launches_per_step": 1}
    att_rec = {"bound": "hbm", "kernel": "attend_decode (gathered Top-K + window attention, one layer, 4 queries)",
               "achieved": round(att_achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
               "frac": round(att_achieved / HBM_PEAK_GBPS, 4), "traffic": att_traffic, "traffic_scope": att_scope,
               "bytes_per_launch": ab, "avg_launch_us": round(att_avg_ms * 1e3, 3), "launches": att_launches,
               "launches_per_step": LAYERS}
    # the roofline line is the kernel that takes most of a step's time
    scan_step_us, att_step_us = scan_avg_ms * 1e3, att_avg_ms * 1e3 * LAYERS
    dominant, other = (att_rec, scan_rec) if att_step_us >= scan_step_us else (scan_rec, att_rec)
    step_gbps = step_bytes() / (ms_per_step * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode, batch 4, 1,048,576-token context, fp8 cache (fp32 scale per 64-entry page), "
                               "r=4, Top-1024, W=128, 64 query heads, 4-layer index reuse",
                   "batch": BATCH, "context": CONTEXT, "ratio": RATIO, "k": TOPK, "window": WINDOW,
                   "q_heads": HEADS, "idx_heads": IDX_HEADS, "group_layers": LAYERS, "kv_dtype": "fp8_e4m3",
                   "replicas": len(caches), "parallelism": "none (1 GPU)"},
        "roofline": dominant,
        "step_roofline": {"bound": "hbm", "achieved": round(step_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                          "frac": round(step_gbps / HBM_PEAK_GBPS, 4), "bytes_per_step": step_bytes(),
                          "scope": "algorithmic bytes of the whole step over its graph-replay time"},
        "scan_roofline" if other is scan_rec else "attend_roofline": other,
        "read_ceiling": {"kernel": "streaming read, 16-byte non-temporal loads, 8 rotating buffers",
                         "bytes": sb, "avg_launch_us": round(ref_us, 3), "achieved": round(ref_gbps, 1),
                         "unit": "GB/s", "scan_frac": round(achieved / ref_gbps, 4)},
    }
    if not args.no_hier:
        line["hierarchical"] = hier_leg(caches, qi, w, max(10, args.steps // 4), args.seed)
    del caches, graphs, g_all
    torch.cuda.empty_cache()
    if not args.no_swa_fp8:
        line["swa_fp8"] = variant_leg(args.seed, dev, args.replicas, qi, w, qs, args.steps, kv="fp8", swa="fp8")
        torch.cuda.empty_cache()
    if not args.no_fp4:
        line["fp4_kv"] = variant_leg(args.seed, dev, args.replicas, qi, w, qs, args.steps, kv="fp4")
        torch.cuda.empty_cache()
    if not args.no_c2:
        line["c2_batch32_64k"] = c2_leg(args.seed, dev, args.replicas, args.steps)
        torch.cuda.empty_cache()
    if not args.no_c5:
        line["c5_serving_64"] = c5_leg(args.seed, dev, args.replicas, args.steps)
        torch.cuda.empty_cache()
    if not args.no_c1:
        line["c1_batch1_4k_fp32"] = c1_leg(args.seed, dev, args.replicas, args.steps)
    if not args.no_prefill:
        line["prefill"] = prefill_leg(args.seed, dev)
    if not args.no_hca:
        line["hca"] = hca_leg(args.seed, dev)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(args.seed, args.cpu_seconds, dev)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
