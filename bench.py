"""Benchmark of the GQA/MQA attention hot path on one MI355X.

Headline (the JSON line's `value`): single-token GQA decode over a bf16 KV
cache at 32K context, in GB/s of algorithmic KV bytes (sum over the batch of
seq_len x n_kv_head x head_dim x 2 bytes x 2 for K and V) per second.  A step
is one whole decode (per-piece partial softmax states, then their merge) for
the whole batch; inputs are resident in HBM before timing starts and two
independent caches alternate so the 256 MB Infinity Cache cannot serve them.

The same run also measures the other hot-path entry points (decode at 4K,
with Dynamic NTK, with the cache write, over a window, a rolling buffer
(also with a shorter window) and StreamingLLM sinks; causal prefill at 8K
on the matrix cores, also with its fp16-score option, a window and sinks;
top-k sparse decode at 128K, the weighted indexer, QSA, dense MLA and
rope_apply) and times the CPU fp64
oracle on a bounded sample of the headline workload.  All data is synthetic
and seeded.

    python bench.py [--steps K] [--warmup W] [--no-cpu] [--gpus 1]
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GQA decode KV GB/s (% of HBM peak) at 32K ctx; causal prefill TFLOP/s"
HBM_PEAK_GBS = 8000.0          # MI355X published HBM3E bandwidth
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16/fp16 matrix peak
PROFILE_DIR = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", default="", help="comma list of sections (decode32k,decode4k,dynamic,append32k,window,"
                    "sinks,mla,prefill,prefill_fp16,prefill_window,sparse,sparse_weighted,qsa,rope) "
                    "for profiling runs")
    return ap.parse_args()


def precondition(fn, seconds=0.03):
    """Untimed calls of fn for `seconds` of wall time, before the warmup calls.
    An idle or fresh GPU reaches its steady clock only after some
    milliseconds of load: measured on the 32K decode, 20 steps right after
    2 s idle average 270-272 us, later ones 260 us.  A serving loop runs at
    the steady state, so each timed region is preceded by this."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        fn(i)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def timed_loop(fn, steps, warmup):
    """Precondition, run warmup calls, then time exactly `steps` calls
    bracketed by device syncs."""
    import torch
    precondition(fn)
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fn(i)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def region_ms(fn, steps, warmup):
    """Mean GPU time per call of `steps` back-to-back calls of fn on the
    current stream, from one HIP event pair around the whole region (events
    between the calls would add their own packets to what is measured),
    after preconditioning and the warmup calls."""
    import torch
    precondition(fn)
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "mqa_kv_cache_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(profile_name, src_hash):
    """HBM bytes per dispatch recorded from rocprofv3 PMC counters in
    profiles/<profile_name>, or None when absent or taken on other sources."""
    path = os.path.join(PROFILE_DIR, profile_name)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path, encoding="utf-8") as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_sha256_16") != src_hash:
        return None
    try:
        return float(vals["traffic_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------
# sections
# ---------------------------------------------------------------------------

def bench_decode(cfg, steps, warmup, nsets, label):
    import torch

    import mqa_kv_cache_amd as m
    from workloads import device_randn_bf16
    B, Hq, Hkv, D, S = cfg.B, cfg.Hq, cfg.Hkv, cfg.D, cfg.S_max
    lens = torch.from_numpy(cfg.seq_lens()).cuda()
    sets = [(device_randn_bf16((B, Hq, D), cfg.seed * 100 + 10 * i + 1),
             device_randn_bf16((B, Hkv, S, D), cfg.seed * 100 + 10 * i + 2),
             device_randn_bf16((B, Hkv, S, D), cfg.seed * 100 + 10 * i + 3)) for i in range(nsets)]
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(m.gqa_decode_workspace_size(B, Hq, Hkv, D, S), dtype=torch.uint8, device="cuda")
    kv_bytes = int(lens.sum().item()) * Hkv * D * 2 * 2
    rope = cfg.rope()

    def partial(i):
        q, k, v = sets[i % nsets]
        m.gqa_decode_partial(q, k, v, lens, cfg.scale, ws, q_rope=rope)

    def step(i):
        partial(i)
        m.gqa_decode_combine(lens, B, Hq, Hkv, D, S, ws, out)

    # whole steps (partial + combine), nothing else on the stream
    ms = timed_loop(step, steps, warmup)
    # the partial kernel alone, the same launches back to back
    kern_ms = region_ms(partial, steps, warmup)
    log(f"[bench] {label}: step {ms * 1e3:.1f} us, partial kernel {kern_ms * 1e3:.1f} us, "
        f"{kv_bytes / ms / 1e6:.0f} GB/s")
    return dict(ms=ms, kern_ms=kern_ms, kv_bytes=kv_bytes, lens=lens.cpu().numpy(), sets=sets)


def bench_decode_append(cfg, steps, warmup, nsets=2):
    """The decode step with its cache write (gqa_decode_append): the new
    token's rotated key and value go into row seq_lens[b]-1, then it attends."""
    import torch

    import mqa_kv_cache_amd as m
    from workloads import device_randn_bf16
    B, Hq, Hkv, D, S = cfg.B, cfg.Hq, cfg.Hkv, cfg.D, cfg.S_max
    lens = torch.from_numpy(cfg.seq_lens()).cuda()
    sets = [(device_randn_bf16((B, Hq, D), cfg.seed * 100 + 10 * i + 1),
             device_randn_bf16((B, Hkv, S, D), cfg.seed * 100 + 10 * i + 2),
             device_randn_bf16((B, Hkv, S, D), cfg.seed * 100 + 10 * i + 3),
             device_randn_bf16((B, Hkv, D), cfg.seed * 100 + 10 * i + 4),
             device_randn_bf16((B, Hkv, D), cfg.seed * 100 + 10 * i + 5)) for i in range(nsets)]
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(m.gqa_decode_workspace_size(B, Hq, Hkv, D, S), dtype=torch.uint8, device="cuda")
    kv_bytes = int(lens.sum().item()) * Hkv * D * 2 * 2
    rope = cfg.rope()

    def step(i):
        q, k, v, kn, vn = sets[i % nsets]
        m.gqa_decode_append(q, kn, vn, k, v, lens, cfg.scale, q_rope=rope, out=out, workspace=ws)

    ms = timed_loop(step, steps, warmup)
    log(f"[bench] decode+append 32K: step {ms * 1e3:.1f} us, {kv_bytes / ms / 1e6:.0f} GB/s")
    del sets
    torch.cuda.empty_cache()
    return dict(ms=ms, kv_bytes=kv_bytes)


def bench_decode_window(cfg, steps, warmup, window, rolling, nsets=4, sinks=0, buffer=0):
    """gqa_decode_window on the 32K workload's batch, q heads and lengths: a
    `window`-token sliding window over the linear cache, or a rolling buffer
    of `window` slots (contexts longer than the buffer), or of `buffer` slots
    with the `window`-token window (its slots wrap around the buffer's end
    for some contexts); with `sinks` > 0 (gqa_decode_sink_window) the first
    positions stay visible as well."""
    import torch

    import mqa_kv_cache_amd as m
    from workloads import device_randn_bf16
    B, Hq, Hkv, D = cfg.B, cfg.Hq, cfg.Hkv, cfg.D
    S = (buffer or window) if rolling else cfg.S_max
    lens_np = cfg.seq_lens()
    lens = torch.from_numpy(lens_np).cuda()
    sets = [(device_randn_bf16((B, Hq, D), cfg.seed * 100 + 10 * i + 1),
             device_randn_bf16((B, Hkv, S, D), cfg.seed * 100 + 10 * i + 2),
             device_randn_bf16((B, Hkv, S, D), cfg.seed * 100 + 10 * i + 3)) for i in range(nsets)]
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(m.gqa_decode_workspace_size(B, Hq, Hkv, D, S), dtype=torch.uint8, device="cuda")
    if rolling:
        rows = int(sum(min(int(L), window) for L in lens_np))
    else:
        rows = int(sum(min(int(L), window) + min(sinks, max(0, int(L) - window)) for L in lens_np))
    kv_bytes = rows * Hkv * D * 2 * 2
    rope = cfg.rope()

    def step(i):
        q, k, v = sets[i % nsets]
        m.gqa_decode_window(q, k, v, lens, cfg.scale, window=window if not rolling or buffer else 0,
                            rolling=rolling, q_rope=rope, out=out, workspace=ws, sinks=sinks)

    ms = timed_loop(step, steps, warmup)
    label = (f"sink{sinks}_" if sinks else "") + (
        f"rolling{buffer}_window{window}" if rolling and buffer else
        f"rolling{window}" if rolling else f"window{window}")
    log(f"[bench] decode {label} (32K contexts): step {ms * 1e3:.1f} us, {kv_bytes / ms / 1e6:.0f} GB/s")
    del sets
    torch.cuda.empty_cache()
    return dict(ms=ms, kv_bytes=kv_bytes, label=label)


def bench_prefill(cfg, steps, warmup, fp16_scores=False):
    """gqa_prefill_causal on the 8K workload (scores from hi + lo operands,
    three products: the matrix cores do 2x the algorithmic flops), or with
    fp16_scores the one-product gqa_prefill_fp16."""
    import torch

    import mqa_kv_cache_amd as m
    from workloads import device_randn_bf16
    B, T, Hq, Hkv, D = cfg.B, cfg.T, cfg.Hq, cfg.Hkv, cfg.D
    q = device_randn_bf16((B, Hq, T, D), cfg.seed * 100 + 1)
    k = device_randn_bf16((B, Hkv, T, D), cfg.seed * 100 + 2)
    v = device_randn_bf16((B, Hkv, T, D), cfg.seed * 100 + 3)
    out = torch.empty_like(q)
    ws = torch.empty(m.gqa_prefill_workspace_size(B, Hkv, T, D, cfg.rope()), dtype=torch.uint8,
                     device="cuda")
    flops = 2 * D * Hq * T * (T + 1) * B       # QK^T and PV over the causal triangle incl. diagonal

    def step(i):
        m.gqa_prefill_causal(q, k, v, cfg.scale, rope=cfg.rope(), out=out, workspace=ws,
                             fp16_scores=fp16_scores)

    ev_ms = region_ms(step, max(steps // 2, 5), max(warmup // 2, 2))
    tf = flops / ev_ms / 1e9
    log(f"[bench] prefill T={T}{' fp16 scores' if fp16_scores else ''}: {ev_ms * 1e3:.1f} us per "
        f"call, {tf:.1f} TFLOP/s")
    return dict(ev_ms=ev_ms, flops=flops, tflops=tf, mfma_work=1.0 if fp16_scores else 2.0)


def bench_prefill_window(cfg, steps, warmup, window=4096, sinks=0):
    """gqa_prefill_window on the 8K prefill with a `window`-token band (and
    `sinks` sink tokens beside it: gqa_prefill_sink_window)."""
    import torch

    import mqa_kv_cache_amd as m
    from workloads import device_randn_bf16
    B, T, Hq, Hkv, D = cfg.B, cfg.T, cfg.Hq, cfg.Hkv, cfg.D
    q = device_randn_bf16((B, Hq, T, D), cfg.seed * 100 + 1)
    k = device_randn_bf16((B, Hkv, T, D), cfg.seed * 100 + 2)
    v = device_randn_bf16((B, Hkv, T, D), cfg.seed * 100 + 3)
    out = torch.empty_like(q)
    ws = torch.empty(m.gqa_prefill_workspace_size(B, Hkv, T, D, cfg.rope()), dtype=torch.uint8,
                     device="cuda")
    # visible (query, key) pairs per head: the band plus the sinks below it
    pairs = sum(min(i + 1, window) + min(sinks, max(0, i + 1 - window)) for i in range(T))
    flops = 4 * D * Hq * pairs * B                          # QK^T and PV, 2 flops per product

    def step(i):
        m.gqa_prefill_causal(q, k, v, cfg.scale, rope=cfg.rope(), out=out, workspace=ws,
                             window=window, sinks=sinks)

    ev_ms = region_ms(step, max(steps // 2, 5), max(warmup // 2, 2))
    tf = flops / ev_ms / 1e9
    label = (f"sink{sinks}_" if sinks else "") + f"window{window}"
    log(f"[bench] prefill T={T} {label}: {ev_ms * 1e3:.1f} us per call, {tf:.1f} TFLOP/s")
    return dict(ev_ms=ev_ms, flops=flops, tflops=tf, label=label)


def bench_sparse(cfg, steps, warmup):
    import torch

    import mqa_kv_cache_amd as m
    from workloads import device_randn_bf16
    B, H, S, k = cfg.B, cfg.H, cfg.S_max, cfg.top_k
    # eight input sets rotate (~1.1 GB of indexer keys and gathered rows
    # between two uses of a set), so the 256 MB Infinity Cache cannot serve
    # the set that comes round again
    nsets = 8
    sets = [(device_randn_bf16((B, H, cfg.Dqk), cfg.seed * 100 + 10 * i + 1),
             device_randn_bf16((B, S, cfg.Dqk), cfg.seed * 100 + 10 * i + 2),
             device_randn_bf16((B, cfg.D_idx), cfg.seed * 100 + 10 * i + 3),
             device_randn_bf16((B, S, cfg.D_idx), cfg.seed * 100 + 10 * i + 4)) for i in range(nsets)]
    lens = torch.from_numpy(cfg.seq_lens()).cuda()
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    out = torch.empty((B, H, cfg.Dv), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(m.topk_sparse_decode_workspace_size(B, H, S, k), dtype=torch.uint8, device="cuda")
    # algorithmic bytes: indexer keys + selected latent rows + q, q_index, outputs
    alg = (B * S * cfg.D_idx * 2 + B * k * cfg.Dqk * 2 + B * H * cfg.Dqk * 2 + B * cfg.D_idx * 2
           + B * k * 4 + B * H * cfg.Dv * 2)

    def step(i):
        q, lat, qi, ki = sets[i % nsets]
        m.topk_sparse_decode(q, lat, qi, ki, lens, k, cfg.scale, topk_idx=idx, out=out, workspace=ws)

    ev_ms = region_ms(step, steps, warmup)
    log(f"[bench] sparse: {ev_ms * 1e3:.1f} us per call, {alg / ev_ms / 1e6:.0f} GB/s algorithmic")
    return dict(ms=ev_ms, alg_bytes=alg, gbs=alg / ev_ms / 1e6)


def bench_sparse_weighted(cfg, steps, warmup, H_I=64):
    """topk_sparse_decode_weighted: the 64-head weighted indexer on the matrix
    cores, then the same top-k and attention."""
    import numpy as np
    import torch

    import mqa_kv_cache_amd as m
    from workloads import device_randn_bf16
    B, H, S, k = cfg.B, cfg.H, cfg.S_max, cfg.top_k
    nsets = 8
    sets = [(device_randn_bf16((B, H, cfg.Dqk), cfg.seed * 100 + 10 * i + 1),
             device_randn_bf16((B, S, cfg.Dqk), cfg.seed * 100 + 10 * i + 2),
             device_randn_bf16((B, H_I, cfg.D_idx), cfg.seed * 100 + 10 * i + 3),
             device_randn_bf16((B, S, cfg.D_idx), cfg.seed * 100 + 10 * i + 4)) for i in range(nsets)]
    w = torch.from_numpy((np.random.default_rng(cfg.seed).standard_normal((B, H_I)) / 8)
                         .astype(np.float32)).cuda()
    lens = torch.from_numpy(cfg.seq_lens()).cuda()
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    out = torch.empty((B, H, cfg.Dv), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(m.topk_sparse_decode_workspace_size(B, H, S, k), dtype=torch.uint8, device="cuda")
    alg = (B * S * cfg.D_idx * 2 + B * k * cfg.Dqk * 2 + B * H * cfg.Dqk * 2 + B * H_I * cfg.D_idx * 2
           + B * k * 4 + B * H * cfg.Dv * 2)

    def step(i):
        q, lat, qi, ki = sets[i % nsets]
        m.topk_sparse_decode_weighted(q, lat, qi, w, ki, lens, k, cfg.scale, topk_idx=idx, out=out,
                                      workspace=ws)

    ev_ms = region_ms(step, steps, warmup)
    log(f"[bench] sparse weighted (H_I={H_I}): {ev_ms * 1e3:.1f} us per call, {alg / ev_ms / 1e6:.0f} GB/s algorithmic")
    return dict(ms=ev_ms, alg_bytes=alg, gbs=alg / ev_ms / 1e6)


def bench_qsa(cfg, steps, warmup):
    """qsa_sparse_decode: micro-block indexer over the 128K context, top 512
    blocks plus the tail, sparse GQA over the <= 2051 tokens."""
    import torch

    import mqa_kv_cache_amd as m
    from workloads import device_randn_bf16
    B, Hq, Hkv, D, S = cfg.B, cfg.Hq, cfg.Hkv, cfg.D, cfg.S_max
    nsets = 2   # 1.2 GB of caches and indexer keys per set
    sets = [(device_randn_bf16((B, Hq, D), cfg.seed * 100 + 10 * i + 1),
             device_randn_bf16((B, Hkv, S, D), cfg.seed * 100 + 10 * i + 2),
             device_randn_bf16((B, Hkv, S, D), cfg.seed * 100 + 10 * i + 3),
             device_randn_bf16((B, cfg.H_I, cfg.D_idx), cfg.seed * 100 + 10 * i + 4),
             device_randn_bf16((B, S, cfg.D_idx), cfg.seed * 100 + 10 * i + 5)) for i in range(nsets)]
    lens = torch.from_numpy(cfg.seq_lens()).cuda()
    tok = torch.empty((B, m.QSA_TOKENS), dtype=torch.int32, device="cuda")
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(m.qsa_sparse_decode_workspace_size(B, Hq, S), dtype=torch.uint8, device="cuda")
    rope = cfg.block_rope()
    n_tok = min(512, S // 4) * 4 + S % 4
    alg = (B * S * cfg.D_idx * 2 + B * Hkv * n_tok * D * 2 * 2 + B * Hq * D * 2 * 2
           + B * cfg.H_I * cfg.D_idx * 2 + B * m.QSA_TOKENS * 4)

    def step(i):
        q, kc, vc, qi, ki = sets[i % nsets]
        m.qsa_sparse_decode(q, kc, vc, qi, ki, lens, cfg.scale, block_rope=rope, token_idx=tok,
                            out=out, workspace=ws)

    ev_ms = region_ms(step, steps, warmup)
    log(f"[bench] qsa: {ev_ms * 1e3:.1f} us per call, {alg / ev_ms / 1e6:.0f} GB/s algorithmic")
    return dict(ms=ev_ms, alg_bytes=alg, gbs=alg / ev_ms / 1e6)


def bench_mla(cfg, steps, warmup):
    """Dense absorbed-MLA decode over the full latent cache (no selection)."""
    import torch

    import mqa_kv_cache_amd as m
    from workloads import device_randn_bf16
    B, H, S = cfg.B, cfg.H, cfg.S_max
    # two sets (604 MB of latent rows each) rotate past the 256 MB Infinity Cache
    nsets = 2
    sets = [(device_randn_bf16((B, H, cfg.Dqk), cfg.seed * 100 + 10 * i + 5),
             device_randn_bf16((B, S, cfg.Dqk), cfg.seed * 100 + 10 * i + 6)) for i in range(nsets)]
    lens = torch.from_numpy(cfg.seq_lens()).cuda()
    out = torch.empty((B, H, cfg.Dv), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(m.mla_decode_workspace_size(B, H, S), dtype=torch.uint8, device="cuda")
    rows = int(cfg.seq_lens().sum())
    alg = rows * cfg.Dqk * 2 + B * H * cfg.Dqk * 2 + B * H * cfg.Dv * 2
    flops = 2 * rows * H * (cfg.Dqk + cfg.Dv)

    def step(i):
        q, lat = sets[i % nsets]
        m.mla_decode(q, lat, lens, cfg.scale, out=out, workspace=ws)

    ev_ms = region_ms(step, steps, warmup)
    log(f"[bench] mla dense: {ev_ms * 1e3:.1f} us per call, {alg / ev_ms / 1e6:.0f} GB/s, "
        f"{flops / ev_ms / 1e9:.0f} TFLOP/s")
    return dict(ms=ev_ms, alg_bytes=alg, flops=flops, gbs=alg / ev_ms / 1e6,
                tflops=flops / ev_ms / 1e9)


def bench_rope(cfg, steps, warmup):
    import torch

    import mqa_kv_cache_amd as m
    from workloads import device_randn_bf16
    T, Hq, D = cfg.T, cfg.Hq, cfg.D
    # four (input, output) pairs rotate (512 MiB) so the 256 MB Infinity Cache
    # cannot serve a pair that comes round again
    nsets = 4
    xs = [device_randn_bf16((T, Hq, D), 7 + i) for i in range(nsets)]
    ys = [torch.empty_like(xs[0]) for _ in range(nsets)]
    pos = torch.arange(T, dtype=torch.int32, device="cuda")
    byts = 2 * T * Hq * D * 2

    def step(i):
        m.rope_apply(xs[i % nsets], pos, cfg.rope(), out=ys[i % nsets])

    ev_ms = region_ms(step, steps, warmup)
    log(f"[bench] rope_apply: {ev_ms * 1e3:.1f} us, {byts / ev_ms / 1e6:.0f} GB/s")
    return dict(ms=ev_ms, gbs=byts / ev_ms / 1e6)


def cpu_baseline(cfg, dec, budget_s=12.0):
    """The fp64 oracle on the host cores, on a bounded sample of the headline
    workload: whole sequences (every q head) of the headline batch, taken in
    order until about `budget_s` seconds of oracle time.  Inputs are copied to
    host float64 beforehand; only the oracle calls are timed."""
    from oracle import attention as oatt
    from workloads import bf16_tensor_to_f64
    q, k, v = dec["sets"][0]
    lens = dec["lens"]
    Hq, Hkv, D = cfg.Hq, cfg.Hkv, cfg.D
    g = Hq // Hkv
    wall = cpu = 0.0
    rows = nb = 0
    for b in range(cfg.B):
        L = int(lens[b])
        qf = bf16_tensor_to_f64(q[b])
        kvs = [(bf16_tensor_to_f64(k[b, kv, :L]), bf16_tensor_to_f64(v[b, kv, :L])) for kv in range(Hkv)]
        c0, t0 = time.process_time(), time.perf_counter()
        for kv, (kb, vb) in enumerate(kvs):
            for hl in range(g):
                oatt.decode_one(qf[kv * g + hl], kb, vb, L, cfg.scale, cfg.rope())
        wall += time.perf_counter() - t0
        cpu += time.process_time() - c0
        rows += L
        nb += 1
        del kvs
        if wall >= budget_s:
            break
    sample_bytes = rows * Hkv * D * 2 * 2
    return {"value": round(sample_bytes / wall / 1e9, 3), "unit": "GB/s",
            "cores": max(1, round(cpu / wall)), "kind": "oracle",
            "sample": f"all {Hq} q heads of the first {nb} of {cfg.B} sequences of the headline "
                      f"batch ({rows} context rows, {sample_bytes} KV bytes), numpy float64 oracle; "
                      f"{wall:.1f} s wall, {cpu:.1f} s CPU; os.cpu_count()={os.cpu_count()}"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    import mqa_kv_cache_amd as m  # noqa: F401  (fails loudly without the HIP library)
    from workloads import DECODE_4K, DECODE_32K_YARN, PREFILL_8K, QSA_128K, SPARSE_128K
    torch.cuda.set_device(0)
    only = set(s for s in args.only.split(",") if s)
    want = (lambda s: not only or s in only)
    K, W = args.steps, args.warmup

    res = {}
    if want("decode32k"):
        res["d32"] = bench_decode(DECODE_32K_YARN, K, W, nsets=2, label="decode 32K")
    if want("decode4k"):
        res["d4"] = bench_decode(DECODE_4K, K, W, nsets=4, label="decode 4K")
    if want("dynamic"):
        res["dd"] = bench_decode(dataclasses.replace(DECODE_32K_YARN, rope_kind="dynamic_ntk"), K, W,
                                 nsets=2, label="decode 32K dynamic NTK")
    if want("append32k"):
        res["da"] = bench_decode_append(DECODE_32K_YARN, K, W)
    if want("window"):
        res["dw"] = bench_decode_window(DECODE_32K_YARN, K, W, 4096, False)
        res["dr"] = bench_decode_window(DECODE_32K_YARN, K, W, 4096, True)
        res["drw"] = bench_decode_window(DECODE_32K_YARN, K, W, 4096, True, buffer=8192)
    if want("sinks"):
        res["ds"] = bench_decode_window(DECODE_32K_YARN, K, W, 4096, False, sinks=4)
    if want("prefill"):
        res["p"] = bench_prefill(PREFILL_8K, K, W)
    if want("prefill_fp16"):
        res["pf"] = bench_prefill(PREFILL_8K, K, W, fp16_scores=True)
    if want("prefill_window"):
        res["pw"] = bench_prefill_window(PREFILL_8K, K, W)
        res["pws"] = bench_prefill_window(PREFILL_8K, K, W, sinks=4)
    if want("sparse"):
        res["s"] = bench_sparse(SPARSE_128K, K, W)
    if want("sparse_weighted"):
        res["sw"] = bench_sparse_weighted(SPARSE_128K, K, W)
    if want("qsa"):
        res["qsa"] = bench_qsa(QSA_128K, K, W)
    if want("mla"):
        res["mla"] = bench_mla(SPARSE_128K, K, W)
    if want("rope"):
        res["r"] = bench_rope(PREFILL_8K, K, W)
    if only and "d32" not in res:
        return

    d = res["d32"]
    cfg = DECODE_32K_YARN
    value = d["kv_bytes"] / d["ms"] / 1e6
    achieved = d["kv_bytes"] / d["kern_ms"] / 1e6
    src = source_hash("decode.hip", "device_common.h")
    traffic = recorded_traffic("decode_split_kernel_decode32k_yarn.pmc.txt", src)
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(d["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"gqa_decode: B={cfg.B} sequences x 1 new token, Hq={cfg.Hq}, "
                         f"Hkv={cfg.Hkv}, D={cfg.D}, S_max={cfg.S_max}, seq_lens~U[{cfg.ragged_lo},"
                         f"{cfg.S_max}] (seed {cfg.seed}), YaRN s=4 on q, bf16 KV cache"),
            "global_batch": cfg.B,
            "seq_len": cfg.S_max,
            "parallelism": "single GPU",
        },
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_split_kernel<128,1>",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes": d["kv_bytes"],
            "kernel_ms": round(d["kern_ms"], 5),
            "source_sha256_16": src,
        },
    }
    if "d4" in res:
        d4 = res["d4"]
        line["decode_4k"] = {"GB/s": round(d4["kv_bytes"] / d4["ms"] / 1e6, 1),
                             "kernel_GB/s": round(d4["kv_bytes"] / d4["kern_ms"] / 1e6, 1),
                             "pct_of_hbm_peak": round(100 * d4["kv_bytes"] / d4["ms"] / 1e6 / HBM_PEAK_GBS, 2),
                             "ms_per_step": round(d4["ms"], 5)}
    if "dd" in res:
        dd = res["dd"]
        line["decode_dynamic_ntk_32k"] = {"GB/s": round(dd["kv_bytes"] / dd["ms"] / 1e6, 1),
                                          "pct_of_hbm_peak": round(100 * dd["kv_bytes"] / dd["ms"] / 1e6 / HBM_PEAK_GBS, 2),
                                          "ms_per_step": round(dd["ms"], 5)}
    if "da" in res:
        da = res["da"]
        line["decode_append_32k"] = {"GB/s": round(da["kv_bytes"] / da["ms"] / 1e6, 1),
                                     "pct_of_hbm_peak": round(100 * da["kv_bytes"] / da["ms"] / 1e6 / HBM_PEAK_GBS, 2),
                                     "ms_per_step": round(da["ms"], 5)}
    for key in ("dw", "dr", "drw", "ds"):
        if key in res:
            r = res[key]
            line[f"decode_{r['label']}_32k"] = {
                "GB/s": round(r["kv_bytes"] / r["ms"] / 1e6, 1),
                "pct_of_hbm_peak": round(100 * r["kv_bytes"] / r["ms"] / 1e6 / HBM_PEAK_GBS, 2),
                "ms_per_step": round(r["ms"], 5)}
    for key, name in (("p", "prefill_8k"), ("pf", "prefill_8k_fp16_scores")):
        if key in res:
            p = res[key]
            line[name] = {"TFLOP/s": round(p["tflops"], 1),
                          "pct_of_mfma_peak": round(100 * p["tflops"] / BF16_PEAK_TFLOPS, 2),
                          "ms_per_call": round(p["ev_ms"], 4), "flops": p["flops"],
                          "matrix_core_flops_per_flop": p["mfma_work"],
                          "bound": "mfma", "peak": BF16_PEAK_TFLOPS}
    for key in ("pw", "pws"):
        if key in res:
            pw = res[key]
            line[f"prefill_8k_{pw['label']}"] = {
                "TFLOP/s": round(pw["tflops"], 1),
                "pct_of_mfma_peak": round(100 * pw["tflops"] / BF16_PEAK_TFLOPS, 2),
                "ms_per_call": round(pw["ev_ms"], 4), "flops": pw["flops"]}
    if "s" in res:
        s = res["s"]
        line["sparse_128k"] = {"GB/s": round(s["gbs"], 1), "ms_per_call": round(s["ms"], 5),
                               "algorithmic_bytes": s["alg_bytes"],
                               "pct_of_hbm_peak": round(100 * s["gbs"] / HBM_PEAK_GBS, 2)}
    if "sw" in res:
        sw = res["sw"]
        line["sparse_weighted64_128k"] = {"GB/s": round(sw["gbs"], 1), "ms_per_call": round(sw["ms"], 5),
                                          "algorithmic_bytes": sw["alg_bytes"],
                                          "pct_of_hbm_peak": round(100 * sw["gbs"] / HBM_PEAK_GBS, 2)}
    if "qsa" in res:
        r = res["qsa"]
        line["qsa_128k"] = {"GB/s": round(r["gbs"], 1), "ms_per_call": round(r["ms"], 5),
                            "algorithmic_bytes": r["alg_bytes"],
                            "pct_of_hbm_peak": round(100 * r["gbs"] / HBM_PEAK_GBS, 2)}
    if "mla" in res:
        ml = res["mla"]
        line["mla_dense_128k"] = {"GB/s": round(ml["gbs"], 1), "TFLOP/s": round(ml["tflops"], 1),
                                  "pct_of_hbm_peak": round(100 * ml["gbs"] / HBM_PEAK_GBS, 2),
                                  "pct_of_mfma_peak": round(100 * ml["tflops"] / BF16_PEAK_TFLOPS, 2),
                                  "ms_per_call": round(ml["ms"], 5), "flops": ml["flops"],
                                  "algorithmic_bytes": ml["alg_bytes"]}
    if "r" in res:
        line["rope_apply"] = {"GB/s": round(res["r"]["gbs"], 1), "ms_per_call": round(res["r"]["ms"], 5)}
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(cfg, d)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
