"""Benchmark of the paged-attention hot path on one MI355X.

Headline workload (c4, Qwen3-8B-shaped decode): one step = paged decode
attention of 256 sequences (32 query / 8 KV heads, head_dim 128, bf16,
contexts uniform in [1024, 8192], a random half sharing one 1024-token
prefix) over 256-token blocks drawn from a shuffled pool, one launch
(pa_paged_attn_decode). Its 6 GB of pools are far larger than every cache,
so each step reads its K/V from HBM.

The timed region holds exactly --steps steps, bracketed by device
synchronisation, with no per-kernel events inside it; one HIP event pair on
the launch stream brackets it, and its average is the kernel's launch
duration for the roofline. Each workload is also timed as 30 reps, each after
a sweep that reads a 1 GiB buffer on the same stream (every cache line of the
previous rep evicted, the caches left clean), for the median, min and p90;
the headline also after a 1 GiB overwrite (caches left dirty).

Printed: one JSON line with the headline value (decode KV throughput in
TB/s), the roofline of its kernel, the fp64 CPU oracle timed on the host on a
bounded sample of the same workload (and of the prefill and verify
workloads, in GFLOP/s), and secondary measurements of the other workloads:
the Qwen3-0.6B-shaped decode step (store + decode, one launch, on rotating
pool copies, with its own roofline), chunked prefill, the RoPE store,
speculative verify, fp8 decode, decode-step graphs and the host block
manager.
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published (no sparsity)
METRIC = "paged-attn decode KV TB/s (% HBM peak); prefill TFLOP/s (% MFMA peak)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "decode": os.path.join(ROOT, "paged_kv_cache_209_amd", "csrc", "decode.hip"),
    "decode_store": os.path.join(ROOT, "paged_kv_cache_209_amd", "csrc", "decode.hip"),
    "prefill": os.path.join(ROOT, "paged_kv_cache_209_amd", "csrc", "prefill.hip"),
    "kv_store": os.path.join(ROOT, "paged_kv_cache_209_amd", "csrc", "kv_store.hip"),
    "rope_store": os.path.join(ROOT, "paged_kv_cache_209_amd", "csrc", "rope_store.hip"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(kernel: str) -> str:
    with open(KERNEL_SOURCES[kernel], "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    try:
        data = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    rec = data.get(f"{kernel}:{workload}")
    if not rec or rec.get("source_sha") != source_sha(kernel):
        return None
    return rec.get("bytes_per_launch")


def decode_bytes(case) -> dict:
    """Algorithmic bytes of one decode launch: every K/V row of every context
    once (shared prefix rows once), q and out, the block-table entries read,
    and the context lengths."""
    import workloads as w

    elt = case.q.element_size()
    hkv, d = case.num_kv_heads, case.head_dim
    ctx = case.context_lens.tolist()
    seen = set()
    unique_rows = 0
    for i, L in enumerate(ctx):
        for b in range(w.blocks_for(L)):
            blk = int(case.block_tables[i, b])
            rows = min(256, L - 256 * b)
            if blk in seen:
                continue  # a shared block (same id) is read from HBM once
            seen.add(blk)
            unique_rows += rows
    kv_row = hkv * d * elt * 2
    logical = sum(ctx) * kv_row
    qo = 2 * case.q.numel() * elt
    meta = sum(w.blocks_for(L) for L in ctx) * 4 + len(ctx) * 4
    return {"unique_kv": unique_rows * kv_row, "logical_kv": logical, "q_out": qo, "meta": meta,
            "total": unique_rows * kv_row + qo + meta}


def decode_flops(case) -> float:
    return 4.0 * case.head_dim * case.num_q_heads * float(case.context_lens.sum())


def prefill_flops(case) -> float:
    cu = case.cu_seqlens.tolist()
    tot = 0.0
    for i, L in enumerate(case.context_lens.tolist()):
        n = cu[i + 1] - cu[i]
        c = L - n
        tot += n * c + n * (n + 1) / 2
    return 4.0 * case.head_dim * case.num_q_heads * tot


def prefill_bytes(case) -> dict:
    import workloads as w

    elt = case.q.element_size()
    hkv, d = case.num_kv_heads, case.head_dim
    cu = case.cu_seqlens.tolist()
    seen = set()
    unique_rows = 0
    logical = 0
    for i, L in enumerate(case.context_lens.tolist()):
        c = L - (cu[i + 1] - cu[i])
        logical += c
        for b in range(w.blocks_for(c)):
            blk = int(case.block_tables[i, b])
            if blk in seen:
                continue
            seen.add(blk)
            unique_rows += min(256, c - 256 * b)
    kv_row = hkv * d * elt * 2
    new = case.total_q * (2 * case.num_q_heads + 2 * hkv) * d * elt  # q, out, k, v
    meta = (len(cu) + case.num_seqs) * 4
    return {"unique_kv": unique_rows * kv_row, "logical_kv": logical * kv_row, "new_tokens": new,
            "total": unique_rows * kv_row + new + meta}


class Timer:
    """Pairs of HIP events on the current stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.append([e, None])

    def stop(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs[-1][1] = e

    def ms(self):
        return [a.elapsed_time(b) for a, b in self.pairs]


def time_launches(torch, fn, count):
    """Average duration (ms) of `count` back-to-back calls of fn(i), bracketed
    by one HIP event pair on the current stream (the stream the library
    launches on). Nothing else is enqueued between the calls."""
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for i in range(count):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / count


def run_decode_workload(torch, pa, case, steps, warmup, copies, with_store):
    """Time `steps` decode steps (optionally with the store) on rotating pool
    copies, then the decode launches alone.

    The timed region holds exactly `steps` steps and no per-kernel events (an
    event pair around each launch adds several microseconds per step on this
    stack). Kernel durations come from separate passes of `steps` back-to-back
    launches of one kernel, each bracketed by one event pair on the launch
    stream."""
    dev = "cuda:0"
    kcs = [case.k_cache.to(dev)]
    vcs = [case.v_cache.to(dev)]
    for _ in range(copies - 1):
        kcs.append(kcs[0].clone())
        vcs.append(vcs[0].clone())
    q = case.q.to(dev)
    out = torch.empty_like(q)
    bt = case.block_tables.to(dev)
    cl = case.context_lens.to(dev)
    if with_store:
        kn, vn, sm = case.k_new.to(dev), case.v_new.to(dev), case.slot_mapping.to(dev)
    maxc = case.max_context_len
    ws = pa._lib.workspace(q.device, pa.decode_workspace_bytes(case.num_seqs, case.num_q_heads, case.head_dim, maxc))

    def store(i):
        pa.kv_store(kcs[i % copies], vcs[i % copies], kn, vn, sm)

    def decode(i):
        pa.paged_attn_decode(out, q, kcs[i % copies], vcs[i % copies], bt, cl, case.scale, maxc,
                             workspace_tensor=ws)

    def step(i):
        if with_store:
            store(i)
        decode(i)

    def fused(i):
        pa.paged_attn_decode_store(out, q, kcs[i % copies], vcs[i % copies], kn, vn, sm, bt, cl, case.scale, maxc,
                                   workspace_tensor=ws)

    def timed_steps(fn):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        t_all = Timer(torch)
        t0 = time.perf_counter()
        t_all.start()
        for i in range(steps):
            fn(warmup + i)
        t_all.stop()
        torch.cuda.synchronize()
        return t_all.ms()[0] / steps, (time.perf_counter() - t0) * 1e3 / steps

    step_ms, wall_ms = timed_steps(step)
    res = {"step_ms": step_ms, "wall_ms": wall_ms, "decode_ms": time_launches(torch, decode, steps)}
    if with_store:
        res["store_ms"] = time_launches(torch, store, steps)
        res["fused_step_ms"], res["fused_wall_ms"] = timed_steps(fused)
        res["fused_ms"] = time_launches(torch, fused, steps)
    del kcs, vcs
    torch.cuda.empty_cache()
    return res


def run_prefill_workload(torch, pa, case, steps, warmup, with_store, flush_buf):
    """Average prefill launch time (ms) over `steps` back-to-back launches
    (the new tokens are stored once beforehand when the case has a slot
    mapping), the store's own average when it has one, and the median, min
    and p90 of 30 flushed reps of each (every rep after a 1 GiB flush)."""
    dev = "cuda:0"
    kc, vc = case.k_cache.to(dev), case.v_cache.to(dev)
    q, k, v = case.q.to(dev), case.k.to(dev), case.v.to(dev)
    out = torch.empty_like(q)
    bt, cl, cu = case.block_tables.to(dev), case.context_lens.to(dev), case.cu_seqlens.to(dev)
    sm = case.slot_mapping.to(dev) if with_store else None
    mq, mc = case.max_q_len, case.max_context_len

    def store(_i):
        pa.kv_store(kc, vc, k, v, sm)

    def prefill(_i):
        pa.paged_attn_prefill(out, q, k, v, kc, vc, bt, cl, cu, case.scale, mq, mc)

    for i in range(warmup):
        if with_store:
            store(i)
        prefill(i)
    res = {"prefill_ms": time_launches(torch, prefill, steps), "reps": rep_stats(flushed_reps(torch, prefill,
                                                                                              flush_buf))}
    if with_store:
        res["store_ms"] = time_launches(torch, store, steps)
        res["store_reps"] = rep_stats(flushed_reps(torch, store, flush_buf))
    del kc, vc
    torch.cuda.empty_cache()
    return res


ROPE_THETA = 1.0e6  # Qwen3's rotary base


def run_rope_store(torch, pa, w, steps):
    """Rotary embedding + KV store of the chunked-prefill workload's 4096 new
    tokens (16 Q / 8 KV heads, D 128, bf16; positions continue each cached
    prefix; 1/8 of the slots -1): average launch time and HBM rate of the
    algorithmic bytes (q read and written, k and v read, stored rows written,
    positions and slots read)."""
    c = w.config3()
    dev = "cuda:0"
    n = (c.cu_seqlens[1:] - c.cu_seqlens[:-1]).tolist()
    cached = [int(L) - m for L, m in zip(c.context_lens.tolist(), n)]
    pos = torch.cat([torch.arange(cached[i], cached[i] + n[i], dtype=torch.int32) for i in range(len(n))])
    q, k, v = c.q.to(dev), c.k.to(dev), c.v.to(dev)
    kc, vc = c.k_cache.to(dev), c.v_cache.to(dev)
    q_out = torch.empty_like(q)
    pos_d, sm = pos.to(dev), c.slot_mapping.to(dev)

    def rope(_i):
        pa.rope_kv_store(q_out, kc, vc, q, k, v, pos_d, sm, ROPE_THETA)

    qw = torch.ones(q.shape[2], dtype=q.dtype, device=dev)
    kw = torch.ones(q.shape[2], dtype=q.dtype, device=dev)

    def qknorm_rope(_i):
        pa.qknorm_rope_kv_store(q_out, kc, vc, q, k, v, qw, kw, 1e-6, pos_d, sm, ROPE_THETA)

    for i in range(3):
        rope(i)
        qknorm_rope(i)
    ms = time_launches(torch, rope, steps)
    ms_norm = time_launches(torch, qknorm_rope, steps)
    elt = q.element_size()
    stored = int((c.slot_mapping >= 0).sum())
    nbytes = (2 * q.numel() + k.numel() + v.numel()) * elt + 2 * stored * k[0].numel() * elt + 2 * 4 * q.shape[0]
    return {"avg_us": round(ms * 1e3, 2), "TBps": round(nbytes / (ms * 1e-3) / 1e12, 4),
            "frac_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "qknorm_avg_us": round(ms_norm * 1e3, 2),
            "qknorm_frac_hbm_peak": round(nbytes / (ms_norm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": nbytes, "tokens": int(q.shape[0]), "stored_tokens": stored,
            "rope_theta": ROPE_THETA, "traffic": measured_traffic("rope_store", "c3")}


FP8_SCALE = 1.0 / 80.0  # per-pool scale: N(0,1) values stay far inside the +-448 code range


def run_fp8_decode(torch, pa, case, steps, copies):
    """Decode over fp8 (E4M3) copies of the workload's pools: the bf16 pools
    are quantised on the GPU by pa_kv_store_fp8 (every slot), then `steps`
    back-to-back fp8 decode launches on rotating copies are timed with one
    event pair. Algorithmic bytes: the fp8 K and V rows of every context once
    (shared rows once), bf16 q and out, block-table entries and lengths."""
    dev = "cuda:0"
    nb, bs, hkv, d = case.k_cache.shape
    slots = torch.arange(nb * bs, dtype=torch.int32, device=dev)
    kq = torch.empty((nb, bs, hkv, d), dtype=torch.uint8, device=dev)
    vq = torch.empty_like(kq)
    pa.kv_store_fp8(kq, vq, case.k_cache.to(dev).reshape(nb * bs, hkv, d), case.v_cache.to(dev).reshape(nb * bs, hkv, d),
                    slots, FP8_SCALE, FP8_SCALE)
    kqs, vqs = [kq], [vq]
    for _ in range(copies - 1):
        kqs.append(kq.clone())
        vqs.append(vq.clone())
    q = case.q.to(dev)
    out = torch.empty_like(q)
    bt, cl = case.block_tables.to(dev), case.context_lens.to(dev)
    maxc = case.max_context_len
    ws = torch.zeros(pa.decode_fp8_workspace_bytes(case.num_seqs, case.num_q_heads, d, maxc), dtype=torch.uint8,
                     device=dev)

    def decode(i):
        pa.paged_attn_decode_fp8(out, q, kqs[i % copies], vqs[i % copies], bt, cl, case.scale, FP8_SCALE, FP8_SCALE,
                                 maxc, workspace_tensor=ws)

    for i in range(3):
        decode(i)
    ms = time_launches(torch, decode, steps)
    db = decode_bytes(case)
    kv_fp8 = db["unique_kv"] // case.q.element_size()  # one byte per element instead of two
    nbytes = db["total"] - db["unique_kv"] + kv_fp8
    del kqs, vqs, kq, vq
    torch.cuda.empty_cache()
    return {"decode_avg_us": round(ms * 1e3, 2), "algorithmic_bytes": nbytes,
            "TBps": round(nbytes / (ms * 1e-3) / 1e12, 4),
            "frac_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "context_tokens_per_s": round(int(case.context_lens.sum()) / (ms * 1e-3), 1),
            "scale": FP8_SCALE, "pool_copies_rotated": copies}


def run_decode_graphs(torch, pa, steps):
    """Decode steps (store of the new tokens + paged decode) issued eagerly
    (two binding calls per step, exact max context), eagerly as one launch
    (pa_paged_attn_decode_store) and as one graph launch per step (bucket
    graphs of that one kernel, captured for the table's 4096-token bound), at
    batch sizes 1, 4, 16 and 64 of Qwen3-0.6B-shaped sequences (16 Q / 8 KV
    heads, D 128, bf16, contexts uniform in [128, 4096]). Per step: wall time
    of `steps` back-to-back steps (host issue included) and GPU time from one
    event pair around them."""
    import numpy as np

    from paged_kv_cache_209_amd.decode_graphs import DecodeGraphs

    dev = "cuda:0"
    hq, hkv, d, bs, mb, maxb = 16, 8, 128, 256, 16, 64
    rng = np.random.default_rng(7)
    ctx = rng.integers(128, 4096, endpoint=True, size=maxb).astype(np.int32)
    need = [-(-int(c) // bs) for c in ctx]
    nb = int(1.25 * sum(need)) + 1
    ids = rng.permutation(nb)[:sum(need)]
    bt = np.full((maxb, mb), -1, dtype=np.int32)
    slots = np.empty(maxb, dtype=np.int32)
    k = 0
    for i, c in enumerate(ctx):
        bt[i, :need[i]] = ids[k:k + need[i]]
        k += need[i]
        slots[i] = bt[i, (c - 1) // bs] * bs + (c - 1) % bs
    g = torch.Generator(device=dev).manual_seed(7)
    kc = torch.randn((nb, bs, hkv, d), generator=g, device=dev).to(torch.bfloat16)
    vc = torch.randn((nb, bs, hkv, d), generator=g, device=dev).to(torch.bfloat16)
    ws_bytes = pa.decode_workspace_bytes(maxb, hq, d, mb * bs)
    bufs = {"out": torch.zeros((maxb, hq, d), dtype=torch.bfloat16, device=dev),
            "q": torch.randn((maxb, hq, d), generator=g, device=dev).to(torch.bfloat16),
            "k_new": torch.randn((maxb, hkv, d), generator=g, device=dev).to(torch.bfloat16),
            "v_new": torch.randn((maxb, hkv, d), generator=g, device=dev).to(torch.bfloat16),
            "slot_mapping": torch.from_numpy(slots).to(dev),
            "block_tables": torch.from_numpy(bt).to(dev),
            "context_lens": torch.from_numpy(ctx).to(dev),
            "k_cache": kc, "v_cache": vc,
            "workspace": torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)}
    graphs = DecodeGraphs(bufs, d ** -0.5)
    eager_ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    res = {}
    for n in (1, 4, 16, 64):
        sm, ctx_n = bufs["slot_mapping"][:n].clone(), bufs["context_lens"][:n].clone()
        maxc = int(ctx[:n].max())

        def eager(_i):
            pa.kv_store(kc, vc, bufs["k_new"][:n], bufs["v_new"][:n], sm)
            pa.paged_attn_decode(bufs["out"][:n], bufs["q"][:n], kc, vc, bufs["block_tables"][:n], ctx_n,
                                 d ** -0.5, maxc, workspace_tensor=eager_ws)

        def eager_one(_i):
            pa.paged_attn_decode_store(bufs["out"][:n], bufs["q"][:n], kc, vc, bufs["k_new"][:n], bufs["v_new"][:n],
                                       sm, bufs["block_tables"][:n], ctx_n, d ** -0.5, maxc,
                                       workspace_tensor=eager_ws)

        def graph(_i):
            graphs.launch(n)

        row = {}
        for name, fn in (("eager", eager), ("eager_one_launch", eager_one), ("graph", graph)):
            for i in range(5):
                fn(i)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            ms = time_launches(torch, fn, steps)
            row[f"{name}_wall_us"] = round((time.perf_counter() - t0) / steps * 1e6, 2)
            row[f"{name}_gpu_us"] = round(ms * 1e3, 2)
            # padding rows of the graph's buckets are reset by each launch; restore them
            bufs["slot_mapping"].copy_(torch.from_numpy(slots).to(dev))
            bufs["context_lens"].copy_(torch.from_numpy(ctx).to(dev))
        row["bucket"] = graphs.bucket(n)
        res[f"batch_{n}"] = row
    graphs.close()
    del kc, vc, bufs
    torch.cuda.empty_cache()
    return res


def block_manager_workload(num_seqs, lo, hi, seed, steps):
    """Prompts of num_seqs sequences with contexts uniform in [lo, hi], the
    odd-numbered ones longer than 1024 tokens opening with one shared
    1024-token system prompt; a pool of 256-token blocks 1.25x their need
    (plus room for `steps` decode tokens) and the table width."""
    import numpy as np

    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi, endpoint=True, size=num_seqs)
    system = [int(x) for x in rng.integers(0, 150000, size=1024)]
    prompts = []
    for i, L in enumerate(lens):
        share = i % 2 == 1 and L > 1024
        tail = [int(x) for x in rng.integers(0, 150000, size=int(L) - (1024 if share else 0))]
        prompts.append((system if share else []) + tail)
    nb = int(1.25 * sum(-(-len(p) // 256) for p in prompts)) + num_seqs * ((steps + 3) // 256 + 2)
    width = max(-(-len(p) // 256) for p in prompts) + (steps + 3) // 256 + 2
    return prompts, nb, width


def run_block_manager(num_seqs, lo, hi, seed, steps):
    """Host time of one decode step's metadata from the native block manager
    (append one token to every sequence, then prepare_decode into preallocated
    buffers) after the whole prompts are admitted and prefilled."""
    import torch

    from paged_kv_cache_209_amd.block_manager import BlockManager

    prompts, nb, width = block_manager_workload(num_seqs, lo, hi, seed, steps)
    m = BlockManager(nb, 256)
    for i, p in enumerate(prompts):
        m.allocate(i, p)
    m.prepare_prefill(list(range(num_seqs)), width)
    id_t = torch.arange(num_seqs, dtype=torch.int64)
    tok_t = torch.full((num_seqs,), 7, dtype=torch.int32)
    bufs = {"positions": torch.empty(num_seqs, dtype=torch.int32),
            "slot_mapping": torch.empty(num_seqs, dtype=torch.int32),
            "context_lens": torch.empty(num_seqs, dtype=torch.int32),
            "block_tables": torch.empty((num_seqs, width), dtype=torch.int32)}
    for _ in range(3):
        m.append_tokens(id_t, tok_t)
        m.prepare_decode(id_t, width, out=bufs)
    t0 = time.perf_counter()
    for _ in range(steps):
        m.append_tokens(id_t, tok_t)
        m.prepare_decode(id_t, width, out=bufs)
    return {"native_us_per_step": round((time.perf_counter() - t0) / steps * 1e6, 1), "num_seqs": num_seqs,
            "context_range": [lo, hi], "steps": steps, "num_blocks": nb}


def cpu_baseline(case, budget_s: float):
    """The fp64 oracle (unchanged) on the host cores, on the headline decode
    workload (host copies of its pools), one sequence at a time in order
    until `budget_s` has passed. The rate counts the algorithmic bytes of the
    sequences done (their K/V rows, a block shared with an earlier sampled
    sequence once; q, out and metadata), as the GPU figure does."""
    import torch

    import oracle
    import workloads as w

    cores = len(os.sched_getaffinity(0))
    torch.set_num_threads(cores)
    kc, vc = case.k_cache.cpu(), case.v_cache.cpu()
    q = case.q.cpu()
    elt = q.element_size()
    kv_row = case.num_kv_heads * case.head_dim * elt * 2
    seen = set()
    nbytes = 0
    done = 0
    t0 = time.perf_counter()
    for i in range(case.num_seqs):
        oracle.paged_attn_decode(q, kc, vc, case.block_tables, case.context_lens, case.scale, seqs=[i])
        L = int(case.context_lens[i])
        for b in range(w.blocks_for(L)):
            blk = int(case.block_tables[i, b])
            if blk not in seen:
                seen.add(blk)
                nbytes += min(256, L - 256 * b) * kv_row
        nbytes += 2 * case.num_q_heads * case.head_dim * elt + 4 * (w.blocks_for(L) + 1)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": nbytes / el / 1e12, "unit": "TB/s", "cores": torch.get_num_threads(), "kind": "oracle",
            "sample": f"{done} of the {case.num_seqs} sequences of the Qwen3-8B-shaped decode (contexts "
                      f"U[1024,8192], half sharing a 1024-token prefix), {nbytes / 1e9:.3f} GB of algorithmic bytes, in {el:.1f} s on {cores} host cores, "
                      "fp64",
            "block_manager_oracle_us_per_step": block_manager_oracle_step_us(64, 128, 4096, 1, 200)}


def block_manager_oracle_step_us(num_seqs, lo, hi, seed, steps):
    """The plain-Python oracle of the block manager on the same decode steps
    as the native leg (append one token to every sequence, prepare_decode)."""
    import oracle.block_manager as obm

    prompts, nb, width = block_manager_workload(num_seqs, lo, hi, seed, steps)
    m = obm.OracleBlockManager(nb, 256)
    for i, p in enumerate(prompts):
        m.allocate(i, p)
    ids = list(range(num_seqs))
    m.prepare_prefill(ids, None, width, 1 << 30)
    toks = [7] * num_seqs
    for _ in range(3):
        m.append_tokens(ids, toks)
        m.prepare_decode(ids, width)
    t0 = time.perf_counter()
    for _ in range(steps):
        m.append_tokens(ids, toks)
        m.prepare_decode(ids, width)
    return round((time.perf_counter() - t0) / steps * 1e6, 1)


def run_environment(torch, pa):
    """Where the numbers were taken: GPU, compute units, host CPU and cores."""
    props = torch.cuda.get_device_properties(0)
    cpu = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"gpu": getattr(props, "gcnArchName", props.name), "compute_units": props.multi_processor_count,
            "gpu_memory_gib": round(props.total_memory / 2**30, 1), "library": pa.version(),
            "torch": torch.__version__, "hip": torch.version.hip, "cpu_model": cpu,
            "host_cores_available": len(os.sched_getaffinity(0)), "host_cpu_count": os.cpu_count()}


FLUSH_BYTES = 1 << 30  # larger than the 256 MB memory-side cache and every L2
FLUSH_REPS = 30


def flushed_reps(torch, fn, flush_buf, reps=FLUSH_REPS, write=False):
    """Durations (ms) of `reps` calls of fn(i), each preceded on the same
    stream by a sweep over the 1 GiB flush buffer and bracketed by its own
    HIP event pair. The sweep reads the buffer (a sum), so every cache line
    of the previous call is evicted and the caches are left holding clean
    data, as after the weight reads that precede an attention launch in a
    model step; with write=True it overwrites the buffer instead, leaving
    every cache full of dirty lines that a cache-allocating load must write
    back first."""
    pairs = []
    torch.cuda.synchronize()
    for i in range(reps):
        if write:
            flush_buf.fill_(float(i & 0x7F))
        else:
            flush_buf.sum()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn(i)
        b.record()
        pairs.append((a, b))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in pairs]


def rep_stats(ms_list, write=False):
    """Median, min and p90 (nearest rank) of per-rep durations, in us."""
    xs = sorted(ms_list)
    n = len(xs)
    med = xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])
    p90 = xs[min(n - 1, max(0, math.ceil(0.9 * n) - 1))]
    how = "overwrite" if write else "read"
    return {"median_us": round(med * 1e3, 2), "min_us": round(xs[0] * 1e3, 2), "p90_us": round(p90 * 1e3, 2),
            "reps": n, "timing": f"each rep after a 1 GiB flush ({how}) on the launch stream, own event pair "
                                 "(~3 us of event overhead included)"}


def run_c4_headline(torch, pa, w, steps, warmup, flush_buf):
    """The headline: paged decode of the Qwen3-8B-shaped batch (256 sequences,
    32 Q / 8 KV heads, D 128, bf16, contexts U[1024, 8192], half sharing a
    1024-token prefix), one launch per step. Its 6 GB of pools dwarf every
    cache, so back-to-back steps read their K/V from HBM. Returns the case
    (pools on the device) and the timings."""
    c4 = w.config4(device="cuda:0")
    dev = "cuda:0"
    q = c4.q
    out = torch.empty_like(q)
    bt, cl = c4.block_tables.to(dev), c4.context_lens.to(dev)
    maxc = c4.max_context_len
    ws = pa._lib.workspace(q.device, pa.decode_workspace_bytes(c4.num_seqs, c4.num_q_heads, c4.head_dim, maxc))

    def decode(_i):
        pa.paged_attn_decode(out, q, c4.k_cache, c4.v_cache, bt, cl, c4.scale, maxc, workspace_tensor=ws)

    for i in range(warmup):
        decode(i)
    torch.cuda.synchronize()
    t_all = Timer(torch)
    t0 = time.perf_counter()
    t_all.start()
    for i in range(steps):
        decode(i)
    t_all.stop()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    step_ms = t_all.ms()[0] / steps
    reps = rep_stats(flushed_reps(torch, decode, flush_buf))
    reps_w = rep_stats(flushed_reps(torch, decode, flush_buf, write=True), write=True)
    pa.check_workspace(ws)
    return c4, {"step_ms": step_ms, "wall_ms": wall_ms, "reps": reps, "reps_write": reps_w}


def c2_secondary(torch, pa, w, steps, warmup, copies):
    """The Qwen3-0.6B-shaped decode step: store of the 64 new tokens' K/V +
    decode, as one launch (pa_paged_attn_decode_store) and as two, on
    rotating pool copies; with the one-launch kernel's roofline."""
    c2 = w.config2(device="cuda:0")
    r = run_decode_workload(torch, pa, c2, steps, warmup, copies, with_store=True)
    db = decode_bytes(c2)
    store_bytes = 2 * 2 * c2.k_new.numel() * c2.k_new.element_size()  # read + write of k and v rows
    step_bytes = db["total"] + store_bytes
    achieved = step_bytes / (r["fused_ms"] * 1e-3) / 1e9
    res = {
        "what": "store of 64 new tokens' K/V through slot_mapping + paged decode, one launch "
                "(pa_paged_attn_decode_store), batch 64, 16 Q / 8 KV heads, head_dim 128, contexts U[128,4096]",
        "ms_per_step": round(r["fused_step_ms"], 5),
        "value_tb_s": round(step_bytes / (r["fused_step_ms"] * 1e-3) / 1e12, 4),
        "wall_ms_per_step": round(r["fused_wall_ms"], 5),
        "pool_copies_rotated": copies,
        "step_bytes": step_bytes,
        "roofline": {
            "kernel": "paged_decode_kernel<bf16,128,2,fused store>",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("decode_store", "c2"),
            "algorithmic_bytes_per_launch": step_bytes,
            "avg_launch_us": round(r["fused_ms"] * 1e3, 2),
        },
        "two_launch_step": {
            "what": "the same step as pa_kv_store then pa_paged_attn_decode",
            "ms_per_step": round(r["step_ms"], 5),
            "value_tb_s": round(step_bytes / (r["step_ms"] * 1e-3) / 1e12, 4),
            "store_avg_us": round(r["store_ms"] * 1e3, 2),
            "decode_avg_us": round(r["decode_ms"] * 1e3, 2),
            "decode_frac_hbm_peak": round(db["total"] / (r["decode_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "decode_algorithmic_bytes_per_launch": db["total"],
            "decode_traffic": measured_traffic("decode", "c2"),
        },
    }
    del c2
    torch.cuda.empty_cache()
    return res


def cpu_baseline_prefill(case, budget_s: float, label: str):
    """The fp64 oracle (unchanged) on the host cores, one sequence at a time
    of a prefill / verify workload (host copies of its tensors), until
    `budget_s` has passed: GFLOP/s of the causal work done."""
    import torch

    import oracle

    cores = len(os.sched_getaffinity(0))
    torch.set_num_threads(cores)
    cu = case.cu_seqlens.tolist()
    t0 = time.perf_counter()
    flops = 0.0
    done = 0
    for i in range(case.num_seqs):
        oracle.paged_attn_prefill(case.q, case.k, case.v, case.k_cache, case.v_cache, case.block_tables,
                                  case.context_lens, case.cu_seqlens, case.scale, seqs=[i])
        n = cu[i + 1] - cu[i]
        c = int(case.context_lens[i]) - n
        flops += 4.0 * case.head_dim * case.num_q_heads * (n * c + n * (n + 1) / 2)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": round(flops / el / 1e9, 3), "unit": "GFLOP/s", "cores": torch.get_num_threads(),
            "kind": "oracle", "sample": f"{done} of {case.num_seqs} sequences of the {label} workload in {el:.1f} s "
                                        f"on {cores} host cores, fp64"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--copies", type=int, default=4, help="pool copies rotated between C2 steps")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--skip-secondary", action="store_true")
    ap.add_argument("--only", default="",
                    help="run just one workload: c4 | c2 | c3 | rope | c5 | fp8 | graphs | bm (profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy --steps times (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the paged-attention kernels run on a single device and the "
              "library has no multi-GPU path (per-GPU work would be sharded by sequence or KV head with no "
              "exchange). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 1 << 30, "launches": args.steps}), flush=True)
        return

    import paged_kv_cache_209_amd as pa
    import workloads as w

    pa.library()
    log(f"{pa.version()} on {torch.cuda.get_device_name(0)}")
    flush_buf = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda:0")

    secondary = {}
    c4_case = None
    if args.only in ("", "c4"):
        c4_case, r = run_c4_headline(torch, pa, w, args.steps, args.warmup, flush_buf)
        db = decode_bytes(c4_case)
        step_bytes = db["total"]
        achieved = step_bytes / (r["step_ms"] * 1e-3) / 1e9
        result = {
            "metric": METRIC,
            "value": round(step_bytes / (r["step_ms"] * 1e-3) / 1e12, 4),
            "unit": "TB/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(r["step_ms"], 5),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16",
            "data": "synthetic",
            "config": {
                "workload": "c4_qwen3_8b_decode_shared_prefix: paged decode attention (pa_paged_attn_decode, one "
                            "launch per step) of 256 sequences, 32 Q / 8 KV heads, head_dim 128, 256-token blocks, "
                            "contexts U[1024,8192], a random half sharing one 1024-token prefix (4 block ids), "
                            "shuffled pool 1.25x the unique blocks, bf16 inputs, fp32 accumulation",
                "num_seqs": c4_case.num_seqs,
                "total_context_tokens": int(c4_case.context_lens.sum()),
                "decode_workgroups": pa.decode_num_workgroups(256, 32, 8, 128, c4_case.max_context_len),
                "step_bytes": step_bytes,
                "logical_kv_bytes": db["logical_kv"],
                "parallelism": "single GPU",
            },
            "roofline": {
                "kernel": "paged_decode_kernel<bf16,128,4,false>",
                "bound": "hbm",
                "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS,
                "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic("decode", "c4"),
                "algorithmic_bytes_per_launch": step_bytes,
                "avg_launch_us": round(r["step_ms"] * 1e3, 2),
                "timing": f"the timed region: {args.steps} back-to-back launches (each reads its 4.3 GB of unique "
                          "K/V from HBM), one HIP event pair on the launch stream",
            },
            "wall_ms_per_step": round(r["wall_ms"], 5),
            "flushed_reps": r["reps"],
            "flushed_reps_overwrite": r["reps_write"],
        }
    else:
        result = {"metric": METRIC, "value": None, "note": f"--only {args.only}"}

    if not args.skip_secondary and args.only in ("", "c2"):
        secondary["c2_qwen3_0.6b_decode_step"] = c2_secondary(torch, pa, w, args.steps, args.warmup, args.copies)

    if not args.skip_secondary and args.only in ("", "c3"):
        c3 = w.config3(device="cuda:0")
        r3 = run_prefill_workload(torch, pa, c3, max(10, args.steps), 3, with_store=True, flush_buf=flush_buf)
        avg = r3["prefill_ms"]
        fl = prefill_flops(c3)
        pb = prefill_bytes(c3)
        med = r3["reps"]["median_us"] * 1e-6
        secondary["c3_chunked_prefill_prefix_cache"] = {
            "prefill_avg_us": round(avg * 1e3, 2),
            "store_avg_us": round(r3["store_ms"] * 1e3, 2),
            "TFLOPs": round(fl / (avg * 1e-3) / 1e12, 2),
            "frac_mfma_bf16_peak": round(fl / (avg * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "flushed_reps": r3["reps"],
            "flushed_median_TFLOPs": round(fl / med / 1e12, 2),
            "flushed_median_frac_mfma_bf16_peak": round(fl / med / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "store_flushed_reps": r3["store_reps"],
            "flops": fl,
            "algorithmic_bytes": pb["total"],
            "traffic": measured_traffic("prefill", "c3"),
            "store_traffic": measured_traffic("kv_store", "c3"),
        }
        del c3
    if not args.skip_secondary and args.only in ("", "c3", "rope"):
        secondary["c3_rope_kv_store"] = run_rope_store(torch, pa, w, max(10, args.steps))
        torch.cuda.empty_cache()
    c5_case = None
    if not args.skip_secondary and args.only in ("", "c5"):
        c5_case = w.config5(device="cuda:0")
        r5 = run_prefill_workload(torch, pa, c5_case, max(20, args.steps // 2), 5, with_store=False,
                                  flush_buf=flush_buf)
        avg = r5["prefill_ms"]
        fl = prefill_flops(c5_case)
        pb = prefill_bytes(c5_case)
        med = r5["reps"]["median_us"] * 1e-6
        secondary["c5_spec_verify"] = {
            "verify_avg_us": round(avg * 1e3, 1),
            "TBps": round(pb["total"] / (avg * 1e-3) / 1e12, 4),
            "frac_hbm_peak": round(pb["total"] / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "TFLOPs": round(fl / (avg * 1e-3) / 1e12, 2),
            "frac_mfma_bf16_peak": round(fl / (avg * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "flushed_reps": r5["reps"],
            "flushed_median_frac_hbm_peak": round(pb["total"] / med / 1e9 / HBM_PEAK_GBS, 4),
            "flops": fl,
            "algorithmic_bytes": pb["total"],
            "traffic": measured_traffic("prefill", "c5"),
        }
    if not args.skip_secondary and args.only in ("", "fp8"):
        c2f = w.config2(device="cuda:0")
        fp8 = {"c2_qwen3_0.6b": run_fp8_decode(torch, pa, c2f, max(20, args.steps), args.copies)}
        del c2f
        torch.cuda.empty_cache()
        c4f = c4_case if c4_case is not None else w.config4(device="cuda:0")
        fp8["c4_qwen3_8b_shared_prefix"] = run_fp8_decode(torch, pa, c4f, max(20, args.steps // 2), 1)
        del c4f
        torch.cuda.empty_cache()
        secondary["fp8_kv_decode"] = fp8
    if not args.skip_secondary and args.only in ("", "graphs"):
        secondary["decode_step_graphs_vs_eager"] = run_decode_graphs(torch, pa, max(50, args.steps))
    if not args.skip_secondary and args.only in ("", "bm"):
        secondary["block_manager_decode_step_host"] = {
            "c2_shape": run_block_manager(64, 128, 4096, 1, 200),
            "c4_shape": run_block_manager(256, 1024, 8192, 3, 200),
        }
    if secondary:
        result["secondary"] = secondary
    result["env"] = run_environment(torch, pa)
    del flush_buf
    if not args.skip_cpu and args.only in ("", "c4"):
        log("timing the fp64 oracle on the host ...")
        base = cpu_baseline(c4_case, args.cpu_seconds)
        del c4_case
        torch.cuda.empty_cache()
        base["c3_prefill"] = cpu_baseline_prefill(w.config3(), 5.0, "chunked-prefill (8 sequences x 512 new tokens after cached prefixes)")
        if c5_case is not None:
            host5 = w.PrefillCase(c5_case.name, c5_case.q.cpu(), c5_case.k.cpu(), c5_case.v.cpu(),
                                  c5_case.k_cache.cpu(), c5_case.v_cache.cpu(), c5_case.block_tables,
                                  c5_case.context_lens, c5_case.cu_seqlens, c5_case.scale)
            del c5_case
            torch.cuda.empty_cache()
            base["c5_verify"] = cpu_baseline_prefill(host5, 5.0, "speculative-verify (128 sequences x 5 draft tokens, contexts U[2048,16384])")
            del host5
        result["cpu_baseline"] = base
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
