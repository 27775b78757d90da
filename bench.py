#!/usr/bin/env python3
"""Benchmark of the paged-attention hot path on one MI355X.

A step is one paged_attn_decode call (partition pass + log-sum-exp merge) over
the LLaMA-7B-shaped decode workload: 64 sequences, 32 heads, head_dim 128,
block_size 16, contexts uniform in [512, 4096], fp16, inputs resident in HBM.
The headline value is its algorithmic KV bandwidth (GB/s).  The same run also
measures the GQA bf16 and long-context split-KV decode workloads, the causal
paged prefill (TFLOP/s), the block copy, the KV append and the host<->device
swap (GB/s), and times the fp64 CPU oracle on a bounded sample of the
headline workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]

Prints one JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16/fp16 matrix peak

METRIC = "paged decode KV GB/s (% of 8 TB/s HBM peak); prefill TFLOP/s (% MFMA peak)"

# Sources of each kernel: a kernel's HBM traffic figure (profiles/hbm_traffic.md)
# is only reported while these match the version the counters were taken on.
_CSRC = "paged_kv_cache_248_amd/csrc/"
SOURCES = {
    "decode": [_CSRC + "decode.hip", _CSRC + "pa_device.h"],
    "prefill": [_CSRC + "prefill.hip", _CSRC + "prefill_common.h", _CSRC + "pa_device.h"],
    "copy": [_CSRC + "copy_blocks.hip", _CSRC + "pa_device.h"],
    "append": [_CSRC + "append.hip", _CSRC + "pa_device.h"],
}


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


class KernelTimer:
    """HIP events that the library has the runtime record as part of its main
    kernel's dispatch (start and end of that kernel's execution)."""

    def __init__(self, pa, torch, n: int):
        self.pa, self.torch = pa, torch
        self.pairs = []
        for _ in range(n):
            s = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            s.record()                 # materialise the underlying hipEvent_t
            e.record()
            self.pairs.append((s, e))
        self.lib = pa.load_library()
        self.i = 0

    def arm(self) -> None:
        s, e = self.pairs[self.i]
        st = self.lib.pa_set_profile_events(s.cuda_event, e.cuda_event)
        assert st == 0
        self.i += 1

    def disarm(self) -> None:
        self.lib.pa_set_profile_events(None, None)

    def mean_ms(self) -> float:
        self.torch.cuda.synchronize()
        ts = [s.elapsed_time(e) for s, e in self.pairs[:self.i]]
        return float(np.mean(ts)) if ts else float("nan")


def timed_steps(torch, fn, steps: int, warmup: int, timer=None, between=None):
    for _ in range(warmup):
        fn()
        if between:
            between()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        if timer:
            timer.arm()
        fn()
        if between:
            between()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if timer:
        timer.disarm()
    return (t1 - t0) * 1e3 / steps


def bench_decode(pa, torch, wl, case, steps, warmup):
    """Decode steps over two copies of the inputs (query, pools, tables,
    lengths) in turn, so that no step finds the previous step's K/V in the
    caches (the 256 MB Infinity Cache and the L2s): every timed step streams
    its K/V from HBM.  A shorter run that repeats one copy is reported beside
    it (`*_same_input`) to show what warm caches would add."""
    kv = case.kv
    B, Hq, D = case.query.shape
    Hkv = kv.k_cache.shape[1]
    maxctx = kv.max_context_len
    copies = [(case.query, kv.k_cache, kv.v_cache, kv.block_tables, kv.context_lens),
              tuple(t.clone() for t in (case.query, kv.k_cache, kv.v_cache, kv.block_tables,
                                          kv.context_lens))]
    outs = [torch.empty_like(case.query) for _ in copies]
    wss = [torch.empty(pa.paged_attn_decode_workspace_size(B, Hq, Hkv, D, maxctx,
                                                           case.partition_size),
                       dtype=torch.uint8, device=case.query.device) for _ in copies]
    n = [0]

    def step():
        i = n[0] & 1
        n[0] += 1
        q, kc, vc, bt, cl = copies[i]
        pa.paged_attn_decode(outs[i], q, kc, vc, bt, cl, case.scale, maxctx,
                             partition_size=case.partition_size, workspace=wss[i])

    def step_same():
        q, kc, vc, bt, cl = copies[0]
        pa.paged_attn_decode(outs[0], q, kc, vc, bt, cl, case.scale, maxctx,
                             partition_size=case.partition_size, workspace=wss[0])

    timer = KernelTimer(pa, torch, steps)
    ms = timed_steps(torch, step, steps, warmup, timer)
    kms = timer.mean_ms()
    same_steps = max(10, steps // 2)
    timer_same = KernelTimer(pa, torch, same_steps)
    ms_same = timed_steps(torch, step_same, same_steps, max(10, warmup // 10), timer_same)
    kms_same = timer_same.mean_ms()
    assert torch.equal(outs[0], outs[1]), "the two input copies gave different outputs"
    del copies
    ctx = kv.context_lens.cpu().numpy()
    nbytes = wl.decode_kv_bytes(ctx, Hq, Hkv, D, kv.block_size, wl.ELEM_BYTES[case.dtype])
    return {
        "workload": case.name, "ms_per_step": ms, "kernel_ms": kms, "bytes": nbytes,
        "GBps": nbytes / (ms * 1e-3) / 1e9, "kernel_GBps": nbytes / (kms * 1e-3) / 1e9,
        "tokens_per_s": B / (ms * 1e-3),
        "frac_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "timing": "two input copies alternated: every step reads its K/V from HBM",
        "ms_per_step_same_input": ms_same, "kernel_ms_same_input": kms_same,
        "kernel_GBps_same_input": nbytes / (kms_same * 1e-3) / 1e9,
        "num_seqs": B, "num_heads": Hq, "num_kv_heads": Hkv, "head_dim": D,
        "block_size": kv.block_size, "dtype": case.dtype,
        "context_mean": float(ctx.mean()), "context_min": int(ctx.min()),
        "context_max": int(ctx.max()), "pool_blocks": int(kv.k_cache.shape[0]),
        "partition_size": case.partition_size or pa.default_partition(Hq, Hkv),
    }


def bench_prefill(pa, torch, wl, case, steps, warmup, kernel="pingpong"):
    """kernel: "pingpong" (paged_attn_prefill) or "halftile"
    (paged_attn_prefill_halftile, the second schedule, for comparison)."""
    kv = case.kv
    out = torch.empty_like(case.query)
    fn = pa.paged_attn_prefill if kernel == "pingpong" else pa.paged_attn_prefill_halftile

    def step():
        fn(out, case.query, kv.k_cache, kv.v_cache, kv.block_tables, kv.context_lens,
           case.query_start_loc, case.scale, case.max_query_len, kv.max_context_len)

    timer = KernelTimer(pa, torch, steps)
    ms = timed_steps(torch, step, steps, warmup, timer)
    kms = timer.mean_ms()
    ctx = kv.context_lens.cpu().numpy()
    qsl = case.query_start_loc.cpu().numpy()
    ql = np.diff(qsl)
    T, Hq, D = case.query.shape
    flops = wl.prefill_flops(ctx, ql, Hq, D)
    Hkv = kv.k_cache.shape[1]
    e = wl.ELEM_BYTES[case.dtype]
    # compulsory HBM bytes: Q read and O written once, K and V of every key
    # of every (sequence, kv head) read once
    hbm_bytes = 2 * T * Hq * D * e + 2 * int(ctx.sum()) * Hkv * D * e
    return {
        "workload": case.name, "kernel": kernel, "ms_per_step": ms, "kernel_ms": kms,
        "flops": flops, "hbm_bytes": hbm_bytes,
        "TFLOPs": flops / (ms * 1e-3) / 1e12, "kernel_TFLOPs": flops / (kms * 1e-3) / 1e12,
        "frac_mfma_peak": flops / (kms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS,
        "tokens_per_s": T / (ms * 1e-3), "num_seqs": len(ctx), "new_tokens": int(T),
        "prefix_lens": (ctx - ql).tolist(), "num_heads": Hq, "num_kv_heads": kv.k_cache.shape[1],
        "head_dim": D, "block_size": kv.block_size, "dtype": case.dtype,
    }


def bench_prefill_unfused(pa, torch, wl, case, steps, warmup):
    """The same prefill computed unfused (S and P through HBM, library
    GEMMs); timed per call on the stream it runs on."""
    kv = case.kv
    out = torch.empty_like(case.query)
    ctx = kv.context_lens.cpu()
    qsl = case.query_start_loc.cpu()
    ql = (qsl[1:] - qsl[:-1]).numpy()
    T, Hq, D = case.query.shape
    ws = torch.empty(pa.paged_attn_prefill_unfused_workspace_size(
        int(ql.max()), int(ctx.max()), Hq, kv.k_cache.shape[1], D, case.query.dtype),
        dtype=torch.uint8, device=case.query.device)

    def step():
        pa.paged_attn_prefill_unfused(out, case.query, kv.k_cache, kv.v_cache, kv.block_tables,
                                      ctx, qsl, case.scale, workspace=ws)

    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    c = ctx.numpy()
    flops = wl.prefill_flops(c, ql, Hq, D)
    e = wl.ELEM_BYTES[case.dtype]
    # S (fp32) and P (dtype) of every head: written once and read once each
    sp_bytes = int(sum(2 * Hq * int(q) * int(n) * (4 + e) for q, n in zip(ql, c)))
    return {
        "workload": case.name + " (unfused)", "ms_per_step": ms, "flops": flops,
        "TFLOPs": flops / (ms * 1e-3) / 1e12, "tokens_per_s": T / (ms * 1e-3),
        "s_p_hbm_bytes": sp_bytes, "steps": steps, "warmup": warmup,
    }


def bench_tiny_decode(pa, torch, wl, steps, warmup):
    """The tiny fp32 decode (4 sequences, contexts up to 200 tokens): a
    launch-bound call, reported in microseconds per call, issued eagerly and
    as the replay of a captured HIP graph (its launches recorded once).
    Beside each GPU-timeline rate: the host time to issue one call (the loop
    without the final synchronisation) and, for the eager calls, the kernel's
    own duration from the library's events, which show what bounds each
    rate."""
    case = wl.tiny_decode_f32(device="cuda:0")
    kv = case.kv
    out = torch.empty_like(case.query)
    B, Hq, D = case.query.shape
    maxctx = kv.max_context_len
    ws = torch.empty(max(1, pa.paged_attn_decode_workspace_size(B, Hq, kv.k_cache.shape[1], D,
                                                                maxctx, 0)),
                     dtype=torch.uint8, device="cuda:0")

    def call():
        pa.paged_attn_decode(out, case.query, kv.k_cache, kv.v_cache, kv.block_tables,
                             kv.context_lens, case.scale, maxctx, workspace=ws)

    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)

    def rate(fn):
        """(GPU-timeline us per call, host us to issue one call)"""
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        start.record()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        t1 = time.perf_counter()
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop) * 1e3 / steps, (t1 - t0) * 1e6 / steps

    eager_us, eager_host_us = rate(call)
    timer = KernelTimer(pa, torch, steps)
    timed_steps(torch, call, steps, 10, timer)
    kernel_us = timer.mean_ms() * 1e3
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    graph_us, graph_host_us = rate(g.replay)
    ctx = kv.context_lens.cpu().numpy()
    return {"workload": "tiny_decode_f32", "eager_us_per_call": eager_us,
            "eager_host_us_per_call": eager_host_us, "kernel_us": kernel_us,
            "graph_us_per_call": graph_us, "graph_host_us_per_replay": graph_host_us,
            "num_seqs": B, "num_heads": Hq, "head_dim": D,
            "context_lens": ctx.tolist(), "steps": steps, "warmup": warmup}


def bench_block_manager(pa, wl, steps: int = 200):
    """Host bookkeeping of one decode step (one more token for each of 256
    requests, then the kernels' block tables for the batch) in the native
    block manager, and the same with the Python oracle (the baseline).
    Requests start from lognormal prompts (median 2048, sigma 1), 16-token
    blocks, the pool sized to the prompts plus room for every appended token."""
    from oracle.block_manager_oracle import BlockManagerOracle
    rng = np.random.default_rng(2486)
    n_req, bs = 256, 16
    prompts = np.clip(np.round(2048 * np.exp(rng.standard_normal(n_req))), 16, 32768).astype(int)
    pool = int(sum((p + steps + bs - 1) // bs for p in prompts) * 1.1)
    ids = list(range(n_req))
    mbps = int(max((p + steps + bs - 1) // bs for p in prompts))
    bm = pa.BlockManager(pool, bs)
    ref = BlockManagerOracle(pool, bs)
    for i, p in enumerate(prompts):
        bm.register(i, int(p))
        ref.register(i, int(p))
    import torch
    out = (torch.empty((n_req, mbps), dtype=torch.int32), torch.empty(n_req, dtype=torch.int32))
    t0 = time.perf_counter()
    for _ in range(steps):
        bm.append_tokens(ids)
        bm.batch_tables(ids, mbps, out=out)
    native_us = (time.perf_counter() - t0) * 1e6 / steps
    ref_steps = max(1, steps // 10)
    t0 = time.perf_counter()
    for _ in range(ref_steps):
        for i in ids:
            ref.append_token(i)
        tables = np.full((n_req, mbps), -1, dtype=np.int32)
        for i in ids:
            tables[i, :len(ref.tables[i])] = ref.tables[i]
        lens = np.array([ref.tokens[i] for i in ids], dtype=np.int32)
    oracle_us = (time.perf_counter() - t0) * 1e6 / ref_steps
    return {"workload": "block_manager_decode_step", "requests": n_req, "block_size": bs,
            "pool_blocks": pool, "native_us_per_step": native_us,
            "oracle_us_per_step": oracle_us, "steps": steps, "oracle_steps": ref_steps}


def bench_copy(pa, torch, wl, case, steps, warmup):
    n = wl.copy_count_unique(case.src_to_dst.cpu().numpy(), case.src_k.shape[0],
                             case.dst_k.shape[0])
    block_bytes = case.src_k[0].numel() * case.src_k.element_size()
    ws = torch.empty(pa.paged_kv_copy_blocks_workspace_size(case.dst_k.shape[0]),
                     dtype=torch.uint8, device=case.src_k.device)
    # The working set (~0.5 GB) is near the 256 MB Infinity Cache: overwrite a
    # 1 GiB scratch buffer between steps so every step starts from cold caches.
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=case.src_k.device)

    def step():
        pa.paged_kv_copy_blocks(case.src_k, case.src_v, case.dst_k, case.dst_v,
                                case.src_to_dst, workspace=ws)

    timer = KernelTimer(pa, torch, steps)
    ms = timed_steps(torch, step, steps, warmup, timer, between=lambda: scratch.fill_(1))
    kms = timer.mean_ms()
    nbytes = wl.copy_bytes(n, block_bytes)
    return {
        "workload": case.name, "kernel_ms": kms, "bytes": nbytes, "copies": n,
        "kernel_GBps": nbytes / (kms * 1e-3) / 1e9,
        "frac_hbm_peak": nbytes / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "step_ms_incl_cache_flush": ms,
    }


def bench_append(pa, torch, wl, case, steps, warmup):
    kv = case.kv
    T, Hkv, D = case.key.shape
    # Rows (64 MiB) and touched pool slots fit the 256 MB Infinity Cache:
    # overwrite a 1 GiB scratch buffer between steps so every step starts cold.
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=case.key.device)

    def step():
        pa.paged_kv_append(kv.k_cache, kv.v_cache, case.key, case.value, kv.block_tables,
                           kv.context_lens, case.query_start_loc)

    timer = KernelTimer(pa, torch, steps)
    ms = timed_steps(torch, step, steps, warmup, timer, between=lambda: scratch.fill_(1))
    kms = timer.mean_ms()
    nbytes = wl.append_bytes(T, kv.context_lens.numel(), Hkv, D, kv.block_size,
                             wl.ELEM_BYTES[case.dtype])
    return {
        "workload": case.name, "kernel_ms": kms, "bytes": nbytes, "new_tokens": T,
        "kernel_GBps": nbytes / (kms * 1e-3) / 1e9,
        "frac_hbm_peak": nbytes / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "step_ms_incl_cache_flush": ms,
    }


def bench_swap(pa, torch, wl, case, steps, warmup):
    """Swap out (device -> pinned host pools) and swap in (host -> device)
    through paged_kv_copy_blocks; bytes are those crossing the host link (each
    moved block of K and V once).  The link ceiling is a plain pinned copy of
    the same size in each direction (the copy engines)."""
    block_bytes = case.dev_k[0].numel() * case.dev_k.element_size()
    ws = torch.empty(pa.paged_kv_copy_blocks_workspace_size(max(case.dev_k.shape[0],
                                                                case.host_k.shape[0])),
                     dtype=torch.uint8, device=case.dev_k.device)
    res = {"workload": case.name, "block_bytes": block_bytes}
    for direction in ("out", "in"):
        if direction == "out":
            args = (case.dev_k, case.dev_v, case.host_k, case.host_v, case.out_map)
            n = wl.copy_count_unique(case.out_map.cpu().numpy(), case.dev_k.shape[0], case.host_k.shape[0])
        else:
            args = (case.host_k, case.host_v, case.dev_k, case.dev_v, case.in_map)
            n = wl.copy_count_unique(case.in_map.cpu().numpy(), case.host_k.shape[0], case.dev_k.shape[0])
        timer = KernelTimer(pa, torch, steps)
        timed_steps(torch, lambda: pa.paged_kv_copy_blocks(*args, workspace=ws), steps, warmup, timer)
        kms = timer.mean_ms()
        nbytes = 2 * n * block_bytes
        res[f"{direction}_kernel_ms"] = kms
        res[f"{direction}_bytes"] = nbytes
        res[f"{direction}_GBps"] = nbytes / (kms * 1e-3) / 1e9
    # link ceiling: contiguous pinned <-> device copies of the swapped size
    nb = res["out_bytes"]
    host = torch.empty(nb, dtype=torch.uint8, pin_memory=True)
    dev = torch.empty(nb, dtype=torch.uint8, device=case.dev_k.device)
    for direction, fn in (("d2h", lambda: host.copy_(dev, non_blocking=True)),
                          ("h2d", lambda: dev.copy_(host, non_blocking=True))):
        ms = timed_steps(torch, fn, steps, warmup)
        res[f"link_{direction}_GBps"] = nb / (ms * 1e-3) / 1e9
    return res


def bench_stream_copy(torch, steps, warmup, nbytes: int = 2 << 30):
    """A plain device-to-device copy of known size: the practical HBM ceiling
    for a read+write stream, and the reference that scales the FETCH_SIZE /
    WRITE_SIZE counters to bytes."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    for _ in range(warmup):
        dst.copy_(src)
    ts = []
    for _ in range(steps):
        s.record()
        dst.copy_(src)
        e.record()
        torch.cuda.synchronize()
        ts.append(s.elapsed_time(e))
    ms = float(np.median(ts))
    return {"workload": "stream_copy", "bytes_read": nbytes, "bytes_written": nbytes,
            "ms": ms, "GBps": 2 * nbytes / (ms * 1e-3) / 1e9}


def bench_stream_copy_lib(pa, torch, steps, warmup, nbytes: int = 2 << 30, shapes=(0, 32, 128)):
    """The library's own read+write stream (pa_stream_copy: the non-temporal
    16-byte loads and stores of the block copy and the append) over a 2 GiB
    copy, for a few grid sizes; the fastest is the practical read+write
    ceiling the copy and append kernels are set beside.  Shapes: one 4 KiB
    chunk per work-group, and grid-stride loops over 32 or 128 work-groups
    per CU."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(3)
    dst = torch.empty_like(src)
    best = None
    sweep = {}
    for wgs in shapes:                    # 0: one 4 KiB chunk per work-group
        timer = KernelTimer(pa, torch, steps)
        for _ in range(warmup):
            pa.pa_stream_copy(src, dst, wgs)
        torch.cuda.synchronize()
        for _ in range(steps):
            timer.arm()
            pa.pa_stream_copy(src, dst, wgs)
            timer.disarm()
        torch.cuda.synchronize()
        ms = float(np.median([s.elapsed_time(e) for s, e in timer.pairs[:timer.i]]))
        gbps = 2 * nbytes / (ms * 1e-3) / 1e9
        sweep[str(wgs)] = round(gbps, 1)
        if best is None or gbps > best[1]:
            best = (wgs, gbps, ms)
    return {"workload": "stream_copy_lib", "bytes_read": nbytes, "bytes_written": nbytes,
            "ms": best[2], "GBps": best[1], "wgs_per_cu": best[0], "sweep_GBps": sweep,
            "frac_hbm_peak": best[1] / HBM_PEAK_GBS}


def bench_stream_read(pa, torch, steps, warmup, nbytes: int = 4 << 30):
    """A plain device read of known size (the library's read-stream probe):
    the practical HBM ceiling for the read-dominated decode kernels."""
    src = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda:0")
    src.copy_(torch.arange(src.numel(), dtype=torch.int32, device="cuda:0"))
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda:0")
    timer = KernelTimer(pa, torch, steps)
    for _ in range(warmup):
        pa.pa_stream_read(src, sink)
    torch.cuda.synchronize()
    ts = []
    for _ in range(steps):
        timer.arm()
        pa.pa_stream_read(src, sink)
        timer.disarm()
    torch.cuda.synchronize()
    ts = [s.elapsed_time(e) for s, e in timer.pairs[:timer.i]]
    ms = float(np.median(ts))
    return {"workload": "stream_read", "bytes_read": nbytes, "ms": ms,
            "GBps": nbytes / (ms * 1e-3) / 1e9, "frac_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


def bench_mfma_stream(pa, torch, steps, warmup, iters: int = 20000, shapes=(1, 2)):
    """Back-to-back bf16 MFMA 32x32x16 on random operands over the whole GPU
    (the library's matrix-core stream probe), at 1 and 2 work-groups of four
    wavefronts per CU: the matrix cores' practical rate under the power limit
    for random data, the ceiling the prefill is set beside."""
    g = torch.Generator(device="cuda:0").manual_seed(2489)
    ops = torch.randn(1 << 22, device="cuda:0", generator=g).to(torch.bfloat16)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sweep = {}
    best = None
    for w in shapes:
        sink = torch.zeros(cus * w, dtype=torch.float32, device="cuda:0")
        timer = KernelTimer(pa, torch, steps)
        for _ in range(warmup):
            pa.pa_mfma_stream(ops, sink, w, iters)
        torch.cuda.synchronize()
        for _ in range(steps):
            timer.arm()
            pa.pa_mfma_stream(ops, sink, w, iters)
            timer.disarm()
        torch.cuda.synchronize()
        ms = float(np.median([s.elapsed_time(e) for s, e in timer.pairs[:timer.i]]))
        flops = cus * w * 4 * iters * 32 * 2 * 32 * 32 * 16
        tf = flops / (ms * 1e-3) / 1e12
        sweep[str(w)] = round(tf, 1)
        if best is None or tf > best[1]:
            best = (w, tf, ms, flops)
    w, tf, ms, flops = best
    return {"workload": "mfma_stream_bf16", "wgs_per_cu": w, "waves_per_simd": w,
            "flops": flops, "ms": ms, "TFLOPs": tf, "frac_mfma_peak": tf / MFMA_BF16_PEAK_TFS,
            "sweep_TFLOPs": sweep}


def cpu_baseline(torch, wl, case, budget_s: float, min_s: float = 10.0):
    """The fp64 oracle on the host cores, sequence by sequence, until the time
    budget is spent (whole passes are repeated until at least ``min_s``);
    reported in the metric's unit (KV GB/s)."""
    from oracle import decode_ref
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    kv = case.kv
    B, Hq, D = case.query.shape
    Hkv = kv.k_cache.shape[1]
    ctx_all = kv.context_lens.cpu().numpy()
    bs = kv.block_size
    calls, nbytes, spent, passes = 0, 0, 0.0, 0
    cache = {}
    while spent < max(min_s, 1e-9) and passes < 50:
        for b in range(B):
            n = int(ctx_all[b])
            nb = (n + bs - 1) // bs
            if b not in cache:
                ids = kv.block_tables[b, :nb].long()
                k = kv.k_cache.index_select(0, ids).cpu()
                v = kv.v_cache.index_select(0, ids).cpu()
                q = case.query[b:b + 1].cpu()
                cache[b] = tuple((x.float() if x.dtype == torch.bfloat16 else x).numpy()
                                 for x in (q, k, v))
            q, k, v = cache[b]
            t0 = time.perf_counter()
            decode_ref(q, k, v, np.arange(nb, dtype=np.int32)[None], np.array([n]), case.scale)
            spent += time.perf_counter() - t0
            calls += 1
            nbytes += wl.decode_kv_bytes([n], Hq, Hkv, D, bs, wl.ELEM_BYTES[case.dtype])
            if spent >= budget_s:
                break
        passes += 1
        if spent >= budget_s:
            break
    return {
        "value": nbytes / spent / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
        "sample": f"{calls} single-sequence oracle calls over the {B} sequences of {case.name} "
                  f"(all {Hq} heads, {passes} pass(es)), {spent:.1f} s of fp64 numpy",
        "seconds": spent, **host_info(),
    }


def host_info() -> dict:
    """The host the CPU baseline ran on: logical CPUs, the CPUs this process
    may use, and the CPU model."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"os_cpu_count": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "cpu_model": model}


def cpu_prefill_sample(torch, wl, case, budget_s: float = 5.0):
    """The fp64 prefill oracle on the host cores over a bounded sample of the
    prefill workload: every 32nd new-token row of its shortest sequence, all
    heads, repeated until ``budget_s``; reported in GFLOP/s of the visible
    (query, key) pairs, the formula the GPU figure uses."""
    from oracle import prefill_ref
    kv = case.kv
    ctx = kv.context_lens.cpu().numpy()
    qsl = case.query_start_loc.cpu().numpy()
    b = int(np.argmin(ctx))
    n = int(ctx[b])
    q_b = int(qsl[b + 1] - qsl[b])
    nb = (n + kv.block_size - 1) // kv.block_size
    ids = kv.block_tables[b, :nb].long()
    k = kv.k_cache.index_select(0, ids).float().cpu().numpy()
    v = kv.v_cache.index_select(0, ids).float().cpu().numpy()
    q = case.query[int(qsl[b]):int(qsl[b + 1])].float().cpu().numpy()
    rows = np.arange(0, q_b, 32)
    T, Hq, D = case.query.shape
    pairs = int(sum(n - q_b + int(t) + 1 for t in rows))
    flops_per_call = 4 * D * Hq * pairs
    calls, spent = 0, 0.0
    while spent < budget_s and calls < 20:
        t0 = time.perf_counter()
        prefill_ref(q, k, v, np.arange(nb, dtype=np.int32)[None], np.array([n]),
                    np.array([0, q_b]), case.scale, rows=rows)
        spent += time.perf_counter() - t0
        calls += 1
    return {"value": flops_per_call * calls / spent / 1e9, "unit": "GFLOP/s", "kind": "oracle",
            "sample": f"{len(rows)} of the {q_b} new-token rows (every 32nd) of the shortest "
                      f"sequence ({n} keys), all {Hq} heads, {calls} call(s), {spent:.1f} s of fp64 numpy"}


def cpu_copy_sample(torch, wl, case):
    """The block-copy oracle on the host cores over the whole copy workload
    (K and V pools, one call each), in GB/s of the copy formula."""
    from oracle import copy_blocks_ref
    m = case.src_to_dst.cpu().numpy()
    n = wl.copy_count_unique(m, case.src_k.shape[0], case.dst_k.shape[0])
    block_bytes = case.src_k[0].numel() * case.src_k.element_size()
    host = [t.cpu().view(torch.int16).numpy() for t in (case.src_k, case.dst_k, case.src_v, case.dst_v)]
    t0 = time.perf_counter()
    copy_blocks_ref(host[0], host[1], m)
    copy_blocks_ref(host[2], host[3], m)
    spent = time.perf_counter() - t0
    return {"value": wl.copy_bytes(n, block_bytes) / spent / 1e9, "unit": "GB/s", "kind": "oracle",
            "sample": f"the whole {case.name or 'copy'} workload ({n} blocks of K and of V), "
                      f"{spent:.2f} s"}


def roofline(bound: str, kernel: str, achieved: float, peak: float, unit: str, kernel_ms: float,
             work: int, work_unit: str, traffic, **extra) -> dict:
    """One roofline object: the kernel's algorithmic work per launch over its
    event-timed duration, against the MI355X peak of its bound."""
    return {"bound": bound, "kernel": kernel, "achieved": round(achieved, 2), "peak": peak,
            "unit": unit, "frac": round(achieved / peak, 4), "traffic": traffic,
            "kernel_ms": round(kernel_ms, 5), "work_per_launch": work, "work_unit": work_unit,
            **extra}


def hbm_traffic(kernel_files, launches_key: str):
    """Calibrated HBM bytes per launch from the committed PMC summary, or None
    when the kernel sources changed since the counters were taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", "hbm_traffic.md")
    try:
        text = open(path).read()
        data = json.loads(re.search(r"```json\n(.*?)\n```", text, re.S).group(1))
    except Exception:
        return None
    h = hashlib.sha256()
    for f in kernel_files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    entry = data.get(launches_key)
    if not entry or entry.get("source_sha256") != h.hexdigest():
        return None
    return entry.get("bytes_per_launch")


def rooflines(extra: dict, head: dict) -> dict:
    """One roofline object per workload: the decode kernels, the copy and the
    append against HBM, the prefill kernel against the dense bf16 matrix
    peak (its HBM traffic is reported beside it)."""
    out = {"llama7b_decode_f16": roofline(
        "hbm", "decode_kernel", head["kernel_GBps"], HBM_PEAK_GBS, "GB/s", head["kernel_ms"],
        head["bytes"], "bytes", hbm_traffic(SOURCES["decode"], "decode_kernel/llama7b_decode_f16"))}
    kernels = {"gqa_decode_bf16": "decode_mfma_kernel", "long_decode_f16": "decode_kernel"}
    for name, kern in kernels.items():
        r = extra.get(name)
        if r:
            out[name] = roofline("hbm", kern, r["kernel_GBps"], HBM_PEAK_GBS, "GB/s",
                                 r["kernel_ms"], r["bytes"], "bytes",
                                 hbm_traffic(SOURCES["decode"], f"{kern}/{name}"))
    r = extra.get("prefill_bf16")
    if r:
        out["prefill_bf16"] = roofline(
            "mfma", "prefill_kernel", r["kernel_TFLOPs"], MFMA_BF16_PEAK_TFS, "TFLOP/s",
            r["kernel_ms"], r["flops"], "flop",
            hbm_traffic(SOURCES["prefill"], "prefill_kernel/prefill_bf16"),
            algorithmic_hbm_bytes=r.get("hbm_bytes"))
    for name, kern, src in (("copy_bf16", "copy_kernel", "copy"),
                            ("append_bf16", "append_kernel", "append")):
        r = extra.get(name)
        if r:
            out[name] = roofline("hbm", kern, r["kernel_GBps"], HBM_PEAK_GBS, "GB/s",
                                 r["kernel_ms"], r["bytes"], "bytes",
                                 hbm_traffic(SOURCES[src], f"{kern}/{name}"))
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # A GPU fresh from idle raises its shader clock over the first few
    # hundred milliseconds of load; 300 untimed steps of each workload
    # (0.1-0.4 s) let the timed steps run at the clock the kernel sustains.
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--quick", action="store_true", help="headline workload only")
    ap.add_argument("--only", default=None, choices=["llama7b_decode_f16", "gqa_decode_bf16",
                                                       "long_decode_f16", "prefill_bf16",
                                                       "prefill_bf16_halftile",
                                                       "copy_bf16", "append_bf16", "swap_bf16",
                                                       "stream_copy", "stream_copy_lib", "stream_read",
                                                       "mfma_stream", "prefill_unfused_bf16",
                                                       "tiny_decode_f32", "block_manager"],
                    help="run one workload, print its result object and exit (profiling)")
    ap.add_argument("--cpu-budget", type=float, default=20.0,
                    help="seconds of oracle time for the CPU baseline (0 = skip)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures a single GPU; --gpus {args.gpus} is not supported "
              "(this library has no multi-GPU path)", file=sys.stderr)
        return 2

    import torch

    import paged_kv_cache_248_amd as pa
    import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    dev = "cuda:0"
    pa.load_library()
    props = torch.cuda.get_device_properties(0)
    log(f"device: {props.name} ({getattr(props, 'gcnArchName', '?')}), "
        f"{props.multi_processor_count} CUs")

    if args.only == "stream_copy":
        print(json.dumps(bench_stream_copy(torch, args.steps, args.warmup)), flush=True)
        return 0
    if args.only == "block_manager":
        print(json.dumps(bench_block_manager(pa, wl)), flush=True)
        return 0
    if args.only == "tiny_decode_f32":
        print(json.dumps(bench_tiny_decode(pa, torch, wl, args.steps, args.warmup)), flush=True)
        return 0
    if args.only == "stream_copy_lib":
        print(json.dumps(bench_stream_copy_lib(pa, torch, args.steps, args.warmup)), flush=True)
        return 0
    if args.only == "stream_read":
        print(json.dumps(bench_stream_read(pa, torch, args.steps, args.warmup)), flush=True)
        return 0
    if args.only == "mfma_stream":
        print(json.dumps(bench_mfma_stream(pa, torch, min(args.steps, 20), min(args.warmup, 20))),
              flush=True)
        return 0
    if args.only == "prefill_unfused_bf16":
        log("generating prefill_bf16 ...")
        case = wl.prefill_bf16(device=dev)
        r = bench_prefill_unfused(pa, torch, wl, case, max(3, args.steps // 10),
                                  max(2, args.warmup // 100))
        print(json.dumps(r), flush=True)
        return 0
    if args.only == "prefill_bf16_halftile":
        log("generating prefill_bf16 ...")
        case = wl.prefill_bf16(device=dev)
        r = bench_prefill(pa, torch, wl, case, args.steps, args.warmup, kernel="halftile")
        print(json.dumps(r), flush=True)
        return 0
    if args.only:
        log(f"generating {args.only} ...")
        case = wl.WORKLOADS[args.only](device=dev)
        if args.only.startswith("prefill"):
            r = bench_prefill(pa, torch, wl, case, args.steps, args.warmup)
        elif args.only.startswith("copy"):
            r = bench_copy(pa, torch, wl, case, args.steps, args.warmup)
        elif args.only.startswith("append"):
            r = bench_append(pa, torch, wl, case, args.steps, args.warmup)
        elif args.only.startswith("swap"):
            r = bench_swap(pa, torch, wl, case, max(5, args.steps // 10), max(5, args.warmup // 30))
        else:
            r = bench_decode(pa, torch, wl, case, args.steps, args.warmup)
        print(json.dumps(r), flush=True)
        return 0

    log("generating llama7b_decode_f16 ...")
    head = wl.llama7b_decode_f16(device=dev)
    res = bench_decode(pa, torch, wl, head, args.steps, args.warmup)
    log(f"  decode: {res['ms_per_step']:.3f} ms/step, {res['GBps']:.0f} GB/s "
        f"(kernel {res['kernel_ms']:.3f} ms, {res['kernel_GBps']:.0f} GB/s)")

    extra = {}
    cpu_other = {}
    if not args.quick:
        r = bench_tiny_decode(pa, torch, wl, args.steps, args.warmup)
        log(f"  tiny_decode_f32: {r['eager_us_per_call']:.1f} us/call eager, "
            f"{r['graph_us_per_call']:.1f} us/call as a graph replay")
        extra["tiny_decode_f32"] = r
        for name in ("gqa_decode_bf16", "long_decode_f16"):
            log(f"generating {name} ...")
            case = wl.WORKLOADS[name](device=dev)
            r = bench_decode(pa, torch, wl, case, args.steps, args.warmup)
            log(f"  {name}: {r['ms_per_step']:.3f} ms/step, {r['GBps']:.0f} GB/s "
                f"(kernel {r['kernel_GBps']:.0f} GB/s)")
            extra[name] = r
            del case
            torch.cuda.empty_cache()
        log("generating prefill_bf16 ...")
        pc = wl.prefill_bf16(device=dev)
        r = bench_prefill(pa, torch, wl, pc, args.steps, args.warmup)
        log(f"  prefill: {r['ms_per_step']:.3f} ms/step, {r['kernel_TFLOPs']:.0f} TFLOP/s")
        extra["prefill_bf16"] = r
        h = bench_prefill(pa, torch, wl, pc, args.steps, args.warmup, kernel="halftile")
        h["vs_pingpong"] = h["kernel_TFLOPs"] / r["kernel_TFLOPs"]
        log(f"  prefill, half-tile schedule: {h['kernel_TFLOPs']:.0f} TFLOP/s "
            f"({h['vs_pingpong']:.3f} of the ping-pong kernel)")
        extra["prefill_bf16_halftile"] = h
        u = bench_prefill_unfused(pa, torch, wl, pc, max(3, args.steps // 10),
                                  max(2, args.warmup // 100))
        u["fused_speedup"] = u["ms_per_step"] / r["ms_per_step"]
        log(f"  unfused prefill: {u['ms_per_step']:.3f} ms/step, {u['TFLOPs']:.0f} TFLOP/s; "
            f"fused is {u['fused_speedup']:.2f}x faster")
        extra["prefill_unfused_bf16"] = u
        if args.cpu_budget > 0:
            log("timing the fp64 prefill oracle on a sample ...")
            cpu_other["prefill_bf16"] = cpu_prefill_sample(torch, wl, pc)
            log(f"  prefill oracle: {cpu_other['prefill_bf16']['value']:.2f} GFLOP/s")
        del pc
        torch.cuda.empty_cache()
        log("generating copy_bf16 ...")
        cc = wl.copy_bf16(device=dev)
        r = bench_copy(pa, torch, wl, cc, args.steps, args.warmup)
        log(f"  copy: {r['kernel_ms']:.3f} ms, {r['kernel_GBps']:.0f} GB/s")
        extra["copy_bf16"] = r
        if args.cpu_budget > 0:
            cpu_other["copy_bf16"] = cpu_copy_sample(torch, wl, cc)
            log(f"  copy oracle: {cpu_other['copy_bf16']['value']:.2f} GB/s")
        del cc
        torch.cuda.empty_cache()
        log("generating append_bf16 ...")
        ac = wl.append_bf16(device=dev)
        r = bench_append(pa, torch, wl, ac, args.steps, args.warmup)
        log(f"  append: {r['kernel_ms']:.4f} ms, {r['kernel_GBps']:.0f} GB/s")
        extra["append_bf16"] = r
        del ac
        torch.cuda.empty_cache()
        log("generating swap_bf16 ...")
        sc = wl.swap_bf16(device=dev)
        r = bench_swap(pa, torch, wl, sc, max(5, args.steps // 10), max(5, args.warmup // 30))
        log(f"  swap: out {r['out_GBps']:.1f} GB/s, in {r['in_GBps']:.1f} GB/s "
            f"(plain pinned copies: d2h {r['link_d2h_GBps']:.1f}, h2d {r['link_h2d_GBps']:.1f})")
        extra["swap_bf16"] = r
        del sc
        torch.cuda.empty_cache()
        r = bench_block_manager(pa, wl)
        log(f"  block manager decode step (256 requests): {r['native_us_per_step']:.1f} us native, "
            f"{r['oracle_us_per_step']:.0f} us oracle")
        extra["block_manager"] = r
        r = bench_stream_read(pa, torch, min(args.steps, 50), min(args.warmup, 20))
        log(f"  plain read stream: {r['GBps']:.0f} GB/s")
        extra["stream_read"] = r
        r = bench_stream_copy_lib(pa, torch, min(args.steps, 30), min(args.warmup, 10))
        log(f"  library copy stream: {r['GBps']:.0f} GB/s (read + write; shape {r['wgs_per_cu']}: "
            f"0 = 4 KiB per work-group, else work-groups per CU)")
        extra["stream_copy_lib"] = r
        for name in ("copy_bf16", "append_bf16"):
            extra[name]["frac_of_copy_stream"] = round(extra[name]["kernel_GBps"] / r["GBps"], 4)
            # the same probe at the kernel's own size (launch and drain costs
            # weigh more on a small transfer)
            half = extra[name]["bytes"] // 2 // 16 * 16
            rs = bench_stream_copy_lib(pa, torch, min(args.steps, 30), min(args.warmup, 10),
                                       nbytes=half, shapes=(0,))
            extra[name]["copy_stream_same_size_GBps"] = round(rs["GBps"], 1)
            extra[name]["frac_of_copy_stream_same_size"] = round(
                extra[name]["kernel_GBps"] / rs["GBps"], 4)
        for name in ("llama7b_decode_f16", "gqa_decode_bf16", "long_decode_f16"):
            if name in extra:
                extra[name]["frac_of_read_stream"] = round(
                    extra[name]["kernel_GBps"] / extra["stream_read"]["GBps"], 4)
        r = bench_mfma_stream(pa, torch, min(args.steps, 20), min(args.warmup, 20))
        log(f"  matrix-core stream: {r['TFLOPs']:.0f} TFLOP/s bf16 "
            f"({r['wgs_per_cu']} work-group(s) of 4 waves per CU)")
        extra["mfma_stream"] = r
        if "prefill_bf16" in extra:
            extra["prefill_bf16"]["frac_of_mfma_stream"] = round(
                extra["prefill_bf16"]["kernel_TFLOPs"] / r["TFLOPs"], 4)
        torch.cuda.empty_cache()

    cpu = None
    if args.cpu_budget > 0:
        log("timing the fp64 oracle on host cores ...")
        cpu = cpu_baseline(torch, wl, head, args.cpu_budget)
        log(f"  oracle: {cpu['value']:.3f} GB/s on {cpu['cores']} threads ({cpu['sample']})")

    line = {
        "metric": METRIC,
        "value": round(res["GBps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "llama7b_decode_f16",
            "num_seqs": res["num_seqs"], "num_heads": res["num_heads"],
            "num_kv_heads": res["num_kv_heads"], "head_dim": res["head_dim"],
            "block_size": res["block_size"], "context": "uniform [512, 4096]",
            "context_mean": res["context_mean"], "pool_blocks": res["pool_blocks"],
            "partition_size": res["partition_size"], "accumulation": "f32",
            "parallelism": "single GPU",
        },
        "roofline": roofline("hbm", "decode_kernel", res["kernel_GBps"], HBM_PEAK_GBS, "GB/s",
                             res["kernel_ms"], res["bytes"], "bytes",
                             hbm_traffic(SOURCES["decode"], "decode_kernel/llama7b_decode_f16"),
                             bytes_per_launch=res["bytes"]),
        "rooflines": rooflines(extra, res),
        "cpu_baseline": cpu,
        "cpu_oracle_other": cpu_other or None,
        "tokens_per_s": round(res["tokens_per_s"], 1),
        "extra": extra,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
