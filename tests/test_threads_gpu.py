"""Decode and prefill called from several host threads at once, each thread
on a stream of its own.  The threads share the library's per-device caches
(CU count, resident work-groups per CU, the prefill kernel's LDS attribute);
every result must be bit-identical to the one a single thread computes."""

import threading

import pytest
import torch

import paged_kv_cache_248_amd as pa
import workloads as wl
from tests._util import log

pytestmark = pytest.mark.gpu

DEV = "cuda"
THREADS = 6
ROUNDS = 4


def _decode(case):
    kv = case.kv
    out = torch.empty_like(case.query)
    pa.paged_attn_decode(out, case.query, kv.k_cache, kv.v_cache, kv.block_tables,
                         kv.context_lens, case.scale, kv.max_context_len,
                         partition_size=case.partition_size)
    return out


def _prefill(case):
    kv = case.kv
    out = torch.empty_like(case.query)
    pa.paged_attn_prefill(out, case.query, kv.k_cache, kv.v_cache, kv.block_tables,
                          kv.context_lens, case.query_start_loc, case.scale, case.max_query_len,
                          kv.max_context_len)
    return out


def test_concurrent_threads_match_single_thread():
    ops = [
        ("decode mha f16", _decode,
         wl.make_decode([1, 40, 700, 1500], 8, 8, 128, 16, "f16", seed=31, device=DEV)),
        ("decode gqa bf16", _decode,
         wl.make_decode([3, 513, 2100, 90], 32, 4, 128, 16, "bf16", seed=32, device=DEV)),
        ("prefill bf16 d128", _prefill,
         wl.make_prefill([0, 200, 35], [130, 64, 7], 16, 4, 128, 16, "bf16", seed=33,
                         device=DEV)),
        ("prefill f16 d64", _prefill,
         wl.make_prefill([17, 0], [90, 200], 8, 8, 64, 32, "f16", seed=34, device=DEV)),
    ]
    torch.cuda.synchronize()
    expected = [fn(case) for _, fn, case in ops]
    torch.cuda.synchronize()

    results = [[None] * len(ops) for _ in range(THREADS)]
    errors = []

    def worker(t):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for r in range(ROUNDS):
                    # each thread starts at a different op so the calls overlap
                    for i in range(len(ops)):
                        k = (i + t + r) % len(ops)
                        results[t][k] = ops[k][1](ops[k][2])
            s.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append((t, repr(e)))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(THREADS)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=60)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for t in range(THREADS):
        for k, (name, _, _) in enumerate(ops):
            assert torch.equal(results[t][k], expected[k]), f"thread {t}: {name} differs"
    log(f"{THREADS} threads x {ROUNDS} rounds x {len(ops)} ops: bit-identical")
