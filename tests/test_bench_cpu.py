"""bench.py contract checks that need no GPU: one GPU only, and the host
helpers (algorithmic work formulas, CPU oracle samples, block-manager step)
on small synthetic inputs."""

import os
import subprocess
import sys

import numpy as np
import torch

from conftest import ROOT

import bench
import paged_kv_cache_248_amd as pa
import workloads as wl


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "single GPU" in r.stderr and r.stdout == ""


def test_decode_bytes_follow_the_kv_formula():
    # K and V of every token once per kv head, q read + out written, table ids, lengths
    ctx = np.array([100, 37])
    got = wl.decode_kv_bytes(ctx, 8, 2, 128, 16, 2)
    want = (137 * 2 * 128 * 2 * 2) + 2 * 2 * 8 * 128 * 2 + 4 * (7 + 3) + 4 * 2
    assert got == want


def test_prefill_flops_count_visible_pairs_only():
    # one sequence, prefix 3, two new tokens: rows see 4 and 5 keys
    assert wl.prefill_flops(np.array([5]), np.array([2]), 4, 64) == 4 * 64 * 4 * (4 + 5)


def test_cpu_oracle_samples_on_small_inputs():
    c = wl.make_prefill([100, 40], [64, 33], 8, 2, 128, 16, "bf16", seed=3)
    r = bench.cpu_prefill_sample(torch, wl, c, budget_s=0.2)
    assert r["unit"] == "GFLOP/s" and r["value"] > 0 and r["kind"] == "oracle"
    cc = wl.make_copy(64, 32, (2, 16, 64), "bf16", seed=5)
    r = bench.cpu_copy_sample(torch, wl, cc)
    assert r["unit"] == "GB/s" and r["value"] > 0


def test_block_manager_step_runs_native_and_oracle():
    r = bench.bench_block_manager(pa, wl, steps=10)
    assert r["native_us_per_step"] > 0 and r["oracle_us_per_step"] > 0
