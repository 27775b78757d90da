"""Unfused causal paged prefill (S and P written to HBM, library GEMMs) on
the GPU against the fp64 oracle: the same function as the fused prefill."""

import zlib

import numpy as np
import pytest
import torch

import paged_kv_cache_248_amd as pa
import workloads as wl
from oracle import prefill_ref
from tests._util import assert_close, compact_pool, host, log

pytestmark = pytest.mark.gpu

DEV = "cuda"


def run_unfused(case, workspace=None):
    kv = case.kv
    out = torch.full_like(case.query, float("nan"))
    pa.paged_attn_prefill_unfused(out, case.query, kv.k_cache, kv.v_cache, kv.block_tables,
                                  kv.context_lens, case.query_start_loc, case.scale,
                                  workspace=workspace)
    torch.cuda.synchronize()
    return out


def oracle_full(case):
    kv = case.kv
    return prefill_ref(host(case.query), host(kv.k_cache), host(kv.v_cache),
                       host(kv.block_tables), host(kv.context_lens),
                       host(case.query_start_loc), case.scale)


SMALL = [(dtype, D, Hq, Hkv, bs) for dtype in ("f16", "bf16") for D in (64, 128)
         for (Hq, Hkv) in ((4, 4), (8, 2), (6, 2)) for bs in (16, 32)]


@pytest.mark.parametrize("dtype,D,Hq,Hkv,bs", SMALL)
def test_unfused_small_against_oracle(dtype, D, Hq, Hkv, bs):
    rng = np.random.default_rng(zlib.crc32(repr(("unfused", dtype, D, Hq, Hkv, bs)).encode()))
    # one new token, none (skipped), a ragged tail, several hundred
    ql = np.array([1, 0, 37, int(rng.integers(150, 400))])
    pre = np.array([0, 20, int(rng.integers(0, 70)), int(rng.integers(100, 300))])
    log(f"unfused small dtype={dtype} D={D} Hq={Hq} Hkv={Hkv} bs={bs} pre={pre.tolist()} "
        f"q={ql.tolist()}")
    case = wl.make_prefill(pre, ql, Hq, Hkv, D, bs, dtype, seed=int(rng.integers(1 << 30)),
                           device=DEV, poison=True)
    e = assert_close(host(run_unfused(case)), oracle_full(case), dtype, "unfused small")
    log(f"  max rel err {e:.3e}")


@pytest.mark.parametrize("bs", [8, 256])
def test_unfused_block_sizes(bs):
    case = wl.make_prefill([5, 300], [64, 90], 8, 2, 128, bs, "bf16", seed=bs, device=DEV,
                           poison=True)
    assert_close(host(run_unfused(case)), oracle_full(case), "bf16", f"unfused bs={bs}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_unfused_long_rows(dtype):
    """Contexts of 20000 and 32768 keys: the softmax holds 32 four-key chunks
    per thread (its largest row form) and S rows of 80-128 KiB."""
    case = wl.make_prefill([20000 - 3, 32768 - 2], [3, 2], 8, 2, 128, 32, dtype, seed=21,
                           device=DEV, poison=True)
    e = assert_close(host(run_unfused(case)), oracle_full(case), dtype, "unfused long rows")
    log(f"unfused long rows {dtype}: max rel err {e:.3e}")


def test_unfused_matches_fused_prefill():
    case = wl.make_prefill([0, 130, 700], [200, 129, 64], 16, 4, 128, 16, "bf16", seed=5,
                           device=DEV)
    kv = case.kv
    fused = torch.empty_like(case.query)
    pa.paged_attn_prefill(fused, case.query, kv.k_cache, kv.v_cache, kv.block_tables,
                          kv.context_lens, case.query_start_loc, case.scale, case.max_query_len,
                          kv.max_context_len)
    unf = run_unfused(case)
    ref = oracle_full(case)
    assert_close(host(fused), ref, "bf16", "fused")
    assert_close(host(unf), ref, "bf16", "unfused")


def test_unfused_block_permutation_is_bit_identical():
    case = wl.make_prefill([10, 200], [90, 150], 8, 2, 128, 16, "bf16", seed=12, device=DEV)
    kv = case.kv
    base = run_unfused(case)
    g = torch.Generator(device="cpu").manual_seed(2)
    perm = torch.randperm(kv.k_cache.shape[0], generator=g).to(DEV)
    k2 = torch.empty_like(kv.k_cache)
    v2 = torch.empty_like(kv.v_cache)
    k2[perm] = kv.k_cache
    v2[perm] = kv.v_cache
    out = torch.empty_like(base)
    pa.paged_attn_prefill_unfused(out, case.query, k2, v2,
                                  perm[kv.block_tables.long()].to(torch.int32), kv.context_lens,
                                  case.query_start_loc, case.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, base)


def test_unfused_workload_full_size_sampled():
    """The 8-sequence bf16 workload (2048 new tokens each, prefixes up to
    8192) in the configuration the benchmark times, on sampled rows."""
    case = wl.prefill_bf16(device=DEV)
    kv = case.kv
    ctx = host(kv.context_lens)
    qsl = host(case.query_start_loc)
    out = run_unfused(case)
    assert torch.isfinite(out.float()).all()
    order = np.argsort(ctx)
    seqs = sorted({int(order[0]), int(order[-1])})
    k, v, tables, cl = compact_pool(kv, seqs)
    rng = np.random.default_rng(1)
    for i, b in enumerate(seqs):
        q_b = int(qsl[b + 1] - qsl[b])
        rows = np.unique(np.concatenate([[0, 1, 63, 64, q_b - 1], rng.integers(0, q_b, size=16)]))
        q = host(case.query[int(qsl[b]):int(qsl[b + 1])])
        heads = [0, 5, 31]
        ref = prefill_ref(q, k, v, tables[i:i + 1], cl[i:i + 1], np.array([0, q_b]), case.scale,
                          rows=rows, heads=heads)
        got = host(out[int(qsl[b]):int(qsl[b + 1])])
        e = assert_close(got[rows][:, heads], ref[rows][:, heads], "bf16", f"seq {b}")
        log(f"  unfused seq {b} (ctx {ctx[b]}): {len(rows)} rows x {len(heads)} heads, "
            f"max rel err {e:.3e}")
