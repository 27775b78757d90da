"""Causal paged prefill on the GPU against the fp64 oracle, for both kernel
schedules the library exports (paged_attn_prefill, the ping-pong default, and
paged_attn_prefill_halftile)."""

import zlib

import numpy as np
import pytest
import torch

import paged_kv_cache_248_amd as pa
import workloads as wl
from oracle import decode_ref, prefill_ref
from tests._util import TOL, assert_close, compact_pool, host, log, rel_err

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(params=["pingpong", "halftile"])
def prefill(request):
    """The prefill entry point under test."""
    return {"pingpong": pa.paged_attn_prefill,
            "halftile": pa.paged_attn_prefill_halftile}[request.param]


def run_prefill(case, prefill):
    kv = case.kv
    out = torch.full_like(case.query, float("nan"))
    prefill(out, case.query, kv.k_cache, kv.v_cache, kv.block_tables, kv.context_lens,
            case.query_start_loc, case.scale, case.max_query_len, kv.max_context_len)
    torch.cuda.synchronize()
    return out


def oracle_full(case):
    kv = case.kv
    return prefill_ref(host(case.query), host(kv.k_cache), host(kv.v_cache),
                       host(kv.block_tables), host(kv.context_lens),
                       host(case.query_start_loc), case.scale)


SMALL = []
for dtype in ("f16", "bf16"):
    for D in (64, 128):
        for (Hq, Hkv) in ((4, 4), (8, 2), (8, 4), (16, 2), (6, 2)):
            for bs in (16, 32):
                SMALL.append((dtype, D, Hq, Hkv, bs))


@pytest.mark.parametrize("dtype,D,Hq,Hkv,bs", SMALL)
def test_prefill_small_against_oracle(dtype, D, Hq, Hkv, bs, prefill):
    rng = np.random.default_rng(zlib.crc32(repr(("prefill", dtype, D, Hq, Hkv, bs)).encode()))
    # ragged new-token counts (one, under a tile, several tiles plus a tail)
    ql = np.array([1, 37, 130, int(rng.integers(2, 200))])
    pre = np.array([0, int(rng.integers(0, 70)), 65, int(rng.integers(100, 300))])
    log(f"prefill small dtype={dtype} D={D} Hq={Hq} Hkv={Hkv} bs={bs} pre={pre.tolist()} q={ql.tolist()}")
    case = wl.make_prefill(pre, ql, Hq, Hkv, D, bs, dtype, seed=int(rng.integers(1 << 30)),
                           device=DEV, poison=True)
    e = assert_close(host(run_prefill(case, prefill)), oracle_full(case), dtype, "prefill small")
    log(f"  max rel err {e:.3e}")


BLOCK_SIZES = [(dtype, D, bs) for dtype in ("f16", "bf16") for D in (64, 128)
               for bs in (8, 64, 128, 256)]


@pytest.mark.parametrize("dtype,D,bs", BLOCK_SIZES)
def test_prefill_block_sizes(dtype, D, bs, prefill):
    """Pages smaller than a wavefront's 16 keys of a tile (8) and larger than a
    64-key tile (128, 256): block ids per load instruction and slot offsets
    that change from tile to tile inside one page; contexts ending mid-page."""
    rng = np.random.default_rng(zlib.crc32(repr(("prefill-bs", dtype, D, bs)).encode()))
    ql = np.array([3, 64, 129, int(rng.integers(40, 260))])
    pre = np.array([int(rng.integers(0, 9)), 250, int(rng.integers(300, 700)), 1])
    log(f"prefill block size dtype={dtype} D={D} bs={bs} pre={pre.tolist()} q={ql.tolist()}")
    case = wl.make_prefill(pre, ql, 8, 2, D, bs, dtype, seed=int(rng.integers(1 << 30)),
                           device=DEV, poison=True)
    e = assert_close(host(run_prefill(case, prefill)), oracle_full(case), dtype, "prefill block size")
    log(f"  max rel err {e:.3e}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prefill_large_score_gap_inside_a_tile(dtype, prefill):
    """Keys 4..7 of every 8 score about 255 log2 units above the others.  In
    the S^T accumulator those keys sit in the other half of the wavefront
    (lane l vs l + 32), so the row maximum must combine both halves: a
    maximum over one half only would overflow exp2 on the other."""
    ql = np.array([40, 100])
    pre = np.array([30, 200])
    case = wl.make_prefill(pre, ql, 8, 2, 128, 16, dtype, seed=11, device=DEV)
    kv = case.kv
    slots = torch.arange(kv.k_cache.shape[2], device=DEV)
    big = (slots % 8 >= 4).view(1, 1, -1, 1)
    kv.k_cache.copy_(torch.where(big, torch.full_like(kv.k_cache, 4.0),
                                 torch.full_like(kv.k_cache, 0.1)))
    case.query.fill_(4.0)
    out = run_prefill(case, prefill)
    assert torch.isfinite(out.float()).all()
    assert_close(host(out), oracle_full(case), dtype, "prefill score gap")


def test_prefill_no_prefix_is_plain_causal(prefill):
    case = wl.make_prefill([0, 0], [200, 64], 8, 2, 128, 16, "bf16", seed=3, device=DEV)
    assert_close(host(run_prefill(case, prefill)), oracle_full(case), "bf16", "no prefix")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prefill_single_new_token_matches_decode(dtype, prefill):
    ctx = np.array([1, 20, 300, 1500])
    case = wl.make_decode(ctx, 8, 2, 128, 16, dtype, seed=4, device=DEV)
    kv = case.kv
    dec = torch.empty_like(case.query)
    pa.paged_attn_decode(dec, case.query, kv.k_cache, kv.v_cache, kv.block_tables,
                         kv.context_lens, case.scale, kv.max_context_len)
    pre = torch.empty_like(case.query)
    qsl = torch.arange(len(ctx) + 1, dtype=torch.int32, device=DEV)
    prefill(pre, case.query, kv.k_cache, kv.v_cache, kv.block_tables, kv.context_lens, qsl,
            case.scale, 1, kv.max_context_len)
    torch.cuda.synchronize()
    assert rel_err(host(pre), host(dec).astype(np.float64)) <= TOL[dtype]
    ref = decode_ref(host(case.query), host(kv.k_cache), host(kv.v_cache), host(kv.block_tables),
                     host(kv.context_lens), case.scale)
    assert_close(host(pre), ref, dtype, "q=1 prefill")


def test_prefill_block_permutation_is_bit_identical(prefill):
    case = wl.make_prefill([10, 200], [90, 150], 8, 2, 128, 16, "bf16", seed=12, device=DEV)
    kv = case.kv
    base = run_prefill(case, prefill)
    g = torch.Generator(device="cpu").manual_seed(2)
    perm = torch.randperm(kv.k_cache.shape[0], generator=g).to(DEV)
    k2 = torch.empty_like(kv.k_cache)
    v2 = torch.empty_like(kv.v_cache)
    k2[perm] = kv.k_cache
    v2[perm] = kv.v_cache
    out = torch.empty_like(base)
    prefill(out, case.query, k2, v2, perm[kv.block_tables.long()].to(torch.int32),
            kv.context_lens, case.query_start_loc, case.scale, case.max_query_len,
            kv.max_context_len)
    torch.cuda.synchronize()
    assert torch.equal(out, base)


def test_prefill_workload_full_size_sampled(prefill):
    case = wl.prefill_bf16(device=DEV)
    kv = case.kv
    ctx = host(kv.context_lens)
    qsl = host(case.query_start_loc)
    log(f"prefill_bf16: ctx={ctx.tolist()} T={case.query.shape[0]}")
    out = run_prefill(case, prefill)
    assert torch.isfinite(out.float()).all()
    order = np.argsort(ctx)
    seqs = sorted({int(order[0]), int(order[-1])})
    k, v, tables, cl = compact_pool(kv, seqs)
    rng = np.random.default_rng(0)
    for i, b in enumerate(seqs):
        q_b = int(qsl[b + 1] - qsl[b])
        rows = np.unique(np.concatenate([[0, 1, 31, 32, 63, 64, q_b - 1],
                                         rng.integers(0, q_b, size=24)]))
        q = host(case.query[int(qsl[b]):int(qsl[b + 1])])
        heads = [0, 3, 4, 31]
        ref = prefill_ref(q, k, v, tables[i:i + 1], cl[i:i + 1], np.array([0, q_b]), case.scale,
                          rows=rows, heads=heads)
        got = host(out[int(qsl[b]):int(qsl[b + 1])])
        e = assert_close(got[rows][:, heads], ref[rows][:, heads], "bf16", f"seq {b}")
        log(f"  seq {b} (ctx {ctx[b]}): {len(rows)} rows x {len(heads)} heads, max rel err {e:.3e}")


@pytest.mark.parametrize("dtype,bs", [("bf16", 32), ("f16", 16), ("bf16", 8)])
def test_prefill_long_context(dtype, bs, prefill):
    """Contexts of 32768 and 20000 keys (prefixes of 32568 and 19900 tokens):
    page indices and key offsets at the top of the supported range, several
    hundred key tiles per query tile; sampled rows against the oracle."""
    pre = np.array([32768 - 200, 20000 - 100])
    ql = np.array([200, 100])
    case = wl.make_prefill(pre, ql, 8, 2, 128, bs, dtype, seed=41 + bs, device=DEV, poison=True)
    kv = case.kv
    out = run_prefill(case, prefill)
    assert torch.isfinite(out.float()).all()
    rows = np.array([0, 1, 63, 64, 127, 199, 200, 201, 263, 299])
    ref = prefill_ref(host(case.query), host(kv.k_cache), host(kv.v_cache),
                      host(kv.block_tables), host(kv.context_lens),
                      host(case.query_start_loc), case.scale, rows=rows)
    e = assert_close(host(out)[rows], ref[rows], dtype, "long-context prefill")
    log(f"long-context prefill {dtype} bs={bs}: max rel err {e:.3e}")
