"""Paged decode on the GPU against the fp64 oracle (same seeded inputs)."""

import zlib

import numpy as np
import pytest
import torch

import paged_kv_cache_248_amd as pa
import workloads as wl
from oracle import decode_ref
from tests._util import TOL, assert_close, compact_pool, host, log, rel_err

pytestmark = pytest.mark.gpu

DEV = "cuda"


def run_decode(case, partition_size=None, max_context_len=None):
    kv = case.kv
    out = torch.full_like(case.query, float("nan"))
    part = case.partition_size if partition_size is None else partition_size
    pa.paged_attn_decode(out, case.query, kv.k_cache, kv.v_cache, kv.block_tables,
                         kv.context_lens, case.scale,
                         kv.max_context_len if max_context_len is None else max_context_len,
                         partition_size=part)
    torch.cuda.synchronize()
    return out


def oracle_full(case):
    kv = case.kv
    return decode_ref(host(case.query), host(kv.k_cache), host(kv.v_cache),
                      host(kv.block_tables), host(kv.context_lens), case.scale)


def oracle_sampled(case, seqs, heads):
    kv = case.kv
    k, v, tables, cl = compact_pool(kv, seqs)
    q = host(case.query[seqs])
    ref = decode_ref(q, k, v, tables, cl, case.scale, heads=heads)
    return ref


SMALL = []
for dtype in ("f32", "f16", "bf16"):
    for D in (64, 128):
        for (Hq, Hkv) in ((4, 4), (8, 2), (8, 4), (16, 2), (12, 2)):
            for bs in (16, 32):
                SMALL.append((dtype, D, Hq, Hkv, bs))


@pytest.mark.parametrize("dtype,D,Hq,Hkv,bs", SMALL)
def test_decode_small_against_oracle(dtype, D, Hq, Hkv, bs):
    rng = np.random.default_rng(zlib.crc32(repr((dtype, D, Hq, Hkv, bs)).encode()))
    ctx = np.concatenate([[1, bs, bs + 1, 129], rng.integers(2, 700, size=3)])
    log(f"decode small dtype={dtype} D={D} Hq={Hq} Hkv={Hkv} bs={bs} ctx={ctx.tolist()}")
    case = wl.make_decode(ctx, Hq, Hkv, D, bs, dtype, seed=int(rng.integers(1 << 30)), device=DEV,
                          poison=True)
    ref = oracle_full(case)
    for part in (-1, 64, 256):
        out = run_decode(case, partition_size=part)
        assert_close(host(out), ref, dtype, f"partition {part}")


BLOCK_SIZES = [(dtype, D, bs) for dtype in ("f32", "f16", "bf16") for D in (64, 128)
               for bs in (8, 64, 128, 256)]


@pytest.mark.parametrize("dtype,D,bs", BLOCK_SIZES)
def test_decode_block_sizes(dtype, D, bs):
    """Pages of 8 tokens (a load's tokens fill one page exactly for fp32 rows)
    and pages larger than a partition (64-token partitions inside 128/256-slot
    pages); contexts ending mid-page and mid-tile."""
    rng = np.random.default_rng(zlib.crc32(repr(("decode-bs", dtype, D, bs)).encode()))
    ctx = np.concatenate([[1, bs - 1, bs + 3, 300], rng.integers(2, 900, size=2)])
    log(f"decode block size dtype={dtype} D={D} bs={bs} ctx={ctx.tolist()}")
    case = wl.make_decode(ctx, 8, 2, D, bs, dtype, seed=int(rng.integers(1 << 30)), device=DEV,
                          poison=True)
    ref = oracle_full(case)
    for part in (-1, 64):
        out = run_decode(case, partition_size=part)
        assert_close(host(out), ref, dtype, f"block size {bs} partition {part}")


LARGE_GROUPS = [(dtype, D, Hq) for dtype in ("f16", "bf16") for D in (64, 128)
                for Hq in (32, 40, 64)]


@pytest.mark.parametrize("dtype,D,Hq", LARGE_GROUPS)
def test_decode_large_groups(dtype, D, Hq):
    """16, 20 and 32 query heads per kv head: one full block of 16 heads, a
    full block plus a 4-head block, and two full blocks per work item chunk."""
    rng = np.random.default_rng(zlib.crc32(repr(("decode-groups", dtype, D, Hq)).encode()))
    ctx = np.concatenate([[1, 16, 17, 1000], rng.integers(2, 1500, size=2)])
    log(f"decode large group dtype={dtype} D={D} Hq={Hq} Hkv=2 ctx={ctx.tolist()}")
    case = wl.make_decode(ctx, Hq, 2, D, 16, dtype, seed=int(rng.integers(1 << 30)), device=DEV,
                          poison=True)
    ref = oracle_full(case)
    for part in (-1, 0, 128):
        out = run_decode(case, partition_size=part)
        assert_close(host(out), ref, dtype, f"group {Hq // 2} partition {part}")


def test_tiny_decode_f32_workload():
    case = wl.tiny_decode_f32(device=DEV, poison=True)
    log(f"tiny decode f32 ctx={case.kv.context_lens.tolist()}")
    e = assert_close(host(run_decode(case)), oracle_full(case), "f32", "tiny f32")
    log(f"  max rel err {e:.3e}")


@pytest.mark.parametrize("name,seqs_pick", [
    ("llama7b_decode_f16", "extremes"),
    ("gqa_decode_bf16", "extremes"),
    ("long_decode_f16", "first"),
])
def test_full_size_workloads_sampled(name, seqs_pick):
    case = wl.WORKLOADS[name](device=DEV)
    kv = case.kv
    ctx = kv.context_lens.cpu().numpy()
    log(f"{name}: B={len(ctx)} pool={kv.k_cache.shape[0]} ctx range [{ctx.min()}, {ctx.max()}]")
    out = run_decode(case)
    if seqs_pick == "extremes":
        order = np.argsort(ctx)
        seqs = sorted({int(order[0]), int(order[1]), int(order[len(order) // 2]), int(order[-2]),
                       int(order[-1])})
    else:
        seqs = [0, len(ctx) - 1]
    Hq = case.query.shape[1]
    heads = sorted({0, 1, Hq // 2, Hq - 1})
    ref = oracle_sampled(case, seqs, heads)
    got = host(out[seqs])[:, heads]
    e = assert_close(got, ref[:, heads], case.dtype, name)
    log(f"  sampled seqs {seqs} heads {heads}: max rel err {e:.3e}")
    # every output row is finite (no stray NaN from unwritten rows)
    assert torch.isfinite(out.float()).all()


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_one_token_context_is_bit_exact(dtype):
    case = wl.make_decode(np.ones(9, dtype=np.int64), 8, 2, 128, 16, dtype, seed=5, device=DEV,
                          poison=True)
    kv = case.kv
    out = run_decode(case)
    first = kv.block_tables[:, 0].long()
    want = kv.v_cache[first, :, 0, :].repeat_interleave(4, dim=1)     # [B, Hq, D]
    assert torch.equal(out.view(torch.int16 if dtype != "f32" else torch.int32),
                       want.contiguous().view(torch.int16 if dtype != "f32" else torch.int32))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_block_permutation_is_bit_identical(dtype):
    ctx = np.array([1, 15, 16, 17, 300, 1025, 2100])
    case = wl.make_decode(ctx, 8, 2, 128, 16, dtype, seed=6, device=DEV)
    kv = case.kv
    base = run_decode(case, partition_size=512)
    g = torch.Generator(device="cpu").manual_seed(1)
    perm = torch.randperm(kv.k_cache.shape[0], generator=g).to(DEV)
    k2 = torch.empty_like(kv.k_cache)
    v2 = torch.empty_like(kv.v_cache)
    k2[perm] = kv.k_cache
    v2[perm] = kv.v_cache
    bt2 = perm[kv.block_tables.long()].to(torch.int32)
    out = torch.empty_like(base)
    pa.paged_attn_decode(out, case.query, k2, v2, bt2, kv.context_lens, case.scale,
                         kv.max_context_len, partition_size=512)
    torch.cuda.synchronize()
    assert torch.equal(out, base)


def test_split_partition_covering_context_equals_unsplit_bitwise():
    ctx = np.array([3, 64, 200, 511, 512])
    case = wl.make_decode(ctx, 8, 8, 128, 16, "f16", seed=7, device=DEV)
    a = run_decode(case, partition_size=-1)
    b = run_decode(case, partition_size=512)
    assert torch.equal(a, b)
    c = run_decode(case, partition_size=64)        # genuinely split: within tolerance
    assert rel_err(host(c), host(a).astype(np.float64)) <= 2 * TOL["f16"]


def test_gqa_matches_mha_on_replicated_kv():
    ctx = np.array([5, 100, 777])
    case = wl.make_decode(ctx, 16, 4, 128, 16, "bf16", seed=8, device=DEV)
    kv = case.kv
    gqa = run_decode(case)
    k4 = kv.k_cache.repeat_interleave(4, dim=1).contiguous()
    v4 = kv.v_cache.repeat_interleave(4, dim=1).contiguous()
    mha = torch.empty_like(gqa)
    pa.paged_attn_decode(mha, case.query, k4, v4, kv.block_tables, kv.context_lens, case.scale,
                         kv.max_context_len)
    torch.cuda.synchronize()
    assert rel_err(host(gqa), host(mha).astype(np.float64)) <= TOL["bf16"]
    log(f"  gqa vs mha bit-identical: {torch.equal(gqa, mha)}")


def test_constant_value_returns_constant():
    ctx = np.array([1, 33, 999, 4000])
    case = wl.make_decode(ctx, 4, 4, 128, 16, "f16", seed=9, device=DEV)
    case.kv.v_cache.fill_(0.625)
    out = run_decode(case)
    assert torch.allclose(out.float(), torch.full_like(out.float(), 0.625), atol=2e-3, rtol=0)


def test_partial_max_context_clamps_without_fault():
    # contexts above max_context_len are cut to it: memory-safe, defined output
    ctx = np.array([100, 300])
    case = wl.make_decode(ctx, 4, 4, 64, 16, "f32", seed=10, device=DEV)
    out = run_decode(case, max_context_len=128)
    kv = case.kv
    ref = decode_ref(host(case.query), host(kv.k_cache), host(kv.v_cache), host(kv.block_tables),
                     np.minimum(host(kv.context_lens), 128), case.scale)
    assert_close(host(out), ref, "f32", "clamped")


def test_empty_batch_is_a_no_op():
    q = torch.zeros(0, 4, 64, device=DEV)
    kc = torch.zeros(4, 4, 16, 64, device=DEV)
    pa.paged_attn_decode(q, q, kc, kc, torch.zeros(0, 2, dtype=torch.int32, device=DEV),
                         torch.zeros(0, dtype=torch.int32, device=DEV), 0.125, 32)
    torch.cuda.synchronize()


def test_tiny_decode_graph_replays_match_eager():
    """Decode captured into a HIP graph (plan + attention launches, no memset
    nodes): every replay, with new query values written into the captured
    input between replays and eager work interleaved, equals the eager call
    on the same inputs bit for bit."""
    case = wl.tiny_decode_f32(device=DEV, poison=True)
    kv = case.kv
    B, Hq, D = case.query.shape
    maxctx = kv.max_context_len            # host value, read before the capture
    ws = torch.empty(max(1, pa.paged_attn_decode_workspace_size(B, Hq, kv.k_cache.shape[1], D,
                                                                maxctx, 0)),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty_like(case.query)

    def call(o, w):
        pa.paged_attn_decode(o, case.query, kv.k_cache, kv.v_cache, kv.block_tables,
                             kv.context_lens, case.scale, maxctx, workspace=w)

    call(out, ws)                          # first call outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, ws)
    gen = torch.Generator(device="cpu").manual_seed(9)
    eager_out = torch.empty_like(out)
    eager_ws = torch.empty_like(ws)
    for r in range(4):
        case.query.copy_(torch.randn(case.query.shape, generator=gen).to(DEV))
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        call(eager_out, eager_ws)          # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, eager_out), f"replay {r}"
    ref = oracle_full(case)
    assert_close(host(out), ref, "f32", "graph replay")


@pytest.mark.parametrize("dtype,long_ctx", [("f32", False), ("f16", True), ("bf16", True)])
def test_empty_contexts_leave_their_rows_unwritten(dtype, long_ctx):
    """context_lens of 0 or below: that sequence's output rows keep their
    previous bytes, in the single-partition launch (all contexts short) and
    in the split launch (one context spans several partitions); the other
    rows match the oracle."""
    ctx = np.array([40, 3, 700 if long_ctx else 90, 17])
    Hq, Hkv = (8, 2) if dtype != "f32" else (4, 4)
    case = wl.make_decode(ctx, Hq, Hkv, 128, 16, dtype, seed=31, device=DEV)
    kv = case.kv
    cl = kv.context_lens.clone()
    cl[1] = 0
    cl[3] = -5
    out = torch.full_like(case.query, 7.0)
    pa.paged_attn_decode(out, case.query, kv.k_cache, kv.v_cache, kv.block_tables, cl,
                         case.scale, int(ctx.max()), partition_size=256 if long_ctx else 0)
    torch.cuda.synchronize()
    got = host(out)
    assert (got[1] == 7.0).all() and (got[3] == 7.0).all()
    ref = decode_ref(host(case.query), host(kv.k_cache), host(kv.v_cache), host(kv.block_tables),
                     host(kv.context_lens), case.scale)
    assert_close(got[[0, 2]], ref[[0, 2]], dtype, "rows with keys")
