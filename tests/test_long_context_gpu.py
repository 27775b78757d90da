"""Long-context parity with planted keys, and the merge of many partitions.

With N(0, 1) inputs and tens of thousands of keys every softmax weight is
tiny and the outputs shrink to about 1/sqrt(keys), so a dropped or doubled
partition moves them by less than the tolerance.  Here a few keys per
(sequence, head) are planted with large scores (k = alpha * q, score 12 to
13.5 against a background of about e^10.9 total weight): each planted key
carries 5-25% of the softmax mass, so the output is an O(1) mix of their V
rows and any partition, tile or merge step that is lost, repeated or
mis-weighted shows up far above the tolerance.  The oracle sees the same
planted pool (OnlineSoftmax M/L/O merge, "vLLM中FlashAttention与KVCache交换机制解析").
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_248_amd as pa
import workloads as wl
from oracle import decode_ref, prefill_ref
from tests._util import TOL, assert_close, compact_pool, host, log

pytestmark = pytest.mark.gpu

DEV = "cuda"


def plant(kv, query_rows, seq_of_row, pos_lists, group, scores):
    """For query row r (a [Hq, D] tensor of queries, sequence seq_of_row[r])
    and each head h, set the K row of kv head h // group at every logical
    position in pos_lists[r][h] to alpha * q[h], alpha chosen so that the
    scaled score is the matching entry of scores[r][h].  Rows are written in
    the storage dtype, so the oracle and the kernel see the same bytes."""
    bs = kv.block_size
    tables = kv.block_tables.cpu().numpy()
    D = kv.k_cache.shape[-1]
    scale = 1.0 / np.sqrt(D)
    for r, q in enumerate(query_rows):
        b = seq_of_row[r]
        qf = q.float()
        for h, positions in enumerate(pos_lists[r]):
            g = h // group
            qh = qf[h]
            norm2 = float((qh * qh).sum())
            for j, s in zip(positions, scores[r][h]):
                blk = int(tables[b, j // bs])
                alpha = float(s) / (scale * norm2)
                kv.k_cache[blk, g, j % bs] = (alpha * qh).to(kv.k_cache.dtype)


def rel_to_row_max(got, ref):
    """Largest per-row error relative to that row's max |ref| (rows = all but
    the last axis)."""
    g = np.asarray(got, np.float64).reshape(-1, got.shape[-1])
    r = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    return float(np.max(np.abs(g - r).max(axis=1) / np.maximum(np.abs(r).max(axis=1), 1e-30)))


@pytest.mark.parametrize("dtype,Hq,Hkv,bs,part", [
    ("f16", 32, 32, 32, 512),      # the long-context workload's shape and partitions
    ("bf16", 32, 8, 16, 4096),     # GQA on the matrix-core kernel, default partitions
    ("bf16", 32, 8, 16, 2048),
    ("bf16", 32, 8, 16, 512),
])
def test_decode_planted_keys_long_context(dtype, Hq, Hkv, bs, part):
    ctx = np.array([32768, 16389])
    seed = 4400 + Hkv + part
    case = wl.make_decode(ctx, Hq, Hkv, 128, bs, dtype, seed=seed, device=DEV)
    kv = case.kv
    rng = np.random.default_rng(seed)
    G = Hq // Hkv
    pos, sc = [], []
    for b, n in enumerate(ctx):
        nparts = (int(n) + part - 1) // part
        ph, sh = [], []
        for h in range(Hq):
            # 8 partitions: first, last and six random ones; inside each a
            # random key, or the partition's first or last key
            chosen = np.unique(np.concatenate([[0, nparts - 1], rng.integers(0, nparts, 6)]))
            js = []
            for p in chosen:
                lo, hi = p * part, min((p + 1) * part, int(n))
                js.append(int(rng.choice([lo, hi - 1, int(rng.integers(lo, hi))])))
            ph.append(js)
            sh.append(12.0 + 1.5 * rng.random(len(js)))
        pos.append(ph)
        sc.append(sh)
    plant(kv, [case.query[b] for b in range(len(ctx))], list(range(len(ctx))), pos, G, sc)
    out = torch.full_like(case.query, float("nan"))
    pa.paged_attn_decode(out, case.query, kv.k_cache, kv.v_cache, kv.block_tables,
                         kv.context_lens, case.scale, kv.max_context_len, partition_size=part)
    torch.cuda.synchronize()
    k, v, tables, cl = compact_pool(kv, [0, 1])
    ref = decode_ref(host(case.query), k, v, tables, cl, case.scale)
    got = host(out)
    assert np.abs(ref).max() > 0.3, "planted keys should dominate the output"
    e = assert_close(got, ref, dtype, f"planted decode {dtype} part {part}")
    log(f"planted decode {dtype} Hq={Hq} Hkv={Hkv} part={part}: max rel err {e:.3e}, "
        f"max err / row max|ref| {rel_to_row_max(got, ref):.3e}, max|ref| {np.abs(ref).max():.2f}")


@pytest.mark.parametrize("kernel", ["pingpong", "halftile"])
@pytest.mark.parametrize("dtype,bs", [("bf16", 16), ("f16", 32)])
def test_prefill_planted_keys_long_context(dtype, bs, kernel):
    """Prefixes of 30000 and 16000 tokens: planted keys for chosen query rows
    across the whole visible range (the first key, the row's own position, the
    key just before it, random keys), so each key tile's contribution to those
    rows is O(1); checked on those rows and on random rows, every head."""
    pre = np.array([30000, 16000])
    ql = np.array([256, 130])
    Hq, Hkv = 8, 2
    G = Hq // Hkv
    case = wl.make_prefill(pre, ql, Hq, Hkv, 128, bs, dtype, seed=4501 + bs, device=DEV)
    kv = case.kv
    qsl = host(case.query_start_loc)
    rng = np.random.default_rng(4502 + bs)
    plant_rows = {0: [0, 69, 255], 1: [0, 64, 129]}
    rows_q, row_seq, pos, sc = [], [], [], []
    for b, ts in plant_rows.items():
        for t in ts:
            p = int(pre[b]) + t                     # this row sees keys 0..p
            rows_q.append(case.query[int(qsl[b]) + t])
            row_seq.append(b)
            ph, sh = [], []
            for h in range(Hq):
                js = sorted({0, p, max(p - 1, 0), *rng.integers(0, p + 1, 5).tolist()})
                ph.append(js)
                sh.append(12.0 + 1.5 * rng.random(len(js)))
            pos.append(ph)
            sc.append(sh)
    # rows of one sequence share kv heads: plant row by row (a later row's
    # key wins where two name the same position)
    plant(kv, rows_q, row_seq, pos, G, sc)
    out = torch.full_like(case.query, float("nan"))
    fn = pa.paged_attn_prefill if kernel == "pingpong" else pa.paged_attn_prefill_halftile
    fn(out, case.query, kv.k_cache, kv.v_cache, kv.block_tables, kv.context_lens,
       case.query_start_loc, case.scale, case.max_query_len, kv.max_context_len)
    torch.cuda.synchronize()
    got_all = host(out)
    k, v, tables, cl = compact_pool(kv, [0, 1])
    for b in (0, 1):
        q_b = int(ql[b])
        rows = np.unique(np.concatenate([plant_rows[b], rng.integers(0, q_b, 6)]))
        q = host(case.query[int(qsl[b]):int(qsl[b + 1])])
        ref = prefill_ref(q, k, v, tables[b:b + 1], cl[b:b + 1], np.array([0, q_b]), case.scale,
                          rows=rows)
        got = got_all[int(qsl[b]):int(qsl[b + 1])][rows]
        e = assert_close(got, ref[rows], dtype, f"planted prefill seq {b}")
        assert np.abs(ref[plant_rows[b]]).max() > 0.3
        log(f"planted prefill {dtype} bs={bs} seq {b} rows {rows.tolist()}: max rel err {e:.3e}, "
            f"max err / row max|ref| {rel_to_row_max(got, ref[rows]):.3e}")


@pytest.mark.parametrize("dtype,ctx", [("bf16", [70001, 999]), ("f16", [131072])])
def test_decode_merge_over_1024_partitions_large_group(dtype, ctx):
    """16 query heads per kv head, 64-token partitions, contexts over 65536
    keys: 1094 and 2048 (the most allowed) partitions merged by one
    work-group per (sequence, kv head) — the in-kernel merge's largest case
    (16 x 2048 weights, recomputed per partial).  Every row against the
    oracle."""
    ctx = np.array(ctx)
    case = wl.make_decode(ctx, 32, 2, 128, 16, dtype, seed=4600 + len(ctx), device=DEV,
                          poison=True)
    kv = case.kv
    out = torch.full_like(case.query, float("nan"))
    pa.paged_attn_decode(out, case.query, kv.k_cache, kv.v_cache, kv.block_tables,
                         kv.context_lens, case.scale, kv.max_context_len, partition_size=64)
    torch.cuda.synchronize()
    k, v, tables, cl = compact_pool(kv, list(range(len(ctx))))
    ref = decode_ref(host(case.query), k, v, tables, cl, case.scale)
    e = assert_close(host(out), ref, dtype, "many-partition merge")
    log(f"merge of {(int(ctx.max()) + 63) // 64} partitions, group 16, {dtype}: max rel err {e:.3e}")
