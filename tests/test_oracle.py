"""Pins for the fp64 oracle: each checks it against something other than
itself — values the pages print, closed forms, invariants, a library routine,
or brute force on tiny inputs.  CPU only."""

import json
import math
import os

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import (append_kv_ref, attend_two_pass, copy_blocks_ref, decode_ref,
                    decode_split_ref, gather_sequence, online_softmax_ref, prefill_ref,
                    split_merge_ref)


def _np(t):
    """Storage tensor -> numpy with exactly the stored values (bf16 via fp32)."""
    if t.dtype == torch.bfloat16:
        return t.float().numpy()
    return t.numpy()


def _dec_np(case):
    kv = case.kv
    return (_np(case.query), _np(kv.k_cache), _np(kv.v_cache), kv.block_tables.numpy(),
            kv.context_lens.numpy(), case.scale)


# ---------------------------------------------------------------- p1
@pytest.mark.parametrize("n", [1, 2, 7, 64, 1000, 10000])
def test_online_recurrence_equals_two_pass(n):
    """The page's one-pass (M, L, O) recurrence reaches the two-pass softmax
    result for any tiling of the key stream, scores spread widely enough to
    force rescaling."""
    rng = np.random.default_rng(n)
    x = rng.normal(0.0, 30.0, size=n)
    v = rng.normal(size=(n, 8))
    cuts = np.sort(rng.choice(np.arange(1, n), size=min(n - 1, rng.integers(0, 12)), replace=False)) if n > 1 else []
    edges = [0, *cuts.tolist(), n] if n > 1 else [0, 1]
    tiles = list(zip(edges[:-1], edges[1:]))
    M, L, O = online_softmax_ref(x, v, tiles)
    m = x.max()
    w = np.exp(x - m)
    assert M == m
    np.testing.assert_allclose(L, w.sum(), rtol=1e-12)
    # and the oracle's own attend routine (which recomputes scores from q, K)
    ref = (w @ v) / w.sum()
    np.testing.assert_allclose(O, ref, rtol=1e-12, atol=1e-13)


def test_attend_two_pass_matches_closed_form_softmax():
    """Scores supplied through q K^T with an identity K equal q * scale."""
    rng = np.random.default_rng(1)
    q = rng.normal(size=5)
    K = np.eye(5)
    V = rng.normal(size=(5, 3))
    got = attend_two_pass(q, K, V, 0.5)
    s = 0.5 * q
    p = np.exp(s) / np.exp(s).sum()
    np.testing.assert_allclose(got, p @ V, rtol=1e-14)


# ---------------------------------------------------------------- p2, p3
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_one_token_context_returns_its_value(dtype):
    case = wl.make_decode([1, 1, 1], 4, 2, 64, 16, dtype, seed=11, pool_blocks=16, poison=True)
    q, k, v, bt, cl, sc = _dec_np(case)
    out = decode_ref(q, k, v, bt, cl, sc)
    for b in range(3):
        for h in range(4):
            assert np.array_equal(out[b, h], v[bt[b, 0], h // 2, 0].astype(np.float64))


def test_constant_value_returns_constant():
    case = wl.make_decode([1, 17, 100, 333], 4, 4, 64, 16, "f32", seed=12)
    q, k, v, bt, cl, sc = _dec_np(case)
    v = np.full_like(v, 0.625)
    out = decode_ref(q, k, v, bt, cl, sc)
    np.testing.assert_allclose(out, 0.625, rtol=0, atol=1e-15)


# ---------------------------------------------------------------- p4
def test_block_permutation_invariance():
    """Moving physical blocks and rewriting the tables to match leaves the
    result bit-identical."""
    case = wl.make_decode([5, 33, 200, 64], 8, 2, 64, 16, "f16", seed=13)
    q, k, v, bt, cl, sc = _dec_np(case)
    ref = decode_ref(q, k, v, bt, cl, sc)
    rng = np.random.default_rng(99)
    perm = rng.permutation(k.shape[0])           # new home of old block i is perm[i]
    k2 = np.empty_like(k)
    v2 = np.empty_like(v)
    k2[perm] = k
    v2[perm] = v
    out = decode_ref(q, k2, v2, perm[bt].astype(np.int32), cl, sc)
    assert np.array_equal(out, ref)


# ---------------------------------------------------------------- p5
def _brute_decode(q, k, v, bt, cl, scale, group):
    B, H, D = q.shape
    bs = k.shape[2]
    out = np.zeros((B, H, D))
    s64 = float(np.float32(scale))
    for b in range(B):
        n = int(cl[b])
        for h in range(H):
            g = h // group
            scores = []
            for j in range(n):
                blk = int(bt[b][j // bs])
                acc = 0.0
                for d in range(D):
                    acc += float(q[b][h][d]) * float(k[blk][g][j % bs][d])
                scores.append(s64 * acc)
            mx = max(scores)
            ws = [math.exp(s - mx) for s in scores]
            tot = sum(ws)
            for d in range(D):
                num = 0.0
                for j in range(n):
                    blk = int(bt[b][j // bs])
                    num += ws[j] * float(v[blk][g][j % bs][d])
                out[b][h][d] = num / tot
    return out


@pytest.mark.parametrize("bs", [1, 2, 16])
def test_decode_matches_brute_force(bs):
    rng = np.random.default_rng(bs)
    ctx = rng.integers(1, 6, size=2)
    case = wl.make_decode(ctx, 2, 1, 4, bs, "f32", seed=20 + bs)
    q, k, v, bt, cl, sc = _dec_np(case)
    got = decode_ref(q, k, v, bt, cl, sc)
    want = _brute_decode(q, k, v, bt, cl, sc, group=2)
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("bs", [1, 2, 16])
def test_prefill_matches_brute_force(bs):
    pre = [0, 3]
    ql = [3, 2]
    case = wl.make_prefill(pre, ql, 2, 1, 4, bs, "f32", seed=30 + bs)
    kv = case.kv
    q, k, v = _np(case.query), _np(kv.k_cache), _np(kv.v_cache)
    bt, cl, qsl = kv.block_tables.numpy(), kv.context_lens.numpy(), case.query_start_loc.numpy()
    got = prefill_ref(q, k, v, bt, cl, qsl, case.scale)
    s64 = float(np.float32(case.scale))
    for b in range(2):
        n = int(cl[b])
        for t in range(ql[b]):
            row = int(qsl[b]) + t
            pos = n - ql[b] + t
            for h in range(2):
                sc = []
                for j in range(pos + 1):
                    blk = int(bt[b][j // bs])
                    sc.append(s64 * sum(float(q[row][h][d]) * float(k[blk][0][j % bs][d]) for d in range(4)))
                mx = max(sc)
                w = [math.exp(s - mx) for s in sc]
                for d in range(4):
                    num = sum(w[j] * float(v[int(bt[b][j // bs])][0][j % bs][d]) for j in range(pos + 1))
                    assert abs(got[row, h, d] - num / sum(w)) <= 1e-13 * max(1.0, abs(num / sum(w)))


def test_block_table_example_from_page(golden_dir):
    """The page's example tables ([5,12,8], [3,7], [9,14,16,20]) address the
    pool; decoding through them equals attention over the pages laid end to end."""
    g = json.load(open(os.path.join(golden_dir, "block_table_example.json")))
    tables = [g["block_tables"][str(i)] for i in range(3)]
    bs, D = 4, 8
    rng = np.random.default_rng(5)
    k = rng.normal(size=(21, 1, bs, D)).astype(np.float32)
    v = rng.normal(size=(21, 1, bs, D)).astype(np.float32)
    q = rng.normal(size=(3, 1, D)).astype(np.float32)
    bt = np.zeros((3, 4), dtype=np.int32)
    for i, t in enumerate(tables):
        bt[i, :len(t)] = t
    cl = np.array([len(t) * bs - 1 for t in tables], dtype=np.int32)  # last block partly full
    out = decode_ref(q, k, v, bt, cl, 0.25)
    for i, t in enumerate(tables):
        K = np.concatenate([k[p, 0] for p in t])[:cl[i]].astype(np.float64)
        V = np.concatenate([v[p, 0] for p in t])[:cl[i]].astype(np.float64)
        s = 0.25 * (K @ q[i, 0].astype(np.float64))
        w = np.exp(s - s.max())
        np.testing.assert_allclose(out[i, 0], (w @ V) / w.sum(), rtol=1e-13)


# ---------------------------------------------------------------- p6, p7
def test_decode_identity_table_equals_library_sdpa():
    B, H, D, bs, n = 3, 4, 64, 16, 48
    rng = np.random.default_rng(6)
    k = rng.normal(size=(B * n // bs, H, bs, D))
    v = rng.normal(size=(B * n // bs, H, bs, D))
    q = rng.normal(size=(B, H, D))
    bt = np.arange(B * n // bs, dtype=np.int32).reshape(B, n // bs)
    cl = np.full(B, n, dtype=np.int32)
    scale = float(np.float32(1 / 8))
    got = decode_ref(q, k, v, bt, cl, scale)
    K = torch.from_numpy(k).reshape(B, n // bs, H, bs, D).permute(0, 2, 1, 3, 4).reshape(B, H, n, D)
    V = torch.from_numpy(v).reshape(B, n // bs, H, bs, D).permute(0, 2, 1, 3, 4).reshape(B, H, n, D)
    Q = torch.from_numpy(q).reshape(B, H, 1, D)
    want = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)
    np.testing.assert_allclose(got, want.reshape(B, H, D).numpy(), rtol=1e-12, atol=1e-13)


def test_prefill_no_prefix_equals_library_causal_sdpa():
    H, D, bs, n = 2, 32, 16, 40
    rng = np.random.default_rng(7)
    nb = (n + bs - 1) // bs
    k = rng.normal(size=(nb, H, bs, D))
    v = rng.normal(size=(nb, H, bs, D))
    q = rng.normal(size=(n, H, D))
    bt = np.arange(nb, dtype=np.int32)[None]
    got = prefill_ref(q, k, v, bt, np.array([n]), np.array([0, n]), 0.125)
    K = torch.from_numpy(k).permute(1, 0, 2, 3).reshape(H, nb * bs, D)[:, :n][None]
    V = torch.from_numpy(v).permute(1, 0, 2, 3).reshape(H, nb * bs, D)[:, :n][None]
    Q = torch.from_numpy(q).permute(1, 0, 2)[None]
    want = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=0.125)
    np.testing.assert_allclose(got, want[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)


def test_prefill_with_prefix_equals_library_sdpa_with_bottom_right_mask():
    H, D, bs, pre, ql = 2, 16, 8, 13, 9
    n = pre + ql
    rng = np.random.default_rng(8)
    nb = (n + bs - 1) // bs
    k = rng.normal(size=(nb, H, bs, D))
    v = rng.normal(size=(nb, H, bs, D))
    q = rng.normal(size=(ql, H, D))
    bt = rng.permutation(nb).astype(np.int32)[None]
    got = prefill_ref(q, k, v, bt, np.array([n]), np.array([0, ql]), 0.25)
    K = torch.from_numpy(k[bt[0]]).permute(1, 0, 2, 3).reshape(H, nb * bs, D)[:, :n][None]
    V = torch.from_numpy(v[bt[0]]).permute(1, 0, 2, 3).reshape(H, nb * bs, D)[:, :n][None]
    Q = torch.from_numpy(q).permute(1, 0, 2)[None]
    allowed = torch.ones(ql, n, dtype=torch.bool).tril(diagonal=pre)
    want = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=allowed, scale=0.25)
    np.testing.assert_allclose(got, want[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- p8
def test_prefill_single_new_token_equals_decode():
    ctx = np.array([1, 17, 90, 300])
    case = wl.make_decode(ctx, 8, 2, 64, 16, "bf16", seed=14)
    q, k, v, bt, cl, sc = _dec_np(case)
    dec = decode_ref(q, k, v, bt, cl, sc)
    pre = prefill_ref(q, k, v, bt, cl, np.arange(5), sc)     # one new token per sequence
    # equal up to fp64 rounding (BLAS may associate a 1-row and a G-row product differently)
    np.testing.assert_allclose(pre, dec, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- p9
def test_gqa_equals_mha_on_repeated_kv():
    ctx = np.array([3, 40, 129])
    case = wl.make_decode(ctx, 8, 2, 64, 16, "f16", seed=15)
    q, k, v, bt, cl, sc = _dec_np(case)
    gqa = decode_ref(q, k, v, bt, cl, sc)
    k_rep = np.repeat(k, 4, axis=1)     # kv head g becomes heads 4g..4g+3
    v_rep = np.repeat(v, 4, axis=1)
    mha = decode_ref(q, k_rep, v_rep, bt, cl, sc)
    np.testing.assert_allclose(gqa, mha, rtol=1e-13, atol=1e-15)
    # a head-to-group map other than h // G (e.g. h % Hkv) would not match
    wrong = decode_ref(q, np.repeat(k, 1, axis=1)[:, [0, 1] * 4], np.repeat(v, 1, axis=1)[:, [0, 1] * 4],
                       bt, cl, sc)
    assert not np.allclose(gqa, wrong)


# ---------------------------------------------------------------- p10
@pytest.mark.parametrize("part", [1, 16, 64, 512, 100000])
def test_split_merge_equals_unsplit(part):
    ctx = np.array([1, 100, 700, 1500])
    case = wl.make_decode(ctx, 2, 2, 64, 16, "f32", seed=16)
    q, k, v, bt, cl, sc = _dec_np(case)
    a = decode_ref(q, k, v, bt, cl, sc)
    b = decode_split_ref(q, k, v, bt, cl, sc, part)
    np.testing.assert_allclose(b, a, rtol=1e-13, atol=1e-14)


def test_split_merge_wide_scores():
    rng = np.random.default_rng(3)
    x = rng.normal(0, 40, size=3000)
    v = rng.normal(size=(3000, 4))
    w = np.exp(x - x.max())
    np.testing.assert_allclose(split_merge_ref(x, v, 37), (w @ v) / w.sum(), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- p11
def test_copy_page_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "swap_blocks_example.json")))
    rng = np.random.default_rng(0)
    src = rng.normal(size=(g["num_src"], *g["block_shape"])).astype(np.float32)
    dst = np.zeros((g["num_dst"], *g["block_shape"]), dtype=np.float32)
    out = copy_blocks_ref(src, dst, np.array(g["mapping"]))
    for d, s in g["expected_copies"]:
        assert np.array_equal(out[d], src[s])
    for d in g["expected_untouched"]:
        assert np.array_equal(out[d], dst[d])
    filled = int((out.reshape(out.shape[0], -1) != 0).any(axis=1).sum())
    assert filled == g["expected_filled_count"]


def _copy_brute(src, dst, m):
    """One forward pass over the mapping records, per destination, the first
    position naming it; then each recorded (destination, position) pair is
    applied when the position is a source block."""
    first = {}
    for i, d in enumerate(np.asarray(m).tolist()):
        if 0 <= d < dst.shape[0]:
            first.setdefault(d, i)
    out = dst.copy()
    for d, i in first.items():
        if i < src.shape[0]:
            out[d] = src[i]
    return out


@pytest.mark.parametrize("seed", range(40))
def test_copy_matches_brute_force_with_duplicates_and_invalid(seed):
    rng = np.random.default_rng(seed)
    ns, nd = int(rng.integers(1, 9)), int(rng.integers(1, 7))
    nm = int(rng.integers(0, 13))                  # may exceed the source pool
    m = rng.integers(-2, nd + 2, size=nm)          # -2/-1, repeats and out-of-range values
    src = rng.integers(0, 2**16, size=(ns, 3, 5), dtype=np.uint16)
    dst = rng.integers(0, 2**16, size=(nd, 3, 5), dtype=np.uint16)
    assert np.array_equal(copy_blocks_ref(src, dst, m), _copy_brute(src, dst, m))


def test_copy_duplicate_destination_takes_lowest_source():
    src = np.arange(3 * 2, dtype=np.uint16).reshape(3, 2) + 100
    dst = np.zeros((2, 2), dtype=np.uint16)
    out = copy_blocks_ref(src, dst, np.array([1, 1, 0, 1]))
    assert out.tolist() == [src[2].tolist(), src[0].tolist()]
    # first match beyond the source pool: the destination is left alone
    out = copy_blocks_ref(src[:1], dst, np.array([-1, 0, 0]))
    assert out.tolist() == dst.tolist()


def test_copy_is_bytewise_nan_payloads_and_negative_zero():
    src = np.array([[0x7FC1, 0x8000], [0xFFFF, 0x0001]], dtype=np.uint16).view(np.float16)
    dst = np.zeros((2, 2), dtype=np.float16)
    out = copy_blocks_ref(src, dst, np.array([1, 0]))
    assert out.view(np.uint16).tolist() == [[0xFFFF, 0x0001], [0x7FC1, 0x8000]]


# ---------------------------------------------------------------- p12
def test_poisoned_pool_does_not_reach_the_output():
    case = wl.make_decode([7, 16, 33, 50], 4, 4, 64, 16, "f16", seed=17, poison=True)
    q, k, v, bt, cl, sc = _dec_np(case)
    assert np.isnan(k).any()                       # the pool really is poisoned
    out = decode_ref(q, k, v, bt, cl, sc)
    assert np.isfinite(out).all()
    assert np.abs(out).max() < 10.0                # the +1e4 tail slots were not read


# ---------------------------------------------------------------- p13
def test_kv_byte_model_matches_page(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "kv_cache_bytes.json")))
    got = wl.kv_cache_bytes(g["n_layers"], g["n_heads"], g["d_head"], g["seq"], g["batch"],
                            g["elem_bytes"])
    assert got == g["expected_bytes"]
    # one layer of that cache is exactly what decode streams for that batch
    ctx = np.full(g["batch"], g["seq"])
    per_layer = wl.decode_kv_bytes(ctx, g["n_heads"], g["n_heads"], g["d_head"], 16, 2)
    extra = 2 * g["batch"] * g["n_heads"] * g["d_head"] * 2 + 4 * g["batch"] * (g["seq"] // 16) + 4 * g["batch"]
    assert (per_layer - extra) * g["n_layers"] == g["expected_bytes"]


def test_gather_respects_slot_and_block():
    k = np.arange(4 * 1 * 2 * 1, dtype=np.float32).reshape(4, 1, 2, 1)
    got = gather_sequence(k, np.array([3, 0, 2]), 5, 0)[:, 0]
    assert got.tolist() == [6, 7, 0, 1, 4]


def test_prefill_flop_model_small():
    # ctx 5 with 3 new tokens: rows see 3, 4, 5 keys -> 12 pairs
    assert wl.prefill_pairs([5], [3]) == 12
    assert wl.prefill_flops([5], [3], 2, 4) == 4 * 4 * 2 * 12


# ---------------------------------------------------------------- KV append
def _append_example_arrays(g, D=3):
    names = ["req_A", "req_B"]
    tables = [g["block_tables"][n] for n in names]
    bt = np.full((2, 3), -1, dtype=np.int32)
    for i, t in enumerate(tables):
        bt[i, :len(t)] = t
    cl = np.array([g["context_lens"][n] for n in names], dtype=np.int32)
    qsl = np.array([0, cl[0], cl[0] + cl[1]], dtype=np.int32)      # every token is new
    rows = (np.arange(int(qsl[-1]))[:, None, None] + 1 + np.zeros((1, 1, D))).astype(np.float32)
    pool = np.full((g["num_blocks"], 1, g["block_size"], D), -7.0, dtype=np.float32)
    return names, bt, cl, qsl, rows, pool


def test_append_block_manager_example(golden_dir):
    """The page's allocator run (req_A: 20 + 13 tokens over blocks [0, 1, 3];
    req_B: 10 tokens in block 2): each token lands in the block and row the
    allocation implies, and nothing else changes."""
    g = json.load(open(os.path.join(golden_dir, "append_block_manager_example.json")))
    names, bt, cl, qsl, rows, pool = _append_example_arrays(g)
    out = append_kv_ref(pool, rows, bt, cl, qsl)
    for name, tok, blk, row in g["expected_slots"]:
        r = int(qsl[names.index(name)]) + tok
        assert np.array_equal(out[blk, 0, row], rows[r, 0]), (name, tok)
    for blk in g["untouched_blocks"]:
        assert np.array_equal(out[blk], pool[blk])
    for blk, row in g["untouched_rows"]:
        assert np.array_equal(out[blk, 0, row], pool[blk, 0, row])
    assert int((out != pool).any(axis=(1, 3)).sum()) == int(cl.sum())


def test_append_then_gather_returns_the_rows():
    """New tokens appended after a cached prefix read back, through the block
    table, at positions context_len - q_b .. context_len - 1; the prefix and
    every other slot keep their bytes."""
    rng = np.random.default_rng(11)
    bs, Hkv, D, nb = 4, 2, 5, 40
    ctx = np.array([7, 4, 13, 1])
    q = np.array([3, 4, 5, 1])
    qsl = np.concatenate([[0], np.cumsum(q)]).astype(np.int32)
    perm = rng.permutation(nb).astype(np.int32)
    bt = perm[:16].reshape(4, 4)
    pool = rng.integers(0, 2**16, size=(nb, Hkv, bs, D), dtype=np.uint16)
    rows = rng.integers(0, 2**16, size=(int(qsl[-1]), Hkv, D), dtype=np.uint16)
    out = append_kv_ref(pool, rows, bt, ctx, qsl)
    for b in range(4):
        for h in range(Hkv):
            got = gather_sequence(out, bt[b], int(ctx[b]), h)
            old = gather_sequence(pool, bt[b], int(ctx[b]), h)
            n_old = int(ctx[b] - q[b])
            assert np.array_equal(got[:n_old], old[:n_old])
            assert np.array_equal(got[n_old:], rows[qsl[b]:qsl[b + 1], h])
    used = set()
    for b in range(4):
        for j in range(int(ctx[b] - q[b]), int(ctx[b])):
            used.add((int(bt[b, j // bs]), j % bs))
    for blk in range(nb):
        for r in range(bs):
            if (blk, r) not in used:
                assert np.array_equal(out[blk, :, r], pool[blk, :, r])


def test_append_in_two_calls_equals_one_call():
    """Appending a sequence's new tokens in two calls (context_lens counting
    the tokens present after each) leaves the same pool as one call."""
    rng = np.random.default_rng(12)
    bs, nb = 8, 12
    pool = rng.normal(size=(nb, 2, bs, 4)).astype(np.float32)
    bt = rng.permutation(nb)[:6].astype(np.int32).reshape(2, 3)
    ctx = np.array([20, 17])
    q = np.array([9, 17])
    rows = rng.normal(size=(int(q.sum()), 2, 4)).astype(np.float32)
    one = append_kv_ref(pool, rows, bt, ctx, np.array([0, 9, 26]))
    # first call: 4 and 10 of the new tokens; second call: the rest
    first = np.concatenate([rows[0:4], rows[9:19]])
    second = np.concatenate([rows[4:9], rows[19:26]])
    two = append_kv_ref(pool, first, bt, ctx - np.array([5, 7]), np.array([0, 4, 14]))
    two = append_kv_ref(two, second, bt, ctx, np.array([0, 5, 12]))
    assert np.array_equal(one, two)


def test_append_skips_tokens_without_a_destination():
    """Positions before 0 (more new tokens than the context holds), past the
    table row, and table entries that are not pool blocks are not written."""
    bs, nb = 4, 6
    pool = np.zeros((nb, 1, bs, 2), dtype=np.float32)
    bt = np.array([[0, 1], [-1, 2], [3, 99]], dtype=np.int32)
    ctx = np.array([2, 8, 8])                     # seq 0: 3 new tokens but 2 in context
    q = np.array([3, 8, 8])
    qsl = np.concatenate([[0], np.cumsum(q)])
    rows = (np.arange(int(qsl[-1]), dtype=np.float32)[:, None, None] + 1) * np.ones((1, 1, 2))
    out = append_kv_ref(pool, rows, bt, ctx, qsl)
    assert np.array_equal(out[0, 0, 0], rows[1, 0]) and np.array_equal(out[0, 0, 1], rows[2, 0])
    assert np.array_equal(out[2, 0], rows[7:11, 0])      # seq 1, positions 4..7; 0..3 skipped
    assert np.array_equal(out[3, 0], rows[11:15, 0])     # seq 2, positions 0..3; 4..7 skipped
    for blk in (1, 4, 5):
        assert not out[blk].any()
    # positions past the table row (2 blocks of 4) are skipped as well
    out2 = append_kv_ref(pool, rows[:3], bt[:1], np.array([11]), np.array([0, 3]))   # 8, 9, 10
    assert not out2.any()
    out3 = append_kv_ref(pool, rows[:3], bt[:1], np.array([10]), np.array([0, 3]))   # 7 fits
    assert np.array_equal(out3[1, 0, 3], rows[0, 0]) and int((out3 != 0).any(axis=3).sum()) == 1
