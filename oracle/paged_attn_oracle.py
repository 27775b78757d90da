"""Plain, slow, fp64 CPU oracle for paged attention and paged block copy.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the CPU
baseline leg of the benchmark may import this module.  The GPU library never
calls it and shares no code with it.

Pages cited (by title):
  [P-swap]  "vLLM中FlashAttention与KVCache交换机制解析"
  [P-wall]  "大模型长文本推理基座从 FlashAttention 硬件加速机制到 vLLM 核心
             PagedAttention 显存物理布局深度剖析"
  [P-opt]   "vLLM中FlashAttention与KVCache优化解析"

Every routine is the plain definition written out: gather a sequence's K/V
through its block table, score with the scaled dot product, softmax in two
passes (max, then exp/sum), weight V.  Inputs are numpy arrays; floating
inputs are upcast exactly to float64 before any arithmetic, so fp16/bf16/fp32
values enter unchanged.  ``scale`` is taken as the float32 value the GPU sees,
promoted to float64.

Readings of points the pages leave open (all also listed in the design notes):
  * cache layout: separate K and V pools shaped [num_blocks, kv_heads,
    block_size, head_dim]; slot j of a sequence lives in physical block
    block_table[j // block_size] at row j % block_size;
  * GQA: query head h reads kv head h // (num_heads // num_kv_heads);
  * decode: context_lens[b] counts every cached key attended, the current
    token's included;
  * prefill: context_lens[b] counts prefix + new keys; new query t of a
    sequence with q_b new tokens sits at absolute position
    context_lens[b] - q_b + t and sees keys 0..position (bottom-right causal);
  * KV append: context_lens[b] counts the cached tokens after the append
    (as for prefill), so new token i of a sequence with q_b new tokens is
    logical token context_lens[b] - q_b + i; a token whose position is
    negative or past its table row, or whose table entry is not a block of
    the pool, is not written;
  * block copy: src_to_dst[i] = j copies source block i into destination
    block j; when several i name the same j the lowest i is the one taken, and
    it is taken only if it is a valid source index; -1 and any j outside the
    destination pool are ignored; untouched destination blocks keep their
    bytes.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "as_f64",
    "gather_sequence",
    "attend_two_pass",
    "decode_ref",
    "prefill_ref",
    "online_softmax_ref",
    "split_merge_ref",
    "decode_split_ref",
    "copy_blocks_ref",
    "append_kv_ref",
]


def as_f64(a) -> np.ndarray:
    """Exact upcast to float64 (fp16/fp32 numpy arrays, or float32 views of bf16)."""
    a = np.asarray(a)
    return a.astype(np.float64)


def _scale64(scale) -> np.float64:
    # The GPU receives the softmax scale as a float32; the oracle uses that
    # same value, widened.
    return np.float64(np.float32(scale))


def gather_sequence(cache: np.ndarray, table_row: np.ndarray, n: int, kv_head: int) -> np.ndarray:
    """Logical rows 0..n-1 of one sequence for one kv head, in logical order.

    [P-wall] §二.2 and [P-opt] "工程实现关键点 1 Block Table 管理": a logical
    block of ``block_size`` tokens maps through the per-sequence block table to
    a physical block anywhere in the pool.
    """
    block_size = cache.shape[2]
    j = np.arange(n)
    phys = np.asarray(table_row)[j // block_size]
    return cache[phys, kv_head, j % block_size, :]


def attend_two_pass(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale, mask=None) -> np.ndarray:
    """softmax(scale * q K^T) V with the two-pass softmax, float64.

    Attention(Q,K,V) = softmax(QK^T / sqrt(d_k)) V is the formula at the top of
    [P-swap]; the "traditional" softmax the same page describes scans once for
    the maximum, then for the exponential sum, then normalises.

    q: [..., D] query rows; K, V: [n, D]; mask: boolean [..., n], True = visible.
    """
    q = as_f64(q)
    K = as_f64(K)
    V = as_f64(V)
    s = _scale64(scale) * (q @ K.T)
    if mask is not None:
        s = np.where(mask, s, -np.inf)
    m = s.max(axis=-1, keepdims=True)          # pass 1: maximum
    w = np.exp(s - m)                          # pass 2: exponentials ...
    l = w.sum(axis=-1, keepdims=True)          # ... and their sum
    return (w @ V) / l


def decode_ref(query, k_cache, v_cache, block_tables, context_lens, scale,
               seqs=None, heads=None) -> np.ndarray:
    """Paged decode: one query token per sequence against its cached keys.

    query [B, Hq, D]; k_cache, v_cache [num_blocks, Hkv, bs, D];
    block_tables int [B, max_blocks]; context_lens int [B].
    Returns float64 [B, Hq, D]; rows not in (seqs x heads) are NaN.
    """
    query = np.asarray(query)
    B, Hq, D = query.shape
    Hkv = k_cache.shape[1]
    group = Hq // Hkv
    out = np.full((B, Hq, D), np.nan)
    seqs = range(B) if seqs is None else seqs
    heads = range(Hq) if heads is None else heads
    heads = sorted(set(heads))
    for b in seqs:
        n = int(context_lens[b])
        for g in sorted({h // group for h in heads}):
            K = gather_sequence(k_cache, block_tables[b], n, g)
            V = gather_sequence(v_cache, block_tables[b], n, g)
            hs = [h for h in heads if h // group == g]
            out[b, hs] = attend_two_pass(query[b, hs], K, V, scale)
    return out


def prefill_ref(query, k_cache, v_cache, block_tables, context_lens, query_start_loc,
                scale, rows=None, heads=None) -> np.ndarray:
    """Causal paged prefill / append.

    The serving flow in [P-swap] runs prefill through FlashAttention over every
    key of the request; here the new tokens of sequence b are query rows
    query_start_loc[b] .. query_start_loc[b+1]-1 of the packed query
    [T, Hq, D] and keys are read through the block table.  Row t of sequence b
    sits at position context_lens[b] - q_b + t and sees keys 0..position.

    rows: optional iterable of packed query-row indices to evaluate (others NaN).
    """
    query = np.asarray(query)
    T, Hq, D = query.shape
    Hkv = k_cache.shape[1]
    group = Hq // Hkv
    qsl = np.asarray(query_start_loc)
    out = np.full((T, Hq, D), np.nan)
    want = np.ones(T, dtype=bool) if rows is None else np.isin(np.arange(T), np.asarray(list(rows)))
    heads = range(Hq) if heads is None else heads
    heads = sorted(set(heads))
    for b in range(len(qsl) - 1):
        r0, r1 = int(qsl[b]), int(qsl[b + 1])
        sel = np.flatnonzero(want[r0:r1])
        if sel.size == 0:
            continue
        n = int(context_lens[b])
        q_b = r1 - r0
        pos = (n - q_b) + sel                       # absolute positions
        visible = np.arange(n)[None, :] <= pos[:, None]
        for g in sorted({h // group for h in heads}):
            K = gather_sequence(k_cache, block_tables[b], n, g)
            V = gather_sequence(v_cache, block_tables[b], n, g)
            for h in (h for h in heads if h // group == g):
                for c0 in range(0, sel.size, 256):   # bounded memory, same math
                    cs = sel[c0:c0 + 256]
                    out[r0 + cs, h] = attend_two_pass(query[r0 + cs, h], K, V, scale,
                                                      mask=visible[c0:c0 + 256])
    return out


def online_softmax_ref(x: np.ndarray, v: np.ndarray, tiles) -> tuple[float, float, np.ndarray]:
    """The one-pass recurrence of [P-swap] (OnlineSoftmax: M_new, L_new, O_new
    equations), with O kept normalised after every tile, exactly as printed.

    x: [n] scores (already scaled); v: [n, D]; tiles: list of (start, stop)
    covering 0..n in order.  Returns (M, L, O).  Initial state M = -inf, L = 0,
    O = 0 (not stated on the page; the natural empty-prefix values).
    """
    x = as_f64(x)
    v = as_f64(v)
    M, L = -math.inf, 0.0
    O = np.zeros(v.shape[1])
    for (a, b) in tiles:
        Xi, Vi = x[a:b], v[a:b]
        M_new = max(M, float(Xi.max()))
        carry = L * math.exp(M - M_new)            # L_old * exp(M_old - M_new)
        e = np.exp(Xi - M_new)
        L_new = carry + float(e.sum())
        O = (carry / L_new) * O + (e @ Vi) / L_new
        M, L = M_new, L_new
    return M, L, O


def split_merge_ref(x: np.ndarray, v: np.ndarray, partition: int) -> np.ndarray:
    """Split the key stream into partitions of ``partition`` keys, attend
    within each (two-pass: M_p, L_p, O_p), then combine the partials with the
    same rescaling the recurrence uses: M = max_p M_p,
    L = sum_p L_p exp(M_p - M), O = sum_p L_p exp(M_p - M) O_p / L.
    """
    x = as_f64(x)
    v = as_f64(v)
    Ms, Ls, Os = [], [], []
    for a in range(0, x.shape[0], partition):
        xs, vs = x[a:a + partition], v[a:a + partition]
        m = xs.max()
        w = np.exp(xs - m)
        Ms.append(m)
        Ls.append(w.sum())
        Os.append((w @ vs) / w.sum())
    Ms, Ls, Os = np.array(Ms), np.array(Ls), np.array(Os)
    M = Ms.max()
    c = Ls * np.exp(Ms - M)
    return (c[:, None] * Os).sum(axis=0) / c.sum()


def decode_split_ref(query, k_cache, v_cache, block_tables, context_lens, scale,
                     partition: int) -> np.ndarray:
    """Decode computed as per-partition partials merged by log-sum-exp."""
    query = np.asarray(query)
    B, Hq, D = query.shape
    Hkv = k_cache.shape[1]
    group = Hq // Hkv
    out = np.empty((B, Hq, D))
    s64 = _scale64(scale)
    for b in range(B):
        n = int(context_lens[b])
        for h in range(Hq):
            K = as_f64(gather_sequence(k_cache, block_tables[b], n, h // group))
            V = as_f64(gather_sequence(v_cache, block_tables[b], n, h // group))
            x = s64 * (K @ as_f64(query[b, h]))
            out[b, h] = split_merge_ref(x, V, partition)
    return out


def copy_blocks_ref(src: np.ndarray, dst: np.ndarray, src_to_dst) -> np.ndarray:
    """Block copy by mapping, byte for byte; returns the new destination pool.

    [P-swap] swap_blocks signature and its CPU mock: src_to_dst[i] = j means
    copy source block i into destination block j; -1 marks an unused entry.
    For each destination block, the lowest i naming it is chosen, and the copy
    happens only if that i is a valid source block.  [P-opt] "Swap Blocks 机制"
    applies the same mapping to the K pool and to the V pool; callers run this
    once per pool.
    """
    src = np.ascontiguousarray(src)
    out = np.array(dst, copy=True)
    m = np.asarray(src_to_dst).reshape(-1).astype(np.int64)
    num_src, num_dst = src.shape[0], out.shape[0]
    vals, first = np.unique(m, return_index=True)   # lowest index of each value
    take = (vals >= 0) & (vals < num_dst) & (first < num_src)
    sb = src.reshape(num_src, -1).view(np.uint8)
    ob = out.reshape(num_dst, -1).view(np.uint8)
    ob[vals[take]] = sb[first[take]]
    return out


def append_kv_ref(cache: np.ndarray, new_rows: np.ndarray, block_tables, context_lens,
                  query_start_loc) -> np.ndarray:
    """Write new tokens' K (or V) rows into the paged pool; returns the new pool.

    [P-opt] PagedAttention section, the PagedKVCache sketch: ``append`` adds a
    sequence's new KV rows after its cached ones, taking pool blocks through
    the sequence's block table; [P-wall] §二.2: logical token j of a sequence
    lives in physical block block_table[j // block_size] at row
    j % block_size.  new_rows is [total_new_tokens, kv_heads, head_dim]; the
    new tokens of sequence b are rows query_start_loc[b] ..
    query_start_loc[b + 1] - 1, and token i of them is logical token
    context_lens[b] - q_b + i.  Tokens are written one by one in (sequence,
    token) order, every kv head of a token at once, byte for byte; a token
    with no valid destination is skipped.  Callers run this once for the K
    pool and once for the V pool.
    """
    out = np.array(cache, copy=True)
    num_blocks, _, block_size, _ = out.shape
    tables = np.asarray(block_tables)
    ctx = np.asarray(context_lens).astype(np.int64)
    qsl = np.asarray(query_start_loc).astype(np.int64)
    rows = np.asarray(new_rows)
    max_pos = tables.shape[1] * block_size
    for b in range(len(ctx)):
        q_b = int(qsl[b + 1] - qsl[b])
        for i in range(q_b):
            pos = int(ctx[b]) - q_b + i
            if pos < 0 or pos >= max_pos:
                continue
            blk = int(tables[b, pos // block_size])
            if blk < 0 or blk >= num_blocks:
                continue
            out[blk, :, pos % block_size, :] = rows[qsl[b] + i]
    return out
