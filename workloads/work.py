"""Algorithmic work of each path: the bytes or flops the method itself must
move or compute, independent of how a kernel does it.  Used to turn measured
times into GB/s and TFLOP/s.  Scores and probabilities never reach memory, and
split-KV partials are implementation overhead, so neither is counted.
"""

from __future__ import annotations

import numpy as np


def kv_cache_bytes(n_layers: int, n_heads: int, d_head: int, seq: int, batch: int,
                   elem_bytes: int = 2) -> int:
    """Bytes of a dense KV cache: K and V (factor 2), each element ``elem_bytes``.

    This is the memory formula of §一 of "大模型长文本推理基座从 FlashAttention
    硬件加速机制到 vLLM 核心 PagedAttention 显存物理布局深度剖析" (fp16 there).
    """
    return 2 * elem_bytes * n_layers * n_heads * d_head * seq * batch


def decode_kv_bytes(context_lens, num_heads: int, num_kv_heads: int, head_dim: int,
                    block_size: int, elem_bytes: int) -> int:
    """K and V of every attended token once per kv head, the query read, the
    output written, the block-table entries used and the context lengths."""
    ctx = np.asarray(context_lens, dtype=np.int64)
    B = ctx.size
    kv = int(ctx.sum()) * num_kv_heads * head_dim * 2 * elem_bytes
    qo = 2 * B * num_heads * head_dim * elem_bytes
    tables = 4 * int(((ctx + block_size - 1) // block_size).sum())
    return kv + qo + tables + 4 * B


def prefill_pairs(context_lens, query_lens) -> int:
    """Number of visible (query, key) pairs under the bottom-right causal mask:
    sum over sequences of sum_{t < q_b} (ctx_b - q_b + t + 1)."""
    ctx = np.asarray(context_lens, dtype=np.int64)
    ql = np.asarray(query_lens, dtype=np.int64)
    pre = ctx - ql
    return int((ql * pre + ql * (ql + 1) // 2).sum())


def prefill_flops(context_lens, query_lens, num_heads: int, head_dim: int) -> int:
    """QK^T and PV over the visible pairs only: 2 products x 2 flops x D each."""
    return 4 * head_dim * num_heads * prefill_pairs(context_lens, query_lens)


def copy_bytes(num_copied: int, block_bytes: int, pools: int = 2) -> int:
    """Each copied block is read once and written once, in each pool (K and V)."""
    return 2 * pools * num_copied * block_bytes


def copy_count_unique(src_to_dst, num_src: int, num_dst: int) -> int:
    """Copies made by a mapping whose valid destinations are all distinct."""
    m = np.asarray(src_to_dst, dtype=np.int64).reshape(-1)
    i = np.arange(m.size)
    ok = (m >= 0) & (m < num_dst)
    if np.unique(m[ok]).size != int(ok.sum()):
        raise ValueError("mapping names a destination more than once")
    return int((ok & (i < num_src)).sum())


def append_bytes(num_tokens: int, num_seqs: int, num_kv_heads: int, head_dim: int,
                 block_size: int, elem_bytes: int, pools: int = 2) -> int:
    """Each new token's rows are read once and written once, in each pool (K
    and V), plus the per-sequence metadata (query_start_loc, context_lens)
    and one block-table entry per block-sized run of new tokens."""
    rows = 2 * pools * num_tokens * num_kv_heads * head_dim * elem_bytes
    meta = 4 * (num_seqs + 1) + 4 * num_seqs + 4 * ((num_tokens + block_size - 1) // block_size)
    return rows + meta

