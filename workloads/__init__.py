"""Seeded synthetic inputs for paged attention and paged block copy.

This module draws inputs and nothing else: it holds none of the attention or
copy arithmetic.  Both the GPU tests and the fp64 oracle consume what it
produces, so every parity comparison runs on identical bytes.

Recipe (per workload, all seeded):
  * integer metadata (context lengths, block assignment, copy mapping) comes
    from ``numpy.random.default_rng(seed)``, so it is the same on every device;
  * Q/K/V are N(0, 1) drawn in float32 by a ``torch.Generator`` seeded with
    the same seed on the target device, then rounded to the storage dtype
    (round to nearest even);
  * physical blocks are handed out from a seeded permutation of the pool, so a
    sequence's blocks are scattered through the pool, as with the paged KV
    cache the pages describe;
  * with ``poison=True`` every pool block no sequence references is NaN, the
    slots past the context in each sequence's last block hold +1e4, and block
    table padding names a NaN block: a kernel that reads anything outside the
    context shows up in the output.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

from .work import (append_bytes, copy_bytes, copy_count_unique, decode_kv_bytes,  # noqa: F401
                   kv_cache_bytes, prefill_flops, prefill_pairs)

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}

_CHUNK = 1 << 25  # elements per randn call (bounded float32 temporaries)


def _randn_fill(t: torch.Tensor, gen: torch.Generator) -> None:
    flat = t.view(-1)
    for s in range(0, flat.numel(), _CHUNK):
        e = min(s + _CHUNK, flat.numel())
        flat[s:e] = torch.randn(e - s, generator=gen, device=t.device,
                                dtype=torch.float32).to(t.dtype)


def _generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


@dataclass
class PagedKV:
    """A paged K/V pool and the block tables that address it."""
    k_cache: torch.Tensor           # [num_blocks, Hkv, bs, D]
    v_cache: torch.Tensor           # [num_blocks, Hkv, bs, D]
    block_tables: torch.Tensor      # int32 [B, max_blocks_per_seq]
    context_lens: torch.Tensor      # int32 [B]
    free_blocks: np.ndarray         # physical ids referenced by no sequence
    block_size: int

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max().item()) if self.context_lens.numel() else 0


def make_paged_kv(context_lens, num_kv_heads: int, head_dim: int, block_size: int,
                  dtype: str, seed: int, device="cpu", rng=None, pool_blocks=None,
                  free_frac: float = 0.1, poison: bool = False,
                  max_blocks_per_seq=None) -> PagedKV:
    ctx = np.asarray(context_lens, dtype=np.int64)
    rng = np.random.default_rng(seed) if rng is None else rng
    nblk = (ctx + block_size - 1) // block_size
    needed = int(nblk.sum())
    pool = int(math.ceil((1.0 + free_frac) * needed)) if pool_blocks is None else int(pool_blocks)
    pool = max(pool, 1)
    if pool < needed:
        raise ValueError(f"pool of {pool} blocks cannot hold {needed}")
    perm = rng.permutation(pool)
    mbps = int(nblk.max()) if max_blocks_per_seq is None else int(max_blocks_per_seq)
    mbps = max(mbps, 1)
    free = np.sort(perm[needed:])
    pad = int(free[0]) if (poison and free.size) else 0
    tables = np.full((len(ctx), mbps), pad, dtype=np.int32)
    off = 0
    for b, n in enumerate(nblk):
        tables[b, :n] = perm[off:off + n]
        off += n
    dt = DTYPES[dtype]
    gen = _generator(seed, device)
    shape = (pool, num_kv_heads, block_size, head_dim)
    k = torch.empty(shape, dtype=dt, device=device)
    v = torch.empty(shape, dtype=dt, device=device)
    _randn_fill(k, gen)
    _randn_fill(v, gen)
    if poison:
        if free.size:
            fi = torch.as_tensor(free, device=device, dtype=torch.long)
            k[fi] = float("nan")
            v[fi] = float("nan")
        for b, n in enumerate(ctx):
            tail = int(n) % block_size
            if n > 0 and tail:
                last = int(tables[b, nblk[b] - 1])
                k[last, :, tail:, :] = 1e4
                v[last, :, tail:, :] = 1e4
    return PagedKV(k, v, torch.as_tensor(tables, device=device),
                   torch.as_tensor(ctx.astype(np.int32), device=device), free, block_size)


@dataclass
class DecodeInputs:
    query: torch.Tensor             # [B, Hq, D]
    kv: PagedKV
    scale: float
    dtype: str
    partition_size: int = 0         # 0 = library default
    name: str = ""

    @property
    def num_heads(self) -> int:
        return self.query.shape[1]


def make_decode(context_lens, num_heads: int, num_kv_heads: int, head_dim: int,
                block_size: int, dtype: str, seed: int, device="cpu", rng=None,
                name: str = "", partition_size: int = 0, **kv_kw) -> DecodeInputs:
    ctx = np.asarray(context_lens, dtype=np.int64)
    kv = make_paged_kv(ctx, num_kv_heads, head_dim, block_size, dtype, seed, device, rng=rng, **kv_kw)
    q = torch.empty((len(ctx), num_heads, head_dim), dtype=DTYPES[dtype], device=device)
    _randn_fill(q, _generator(seed + 7919, device))
    return DecodeInputs(q, kv, float(np.float32(1.0 / math.sqrt(head_dim))), dtype,
                        partition_size, name)


@dataclass
class PrefillInputs:
    query: torch.Tensor             # packed [T, Hq, D]
    query_start_loc: torch.Tensor   # int32 [B + 1]
    kv: PagedKV                     # context_lens = prefix + new tokens
    scale: float
    dtype: str
    max_query_len: int
    name: str = ""


def make_prefill(prefix_lens, query_lens, num_heads: int, num_kv_heads: int, head_dim: int,
                 block_size: int, dtype: str, seed: int, device="cpu", rng=None,
                 name: str = "", **kv_kw) -> PrefillInputs:
    pre = np.asarray(prefix_lens, dtype=np.int64)
    ql = np.asarray(query_lens, dtype=np.int64)
    kv = make_paged_kv(pre + ql, num_kv_heads, head_dim, block_size, dtype, seed, device,
                       rng=rng, **kv_kw)
    qsl = np.zeros(len(ql) + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(ql)
    q = torch.empty((int(qsl[-1]), num_heads, head_dim), dtype=DTYPES[dtype], device=device)
    _randn_fill(q, _generator(seed + 7919, device))
    return PrefillInputs(q, torch.as_tensor(qsl, device=device), kv,
                         float(np.float32(1.0 / math.sqrt(head_dim))), dtype,
                         int(ql.max()) if ql.size else 0, name)


@dataclass
class AppendInputs:
    kv: PagedKV                     # pools written in place; tables cover prefix + new
    key: torch.Tensor               # [T, Hkv, D] rows of the new tokens
    value: torch.Tensor             # [T, Hkv, D]
    query_start_loc: torch.Tensor   # int32 [B+1]
    dtype: str
    name: str = ""


def make_append(prefix_lens, new_lens, num_kv_heads: int, head_dim: int, block_size: int,
                dtype: str, seed: int, device="cpu", rng=None, name: str = "",
                **kv_kw) -> AppendInputs:
    """A paged pool whose tables already hold blocks for prefix + new tokens
    (context_lens counts both), and fresh N(0,1) K/V rows for the new tokens."""
    pre = np.asarray(prefix_lens, dtype=np.int64)
    ql = np.asarray(new_lens, dtype=np.int64)
    kv = make_paged_kv(pre + ql, num_kv_heads, head_dim, block_size, dtype, seed, device,
                       rng=rng, **kv_kw)
    qsl = np.zeros(len(ql) + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(ql)
    shape = (int(qsl[-1]), num_kv_heads, head_dim)
    key = torch.empty(shape, dtype=DTYPES[dtype], device=device)
    value = torch.empty(shape, dtype=DTYPES[dtype], device=device)
    gen = _generator(seed + 104729, device)
    _randn_fill(key, gen)
    _randn_fill(value, gen)
    return AppendInputs(kv, key, value, torch.as_tensor(qsl, device=device), dtype, name)


@dataclass
class CopyInputs:
    src_k: torch.Tensor
    src_v: torch.Tensor
    dst_k: torch.Tensor
    dst_v: torch.Tensor
    src_to_dst: torch.Tensor        # int64 [num_mappings]
    name: str = ""


def make_copy(num_src: int, num_dst: int, block_shape, dtype: str, seed: int, device="cpu",
              mapping=None, invalid_frac: float = 0.1, num_mappings=None,
              sentinel: float = -3.0, name: str = "") -> CopyInputs:
    """Source pools N(0,1); destination pools pre-filled with ``sentinel``.

    Default mapping: a seeded permutation of 0..num_mappings-1 (num_mappings
    defaults to num_dst) with ``invalid_frac`` of its positions set to -1.
    """
    rng = np.random.default_rng(seed)
    if mapping is None:
        nm = num_dst if num_mappings is None else int(num_mappings)
        m = rng.permutation(nm).astype(np.int64)
        bad = rng.choice(nm, size=int(round(invalid_frac * nm)), replace=False)
        m[bad] = -1
    else:
        m = np.asarray(mapping, dtype=np.int64)
    dt = DTYPES[dtype]
    gen = _generator(seed, device)
    src_k = torch.empty((num_src, *block_shape), dtype=dt, device=device)
    src_v = torch.empty((num_src, *block_shape), dtype=dt, device=device)
    _randn_fill(src_k, gen)
    _randn_fill(src_v, gen)
    dst_k = torch.full((num_dst, *block_shape), sentinel, dtype=dt, device=device)
    dst_v = torch.full((num_dst, *block_shape), sentinel, dtype=dt, device=device)
    return CopyInputs(src_k, src_v, dst_k, dst_v, torch.as_tensor(m, device=device), name)


# ---------------------------------------------------------------------------
# The named workloads.  Seeds 2481..2486 (the append workload reuses the
# prefill draw, 2485).
# ---------------------------------------------------------------------------

def tiny_decode_f32(device="cpu", **kw) -> DecodeInputs:
    """4 sequences, 4 query heads = 4 kv heads, head_dim 64, block_size 16,
    context lengths uniform in [1, 200], a pool of 64 physical blocks handed
    out by a seeded permutation, fp32."""
    rng = np.random.default_rng(2481)
    ctx = rng.integers(1, 200, size=4, endpoint=True)
    return make_decode(ctx, 4, 4, 64, 16, "f32", 2481, device, rng=rng, pool_blocks=64,
                       name="tiny_decode_f32", **kw)


def llama7b_decode_f16(device="cpu", num_seqs: int = 64, **kw) -> DecodeInputs:
    """LLaMA-7B-shaped single-layer decode: 64 sequences, 32 heads = 32 kv
    heads, head_dim 128, block_size 16, context lengths uniform in
    [512, 4096], pool = needed blocks + 10% free, shuffled, fp16."""
    rng = np.random.default_rng(2482)
    ctx = rng.integers(512, 4096, size=num_seqs, endpoint=True)
    return make_decode(ctx, 32, 32, 128, 16, "f16", 2482, device, rng=rng,
                       name="llama7b_decode_f16", **kw)


def gqa_decode_bf16(device="cpu", num_seqs: int = 128, **kw) -> DecodeInputs:
    """GQA decode: 128 sequences, 32 query heads sharing 8 kv heads,
    head_dim 128, block_size 16, context lengths lognormal with median 2048
    and sigma 1 clipped to [16, 32768], pool + 10%, permuted, bf16."""
    rng = np.random.default_rng(2483)
    z = rng.standard_normal(num_seqs)
    ctx = np.clip(np.rint(2048.0 * np.exp(1.0 * z)), 16, 32768).astype(np.int64)
    return make_decode(ctx, 32, 8, 128, 16, "bf16", 2483, device, rng=rng,
                       name="gqa_decode_bf16", **kw)


def long_decode_f16(device="cpu", num_seqs: int = 16, context: int = 32768, **kw) -> DecodeInputs:
    """Long-context split-KV decode: 16 sequences of 32768 cached tokens,
    32 heads = 32 kv heads, head_dim 128, block_size 32, fragmented random
    block tables (pool + 10%), KV partitions of 512 tokens, fp16."""
    rng = np.random.default_rng(2484)
    ctx = np.full(num_seqs, context, dtype=np.int64)
    kw.setdefault("partition_size", 512)
    return make_decode(ctx, 32, 32, 128, 32, "f16", 2484, device, rng=rng,
                       name="long_decode_f16", **kw)


def prefill_bf16(device="cpu", num_seqs: int = 8, query_len: int = 2048, **kw) -> PrefillInputs:
    """Causal paged prefill/append: 8 sequences each appending 2048 new
    tokens to cached prefixes uniform in [0, 8192], 32 query heads sharing
    8 kv heads, head_dim 128, block_size 16, pool + 10% permuted, bf16."""
    rng = np.random.default_rng(2485)
    pre = rng.integers(0, 8192, size=num_seqs, endpoint=True)
    ql = np.full(num_seqs, query_len, dtype=np.int64)
    return make_prefill(pre, ql, 32, 8, 128, 16, "bf16", 2485, device, rng=rng,
                        name="prefill_bf16", **kw)


def append_bf16(device="cpu", num_seqs: int = 8, new_len: int = 2048, **kw) -> AppendInputs:
    """KV append of the prefill workload's new tokens: 8 sequences each
    appending 2048 tokens after cached prefixes uniform in [0, 8192] (the same
    draw and pool as prefill_bf16), 8 kv heads, head_dim 128, block_size 16,
    pool + 10% permuted, bf16; new rows N(0,1)."""
    rng = np.random.default_rng(2485)
    pre = rng.integers(0, 8192, size=num_seqs, endpoint=True)
    ql = np.full(num_seqs, new_len, dtype=np.int64)
    return make_append(pre, ql, 8, 128, 16, "bf16", 2485, device, rng=rng,
                       name="append_bf16", **kw)


@dataclass
class SwapInputs:
    dev_k: torch.Tensor             # device pools [num_dev, *block_shape]
    dev_v: torch.Tensor
    host_k: torch.Tensor            # pinned host pools [num_host, *block_shape]
    host_v: torch.Tensor
    out_map: torch.Tensor           # int64 [num_dev] on the device: dev block i -> host block
    in_map: torch.Tensor            # int64 [num_host] on the device: host block i -> dev block
    name: str = ""


def make_swap(num_dev: int, num_host: int, block_shape, dtype: str, seed: int, device="cuda",
              invalid_frac: float = 0.1, name: str = "") -> SwapInputs:
    """Device pools N(0,1), pinned host pools N(0,1) drawn after them (a
    distinct pattern, so a swap in is visible); each mapping is a seeded
    permutation of the other pool's block ids with ``invalid_frac`` of its
    entries set to -1 (swap out: device block i -> host block out_map[i];
    swap in: host block i -> device block in_map[i])."""
    rng = np.random.default_rng(seed)

    def mapping(n_from, n_to):
        m = rng.permutation(max(n_from, n_to))[:n_from].astype(np.int64)
        m[m >= n_to] = -1
        bad = rng.choice(n_from, size=int(round(invalid_frac * n_from)), replace=False)
        m[bad] = -1
        return m

    out_map, in_map = mapping(num_dev, num_host), mapping(num_host, num_dev)
    dt = DTYPES[dtype]
    gen = _generator(seed, device)
    dev_k = torch.empty((num_dev, *block_shape), dtype=dt, device=device)
    dev_v = torch.empty((num_dev, *block_shape), dtype=dt, device=device)
    _randn_fill(dev_k, gen)
    _randn_fill(dev_v, gen)
    host_k = torch.empty((num_host, *block_shape), dtype=dt, pin_memory=True)
    host_v = torch.empty((num_host, *block_shape), dtype=dt, pin_memory=True)
    tmp = torch.empty((num_host, *block_shape), dtype=dt, device=device)
    _randn_fill(tmp, gen)
    host_k.copy_(tmp)
    _randn_fill(tmp, gen)
    host_v.copy_(tmp)
    del tmp
    return SwapInputs(dev_k, dev_v, host_k, host_v, torch.as_tensor(out_map, device=device),
                      torch.as_tensor(in_map, device=device), name)


def swap_bf16(device="cuda", **kw) -> SwapInputs:
    """Host<->device swap of K and V blocks: 2048 device blocks and 2048
    pinned host blocks of [8, 16, 128] bf16 (32 KiB per block per pool), each
    mapping a seeded permutation with 10% -1 (1843 blocks moved per
    direction)."""
    return make_swap(2048, 2048, (8, 16, 128), "bf16", 2487, device, name="swap_bf16", **kw)


def copy_bf16(device="cpu", **kw) -> CopyInputs:
    """Block copy of K and V pools: source pool 8192 blocks, destination pool
    4096 blocks of [8 heads, 16 slots, 128] bf16, mapping of length 4096 = a
    seeded permutation of 0..4095 with 10% of entries -1."""
    return make_copy(8192, 4096, (8, 16, 128), "bf16", 2486, device, name="copy_bf16", **kw)


WORKLOADS = {
    "tiny_decode_f32": tiny_decode_f32,
    "llama7b_decode_f16": llama7b_decode_f16,
    "gqa_decode_bf16": gqa_decode_bf16,
    "long_decode_f16": long_decode_f16,
    "prefill_bf16": prefill_bf16,
    "copy_bf16": copy_bf16,
    "append_bf16": append_bf16,
    "swap_bf16": swap_bf16,
}
