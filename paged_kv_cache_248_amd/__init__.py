"""MI355X (gfx950) paged attention: Python binding of libpagedattn.so.

Argument marshalling only.  Every step of decode, prefill and block copy runs
in the HIP kernels of the shared library; PyTorch supplies device memory and
the current stream.  The functions carry the names of the C entry points in
include/paged_attn.h and raise ``PagedAttnError`` on a non-zero status.  If
the library has not been built, every call raises: there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "PagedAttnError", "library_path", "load_library",
    "paged_attn_decode", "paged_attn_decode_workspace_size", "paged_attn_decode_noalloc",
    "DECODE_NOALLOC_SCRATCH_BYTES",
    "paged_attn_prefill", "paged_attn_prefill_halftile",
    "paged_attn_prefill_unfused", "paged_attn_prefill_unfused_workspace_size",
    "paged_kv_copy_blocks", "paged_kv_copy_blocks_workspace_size",
    "paged_kv_append", "BlockManager", "OutOfBlocksError",
    "DEFAULT_PARTITION", "DEFAULT_PARTITION_GQA", "default_partition",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_PARTITION = 512       # PA_DEFAULT_PARTITION
DEFAULT_PARTITION_GQA = 4096  # PA_DEFAULT_PARTITION_GQA
DECODE_NOALLOC_SCRATCH_BYTES = 64 << 20   # PA_DECODE_NOALLOC_SCRATCH_BYTES


def default_partition(num_heads: int, num_kv_heads: int) -> int:
    """Partition length decode uses for partition_size=0 (same rule as the library)."""
    return DEFAULT_PARTITION_GQA if num_heads // num_kv_heads >= 4 else DEFAULT_PARTITION

_DTYPE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}

_VP = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

_SIGS = {
    "pa_status_string": (ctypes.c_char_p, [ctypes.c_int32]),
    "pa_set_profile_events": (ctypes.c_int, [_VP, _VP]),
    "paged_attn_decode_workspace_size": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32]),
    "paged_attn_decode": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _I32, _I32,
                                          _I32, _I32, _I32, _I32, ctypes.c_float, ctypes.c_int,
                                          _I32, _VP, _SZ, _VP]),
    "paged_attn_decode_noalloc": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _I32,
                                                  _I32, _I32, _I32, _I32, _I32, ctypes.c_float,
                                                  ctypes.c_int, _I32, _VP]),
    "paged_attn_prefill": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _I32,
                                           _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                           ctypes.c_float, ctypes.c_int, _VP]),
    "paged_attn_prefill_halftile": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _I32,
                                                    _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                                    _I32, ctypes.c_float, ctypes.c_int, _VP]),
    "paged_attn_prefill_unfused_workspace_size": (_SZ, [_I32, _I32, _I32, _I32, _I32,
                                                        ctypes.c_int]),
    "paged_attn_prefill_unfused": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _I32,
                                                   _I32, _I32, _I32, _I32, _I32, _I32,
                                                   ctypes.c_float, ctypes.c_int, _VP, _SZ, _VP]),
    "paged_kv_copy_blocks_workspace_size": (_SZ, [_I64]),
    "pa_host_device_pointer": (ctypes.c_int, [_VP, ctypes.POINTER(ctypes.c_void_p)]),
    "pa_stream_read": (ctypes.c_int, [_VP, _I64, _VP, _I32, _VP]),
    "pa_stream_copy": (ctypes.c_int, [_VP, _VP, _I64, _I32, _VP]),
    "pa_mfma_stream": (ctypes.c_int, [_VP, _I64, _VP, _I32, _I32, _I32, _I32, _VP]),
    "pa_bm_create": (ctypes.c_int, [_I32, _I32, ctypes.POINTER(ctypes.c_void_p)]),
    "pa_bm_destroy": (None, [_VP]),
    "pa_bm_register": (ctypes.c_int, [_VP, _I64, _I64]),
    "pa_bm_append_token": (ctypes.c_int, [_VP, _I64, ctypes.POINTER(_I32), ctypes.POINTER(_I32)]),
    "pa_bm_append_tokens": (ctypes.c_int, [_VP, _VP, _I32, _VP, _VP]),
    "pa_bm_fork": (ctypes.c_int, [_VP, _I64, _I64]),
    "pa_bm_finish": (ctypes.c_int, [_VP, _I64]),
    "pa_bm_free_count": (_I32, [_VP]),
    "pa_bm_block_table": (ctypes.c_int, [_VP, _I64, _VP, _I32, ctypes.POINTER(_I32),
                                         ctypes.POINTER(_I64)]),
    "pa_bm_free_list": (ctypes.c_int, [_VP, _VP, _I32, ctypes.POINTER(_I32)]),
    "pa_bm_ref_count": (ctypes.c_int, [_VP, _I32, ctypes.POINTER(_I32)]),
    "pa_bm_fill_batch": (ctypes.c_int, [_VP, _VP, _I32, _I32, _VP, _VP]),
    "paged_kv_append": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _I32, _I32,
                                        _I32, _I32, _I32, ctypes.c_int, _VP]),
    "paged_kv_copy_blocks": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _I64, _I64, _I64, _I64,
                                             _VP, _SZ, _VP]),
}

_lib = None


class PagedAttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


def library_path() -> str:
    """The in-tree library, or the file PA_LIBRARY names (the host-sanitized
    build, for CPU runs of the host-side tests)."""
    return os.environ.get("PA_LIBRARY") or os.path.join(_HERE, "libpagedattn.so")


def load_library():
    """Load (once) and return the ctypes handle; raises if it is not built."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with `python -m paged_kv_cache_248_amd.build` "
                "(there is no non-HIP fallback)")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load_library().pa_status_string(status).decode()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise PagedAttnError(status, what)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, anchor: torch.Tensor) -> ctypes.c_void_p:
    """Handle of `stream` (None: torch's current stream).  The library works on
    the current HIP device, so the call's device tensors (represented by
    `anchor`) and the stream must belong to it."""
    dev = torch.cuda.current_device()
    if anchor.device.index != dev:
        raise ValueError(f"tensors are on {anchor.device} but the current device is cuda:{dev}; "
                         f"call under torch.cuda.device({anchor.device.index})")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    elif hasattr(stream, "device") and stream.device.index != dev:
        raise ValueError(f"stream belongs to {stream.device}, the current device is cuda:{dev}")
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _need(t: torch.Tensor, name: str, dtype=None, dims=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dims, got {t.dim()}")


def paged_attn_decode_workspace_size(num_seqs: int, num_heads: int, num_kv_heads: int,
                                     head_dim: int, max_context_len: int,
                                     partition_size: int = 0) -> int:
    return int(load_library().paged_attn_decode_workspace_size(
        num_seqs, num_heads, num_kv_heads, head_dim, max_context_len, partition_size))


def _decode_shapes(out, query, k_cache, v_cache, block_tables, context_lens):
    _need(query, "query", dims=3)
    dt = query.dtype
    if dt not in _DTYPE:
        raise ValueError(f"unsupported dtype {dt}")
    _need(out, "out", dt, 3)
    _need(k_cache, "k_cache", dt, 4)
    _need(v_cache, "v_cache", dt, 4)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    if v_cache.shape != k_cache.shape or out.shape != query.shape:
        raise ValueError("k_cache/v_cache or out/query shapes differ")
    B, Hq, D = query.shape
    nblk, Hkv, bs, Dk = k_cache.shape
    if Dk != D or block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("inconsistent shapes")
    return B, Hq, Hkv, D, nblk, bs, block_tables.shape[1], dt


def paged_attn_decode_noalloc(out: torch.Tensor, query: torch.Tensor, k_cache: torch.Tensor,
                              v_cache: torch.Tensor, block_tables: torch.Tensor,
                              context_lens: torch.Tensor, scale: float,
                              max_context_len: Optional[int] = None, partition_size: int = 0,
                              stream=None) -> torch.Tensor:
    """paged_attn_decode without a workspace: the library keeps the work
    list and split-KV partials in its own static device array
    (DECODE_NOALLOC_SCRATCH_BYTES per GPU), so the call allocates nothing.
    Calls that overlap in time on one GPU share that array and race."""
    lib = load_library()
    B, Hq, Hkv, D, nblk, bs, mbps, dt = _decode_shapes(out, query, k_cache, v_cache,
                                                       block_tables, context_lens)
    if max_context_len is None:
        max_context_len = mbps * bs
    st = lib.paged_attn_decode_noalloc(_ptr(out), _ptr(query), _ptr(k_cache), _ptr(v_cache),
                                       _ptr(block_tables), _ptr(context_lens), B, Hq, Hkv, D,
                                       bs, nblk, mbps, int(max_context_len), float(scale),
                                       _DTYPE[dt], int(partition_size), _stream(stream, query))
    _check(st, "paged_attn_decode_noalloc")
    return out


def paged_attn_decode(out: torch.Tensor, query: torch.Tensor, k_cache: torch.Tensor,
                      v_cache: torch.Tensor, block_tables: torch.Tensor,
                      context_lens: torch.Tensor, scale: float,
                      max_context_len: Optional[int] = None, partition_size: int = 0,
                      workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """out[b,h] = softmax(scale * q[b,h] K_b^T) V_b over the paged cache.

    query/out [B, Hq, D]; k_cache/v_cache [num_blocks, Hkv, block_size, D];
    block_tables int32 [B, max_blocks]; context_lens int32 [B].
    ``max_context_len`` (host int) bounds context_lens; None means
    max_blocks * block_size.  partition_size: 0 = default, -1 = never split.
    """
    lib = load_library()
    B, Hq, Hkv, D, nblk, bs, mbps, dt = _decode_shapes(out, query, k_cache, v_cache,
                                                       block_tables, context_lens)
    if max_context_len is None:
        max_context_len = mbps * bs
    need = paged_attn_decode_workspace_size(B, Hq, Hkv, D, max_context_len, partition_size)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=query.device)
    else:
        _need(workspace, "workspace", torch.uint8, 1)
    st = lib.paged_attn_decode(_ptr(out), _ptr(query), _ptr(k_cache), _ptr(v_cache),
                               _ptr(block_tables), _ptr(context_lens), B, Hq, Hkv, D, bs,
                               nblk, mbps, int(max_context_len), float(scale), _DTYPE[dt],
                               int(partition_size), _ptr(workspace), workspace.numel(),
                               _stream(stream, query))
    _check(st, "paged_attn_decode")
    return out


def paged_attn_prefill(out: torch.Tensor, query: torch.Tensor, k_cache: torch.Tensor,
                       v_cache: torch.Tensor, block_tables: torch.Tensor,
                       context_lens: torch.Tensor, query_start_loc: torch.Tensor,
                       scale: float, max_query_len: int, max_context_len: int,
                       stream=None) -> torch.Tensor:
    """Causal prefill/append of packed new tokens over the paged cache.

    query/out [T, Hq, D]; query_start_loc int32 [B+1]; context_lens int32 [B]
    counts prefix + new keys (all already in the cache).
    """
    return _prefill("paged_attn_prefill", out, query, k_cache, v_cache, block_tables,
                    context_lens, query_start_loc, scale, max_query_len, max_context_len, stream)


def paged_attn_prefill_halftile(out: torch.Tensor, query: torch.Tensor, k_cache: torch.Tensor,
                                v_cache: torch.Tensor, block_tables: torch.Tensor,
                                context_lens: torch.Tensor, query_start_loc: torch.Tensor,
                                scale: float, max_query_len: int, max_context_len: int,
                                stream=None) -> torch.Tensor:
    """The same prefill with the library's second (half-tile) kernel schedule."""
    return _prefill("paged_attn_prefill_halftile", out, query, k_cache, v_cache, block_tables,
                    context_lens, query_start_loc, scale, max_query_len, max_context_len, stream)


def _prefill(name, out, query, k_cache, v_cache, block_tables, context_lens, query_start_loc,
             scale, max_query_len, max_context_len, stream):
    lib = load_library()
    _need(query, "query", dims=3)
    dt = query.dtype
    if dt not in _DTYPE:
        raise ValueError(f"unsupported dtype {dt}")
    _need(out, "out", dt, 3)
    _need(k_cache, "k_cache", dt, 4)
    _need(v_cache, "v_cache", dt, 4)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    _need(query_start_loc, "query_start_loc", torch.int32, 1)
    T, Hq, D = query.shape
    nblk, Hkv, bs, Dk = k_cache.shape
    B = context_lens.shape[0]
    if (Dk != D or out.shape != query.shape or v_cache.shape != k_cache.shape
            or block_tables.shape[0] != B or query_start_loc.shape[0] != B + 1):
        raise ValueError("inconsistent shapes")
    st = getattr(lib, name)(_ptr(out), _ptr(query), _ptr(k_cache), _ptr(v_cache),
                            _ptr(block_tables), _ptr(context_lens), _ptr(query_start_loc),
                            B, T, int(max_query_len), int(max_context_len), Hq, Hkv, D, bs,
                            nblk, block_tables.shape[1], float(scale), _DTYPE[dt],
                            _stream(stream, query))
    _check(st, name)
    return out


def paged_attn_prefill_unfused_workspace_size(max_query_len: int, max_context_len: int,
                                              num_heads: int, num_kv_heads: int, head_dim: int,
                                              dtype: torch.dtype) -> int:
    return int(load_library().paged_attn_prefill_unfused_workspace_size(
        int(max_query_len), int(max_context_len), int(num_heads), int(num_kv_heads),
        int(head_dim), _DTYPE[dtype]))


def _host_i32(t, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        t = torch.as_tensor(t)
    if t.dtype != torch.int32 or t.dim() != 1:
        raise ValueError(f"{name} must be a 1-D int32 tensor")
    return t.cpu().contiguous()


def paged_attn_prefill_unfused(out: torch.Tensor, query: torch.Tensor, k_cache: torch.Tensor,
                               v_cache: torch.Tensor, block_tables: torch.Tensor,
                               context_lens, query_start_loc, scale: float,
                               workspace: Optional[torch.Tensor] = None,
                               stream=None) -> torch.Tensor:
    """Prefill computed the unfused way (S and P written to HBM): the
    baseline of paged_attn_prefill, same arguments and result.

    context_lens / query_start_loc are int32 vectors; the C call takes them in
    host memory, so device tensors are copied to the host first (a sync).
    workspace: uint8 device tensor of at least
    paged_attn_prefill_unfused_workspace_size(...) bytes (allocated here if
    None).
    """
    lib = load_library()
    _need(query, "query", dims=3)
    dt = query.dtype
    if dt not in (torch.float16, torch.bfloat16):
        raise ValueError(f"unsupported dtype {dt}")
    _need(out, "out", dt, 3)
    _need(k_cache, "k_cache", dt, 4)
    _need(v_cache, "v_cache", dt, 4)
    _need(block_tables, "block_tables", torch.int32, 2)
    cl = _host_i32(context_lens, "context_lens")
    qsl = _host_i32(query_start_loc, "query_start_loc")
    T, Hq, D = query.shape
    nblk, Hkv, bs, Dk = k_cache.shape
    B = cl.shape[0]
    if (Dk != D or out.shape != query.shape or v_cache.shape != k_cache.shape
            or block_tables.shape[0] != B or qsl.shape[0] != B + 1):
        raise ValueError("inconsistent shapes")
    ql = qsl[1:] - qsl[:-1]
    live = ql > 0
    max_q = int(ql.max()) if B else 0
    max_ctx = int(cl[live].max()) if bool(live.any()) else 0
    need = paged_attn_prefill_unfused_workspace_size(max_q, max_ctx, Hq, Hkv, D, dt)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=query.device)
    _need(workspace, "workspace", torch.uint8, 1)
    st = lib.paged_attn_prefill_unfused(
        _ptr(out), _ptr(query), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        ctypes.c_void_p(cl.data_ptr()), ctypes.c_void_p(qsl.data_ptr()), B, T, Hq, Hkv, D, bs,
        nblk, block_tables.shape[1], float(scale), _DTYPE[dt], _ptr(workspace),
        workspace.numel(), _stream(stream, query))
    _check(st, "paged_attn_prefill_unfused")
    return out


def pa_stream_read(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Read every byte of `src` once on the GPU (measurement probe); work-group
    i writes the XOR of the 32-bit words it read to sink[i] (int32 device
    tensor; at most sink.numel() work-groups)."""
    lib = load_library()
    _need(src, "src")
    _need(sink, "sink", torch.int32, 1)
    _check(lib.pa_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                              sink.numel(), _stream(stream, src)), "pa_stream_read")


def pa_stream_copy(src: torch.Tensor, dst: torch.Tensor, wgs_per_cu: int = 0, stream=None) -> None:
    """Copy-stream probe: dst[:] = src with non-temporal 16-byte accesses
    (measurement of the practical read+write ceiling)."""
    lib = load_library()
    _need(src, "src")
    _need(dst, "dst")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst sizes differ")
    _check(lib.pa_stream_copy(_ptr(src), _ptr(dst), nbytes, int(wgs_per_cu), _stream(stream, src)),
           "pa_stream_copy")


def pa_mfma_stream(operands: torch.Tensor, sink: torch.Tensor, wgs_per_cu: int, iters: int,
                   stream=None) -> None:
    """Matrix-core stream probe: min(CUs x wgs_per_cu, sink.numel()) work-groups
    of four wavefronts, each wavefront `iters` rounds of 32 MFMA 32x32x16 on
    operands (fp16 or bf16, random data) read once; work-group i writes the
    sum of its accumulators to sink[i] (fp32)."""
    lib = load_library()
    _need(operands, "operands")
    _need(sink, "sink", torch.float32)
    if operands.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("operands must be float16 or bfloat16")
    _check(lib.pa_mfma_stream(_ptr(operands), operands.numel() * operands.element_size(),
                              _ptr(sink), sink.numel(), int(wgs_per_cu), int(iters),
                              _DTYPE[operands.dtype], _stream(stream, operands)),
           "pa_mfma_stream")


def paged_kv_append(k_cache: torch.Tensor, v_cache: Optional[torch.Tensor], key: torch.Tensor,
                    value: Optional[torch.Tensor], block_tables: torch.Tensor,
                    context_lens: torch.Tensor, query_start_loc: torch.Tensor,
                    stream=None) -> None:
    """Write new tokens' K (and V) rows [T, Hkv, D] into the paged pools.

    Sequence b's new tokens are rows query_start_loc[b]..query_start_loc[b+1]-1;
    context_lens counts the tokens cached after the append, so new token i is
    logical token context_lens[b] - q_b + i, stored in block
    block_tables[b][pos // block_size] at row pos % block_size.
    """
    lib = load_library()
    _need(key, "key", dims=3)
    dt = key.dtype
    if dt not in _DTYPE:
        raise ValueError(f"unsupported dtype {dt}")
    _need(k_cache, "k_cache", dt, 4)
    if (v_cache is None) != (value is None):
        raise ValueError("v_cache and value must both be given or both be None")
    if v_cache is not None:
        _need(v_cache, "v_cache", dt, 4)
        _need(value, "value", dt, 3)
        if v_cache.shape != k_cache.shape or value.shape != key.shape:
            raise ValueError("K and V shapes differ")
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    _need(query_start_loc, "query_start_loc", torch.int32, 1)
    T, Hkv, D = key.shape
    nblk, Hkv_c, bs, D_c = k_cache.shape
    B = context_lens.shape[0]
    if (Hkv_c != Hkv or D_c != D or block_tables.shape[0] != B
            or query_start_loc.shape[0] != B + 1):
        raise ValueError("inconsistent shapes")
    st = lib.paged_kv_append(_ptr(k_cache), _ptr(v_cache), _ptr(key), _ptr(value),
                             _ptr(block_tables), _ptr(context_lens), _ptr(query_start_loc),
                             B, T, Hkv, D, bs, nblk, block_tables.shape[1], _DTYPE[dt],
                             _stream(stream, key))
    _check(st, "paged_kv_append")


def paged_kv_copy_blocks_workspace_size(num_dst_blocks: int) -> int:
    return int(load_library().paged_kv_copy_blocks_workspace_size(num_dst_blocks))


def _pool_ptr(t: Optional[torch.Tensor], name: str):
    """Device-accessible address of a block pool: a device tensor, or a pinned
    host tensor (the host side of a swap)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.is_cuda:
        return _ptr(t)
    if not t.is_pinned():
        raise ValueError(f"{name} must be a device tensor or pinned host memory")
    if t.numel() == 0:
        return None
    dev = ctypes.c_void_p()
    st = load_library().pa_host_device_pointer(ctypes.c_void_p(t.data_ptr()), ctypes.byref(dev))
    _check(st, "pa_host_device_pointer")
    return dev


def paged_kv_copy_blocks(src_k: torch.Tensor, src_v: Optional[torch.Tensor], dst_k: torch.Tensor,
                         dst_v: Optional[torch.Tensor], src_to_dst: torch.Tensor,
                         workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """dst[j] <- src[i] for src_to_dst[i] = j (lowest i per j, valid i only),
    applied to the K pool pair and, if given, the V pool pair.  Either pool
    pair may be pinned host memory (swap out / swap in); src_to_dst and the
    workspace are device tensors."""
    lib = load_library()
    _pool_ptr(src_k, "src_k")
    _pool_ptr(dst_k, "dst_k")
    _need(src_to_dst, "src_to_dst", torch.int64, 1)
    if (src_v is None) != (dst_v is None):
        raise ValueError("src_v and dst_v must both be given or both be None")
    if src_v is not None:
        _pool_ptr(src_v, "src_v")
        _pool_ptr(dst_v, "dst_v")
        if src_v.shape != src_k.shape or dst_v.shape != dst_k.shape:
            raise ValueError("K and V pools must have matching shapes")
    if src_k.shape[1:] != dst_k.shape[1:] or src_k.dtype != dst_k.dtype:
        raise ValueError("source and destination blocks differ in shape or dtype")
    num_src, num_dst = src_k.shape[0], dst_k.shape[0]
    block_bytes = src_k[0].numel() * src_k.element_size() if num_src else dst_k[0].numel() * dst_k.element_size()
    need = paged_kv_copy_blocks_workspace_size(num_dst)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=src_to_dst.device)
    else:
        _need(workspace, "workspace", torch.uint8, 1)
    st = lib.paged_kv_copy_blocks(_pool_ptr(src_k, "src_k"), _pool_ptr(src_v, "src_v"),
                                  _pool_ptr(dst_k, "dst_k"), _pool_ptr(dst_v, "dst_v"),
                                  _ptr(src_to_dst), src_to_dst.numel(), num_src, num_dst,
                                  block_bytes, _ptr(workspace), workspace.numel(),
                                  _stream(stream, src_to_dst))
    _check(st, "paged_kv_copy_blocks")


class OutOfBlocksError(PagedAttnError):
    """The block manager has no free physical block for the request."""


class BlockManager:
    """Host block manager of the paged KV cache (native, in the library):
    allocation with reference counts from a sorted free list, per-request
    block tables, growth one token at a time, prefix sharing (fork) and
    copy-on-write.  Produces the block_tables / context_lens the kernels read.
    """

    def __init__(self, num_blocks: int, block_size: int):
        self._lib = load_library()
        h = ctypes.c_void_p()
        _check(self._lib.pa_bm_create(int(num_blocks), int(block_size), ctypes.byref(h)),
               "pa_bm_create")
        self._h = h
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.pa_bm_destroy(h)
            self._h = None

    def _st(self, st: int, what: str) -> None:
        if st == -8:
            raise OutOfBlocksError(st, what)
        _check(st, what)

    def register(self, request_id: int, prompt_len: int) -> None:
        self._st(self._lib.pa_bm_register(self._h, int(request_id), int(prompt_len)), "register")

    def append_token(self, request_id: int):
        """None, or the (old, new) block pair of a copy-on-write."""
        a, b = _I32(), _I32()
        self._st(self._lib.pa_bm_append_token(self._h, int(request_id), ctypes.byref(a),
                                              ctypes.byref(b)), "append_token")
        return None if a.value < 0 else (a.value, b.value)

    def append_tokens(self, request_ids):
        """One more token for each listed request, in order (one decode step),
        all or nothing.  Returns (cow_src, cow_dst) int32 arrays with the
        copy-on-write pair of each request, -1 where none."""
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(request_ids, dtype=np.int64))
        src = np.empty(ids.size, dtype=np.int32)
        dst = np.empty(ids.size, dtype=np.int32)
        self._st(self._lib.pa_bm_append_tokens(self._h, ids.ctypes.data_as(ctypes.c_void_p),
                                               int(ids.size), src.ctypes.data_as(ctypes.c_void_p),
                                               dst.ctypes.data_as(ctypes.c_void_p)),
                 "append_tokens")
        return src, dst

    def fork(self, parent_id: int, child_id: int) -> None:
        self._st(self._lib.pa_bm_fork(self._h, int(parent_id), int(child_id)), "fork")

    def finish(self, request_id: int) -> None:
        self._st(self._lib.pa_bm_finish(self._h, int(request_id)), "finish")

    def free_count(self) -> int:
        return int(self._lib.pa_bm_free_count(self._h))

    def table(self, request_id: int) -> list:
        n, t = _I32(), _I64()
        # sizing call: PA_ERR_SHAPE (-3) only says the empty buffer is too small
        st = self._lib.pa_bm_block_table(self._h, int(request_id), None, 0, ctypes.byref(n),
                                         ctypes.byref(t))
        if st not in (0, -3):
            self._st(st, "table")
        buf = (_I32 * max(n.value, 1))()
        self._st(self._lib.pa_bm_block_table(self._h, int(request_id), buf, n.value,
                                              ctypes.byref(n), ctypes.byref(t)), "table")
        return list(buf[:n.value])

    def tokens(self, request_id: int) -> int:
        n, t = _I32(), _I64()
        st = self._lib.pa_bm_block_table(self._h, int(request_id), None, 0, ctypes.byref(n),
                                         ctypes.byref(t))
        if st not in (0, -3):
            self._st(st, "tokens")
        return int(t.value)

    def free_list(self) -> list:
        buf = (_I32 * self.num_blocks)()
        n = _I32()
        self._st(self._lib.pa_bm_free_list(self._h, buf, self.num_blocks, ctypes.byref(n)),
                 "free_list")
        return list(buf[:n.value])

    def ref_count(self, block: int) -> int:
        c = _I32()
        self._st(self._lib.pa_bm_ref_count(self._h, int(block), ctypes.byref(c)), "ref_count")
        return int(c.value)

    def batch_tables(self, request_ids, max_blocks_per_seq: int, out=None):
        """(block_tables int32 [n, max_blocks_per_seq] with -1 padding,
        context_lens int32 [n]) for the kernels, as CPU tensors; ``out`` may
        pass a (tables, lens) pair of contiguous CPU int32 tensors to reuse."""
        ids = torch.as_tensor(list(request_ids), dtype=torch.int64)
        n = ids.numel()
        if out is None:
            tables = torch.empty((n, int(max_blocks_per_seq)), dtype=torch.int32)
            lens = torch.empty(n, dtype=torch.int32)
        else:
            tables, lens = out
            if (tables.dtype != torch.int32 or lens.dtype != torch.int32 or tables.is_cuda
                    or lens.is_cuda or not tables.is_contiguous() or not lens.is_contiguous()
                    or tuple(tables.shape) != (n, int(max_blocks_per_seq))
                    or tuple(lens.shape) != (n,)):
                raise ValueError("out must be contiguous CPU int32 tensors of shapes "
                                 "[n, max_blocks_per_seq] and [n]")
        self._st(self._lib.pa_bm_fill_batch(self._h, ctypes.c_void_p(ids.data_ptr()), n,
                                            int(max_blocks_per_seq),
                                            ctypes.c_void_p(tables.data_ptr()),
                                            ctypes.c_void_p(lens.data_ptr())), "batch_tables")
        return tables, lens

