"""C-ABI checks that need no GPU: the library loads, exports every function
include/paged_attn.h declares, and returns each error status for bad host
arguments before anything is launched."""

import ctypes
import os
import re

import pytest

from conftest import ROOT, gpu_available

import paged_kv_cache_248_amd as pa

HEADER = os.path.join(ROOT, "include", "paged_attn.h")

PA_OK, PA_ERR_NULL, PA_ERR_DTYPE, PA_ERR_SHAPE = 0, -1, -2, -3
PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_LAUNCH, PA_ERR_DEVICE = -4, -5, -6, -7
PA_ERR_NO_BLOCKS, PA_ERR_REQUEST = -8, -9

# Fake device addresses: only ever handed to calls that must fail on host
# validation, before any HIP call could touch them.
P = 0x10000
P2 = 0x20000
P3 = 0x30000


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pa.library_path()):
        pytest.fail("libpagedattn.so is not built (run __graft_entry__.build())")
    return pa.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+char\s*\*|size_t|pa_status_t)\s*(\w+)\s*\(", text, flags=re.M)


def test_header_declares_the_operations():
    names = declared_functions()
    for n in ("paged_attn_decode", "paged_attn_prefill", "paged_kv_copy_blocks",
              "paged_kv_append"):
        assert n in names


def test_library_exports_every_declared_function(lib):
    names = declared_functions()
    assert len(names) >= 6
    raw = ctypes.CDLL(pa.library_path())
    for n in names:
        assert hasattr(raw, n), f"{n} declared but not exported"


def test_status_strings(lib):
    for s in (PA_OK, PA_ERR_NULL, PA_ERR_DTYPE, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED,
              PA_ERR_WORKSPACE, PA_ERR_LAUNCH, PA_ERR_DEVICE, PA_ERR_NO_BLOCKS, PA_ERR_REQUEST):
        assert lib.pa_status_string(s)
        assert b"UNKNOWN" not in lib.pa_status_string(s)
    assert lib.pa_status_string(PA_OK) == b"PA_OK"
    assert b"UNKNOWN" in lib.pa_status_string(12345)


def _decode(lib, **kw):
    a = dict(out=P, query=P, k=P, v=P, bt=P, cl=P, B=2, Hq=8, Hkv=2, D=128, bs=16, nblk=64,
             mbps=8, maxctx=100, scale=0.125, dtype=1, part=0, ws=P3, wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.paged_attn_decode(a["out"], a["query"], a["k"], a["v"], a["bt"], a["cl"], a["B"],
                                 a["Hq"], a["Hkv"], a["D"], a["bs"], a["nblk"], a["mbps"],
                                 a["maxctx"], a["scale"], a["dtype"], a["part"], a["ws"],
                                 a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(dtype=7), PA_ERR_DTYPE),
    (dict(Hq=6, Hkv=4), PA_ERR_SHAPE),
    (dict(Hkv=0), PA_ERR_SHAPE),
    (dict(B=-1), PA_ERR_SHAPE),
    (dict(nblk=0), PA_ERR_SHAPE),
    (dict(D=96), PA_ERR_UNSUPPORTED),
    (dict(bs=12), PA_ERR_UNSUPPORTED),
    (dict(bs=4), PA_ERR_UNSUPPORTED),
    (dict(part=100), PA_ERR_UNSUPPORTED),
    (dict(part=-2), PA_ERR_UNSUPPORTED),
    (dict(part=64, maxctx=64 * 2049, mbps=10000), PA_ERR_UNSUPPORTED),   # too many partitions
    (dict(query=None), PA_ERR_NULL),
    (dict(bt=None), PA_ERR_NULL),
    (dict(out=P + 2), PA_ERR_UNSUPPORTED),
    (dict(ws=None), PA_ERR_WORKSPACE),
    (dict(wsb=16), PA_ERR_WORKSPACE),
    (dict(ws=P3 + 1), PA_ERR_WORKSPACE),   # work list and counter need alignment
    (dict(ws=P3 + 8), PA_ERR_WORKSPACE),
    (dict(B=0), PA_OK),            # nothing to do, nothing launched
    (dict(maxctx=0), PA_OK),
])
def test_decode_validation(lib, kw, want):
    assert _decode(lib, **kw) == want


def test_decode_reports_missing_device(lib):
    if gpu_available():
        pytest.skip("a GPU is present: valid arguments would launch")
    assert _decode(lib) == PA_ERR_DEVICE


def test_decode_workspace_size(lib):
    small = lib.paged_attn_decode_workspace_size(4, 8, 2, 128, 512, 512)
    split = lib.paged_attn_decode_workspace_size(4, 8, 2, 128, 4096, 512)
    assert 0 < small < split
    # 8 partitions of partials: O (D floats) plus M and L per (seq, head, partition)
    assert split - small >= 4 * 8 * 8 * (128 + 2) * 4 - 4096
    assert lib.paged_attn_decode_workspace_size(4, 8, 2, 128, 4096, 100) == 0   # bad partition
    assert lib.paged_attn_decode_workspace_size(4, 8, 2, 128, 4096, -1) == small


def test_decode_default_partition_depends_on_group(lib):
    """partition_size 0 picks 4096 tokens for 4+ heads per kv head, else 512."""
    import paged_kv_cache_248_amd as pa
    ws = lib.paged_attn_decode_workspace_size
    # group 4 (8 heads, 2 kv heads)
    assert ws(4, 8, 2, 128, 16384, 0) == ws(4, 8, 2, 128, 16384, 4096) != ws(4, 8, 2, 128, 16384, 2048)
    # group 2 and MHA
    assert ws(4, 8, 4, 128, 4096, 0) == ws(4, 8, 4, 128, 4096, 512) != ws(4, 8, 4, 128, 4096, 1024)
    assert ws(4, 8, 8, 128, 4096, 0) == ws(4, 8, 8, 128, 4096, 512)
    assert pa.default_partition(8, 2) == 4096 and pa.default_partition(8, 4) == 512
    assert pa.default_partition(32, 32) == pa.DEFAULT_PARTITION == 512


def _prefill(lib, entry="paged_attn_prefill", **kw):
    a = dict(out=P, query=P, k=P, v=P, bt=P, cl=P, qsl=P2, B=2, T=10, maxq=8, maxctx=40, Hq=8,
             Hkv=2, D=128, bs=16, nblk=64, mbps=8, scale=0.125, dtype=2, stream=None)
    a.update(kw)
    return getattr(lib, entry)(a["out"], a["query"], a["k"], a["v"], a["bt"], a["cl"], a["qsl"],
                               a["B"], a["T"], a["maxq"], a["maxctx"], a["Hq"], a["Hkv"], a["D"],
                               a["bs"], a["nblk"], a["mbps"], a["scale"], a["dtype"], a["stream"])


PREFILL_ENTRIES = ["paged_attn_prefill", "paged_attn_prefill_halftile"]


@pytest.mark.parametrize("kw,want", [
    (dict(dtype=0), PA_ERR_DTYPE),          # fp32 prefill is not provided
    (dict(dtype=9), PA_ERR_DTYPE),
    (dict(maxq=50), PA_ERR_SHAPE),          # more new tokens than keys
    (dict(Hq=8, Hkv=3), PA_ERR_SHAPE),
    (dict(D=256), PA_ERR_UNSUPPORTED),
    (dict(bs=48), PA_ERR_UNSUPPORTED),
    (dict(qsl=None), PA_ERR_NULL),
    (dict(v=None), PA_ERR_NULL),
    (dict(k=P + 8), PA_ERR_UNSUPPORTED),
    (dict(scale=0.0), PA_ERR_UNSUPPORTED),
    (dict(scale=-0.125), PA_ERR_UNSUPPORTED),
    (dict(scale=float("nan")), PA_ERR_UNSUPPORTED),
    (dict(T=0), PA_OK),
    (dict(B=0), PA_OK),
])
@pytest.mark.parametrize("entry", PREFILL_ENTRIES)
def test_prefill_validation(lib, kw, want, entry):
    assert _prefill(lib, entry, **kw) == want


@pytest.mark.parametrize("entry", PREFILL_ENTRIES)
def test_prefill_reports_missing_device(lib, entry):
    if gpu_available():
        pytest.skip("a GPU is present: valid arguments would launch")
    assert _prefill(lib, entry) == PA_ERR_DEVICE


def _copy(lib, **kw):
    a = dict(sk=P, sv=P2, dk=P3, dv=P3 + 0x1000, m=P, nm=4, ns=8, nd=4, bb=4096, ws=P2,
             wsb=1 << 20, stream=None)
    a.update(kw)
    return lib.paged_kv_copy_blocks(a["sk"], a["sv"], a["dk"], a["dv"], a["m"], a["nm"], a["ns"],
                                    a["nd"], a["bb"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(bb=0), PA_ERR_SHAPE),
    (dict(nm=-1), PA_ERR_SHAPE),
    (dict(nm=1 << 31), PA_ERR_SHAPE),
    (dict(bb=24), PA_ERR_UNSUPPORTED),
    # one work-group per (pool, destination block, 4 KiB slice) must fit the grid
    (dict(bb=16384, nd=1 << 28), PA_ERR_SHAPE),
    (dict(bb=4096, nd=1 << 30), PA_ERR_SHAPE),
    (dict(sk=None), PA_ERR_NULL),
    (dict(m=None), PA_ERR_NULL),
    (dict(sv=None), PA_ERR_NULL),           # V pair half given
    (dict(dk=P3 + 4), PA_ERR_UNSUPPORTED),
    (dict(ws=None), PA_ERR_WORKSPACE),
    (dict(wsb=8), PA_ERR_WORKSPACE),
    (dict(ws=P2 + 1), PA_ERR_WORKSPACE),    # atomics on an unaligned buffer
    (dict(ws=P2 + 4), PA_ERR_WORKSPACE),
    (dict(nm=0), PA_OK),
    (dict(nd=0), PA_OK),
    (dict(ns=0), PA_OK),
])
def test_copy_validation(lib, kw, want):
    assert _copy(lib, **kw) == want


def test_copy_reports_missing_device(lib):
    if gpu_available():
        pytest.skip("a GPU is present: valid arguments would launch")
    assert _copy(lib) == PA_ERR_DEVICE
    assert _copy(lib, sv=None, dv=None) == PA_ERR_DEVICE


def test_copy_workspace_size(lib):
    assert lib.paged_kv_copy_blocks_workspace_size(4096) == 4096 * 4
    assert lib.paged_kv_copy_blocks_workspace_size(-1) == 0


def test_python_binding_refuses_host_tensors():
    import torch
    q = torch.zeros(2, 4, 64)
    with pytest.raises(ValueError):
        pa.paged_attn_decode(q, q, torch.zeros(4, 4, 16, 64), torch.zeros(4, 4, 16, 64),
                             torch.zeros(2, 4, dtype=torch.int32), torch.ones(2, dtype=torch.int32),
                             0.125)


def test_profile_events_must_be_paired(lib):
    assert lib.pa_set_profile_events(P, None) == PA_ERR_NULL
    assert lib.pa_set_profile_events(None, P) == PA_ERR_NULL
    assert lib.pa_set_profile_events(None, None) == PA_OK


def _append(lib, **kw):
    a = dict(k=P, v=P2, key=P3, value=P3 + 0x1000, bt=P, cl=P, qsl=P2, B=2, T=10, Hkv=2, D=128,
             bs=16, nblk=64, mbps=8, dtype=2, stream=None)
    a.update(kw)
    return lib.paged_kv_append(a["k"], a["v"], a["key"], a["value"], a["bt"], a["cl"], a["qsl"],
                               a["B"], a["T"], a["Hkv"], a["D"], a["bs"], a["nblk"], a["mbps"],
                               a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(dtype=5), PA_ERR_DTYPE),
    (dict(Hkv=0), PA_ERR_SHAPE),
    (dict(B=-1), PA_ERR_SHAPE),
    (dict(T=-1), PA_ERR_SHAPE),
    (dict(nblk=0), PA_ERR_SHAPE),
    (dict(mbps=0), PA_ERR_SHAPE),
    (dict(D=4), PA_ERR_UNSUPPORTED),                 # 8-byte rows: not a multiple of 16
    (dict(bs=12), PA_ERR_UNSUPPORTED),
    (dict(bs=512), PA_ERR_UNSUPPORTED),
    (dict(k=None), PA_ERR_NULL),
    (dict(key=None), PA_ERR_NULL),
    (dict(qsl=None), PA_ERR_NULL),
    (dict(v=None), PA_ERR_NULL),                     # V pool without V rows
    (dict(key=P3 + 8), PA_ERR_UNSUPPORTED),
    (dict(B=0), PA_OK),
    (dict(T=0), PA_OK),
])
def test_append_validation(lib, kw, want):
    assert _append(lib, **kw) == want


def test_append_reports_missing_device(lib):
    if gpu_available():
        pytest.skip("a GPU is present: valid arguments would launch")
    assert _append(lib) == PA_ERR_DEVICE
    assert _append(lib, v=None, value=None) == PA_ERR_DEVICE     # K only is valid


def test_host_device_pointer_rejects_null_and_plain_memory(lib):
    out = ctypes.c_void_p(123)
    assert lib.pa_host_device_pointer(None, ctypes.byref(out)) == PA_ERR_NULL
    assert lib.pa_host_device_pointer(ctypes.c_void_p(P), None) == PA_ERR_NULL
    buf = ctypes.create_string_buffer(4096)                 # ordinary, unpinned host memory
    assert lib.pa_host_device_pointer(ctypes.cast(buf, ctypes.c_void_p), ctypes.byref(out)) == \
        PA_ERR_UNSUPPORTED
    assert not out.value



def _i32(*vals):
    return (ctypes.c_int32 * len(vals))(*vals)


def _unfused(lib, **kw):
    a = dict(out=P, query=P, k=P, v=P, bt=P, cl=_i32(30, 40), qsl=_i32(0, 4, 10), B=2, T=10, Hq=8,
             Hkv=2, D=128, bs=16, nblk=64, mbps=8, scale=0.125, dtype=2, ws=P2, wsb=1 << 30,
             stream=None)
    a.update(kw)
    return lib.paged_attn_prefill_unfused(
        a["out"], a["query"], a["k"], a["v"], a["bt"],
        ctypes.cast(a["cl"], ctypes.c_void_p) if a["cl"] is not None else None,
        ctypes.cast(a["qsl"], ctypes.c_void_p) if a["qsl"] is not None else None,
        a["B"], a["T"], a["Hq"], a["Hkv"], a["D"], a["bs"], a["nblk"], a["mbps"], a["scale"],
        a["dtype"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(dtype=0), PA_ERR_DTYPE),
    (dict(Hq=8, Hkv=3), PA_ERR_SHAPE),
    (dict(D=96), PA_ERR_UNSUPPORTED),
    (dict(bs=48), PA_ERR_UNSUPPORTED),
    (dict(scale=0.0), PA_ERR_UNSUPPORTED),
    (dict(cl=None), PA_ERR_NULL),
    (dict(qsl=None), PA_ERR_NULL),
    (dict(qsl=_i32(1, 4, 10)), PA_ERR_SHAPE),          # does not start at 0
    (dict(qsl=_i32(0, 4, 9)), PA_ERR_SHAPE),           # does not end at total_query_tokens
    (dict(qsl=_i32(0, 6, 4), T=4), PA_ERR_SHAPE),      # decreasing
    (dict(cl=_i32(3, 40)), PA_ERR_SHAPE),              # more new tokens than keys
    (dict(cl=_i32(30, 129)), PA_ERR_SHAPE),            # more keys than the table maps
    (dict(cl=_i32(30, 40000), mbps=4096), PA_ERR_UNSUPPORTED),   # beyond the softmax row limit
    (dict(v=None), PA_ERR_NULL),
    (dict(bt=None), PA_ERR_NULL),
    (dict(k=P + 8), PA_ERR_UNSUPPORTED),
    (dict(ws=None), PA_ERR_WORKSPACE),
    (dict(wsb=1 << 20), PA_ERR_WORKSPACE),
    (dict(T=0, qsl=_i32(0, 0, 0)), PA_OK),
    (dict(B=0), PA_OK),
])
def test_unfused_validation(lib, kw, want):
    assert _unfused(lib, **kw) == want


def test_unfused_reports_missing_device(lib):
    if gpu_available():
        pytest.skip("a GPU is present: valid arguments would launch")
    assert _unfused(lib) == PA_ERR_DEVICE


def test_unfused_workspace_size(lib):
    ws = lib.paged_attn_prefill_unfused_workspace_size
    # S (fp32) and P (bf16) of 32 heads x 2048 rows x 8192 keys dominate
    s_p = 32 * 2048 * 8192 * (4 + 2)
    assert s_p < ws(2048, 8192, 32, 8, 128, 2) < s_p + (80 << 20) + 4 * 2048 * 32 * 128 * 2 + \
        2 * 8 * 8192 * 128 * 2
    # S/P rows are padded to 8 keys: 8190 and 8192 keys differ only in the gathered K/V
    assert 0 < ws(2048, 8192, 32, 8, 128, 2) - ws(2048, 8190, 32, 8, 128, 2) <= 2 * 8 * 2 * 128 * 2
    assert ws(16, 64, 8, 2, 64, 0) == 0            # fp32 is not provided
    assert ws(-1, 64, 8, 2, 64, 2) == 0


def test_stream_read_validation(lib):
    assert lib.pa_stream_read(P, -16, P2, 8, None) == PA_ERR_SHAPE
    assert lib.pa_stream_read(P, 32, P2, 0, None) == PA_ERR_SHAPE            # no sink entries
    assert lib.pa_stream_read(P, 24, P2, 8, None) == PA_ERR_UNSUPPORTED     # not a multiple of 16
    assert lib.pa_stream_read(P + 8, 32, P2, 8, None) == PA_ERR_UNSUPPORTED  # misaligned
    assert lib.pa_stream_read(None, 32, P2, 8, None) == PA_ERR_NULL
    assert lib.pa_stream_read(P, 32, None, 8, None) == PA_ERR_NULL
    assert lib.pa_stream_read(P, 0, P2, 8, None) == PA_OK
    if not gpu_available():
        assert lib.pa_stream_read(P, 32, P2, 8, None) == PA_ERR_DEVICE


def _decode_noalloc(lib, **kw):
    a = dict(out=P, query=P, k=P, v=P, bt=P, cl=P, B=2, Hq=8, Hkv=2, D=128, bs=16, nblk=64,
             mbps=8, maxctx=100, scale=0.125, dtype=1, part=0, stream=None)
    a.update(kw)
    return lib.paged_attn_decode_noalloc(a["out"], a["query"], a["k"], a["v"], a["bt"], a["cl"],
                                         a["B"], a["Hq"], a["Hkv"], a["D"], a["bs"], a["nblk"],
                                         a["mbps"], a["maxctx"], a["scale"], a["dtype"],
                                         a["part"], a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(dtype=7), PA_ERR_DTYPE),
    (dict(Hq=6, Hkv=4), PA_ERR_SHAPE),
    (dict(D=96), PA_ERR_UNSUPPORTED),
    (dict(query=None), PA_ERR_NULL),
    (dict(out=P + 2), PA_ERR_UNSUPPORTED),
    # 128 seqs x 64 heads x 64 partitions x 128 floats of partials: past the
    # library's scratch array, refused before any launch
    (dict(B=128, Hq=64, Hkv=64, mbps=2048, maxctx=32768, part=512), PA_ERR_WORKSPACE),
    (dict(B=0), PA_OK),
])
def test_decode_noalloc_validation(lib, kw, want):
    assert _decode_noalloc(lib, **kw) == want


def test_decode_noalloc_limit_matches_the_workspace_query(lib):
    """The largest call the scratch array takes is the one whose workspace
    query fits PA_DECODE_NOALLOC_SCRATCH_BYTES."""
    limit = pa.DECODE_NOALLOC_SCRATCH_BYTES
    assert "#define PA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in open(HEADER).read()
    fits = lib.paged_attn_decode_workspace_size(128, 32, 8, 128, 32768, 2048)
    assert 0 < fits <= limit
    too_big = lib.paged_attn_decode_workspace_size(128, 64, 64, 128, 32768, 512)
    assert too_big > limit
    if not gpu_available():
        # within the limit, a valid call reaches the device check
        assert _decode_noalloc(lib, B=128, Hq=32, Hkv=8, mbps=2048, maxctx=32768) == PA_ERR_DEVICE


def test_stream_copy_validation(lib):
    assert lib.pa_stream_copy(P, P2 + 0x100000, -16, 0, None) == PA_ERR_SHAPE
    assert lib.pa_stream_copy(P, P2 + 0x100000, 24, 0, None) == PA_ERR_UNSUPPORTED    # not a multiple of 16
    assert lib.pa_stream_copy(P + 8, P2 + 0x100000, 32, 0, None) == PA_ERR_UNSUPPORTED  # misaligned
    assert lib.pa_stream_copy(None, P2, 32, 0, None) == PA_ERR_NULL
    assert lib.pa_stream_copy(P, P + 16, 64, 0, None) == PA_ERR_SHAPE                 # overlapping
    assert lib.pa_stream_copy(P, P2, 0, 0, None) == PA_OK
    if not gpu_available():
        assert lib.pa_stream_copy(P, P2 + 0x100000, 32, 0, None) == PA_ERR_DEVICE


def test_mfma_stream_validation(lib):
    f = lib.pa_mfma_stream
    ok = dict(operands=P, nbytes=8192, sink=P2, words=16, w=1, iters=1, dtype=2)   # bf16

    def call(**kw):
        a = {**ok, **kw}
        return f(a["operands"], a["nbytes"], a["sink"], a["words"], a["w"], a["iters"], a["dtype"],
                 None)

    assert call(dtype=0) == PA_ERR_DTYPE            # fp32 has no such MFMA here
    assert call(dtype=7) == PA_ERR_DTYPE
    assert call(nbytes=2048) == PA_ERR_SHAPE
    assert call(words=0) == PA_ERR_SHAPE
    assert call(w=0) == PA_ERR_SHAPE
    assert call(w=9) == PA_ERR_SHAPE
    assert call(iters=0) == PA_ERR_SHAPE
    assert call(nbytes=8200) == PA_ERR_UNSUPPORTED
    assert call(operands=None) == PA_ERR_NULL
    assert call(sink=None) == PA_ERR_NULL
    assert call(operands=P + 8) == PA_ERR_UNSUPPORTED
