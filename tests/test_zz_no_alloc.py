"""paged_attn_decode_noalloc, the decode entry point that allocates nothing,
against paged_attn_decode on the same inputs.  Both run the same kernels, the
first with the library's static scratch array instead of a caller workspace,
so their outputs must agree bit for bit; the calls come in a row, the second
with a smaller input, so the second reuses the array the first left behind."""

import numpy as np
import pytest
import torch

import paged_kv_cache_248_amd as pa
import workloads as wl
from oracle import decode_ref
from tests._util import assert_close, compact_pool, host, log

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _inputs(dtype, Hq, Hkv, seed):
    rng = np.random.default_rng(seed)
    big = wl.make_decode(rng.integers(512, 4097, size=24), Hq, Hkv, 128, 16, dtype, seed=seed,
                         device=DEV, poison=True)
    small = wl.make_decode(np.concatenate([[1, 16, 513], rng.integers(2, 1500, size=2)]), Hq, Hkv,
                           128, 16, dtype, seed=seed + 1, device=DEV, poison=True)
    return big, small


def _args(case):
    kv = case.kv
    return (case.query, kv.k_cache, kv.v_cache, kv.block_tables, kv.context_lens, case.scale,
            kv.max_context_len)


@pytest.mark.parametrize("dtype,Hq,Hkv,part", [
    ("f16", 32, 32, 512),       # vector-ALU kernel, split into partitions + merge
    ("bf16", 32, 8, 512),       # matrix-core GQA kernel, split + merge
    ("bf16", 32, 8, 0),         # library default partition (4096): mostly one partition
    ("f32", 8, 4, 256),
])
def test_noalloc_matches_workspace_decode_on_consecutive_calls(dtype, Hq, Hkv, part):
    big, small = _inputs(dtype, Hq, Hkv, seed=5100 + Hq + Hkv + part)
    want = []
    for case in (big, small):
        out = torch.full_like(case.query, float("nan"))
        pa.paged_attn_decode(out, *_args(case), partition_size=part)
        want.append(out)
    got = [torch.full_like(c.query, float("nan")) for c in (big, small)]
    # two calls in a row on the same stream: the second (smaller) input
    # reuses the scratch array the first one wrote
    pa.paged_attn_decode_noalloc(got[0], *_args(big), partition_size=part)
    pa.paged_attn_decode_noalloc(got[1], *_args(small), partition_size=part)
    torch.cuda.synchronize()
    for name, w, g in zip(("first", "second"), want, got):
        assert torch.equal(g, w), f"{name} call differs from paged_attn_decode"
    # and both entry points agree with the oracle on the smaller input
    k, v, tables, cl = compact_pool(small.kv, list(range(small.query.shape[0])))
    ref = decode_ref(host(small.query), k, v, tables, cl, small.scale)
    e = assert_close(host(got[1]), ref, dtype, "noalloc second call")
    log(f"noalloc {dtype} Hq={Hq} Hkv={Hkv} part={part}: bit-identical to the workspace path, "
        f"oracle max rel err {e:.3e}")


def test_noalloc_second_call_after_a_split_reuses_scratch_cleanly():
    """A split call (many partitions: the work list and partials fill the
    array), then a call whose work list is shorter and whose partials sit at
    other offsets, then the first input again: all three bit-identical to the
    workspace path."""
    a = wl.make_decode([32768, 20000, 9000], 32, 32, 128, 32, "f16", seed=5200, device=DEV)
    b = wl.make_decode([700, 3000], 32, 32, 128, 32, "f16", seed=5201, device=DEV)
    ref_a = torch.empty_like(a.query)
    ref_b = torch.empty_like(b.query)
    pa.paged_attn_decode(ref_a, *_args(a), partition_size=512)
    pa.paged_attn_decode(ref_b, *_args(b), partition_size=512)
    outs = [torch.full_like(a.query, float("nan")), torch.full_like(b.query, float("nan")),
            torch.full_like(a.query, float("nan"))]
    pa.paged_attn_decode_noalloc(outs[0], *_args(a), partition_size=512)
    pa.paged_attn_decode_noalloc(outs[1], *_args(b), partition_size=512)
    pa.paged_attn_decode_noalloc(outs[2], *_args(a), partition_size=512)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], ref_a)
    assert torch.equal(outs[1], ref_b)
    assert torch.equal(outs[2], ref_a)


def test_noalloc_rejects_a_call_beyond_the_scratch_size():
    """128 sequences x 64 heads x 64 partitions of head_dim 128 need 256 MiB
    of partials: refused on the host before any launch."""
    case = wl.make_decode([8], 64, 64, 128, 16, "f16", seed=5300, device=DEV)
    kv = case.kv
    need = pa.paged_attn_decode_workspace_size(128, 64, 64, 128, 32768, 512)
    assert need > pa.DECODE_NOALLOC_SCRATCH_BYTES
    q = torch.zeros(128, 64, 128, dtype=torch.float16, device=DEV)
    out = torch.full_like(q, 3.0)
    bt = torch.zeros(128, 2048, dtype=torch.int32, device=DEV)
    cl = torch.ones(128, dtype=torch.int32, device=DEV)
    with pytest.raises(pa.PagedAttnError) as ei:
        pa.paged_attn_decode_noalloc(out, q, kv.k_cache, kv.v_cache, bt, cl, 0.1, 32768,
                                     partition_size=512)
    assert ei.value.status == -5
    torch.cuda.synchronize()
    assert (out == 3.0).all()
