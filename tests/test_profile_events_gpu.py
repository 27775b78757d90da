"""The measurement hook: with events set (pa_set_profile_events), every main
kernel is launched with the runtime recording the two events as part of its
dispatch.  Outputs must be bit-identical to the same calls without events,
and each event pair must bracket a positive span no longer than the call's
wall-clock time."""

import time

import pytest
import torch

import paged_kv_cache_248_amd as pa
import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda"


def bits(t: torch.Tensor) -> torch.Tensor:
    return t.view({4: torch.int32, 2: torch.int16}[t.element_size()])


def timed(fn):
    """fn() with events set; returns (event span ms, wall-clock ms)."""
    lib = pa.load_library()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()                             # materialise the hipEvent_t handles
    e.record()
    torch.cuda.synchronize()
    assert lib.pa_set_profile_events(s.cuda_event, e.cuda_event) == 0
    try:
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3
    finally:
        assert lib.pa_set_profile_events(None, None) == 0
    return s.elapsed_time(e), wall


def check_span(span, wall, what):
    assert 0.0 < span <= wall, f"{what}: event span {span} ms, call {wall} ms"


def test_decode_with_events_matches_plain_calls():
    for dtype, Hq, Hkv in (("f16", 8, 8), ("bf16", 32, 8)):
        case = wl.make_decode([700, 33, 4100], Hq, Hkv, 128, 16, dtype, seed=61, device=DEV)
        kv = case.kv
        outs = [torch.empty_like(case.query) for _ in range(2)]

        def call(o):
            pa.paged_attn_decode(o, case.query, kv.k_cache, kv.v_cache, kv.block_tables,
                                 kv.context_lens, case.scale, kv.max_context_len,
                                 partition_size=512)

        call(outs[0])
        span, wall = timed(lambda: call(outs[1]))
        check_span(span, wall, f"decode {dtype}")
        assert torch.equal(bits(outs[0]), bits(outs[1])), f"decode {dtype}"


@pytest.mark.parametrize("fn_name", ["paged_attn_prefill", "paged_attn_prefill_halftile"])
def test_prefill_with_events_matches_plain_calls(fn_name):
    case = wl.make_prefill([100, 0], [70, 130], 8, 2, 128, 16, "bf16", seed=62, device=DEV)
    kv = case.kv
    fn = getattr(pa, fn_name)
    outs = [torch.empty_like(case.query) for _ in range(2)]

    def call(o):
        fn(o, case.query, kv.k_cache, kv.v_cache, kv.block_tables, kv.context_lens,
           case.query_start_loc, case.scale, case.max_query_len, kv.max_context_len)

    call(outs[0])
    span, wall = timed(lambda: call(outs[1]))
    check_span(span, wall, fn_name)
    assert torch.equal(bits(outs[0]), bits(outs[1]))


def test_copy_and_append_with_events_match_plain_calls():
    case = wl.make_copy(40, 30, (2, 16, 128), "bf16", seed=63, device=DEV)
    dsts = [(case.dst_k.clone(), case.dst_v.clone()) for _ in range(2)]
    pa.paged_kv_copy_blocks(case.src_k, case.src_v, *dsts[0], case.src_to_dst)
    span, wall = timed(lambda: pa.paged_kv_copy_blocks(case.src_k, case.src_v, *dsts[1],
                                                       case.src_to_dst))
    check_span(span, wall, "copy")
    assert torch.equal(bits(dsts[0][0]), bits(dsts[1][0]))
    assert torch.equal(bits(dsts[0][1]), bits(dsts[1][1]))

    ap = wl.make_append([10, 0, 40], [7, 20, 3], 2, 128, 16, "bf16", seed=64, device=DEV)
    pools = [(ap.kv.k_cache.clone(), ap.kv.v_cache.clone()) for _ in range(2)]

    def append(kc, vc):
        pa.paged_kv_append(kc, vc, ap.key, ap.value, ap.kv.block_tables, ap.kv.context_lens,
                           ap.query_start_loc)

    append(*pools[0])
    span, wall = timed(lambda: append(*pools[1]))
    check_span(span, wall, "append")
    assert torch.equal(bits(pools[0][0]), bits(pools[1][0]))
    assert torch.equal(bits(pools[0][1]), bits(pools[1][1]))
