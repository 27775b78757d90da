"""The matrix-core stream probe does the MFMAs it is credited with: with
operands in {-1, 0, 1} every partial sum is an integer below 2^24, so each
work-group's sum of accumulators is exact and must equal the closed form
below, computed here from the operand buffer alone.

For C = A B with A 32x16 and B 16x32, the sum of all entries of C is
sum_k (sum_i A[i,k]) (sum_j B[k,j]).  In the 32x32x16 operand layout lane l
holds row / column l mod 32 and k = 8 (l / 32) .. + 7 as one 16-byte
fragment, so column sums of A (row sums of B) are sums over the 32 lanes of
each half-wave, element by element."""

import numpy as np
import pytest
import torch

import paged_kv_cache_248_amd as pa

pytestmark = pytest.mark.gpu


def expected_sink(ops16: np.ndarray, n_wg: int, iters: int) -> np.ndarray:
    """ops16: the operand buffer as float64, grouped in 8-element fragments."""
    frags = ops16.reshape(-1, 8)
    n16 = frags.shape[0]
    out = np.zeros(n_wg)
    for wg in range(n_wg):
        for wave in range(4):
            g = wg * 256 + wave * 64 + np.arange(64)                 # global lanes of the wave
            a = [frags[(g * 16 + k) % n16] for k in range(8)]        # [64, 8] each
            b = [frags[(g * 16 + 8 + k) % n16] for k in range(8)]
            total = 0.0
            for u in range(32):
                A, B = a[u & 7], b[(u >> 2) & 7]
                # per half-wave h: colsum_A[h, e] = sum over lanes of that half
                ca = A.reshape(2, 32, 8).sum(axis=1)
                rb = B.reshape(2, 32, 8).sum(axis=1)
                total += float((ca * rb).sum())
            out[wg] += iters * total
    return out


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_mfma_stream_sums_exact(dtype):
    rng = np.random.default_rng(2490)
    vals = rng.integers(-1, 2, size=1 << 14).astype(np.float32)
    ops = torch.tensor(vals, dtype=dtype, device="cuda")
    n_wg, iters = 16, 3
    sink = torch.full((n_wg,), float("nan"), dtype=torch.float32, device="cuda")
    pa.pa_mfma_stream(ops, sink, 1, iters)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().astype(np.float64)
    want = expected_sink(vals.astype(np.float64), n_wg, iters)
    assert np.abs(want).max() > 0
    assert np.array_equal(got, want), (got[:4], want[:4])


def test_mfma_stream_grid_is_bounded_by_the_sink():
    """With fewer sink entries than CUs x work-groups per CU, only that many
    work-groups run: entries past them stay untouched."""
    ops = torch.ones(4096, dtype=torch.bfloat16, device="cuda")
    sink = torch.full((8,), -7.0, dtype=torch.float32, device="cuda")
    pa.pa_mfma_stream(ops, sink[:5], 2, 1)
    torch.cuda.synchronize()
    s = sink.cpu().numpy()
    # all-ones operands: every MFMA's entries are 16, 32 MFMAs x 1024 entries x 4 waves
    assert np.all(s[:5] == 16.0 * 1024 * 32 * 4)
    assert np.all(s[5:] == -7.0)
