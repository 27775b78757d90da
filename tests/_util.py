"""Helpers shared by the GPU parity tests (not a test module)."""

from __future__ import annotations

import numpy as np
import torch

# Bars: max |gpu - ref| / max(1, |ref|) per element (output scale of 1).
TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 8e-3}


def host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy holding exactly the stored values."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.float().numpy()
    return t.numpy()


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    gpu = np.asarray(gpu, dtype=np.float64)
    ok = ~np.isnan(ref)
    if not ok.any():
        return 0.0
    d = np.abs(gpu[ok] - ref[ok]) / np.maximum(1.0, np.abs(ref[ok]))
    return float(np.nanmax(np.where(np.isnan(d), np.inf, d)))


def assert_close(gpu: np.ndarray, ref: np.ndarray, dtype: str, what: str = "") -> float:
    e = rel_err(gpu, ref)
    assert np.isfinite(gpu[~np.isnan(ref)]).all(), f"{what}: non-finite output"
    assert e <= TOL[dtype], f"{what}: max rel err {e:.3e} > {TOL[dtype]:.1e}"
    return e


def compact_pool(kv, seqs):
    """The blocks the given sequences use, copied to host, with tables
    renumbered into that compact pool (attention does not depend on where a
    block lives, so the oracle may run on the compact copy)."""
    bt = kv.block_tables[seqs].cpu().numpy()
    cl = kv.context_lens[seqs].cpu().numpy()
    bs = kv.block_size
    ids, rows = [], []
    for r, n in zip(bt, cl):
        nb = (int(n) + bs - 1) // bs
        rows.append(np.arange(len(ids), len(ids) + nb))
        ids.extend(r[:nb].tolist())
    idx = torch.as_tensor(np.asarray(ids, dtype=np.int64), device=kv.k_cache.device)
    k = host(kv.k_cache.index_select(0, idx))
    v = host(kv.v_cache.index_select(0, idx))
    width = max(1, max(len(r) for r in rows))
    tables = np.zeros((len(seqs), width), dtype=np.int32)
    for i, r in enumerate(rows):
        tables[i, :len(r)] = r
    return k, v, tables, cl


def log(msg: str) -> None:
    print(msg, flush=True)
