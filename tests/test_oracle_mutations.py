"""Plants plausible mistakes in the oracle (CPU only) and checks that the pins
in test_oracle.py catch every one of them."""

import math

import numpy as np
import pytest

import oracle.paged_attn_oracle as O
import tests.test_oracle as pins


def _gather_slot_major(cache, table_row, n, kv_head):
    # wrong index: walks slots of the first block before moving on
    bs = cache.shape[2]
    j = np.arange(n)
    nb = max(1, (n + bs - 1) // bs)
    return cache[np.asarray(table_row)[j % nb], kv_head, j // nb, :]


def _gather_ignores_table(cache, table_row, n, kv_head):
    # wrong index: physical block taken as the logical block number
    bs = cache.shape[2]
    j = np.arange(n)
    return cache[j // bs, kv_head, j % bs, :]


def _attend_no_scale(q, K, V, scale, mask=None):
    return _orig_attend(q, K, V, 1.0, mask)


def _online_drop_carry(x, v, tiles):
    x, v = O.as_f64(x), O.as_f64(v)
    M, L, Ov = -math.inf, 0.0, np.zeros(v.shape[1])
    for a, b in tiles:
        Mn = max(M, float(x[a:b].max()))
        e = np.exp(x[a:b] - Mn)
        Ln = float(e.sum())                      # dropped L_old * exp(M_old - M_new)
        Ov = (L * math.exp(M - Mn) / max(Ln, 1e-300)) * Ov + (e @ v[a:b]) / Ln
        M, L = Mn, Ln
    return M, L, Ov


def _split_no_rescale(x, v, partition):
    x, v = O.as_f64(x), O.as_f64(v)
    Ls, Os = [], []
    for a in range(0, x.shape[0], partition):
        w = np.exp(x[a:a + partition] - x[a:a + partition].max())
        Ls.append(w.sum())
        Os.append((w @ v[a:a + partition]) / w.sum())
    Ls, Os = np.array(Ls), np.array(Os)
    return (Ls[:, None] * Os).sum(axis=0) / Ls.sum()


def _copy_last_wins(src, dst, m):
    out = np.array(dst, copy=True)
    m = np.asarray(m).reshape(-1)
    for i in range(m.size):
        if 0 <= m[i] < out.shape[0] and i < src.shape[0]:
            out[m[i]] = src[i]
    return out


_orig_attend = O.attend_two_pass


def _prefill_top_left(query, k_cache, v_cache, block_tables, context_lens, qsl, scale, rows=None, heads=None):
    # wrong alignment: new token t sees keys 0..t instead of 0..prefix+t
    q_b = np.diff(np.asarray(qsl))
    return _orig_prefill(query, k_cache, v_cache, block_tables, q_b, qsl, scale, rows, heads)


_orig_prefill = O.prefill_ref


def _decode_mod_group(query, k_cache, v_cache, block_tables, context_lens, scale, seqs=None, heads=None):
    # wrong GQA map h % Hkv
    query = np.asarray(query)
    B, Hq, D = query.shape
    Hkv = k_cache.shape[1]
    out = np.empty((B, Hq, D))
    for b in range(B):
        n = int(context_lens[b])
        for h in range(Hq):
            K = O.gather_sequence(k_cache, block_tables[b], n, h % Hkv)
            V = O.gather_sequence(v_cache, block_tables[b], n, h % Hkv)
            out[b, h] = O.attend_two_pass(query[b, h], K, V, scale)
    return out


_orig_append = O.append_kv_ref


def _append_off_by_one(cache, rows, block_tables, context_lens, qsl):
    # wrong position: token i of a sequence written one slot later
    return _orig_append(cache, rows, block_tables, np.asarray(context_lens) + 1, qsl)


def _append_ignores_table(cache, rows, block_tables, context_lens, qsl):
    # wrong index: logical block number used as the physical block
    nb, _, bs, _ = np.asarray(cache).shape
    ident = np.tile(np.arange(np.asarray(block_tables).shape[1], dtype=np.int64),
                    (len(context_lens), 1))
    return _orig_append(cache, rows, ident, context_lens, qsl)


MUTANTS = [
    ("gather ignores block table", O, "gather_sequence", _gather_ignores_table,
     [lambda: [pins.test_decode_matches_brute_force(bs) for bs in (1, 2, 16)]]),
    ("gather slot-major order", O, "gather_sequence", _gather_slot_major,
     [lambda: [pins.test_prefill_matches_brute_force(bs) for bs in (2, 16)]]),
    ("scale dropped", O, "attend_two_pass", _attend_no_scale,
     [pins.test_decode_identity_table_equals_library_sdpa]),
    ("recurrence carry dropped", pins, "online_softmax_ref", _online_drop_carry,
     [lambda: pins.test_online_recurrence_equals_two_pass(1000)]),
    ("split merge without rescale", O, "split_merge_ref", _split_no_rescale,
     [lambda: pins.test_split_merge_equals_unsplit(64)]),
    ("copy last index wins", pins, "copy_blocks_ref", _copy_last_wins,
     [lambda: [pins.test_copy_matches_brute_force_with_duplicates_and_invalid(s) for s in range(40)],
      pins.test_copy_duplicate_destination_takes_lowest_source]),
    ("prefill top-left causal alignment", pins, "prefill_ref", _prefill_top_left,
     [pins.test_prefill_single_new_token_equals_decode]),
    ("gqa map h % Hkv", pins, "decode_ref", _decode_mod_group,
     [pins.test_gqa_equals_mha_on_repeated_kv]),
    ("append position off by one", pins, "append_kv_ref", _append_off_by_one,
     [lambda: pins.test_append_block_manager_example(pins_golden())]),
    ("append ignores block table", pins, "append_kv_ref", _append_ignores_table,
     [lambda: pins.test_append_block_manager_example(pins_golden()),
      pins.test_append_then_gather_returns_the_rows]),
]


def pins_golden():
    import os
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.mark.parametrize("name,mod,attr,fn,checks", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pin_catches_mutation(monkeypatch, golden_dir, name, mod, attr, fn, checks):
    monkeypatch.setattr(mod, attr, fn)
    if mod is O and hasattr(pins, attr):
        monkeypatch.setattr(pins, attr, fn)
    caught = False
    for chk in checks:
        try:
            chk()
        except (AssertionError, IndexError, ValueError):
            caught = True
    assert caught, f"no pin caught mutation: {name}"
