"""Pins of the block-manager oracle (CPU): the page's allocator run, the
invariants its steps keep, prefix sharing and copy-on-write."""

import json
import os

import numpy as np
import pytest

from oracle.block_manager_oracle import BlockManagerOracle, OutOfBlocks


def replay_page_example(g, make):
    """The simulator run of [P-wall] §三; returns the manager and the free
    count after each step."""
    bm = make(g["num_blocks"], g["block_size"])
    counts = [bm.free_count()]
    bm.register(1, 20)
    counts.append(bm.free_count())
    bm.register(2, 10)
    counts.append(bm.free_count())
    grew_at = None
    for i in range(13):
        before = len(bm_table(bm, 1))
        bm.append_token(1)
        if len(bm_table(bm, 1)) > before and grew_at is None:
            grew_at = i + 1
    counts.append(bm.free_count())
    table_b = list(bm_table(bm, 2))
    bm.finish(2)
    counts.append(bm.free_count())
    return bm, counts, grew_at, table_b


def bm_table(bm, rid):
    return bm.tables[rid] if hasattr(bm, "tables") else bm.table(rid)


def test_page_allocator_run(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "append_block_manager_example.json")))
    bm, counts, grew_at, table_b = replay_page_example(g, BlockManagerOracle)
    assert counts == [s[3] for s in g["run"]["steps"]]
    assert grew_at == g["run"]["expansion_at_append"]
    assert bm.tables[1] == g["block_tables"]["req_A"]
    assert table_b == g["block_tables"]["req_B"]
    assert bm.tokens[1] == g["context_lens"]["req_A"]
    assert bm.free == g["run"]["final_free_list"]


def check_invariants(bm, nblocks, bs):
    refs = np.zeros(nblocks, dtype=int)
    for rid, t in bm.tables.items():
        assert len(t) == (bm.tokens[rid] + bs - 1) // bs
        for b in t:
            refs[b] += 1
    assert list(refs) == bm.ref
    assert bm.free == sorted(bm.free)
    assert set(bm.free) == {b for b in range(nblocks) if refs[b] == 0}
    assert bm.free_count() == len(bm.free)


@pytest.mark.parametrize("seed", range(30))
def test_random_operations_keep_counts_tables_and_free_list_consistent(seed):
    rng = np.random.default_rng(seed)
    nblocks, bs = int(rng.integers(4, 40)), int(rng.choice([1, 2, 4, 16]))
    bm = BlockManagerOracle(nblocks, bs)
    live, next_id = [], 0
    for _ in range(300):
        op = rng.integers(0, 10)
        try:
            if op < 3 or not live:
                bm.register(next_id, int(rng.integers(0, 3 * bs + 2)))
                live.append(next_id)
                next_id += 1
            elif op < 7:
                bm.append_token(int(rng.choice(live)))
            elif op < 8:
                bm.fork(int(rng.choice(live)), next_id)
                live.append(next_id)
                next_id += 1
            else:
                rid = int(rng.choice(live))
                bm.finish(rid)
                live.remove(rid)
        except OutOfBlocks:
            pass
        check_invariants(bm, nblocks, bs)


def test_copy_on_write_of_a_shared_partial_block():
    bm = BlockManagerOracle(8, 4)
    bm.register(1, 6)                 # blocks 0 (full), 1 (2 of 4 slots)
    bm.fork(1, 2)                     # both share 0 and 1
    assert bm.ref[:2] == [2, 2]
    cow = bm.append_token(2)          # writes into shared block 1: copy it first
    assert cow == (1, 2)
    assert bm.tables[2] == [0, 2] and bm.tables[1] == [0, 1]
    assert bm.ref[:3] == [2, 1, 1]
    assert bm.append_token(1) is None  # block 1 is now 1's alone
    assert bm.append_token(2) is None  # block 2 is 2's alone


def test_append_after_a_full_shared_block_allocates_without_copy():
    bm = BlockManagerOracle(8, 4)
    bm.register(1, 8)                 # two full blocks
    bm.fork(1, 2)
    assert bm.append_token(2) is None
    assert bm.tables[2] == [0, 1, 2] and bm.ref[:3] == [2, 2, 1]


def test_out_of_blocks_leaves_state_unchanged():
    bm = BlockManagerOracle(3, 4)
    bm.register(1, 8)
    with pytest.raises(OutOfBlocks):
        bm.register(2, 9)             # needs 3, only 1 free
    assert bm.free == [2] and 2 not in bm.tables
    bm.register(3, 4)
    with pytest.raises(OutOfBlocks):
        bm.append_token(3)            # block full, none free
    assert bm.tokens[3] == 4 and bm.tables[3] == [2]


def test_finish_of_a_fork_keeps_the_shared_blocks():
    bm = BlockManagerOracle(6, 4)
    bm.register(1, 5)
    bm.fork(1, 2)
    bm.finish(1)
    assert bm.tables[2] == [0, 1] and bm.ref[:2] == [1, 1] and bm.free == [2, 3, 4, 5]
    bm.finish(2)
    assert bm.free == list(range(6))


# planted mistakes: each must make one of the pins above fail
class _HighestFirst(BlockManagerOracle):
    # hands out the highest free id instead of the lowest
    def _allocate(self):
        if 0 not in self.ref:
            raise OutOfBlocks()
        b = len(self.ref) - 1 - self.ref[::-1].index(0)
        self.ref[b] = 1
        return b


class _LateGrowth(BlockManagerOracle):
    # grows one token late: the token that fills a new block finds none
    def append_token(self, rid):
        n = self.tokens[rid]
        if n % self.block_size == 1 and n > self.block_size:
            self.tables[rid].append(self._allocate())
        self.tokens[rid] = n + 1
        return None


class _KeepsOnFinish(BlockManagerOracle):
    # a finished request's blocks are never returned
    def finish(self, rid):
        self.tables.pop(rid)
        del self.tokens[rid]


@pytest.mark.parametrize("mutant", [_HighestFirst, _LateGrowth, _KeepsOnFinish])
def test_page_run_catches_mutations(golden_dir, mutant):
    g = json.load(open(os.path.join(golden_dir, "append_block_manager_example.json")))
    bm, counts, grew_at, table_b = replay_page_example(g, mutant)
    ok = (counts == [s[3] for s in g["run"]["steps"]] and grew_at == g["run"]["expansion_at_append"]
          and bm.free == g["run"]["final_free_list"])
    assert not ok
