"""Plain Python block manager: the allocator and per-request block tables of
the paged KV cache, as the pages describe them.

TEST INFRASTRUCTURE ONLY.  Only the test-suite may import this module; the
native block manager shares no code with it.

Page cited (by title):
  [P-wall]  "大模型长文本推理基座从 FlashAttention 硬件加速机制到 vLLM 核心
             PagedAttention 显存物理布局深度剖析" — §三 (the allocator
             simulator: physical blocks with reference counts, a sorted free
             list, per-request block tables, registration, token-by-token
             growth, release) and §四.2 (prefix sharing by reference counts,
             copy-on-write when a request writes into a shared block).

Steps, in the page's order:
  * the pool starts with every block free; the free list is kept sorted, and
    an allocation takes its lowest id and sets that block's count to 1; an
    empty free list is an out-of-blocks error;
  * releasing a block lowers its count if it is above 0; at 0 the block
    returns to the free list (which is sorted again);
  * registering a request of n prompt tokens allocates ceil(n / block_size)
    blocks, in order, and records n tokens;
  * appending one token to a request whose token count is a multiple of
    block_size (its blocks are full) first allocates one more block; if that
    fails the request is left unchanged and the append reports failure;
  * finishing a request releases each of its blocks.
Readings where the page is descriptive only (§四.2):
  * fork: a new request shares every block of an existing one (each count
    + 1) and starts with its token count;
  * append into a partly filled last block whose count is above 1 first
    copies it: a new block is allocated, the old one released, the table's
    last entry replaced, and the (old, new) pair reported so the caller can
    copy the block's bytes; the filled slots are the only ones that matter;
  * a failed registration releases what it had allocated (the page's
    simulator raises part way; a half-registered request is not kept).
"""

from __future__ import annotations


class OutOfBlocks(Exception):
    pass


class BlockManagerOracle:
    def __init__(self, num_blocks: int, block_size: int):
        self.block_size = block_size
        self.ref = [0] * num_blocks
        self.free = list(range(num_blocks))
        self.tables: dict[int, list[int]] = {}
        self.tokens: dict[int, int] = {}

    # -- physical blocks --------------------------------------------------
    def _allocate(self) -> int:
        if not self.free:
            raise OutOfBlocks()
        b = self.free.pop(0)
        self.ref[b] = 1
        return b

    def _release(self, b: int) -> None:
        if self.ref[b] > 0:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
                self.free.sort()

    # -- requests ---------------------------------------------------------
    def register(self, rid: int, prompt_len: int) -> None:
        if rid in self.tables:
            raise KeyError(rid)
        need = (prompt_len + self.block_size - 1) // self.block_size
        got = []
        try:
            for _ in range(need):
                got.append(self._allocate())
        except OutOfBlocks:
            for b in got:
                self._release(b)
            raise
        self.tables[rid] = got
        self.tokens[rid] = prompt_len

    def append_token(self, rid: int):
        """Returns None, or the (old, new) pair of a copy-on-write."""
        table, n = self.tables[rid], self.tokens[rid]
        cow = None
        if n % self.block_size == 0:
            table.append(self._allocate())
        elif self.ref[table[-1]] > 1:
            new = self._allocate()
            old = table[-1]
            self._release(old)
            table[-1] = new
            cow = (old, new)
        self.tokens[rid] = n + 1
        return cow

    def fork(self, parent: int, child: int) -> None:
        if child in self.tables:
            raise KeyError(child)
        for b in self.tables[parent]:
            self.ref[b] += 1
        self.tables[child] = list(self.tables[parent])
        self.tokens[child] = self.tokens[parent]

    def finish(self, rid: int) -> None:
        for b in self.tables.pop(rid):
            self._release(b)
        del self.tokens[rid]

    def free_count(self) -> int:
        return len(self.free)
