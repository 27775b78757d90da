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

What the page fixes (restated as rules, not as its listing):
  * a physical block is free exactly when no request holds it: the manager
    keeps one reference count per block, and the free blocks are those at 0;
  * an allocation hands out the lowest-numbered free block and gives it a
    count of 1; with no free block it is an out-of-blocks error;
  * a release lowers the block's count by one (at 0 the block is free again);
  * a request of n prompt tokens is registered with ceil(n / block_size)
    newly allocated blocks, in logical order, and a token count of n;
  * one more token goes into slot n mod block_size of the last block, so a
    request whose count n is a multiple of block_size needs a new block
    first; if none is free the request is left unchanged and the append fails;
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
        self.ref = [0] * num_blocks            # holders of each physical block
        self.tables: dict[int, list[int]] = {}
        self.tokens: dict[int, int] = {}

    @property
    def free(self) -> list[int]:
        """Free block ids, increasing: the blocks nobody holds."""
        return [b for b, holders in enumerate(self.ref) if holders == 0]

    # -- physical blocks --------------------------------------------------
    def _allocate(self) -> int:
        if 0 not in self.ref:
            raise OutOfBlocks()
        lowest = self.ref.index(0)             # lowest id with no holder
        self.ref[lowest] = 1
        return lowest

    def _release(self, b: int) -> None:
        assert self.ref[b] > 0, "released a block nobody holds"
        self.ref[b] -= 1

    # -- requests ---------------------------------------------------------
    def register(self, rid: int, prompt_len: int) -> None:
        if rid in self.tables:
            raise KeyError(rid)
        blocks = []
        try:
            while len(blocks) * self.block_size < prompt_len:
                blocks.append(self._allocate())
        except OutOfBlocks:
            for b in blocks:
                self._release(b)
            raise
        self.tables[rid] = blocks
        self.tokens[rid] = prompt_len

    def append_token(self, rid: int):
        """Returns None, or the (old, new) pair of a copy-on-write."""
        blocks, n = self.tables[rid], self.tokens[rid]
        slot = n % self.block_size
        cow = None
        if slot == 0:                          # every held slot is filled
            blocks.append(self._allocate())
        elif self.ref[blocks[-1]] > 1:         # the slot is in a shared block
            old, new = blocks[-1], self._allocate()
            self._release(old)
            blocks[-1] = new
            cow = (old, new)
        self.tokens[rid] = n + 1
        return cow

    def fork(self, parent: int, child: int) -> None:
        if child in self.tables:
            raise KeyError(child)
        shared = list(self.tables[parent])
        for b in shared:
            self.ref[b] += 1
        self.tables[child] = shared
        self.tokens[child] = self.tokens[parent]

    def finish(self, rid: int) -> None:
        for b in self.tables.pop(rid):
            self._release(b)
        del self.tokens[rid]

    def free_count(self) -> int:
        return self.ref.count(0)
