"""Reference model of the host-side block manager -- TEST INFRASTRUCTURE ONLY.

Plain Python lists and dicts, one rule per method, so a reader can check each
rule against the pages:

* "PagedAttention (vLLM)" (troisinh.com), section "Cơ chế Block Table": blocks of
  fixed token capacity; a per-sequence table maps logical block j to a physical
  block; a block is taken only when a token needs it, so L tokens hold
  ceil(L/B) blocks (100 tokens -> 7 blocks of 16); freed blocks are reused
  wherever they are, with no defragmentation.
* same page, section "Copy-on-Write cho Beam Search": sequences that share a
  prefix share its physical blocks; a shared block is copied only when one of
  the sharers writes a token that differs, i.e. when it writes into it.
* "KV cache, PagedAttention" (aiwiki.vn), paragraph on paging: waste sits only
  in the last, partly filled block of each sequence; branches with a common
  prefix share blocks instead of duplicating them.

Readings where the pages are silent: the free list is LIFO (the most recently
freed block is handed out first) and starts in the order the caller gives; a
request that cannot be met leaves every piece of state untouched; a write into
a block whose reference count is 1 happens in place.
"""

from __future__ import annotations


class PoolExhausted(RuntimeError):
    pass


class BlockModel:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = list(range(self.num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(self.num_blocks)):
            raise ValueError("free_order must be a permutation of the pool")
        # LIFO: the block handed out next is the last element.
        self.free = list(reversed(order))
        self.refcount = [0] * self.num_blocks
        self.tables = {}   # seq id -> list of physical block ids
        self.lens = {}     # seq id -> number of tokens
        self.copies = []   # (src, dst) pairs emitted by copy-on-write, in order

    # -- helpers ---------------------------------------------------------------
    def _take(self) -> int:
        b = self.free.pop()
        self.refcount[b] = 1
        return b

    def _release(self, b: int) -> None:
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            self.free.append(b)

    def blocks_for(self, n_tokens: int) -> int:
        return -(-int(n_tokens) // self.block_size)

    # -- operations --------------------------------------------------------------
    def add(self, seq, n_tokens: int) -> None:
        """A new sequence holding n_tokens (its prompt)."""
        if seq in self.tables:
            raise KeyError(seq)
        need = self.blocks_for(n_tokens)
        if need > len(self.free):
            raise PoolExhausted("need %d blocks, %d free" % (need, len(self.free)))
        self.tables[seq] = [self._take() for _ in range(need)]
        self.lens[seq] = int(n_tokens)

    def append(self, seq, n_tokens: int = 1) -> None:
        """Write n_tokens more tokens at the end of seq."""
        n_tokens = int(n_tokens)
        L = self.lens[seq]
        table = self.tables[seq]
        new_blocks = self.blocks_for(L + n_tokens) - self.blocks_for(L)
        last_shared = (n_tokens > 0 and L % self.block_size != 0
                       and self.refcount[table[-1]] > 1)
        need = new_blocks + (1 if last_shared else 0)
        if need > len(self.free):
            raise PoolExhausted("need %d blocks, %d free" % (need, len(self.free)))
        if last_shared:
            src = table[-1]
            dst = self._take()
            self.copies.append((src, dst))
            self.refcount[src] -= 1   # still >= 1: another sharer holds it
            table[-1] = dst
        for _ in range(new_blocks):
            table.append(self._take())
        self.lens[seq] = L + n_tokens

    def fork(self, parent, child) -> None:
        """child shares every block of parent (parallel sampling / beam split)."""
        if child in self.tables:
            raise KeyError(child)
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.refcount[b] += 1

    def free_seq(self, seq) -> None:
        for b in self.tables.pop(seq):
            self._release(b)
        del self.lens[seq]

    # -- views -------------------------------------------------------------------
    def check_conservation(self) -> None:
        counted = [0] * self.num_blocks
        for table in self.tables.values():
            for b in table:
                counted[b] += 1
        assert counted == self.refcount, "refcounts disagree with the tables"
        live = sum(1 for c in self.refcount if c > 0)
        assert live + len(self.free) == self.num_blocks, "free + live != pool"
        assert len(set(self.free)) == len(self.free), "a block is free twice"
        assert all(self.refcount[b] == 0 for b in self.free), "a free block is referenced"
        for seq, table in self.tables.items():
            assert len(table) == self.blocks_for(self.lens[seq])
