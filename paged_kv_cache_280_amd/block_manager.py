"""Host-side block manager: the allocation half of the paged KV cache.

What it does, after "PagedAttention (vLLM)" (troisinh.com):
* section "Cơ chế Block Table": the cache is cut into blocks of a fixed number of
  tokens; each sequence owns a table of physical block ids, one per logical
  block; a block is taken from the pool only when a token needs it (L tokens ->
  ceil(L/B) blocks), and a freed block can be reused wherever it sits;
* section "Copy-on-Write cho Beam Search": sequences forked from one another
  (parallel sampling, beam search) share the physical blocks of their common
  prefix; a shared block is copied the moment one sharer writes into it;
* section "Vấn đề": a request that the pool cannot hold is refused.

Design: reference counts and the free list live in numpy arrays; the free list is
a stack (the most recently freed block is reused first, so a sequence that
finishes leaves its blocks at the top for the next admission).  Copy-on-write
decisions are recorded as (src, dst) pairs and handed to the GPU copy_blocks
call in one batch before the tokens are written.  A refused request changes
nothing.
"""

from __future__ import annotations

import numpy as np


class PoolExhausted(RuntimeError):
    """The pool has fewer free blocks than the request needs; nothing changed."""


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        if free_order is None:
            free_order = np.arange(self.num_blocks, dtype=np.int32)
        order = np.asarray(free_order, dtype=np.int32)
        if order.shape != (self.num_blocks,) or not np.array_equal(np.sort(order),
                                                                   np.arange(self.num_blocks)):
            raise ValueError("free_order must be a permutation of the pool's block ids")
        # stack: the next block handed out is _stack[_top - 1]
        self._stack = order[::-1].copy()
        self._top = self.num_blocks
        self.refcount = np.zeros(self.num_blocks, dtype=np.int32)
        self._tables: dict = {}
        self._lens: dict = {}
        self._copies: list = []

    # -- pool ------------------------------------------------------------------
    @property
    def num_free(self) -> int:
        return self._top

    def _take(self, n: int) -> np.ndarray:
        ids = self._stack[self._top - n:self._top][::-1].copy()
        self._top -= n
        self.refcount[ids] = 1
        return ids

    def _give_back(self, ids) -> None:
        for b in ids:
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self._stack[self._top] = b
                self._top += 1

    def blocks_for(self, n_tokens: int) -> int:
        return -(-int(n_tokens) // self.block_size)

    # -- sequences ----------------------------------------------------------------
    def add(self, seq, n_tokens: int) -> None:
        """Admit a sequence whose first n_tokens (its prompt) are about to be written."""
        if seq in self._tables:
            raise KeyError("sequence %r exists" % (seq,))
        need = self.blocks_for(n_tokens)
        if need > self._top:
            raise PoolExhausted("need %d blocks, %d free" % (need, self._top))
        self._tables[seq] = list(self._take(need))
        self._lens[seq] = int(n_tokens)

    def append(self, seq, n_tokens: int = 1):
        """Make room for n_tokens more tokens at the end of seq.  Returns the slots
        (physical block, offset) the new tokens go to.  A shared last block is
        copied first (the pair is queued for copy_blocks)."""
        n_tokens = int(n_tokens)
        table = self._tables[seq]
        L = self._lens[seq]
        B = self.block_size
        grow = self.blocks_for(L + n_tokens) - len(table)
        cow = n_tokens > 0 and L % B != 0 and self.refcount[table[-1]] > 1
        if grow + cow > self._top:
            raise PoolExhausted("need %d blocks, %d free" % (grow + cow, self._top))
        if cow:
            src = table[-1]
            dst = int(self._take(1)[0])
            self.refcount[src] -= 1          # the other sharers keep it
            self._copies.append((int(src), dst))
            table[-1] = dst
        if grow > 0:
            table.extend(int(b) for b in self._take(grow))
        slots = [(table[t // B], t % B) for t in range(L, L + n_tokens)]
        self._lens[seq] = L + n_tokens
        return slots

    def fork(self, parent, child) -> None:
        """child starts as an exact sharer of every block of parent."""
        if child in self._tables:
            raise KeyError("sequence %r exists" % (child,))
        table = self._tables[parent]
        self._tables[child] = list(table)
        self._lens[child] = self._lens[parent]
        np.add.at(self.refcount, np.asarray(table, dtype=np.int64), 1)

    def free(self, seq) -> None:
        self._give_back(self._tables.pop(seq))
        del self._lens[seq]

    # -- views handed to the GPU calls --------------------------------------------
    def take_copies(self) -> np.ndarray:
        """Pending copy-on-write pairs as int32 [P][2] (src, dst); clears the queue."""
        pairs = np.asarray(self._copies, dtype=np.int32).reshape(-1, 2)
        self._copies = []
        return pairs

    def table(self, seq) -> list:
        return list(self._tables[seq])

    def context_len(self, seq) -> int:
        return self._lens[seq]

    def batch(self, seqs, pad_block: int = 0, max_blocks=None):
        """(block_tables int32 [S][M], context_lens int32 [S]) for a decode call.
        Padding entries hold pad_block; they are never read."""
        seqs = list(seqs)
        M = max_blocks or max((len(self._tables[s]) for s in seqs), default=1)
        tables = np.full((len(seqs), max(M, 1)), pad_block, dtype=np.int32)
        lens = np.zeros(len(seqs), dtype=np.int32)
        for i, s in enumerate(seqs):
            t = self._tables[s]
            tables[i, :len(t)] = t
            lens[i] = self._lens[s]
        return tables, lens

    def sequences(self):
        return list(self._tables)

    def internal_waste(self) -> float:
        """Fraction of the slots held by live sequences that hold no token (only the
        tail of each sequence's last block)."""
        held = sum(len(t) for t in self._tables.values()) * self.block_size
        used = sum(self._lens.values())
        return 0.0 if held == 0 else (held - used) / held

    def free_ids(self) -> np.ndarray:
        return self._stack[:self._top].copy()
