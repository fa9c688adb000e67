"""Host-side block manager: the allocation half of the paged KV cache.

What it does, after "PagedAttention (vLLM)" (troisinh.com):
* section "Cơ chế Block Table": the cache is cut into blocks of a fixed number of
  tokens; each sequence owns a table of physical block ids, one per logical
  block; a block is taken from the pool only when a token needs it (L tokens ->
  ceil(L/B) blocks), and a freed block can be reused wherever it sits;
* section "Copy-on-Write cho Beam Search": sequences forked from one another
  (parallel sampling, beam search) share the physical blocks of their common
  prefix; a shared block is copied the moment one sharer writes into it;
* section "Vấn đề": a request that the pool cannot hold is refused;
* prefix caching ("vLLM PagedAttention: Bước đột phá về thông lượng suy luận
  LLM", vi.news.hada.io, list of advanced features): a prompt that begins like
  an earlier one reuses the blocks holding that beginning instead of computing
  its K/V again.

Prefix cache: a full prompt block is keyed by a SHA-256 chain over the token ids
of every block up to and including it (the key of block j hashes the key of
block j-1 and block j's ids), so equal keys mean equal token prefixes.  A new
prompt takes cached blocks from its start up to its first block that is not
cached; its other full blocks join the cache (unless their key is already
there).  A cached block whose last holder leaves keeps its contents and stays
findable (evictable); such blocks are handed out for new contents only once the
free stack is empty, least recently released first, and lose their key then.  A
finished sequence releases its blocks last to first.

Design: reference counts and the free list live in numpy arrays; the free list is
a stack (the most recently freed block is reused first, so a sequence that
finishes leaves its blocks at the top for the next admission).  Copy-on-write
decisions are recorded as (src, dst) pairs and handed to the GPU copy_blocks
call in one batch before the tokens are written.  A refused request changes
nothing.

A batch of copies runs as one copy_blocks call, whose pairs must have distinct
destinations that are not also sources.  So until take_copies hands the batch
over, every block a pending pair names stays out of circulation: a freed source
or destination is held back and joins the free list when the batch is taken, and
a copy whose source is itself a pending destination reads that destination's own
source instead (the bytes the destination will hold once the batch has run).
"""

from __future__ import annotations

import hashlib
from collections import OrderedDict

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
        self._pins: dict = {}                   # block -> pending pairs naming it
        self._held: list = []                   # released while pinned, in release order
        self._src_of: dict = {}                 # pending destination -> its source
        self._cache: dict = {}                  # chain key -> block id
        self._key_of: dict = {}                 # block id -> chain key
        self._evictable: OrderedDict = OrderedDict()  # released cached blocks, oldest first

    # -- pool ------------------------------------------------------------------
    @property
    def num_free(self) -> int:
        """Blocks a request can be given: the free stack plus evictable cached blocks."""
        return self._top + len(self._evictable)

    @property
    def num_cached(self) -> int:
        return len(self._cache)

    def _take(self, n: int) -> np.ndarray:
        k = min(n, self._top)
        ids = self._stack[self._top - k:self._top][::-1].copy()
        self._top -= k
        if k < n:   # the stack ran dry: evict the least recently released cached blocks
            more = []
            for _ in range(n - k):
                b, _ = self._evictable.popitem(last=False)
                del self._cache[self._key_of.pop(b)]
                more.append(b)
            ids = np.concatenate([ids, np.asarray(more, dtype=np.int32)])
        self.refcount[ids] = 1
        return ids

    def _give_back(self, ids) -> None:
        for b in ids:
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                if int(b) in self._pins:
                    self._held.append(int(b))
                else:
                    self._recycle(int(b))

    def _recycle(self, b: int) -> None:
        if b in self._key_of:
            self._evictable[b] = None
        else:
            self._stack[self._top] = b
            self._top += 1

    @staticmethod
    def _chain(prev: bytes, block_tokens) -> bytes:
        return hashlib.sha256(prev + np.asarray(block_tokens, dtype="<i8").tobytes()).digest()

    def blocks_for(self, n_tokens: int) -> int:
        return -(-int(n_tokens) // self.block_size)

    # -- sequences ----------------------------------------------------------------
    def add(self, seq, n_tokens: int, tokens=None) -> int:
        """Admit a sequence whose first n_tokens (its prompt) are about to be written.
        With the prompt's token ids the prefix cache is used: returns the number of
        leading prompt tokens found there (their K/V are already in the pool; only
        the rest must be written)."""
        if seq in self._tables:
            raise KeyError("sequence %r exists" % (seq,))
        n_tokens = int(n_tokens)
        need = self.blocks_for(n_tokens)
        B = self.block_size
        hits, keys = [], []
        if tokens is not None:
            tokens = np.asarray(tokens, dtype=np.int64)
            if tokens.shape != (n_tokens,):
                raise ValueError("one token id per prompt position")
            prev = b""
            for j in range(n_tokens // B):
                prev = self._chain(prev, tokens[j * B:(j + 1) * B])
                keys.append(prev)
            for key in keys:
                b = self._cache.get(key)
                if b is None:
                    break
                hits.append(b)
        revived = sum(1 for b in hits if self.refcount[b] == 0)
        if need - len(hits) > self.num_free - revived:
            raise PoolExhausted("need %d blocks, %d free" % (need - len(hits),
                                                            self.num_free - revived))
        for b in hits:
            if self.refcount[b] == 0:
                del self._evictable[b]
            self.refcount[b] += 1
        new = list(self._take(need - len(hits)))
        for j, b in enumerate(new, start=len(hits)):
            if j < len(keys) and keys[j] not in self._cache:
                self._cache[keys[j]] = int(b)
                self._key_of[int(b)] = keys[j]
        self._tables[seq] = [int(b) for b in hits] + [int(b) for b in new]
        self._lens[seq] = n_tokens
        return len(hits) * B

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
        if grow + cow > self.num_free:
            raise PoolExhausted("need %d blocks, %d free" % (grow + cow, self.num_free))
        if cow:
            shared = table[-1]
            dst = int(self._take(1)[0])
            self.refcount[shared] -= 1       # the other sharers keep it
            # a pending destination holds its source's bytes once the batch has run
            src = self._src_of.get(int(shared), int(shared))
            self._copies.append((src, dst))
            self._src_of[dst] = src
            for b in (src, dst):
                self._pins[b] = self._pins.get(b, 0) + 1
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
        """Release seq's blocks last to first, so that the first blocks of a prompt
        (the ones others can share) are the last to be evicted."""
        self._give_back(self._tables.pop(seq)[::-1])
        del self._lens[seq]

    # -- views handed to the GPU calls --------------------------------------------
    def take_copies(self) -> np.ndarray:
        """Pending copy-on-write pairs as int32 [P][2] (src, dst); clears the queue.
        Destinations are distinct and none is a source, so the pairs may be copied
        in any order.  Blocks released while the batch was pending join the free
        list now, in the order they were released."""
        pairs = np.asarray(self._copies, dtype=np.int32).reshape(-1, 2)
        self._copies = []
        self._pins = {}
        self._src_of = {}
        held, self._held = self._held, []
        for b in held:
            self._recycle(b)
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

    def shared_groups(self, seqs, max_group_size: int):
        """Sharing groups of a decode batch taken in the order of ``seqs``, for
        paged_attn_decode_shared: runs of consecutive sequences (at most
        max_group_size each) that start with the same physical blocks, as forks of
        one prompt do ("PagedAttention (vLLM)", section "Copy-on-Write cho Beam
        Search").  A run grows while the next sequence shares at least the run's
        current prefix with its first member.  The prefix is the positions every
        member holds in common blocks, rounded down to a multiple of
        max(16, block_size).  Returns (group_first int32 [num_groups + 1],
        prefix_lens int32 [len(seqs)]); a group of one has prefix 0."""
        seqs = list(seqs)
        align = max(16, self.block_size)
        B = self.block_size

        def shared_positions(a, b):
            ta, tb = self._tables[a], self._tables[b]
            n = 0
            while n < min(len(ta), len(tb)) and ta[n] == tb[n]:
                n += 1
            p = min(n * B, self._lens[a], self._lens[b])
            return p - p % align

        first, prefix = [0], np.zeros(len(seqs), dtype=np.int32)
        i = 0
        while i < len(seqs):
            j, P = i + 1, 0
            while j < len(seqs) and j - i < max_group_size:
                pj = shared_positions(seqs[i], seqs[j])
                if pj < align or (j > i + 1 and pj < P):
                    break
                P = pj if j == i + 1 else P
                j += 1
            prefix[i:j] = P if j - i > 1 else 0
            first.append(j)
            i = j
        return np.asarray(first, dtype=np.int32), prefix

    def sequences(self):
        return list(self._tables)

    def internal_waste(self) -> float:
        """Fraction of the slots held by live sequences that hold no token (only the
        tail of each sequence's last block)."""
        held = sum(len(t) for t in self._tables.values()) * self.block_size
        used = sum(self._lens.values())
        return 0.0 if held == 0 else (held - used) / held

    def free_ids(self) -> np.ndarray:
        """Blocks on the free stack (holding nothing anyone can find)."""
        return self._stack[:self._top].copy()

    def evictable_ids(self) -> np.ndarray:
        """Cached blocks nobody holds, least recently released first."""
        return np.asarray(list(self._evictable), dtype=np.int32)
