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

* "vLLM PagedAttention: Bước đột phá về thông lượng suy luận LLM"
  (vi.news.hada.io), list of advanced features, prefix caching: requests whose
  prompts begin alike share the KV cache of that common beginning instead of
  computing it again.

Readings where the pages are silent: the free list is LIFO (the most recently
freed block is handed out first) and starts in the order the caller gives; a
request that cannot be met leaves every piece of state untouched; a write into
a block whose reference count is 1 happens in place.

Prefix caching (readings): only full blocks of a prompt are shared, and a block
is identified by every token from position 0 to its end (its K/V depend on all
of them); a new prompt reuses cached blocks from its start up to its first block
that is not cached, its other blocks are taken, and then its new full blocks
join the cache (each unless its key is already there); a cached block whose last user leaves keeps its contents and
stays findable, and is handed out for new contents only when the free list is
empty, least recently released first (its cache entry is then dropped); a
finished sequence releases its blocks last to first.

Copy batches (reading): the copies queued between two take_copies calls are run
together, before the tokens of that batch are written, so within a batch no
block may be both a copy's destination and another copy's source, and no two
copies may share a destination.  Until the batch is taken, a block named by a
queued copy is not handed out again (one released meanwhile waits and joins the
free list when the batch is taken, in release order); a copy out of a block that
is itself a queued destination copies that destination's source (the same bytes
once the batch has run).
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
        self.pinned = set()  # blocks named by a queued copy
        self.waiting = []    # blocks released while pinned, in release order
        self.source_of = {}  # queued destination -> its source
        self.cached = {}     # tuple of tokens 0 .. end of block -> block id
        self.key_of = {}     # block id -> its key in self.cached
        self.evictable = []  # cached blocks nobody holds, least recently released first

    # -- helpers ---------------------------------------------------------------
    def _take(self) -> int:
        if self.free:
            b = self.free.pop()
        else:
            b = self.evictable.pop(0)
            del self.cached[self.key_of.pop(b)]
        self.refcount[b] = 1
        return b

    def _release(self, b: int) -> None:
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            if b in self.pinned:
                self.waiting.append(b)
            else:
                self._to_free_list(b)

    def _to_free_list(self, b: int) -> None:
        if b in self.key_of:
            self.evictable.append(b)
        else:
            self.free.append(b)

    def available(self) -> int:
        return len(self.free) + len(self.evictable)

    def blocks_for(self, n_tokens: int) -> int:
        return -(-int(n_tokens) // self.block_size)

    # -- operations --------------------------------------------------------------
    def add(self, seq, n_tokens: int, tokens=None) -> int:
        """A new sequence holding n_tokens (its prompt).  With the prompt's token
        ids, its leading full blocks come from the prefix cache where they can;
        returns how many of its tokens were found there (their K/V need not be
        written again)."""
        if seq in self.tables:
            raise KeyError(seq)
        n_tokens = int(n_tokens)
        need = self.blocks_for(n_tokens)
        B = self.block_size
        hits = []
        if tokens is not None:
            tokens = [int(t) for t in tokens]
            if len(tokens) != n_tokens:
                raise ValueError("one token id per prompt position")
            for j in range(n_tokens // B):
                key = tuple(tokens[:(j + 1) * B])
                if key not in self.cached:
                    break
                hits.append(self.cached[key])
        revived = sum(1 for b in hits if self.refcount[b] == 0)
        if need - len(hits) > self.available() - revived:
            raise PoolExhausted("need %d blocks, %d free" % (need - len(hits),
                                                            self.available() - revived))
        table = []
        for b in hits:
            if self.refcount[b] == 0:
                self.evictable.remove(b)
            self.refcount[b] += 1
            table.append(b)
        for j in range(len(hits), need):
            table.append(self._take())
        # then the new full blocks join the cache, each unless its key is there
        for j in range(len(hits), need):
            if tokens is not None and (j + 1) * B <= n_tokens:
                key = tuple(tokens[:(j + 1) * B])
                if key not in self.cached:
                    self.cached[key] = table[j]
                    self.key_of[table[j]] = key
        self.tables[seq] = table
        self.lens[seq] = n_tokens
        return len(hits) * B

    def append(self, seq, n_tokens: int = 1) -> None:
        """Write n_tokens more tokens at the end of seq."""
        n_tokens = int(n_tokens)
        L = self.lens[seq]
        table = self.tables[seq]
        new_blocks = self.blocks_for(L + n_tokens) - self.blocks_for(L)
        last_shared = (n_tokens > 0 and L % self.block_size != 0
                       and self.refcount[table[-1]] > 1)
        need = new_blocks + (1 if last_shared else 0)
        if need > self.available():
            raise PoolExhausted("need %d blocks, %d free" % (need, self.available()))
        if last_shared:
            shared = table[-1]
            dst = self._take()
            src = self.source_of.get(shared, shared)
            self.copies.append((src, dst))
            self.source_of[dst] = src
            self.pinned.add(src)
            self.pinned.add(dst)
            self.refcount[shared] -= 1   # still >= 1: another sharer holds it
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
        """Release the blocks last to first: a prompt's first blocks, the ones other
        prompts can share, become the most recently released and are evicted last."""
        for b in reversed(self.tables.pop(seq)):
            self._release(b)
        del self.lens[seq]

    def take_copies(self) -> list:
        """The queued copies, in order; the batch is over: blocks that waited join
        the free list."""
        copies, self.copies = self.copies, []
        self.pinned = set()
        self.source_of = {}
        waiting, self.waiting = self.waiting, []
        for b in waiting:
            self._to_free_list(b)
        return copies

    # -- views -------------------------------------------------------------------
    def check_conservation(self) -> None:
        counted = [0] * self.num_blocks
        for table in self.tables.values():
            for b in table:
                counted[b] += 1
        assert counted == self.refcount, "refcounts disagree with the tables"
        live = sum(1 for c in self.refcount if c > 0)
        assert live + len(self.free) + len(self.evictable) + len(self.waiting) == self.num_blocks, \
            "free + evictable + waiting + live != pool"
        idle = self.free + self.evictable + self.waiting
        assert len(set(idle)) == len(idle), "a block is free twice"
        assert all(self.refcount[b] == 0 for b in idle), "a free block is referenced"
        assert all(b in self.key_of for b in self.evictable), "an evictable block has no key"
        assert all(b not in self.key_of for b in self.free), "a free block is still cached"
        assert all(self.cached[k] == b for b, k in self.key_of.items()), "cache maps disagree"
        for seq, table in self.tables.items():
            assert len(table) == self.blocks_for(self.lens[seq])
