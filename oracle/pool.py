"""Oracle model of the host block pool.  TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Follows [Serving] The Build, Step 4: one pool of fixed-size pages indexed by physical id; a
free list that starts as every id, ``alloc`` takes the id at the END of the list and fails
when the list is empty, ``free`` puts the id back at the end; each sequence owns a page
table (logical block -> physical page) and a token count; appending the token at position
``pos`` opens a new page when ``pos % block_size == 0`` and writes slot ``pos % block_size``
of the last page; finishing a sequence returns its pages in page-table order.

Sharing follows [Chapter] "PagedAttention: KV cache memory" and [Notes] "Fragmentation:
PagedAttention": sequences may point at the same physical blocks until they diverge; a
write into a shared block copies it first (copy-on-write).  The pages give no algorithm
for it; the reading used here (and by the library) is:

* ``fork(parent)`` gives a new sequence the parent's table and length and adds one
  reference to every block of it.
* A write only ever targets position ``len`` (the end of the sequence), so a full shared
  block is never written.  When the first token of an append lands in a partially filled
  last block whose refcount is > 1, a fresh block is taken, the pair (old, new) is
  reported for a whole-block copy, the old block loses one reference and the sequence's
  table points at the new block.
* ``append`` is all-or-nothing: it first counts the blocks it needs and fails with no state
  change when the free list is shorter (the pages' mid-append failure would leave partial
  state, which no caller can use).
* ``free`` drops one reference per block in table order; a block returns to the free list
  when its count reaches zero.
* Sequence ids are the lowest id not currently live.

Prefix caching follows [Serving] The Build, Step 8 ("Prefix caching"): a dictionary from a
block-aligned token prefix to the list of blocks holding it; a lookup tries the longest
block-aligned prefix of the request first and, on a hit, adds one reference to every block of
the match.  The pages show no insertion or release; the reading used here (and by the library):

* ``prefix_insert(seq, tokens)`` registers, for k = 1 .. (full blocks of seq), the prefix
  ``tokens[:16k]`` with the blocks of the prefix ``tokens[:16(k-1)]`` as already registered plus
  seq's block k; a prefix that is already registered keeps its blocks; registration stops at a
  block that is already registered under another prefix.  Only full blocks are registered, so
  a registered block is never written again.
* ``prefix_lookup(tokens)`` starts a new sequence holding the longest registered block-aligned
  prefix of ``tokens`` (the whole request may match).
* A registered block whose count reaches zero is not freed: it waits on an LRU list (least
  recently released first) and can still be matched, which takes it off the list.  The blocks a
  finished sequence releases join the list deepest first (reverse table order), so eviction
  shortens a registered prefix from its end rather than cutting it at the root.
* An allocation with an empty free list evicts the LRU head: every prefix whose blocks include
  it is unregistered, and the blocks left in no registered prefix leave the LRU for the free
  list in LRU order; the evicted block is the one allocated.  An append fails only when the free
  list and the LRU together are too short.
"""
from __future__ import annotations


class OutOfBlocks(Exception):
    """The free list cannot cover an append (the pages' out-of-pages error)."""


class InvalidOp(Exception):
    """Operation on an unknown sequence or with a bad argument."""


class PoolModel:
    def __init__(self, num_blocks: int, block_size: int = 16, free_order=None):
        if num_blocks < 0 or block_size <= 0:
            raise InvalidOp("bad pool size")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        if free_order is None:
            self.free = list(range(self.num_blocks))
        else:
            fo = [int(x) for x in free_order]
            if sorted(fo) != list(range(self.num_blocks)):
                raise InvalidOp("free_order must be a permutation of 0..N-1")
            self.free = fo
        self.refcnt = [0] * self.num_blocks
        self.tables: dict[int, list[int]] = {}
        self.lens: dict[int, int] = {}
        self.entries: dict[tuple, list[int]] = {}  # registered prefix tokens -> its blocks
        self.lru: list[int] = []  # registered blocks with no reference, least recently released first

    # ---- block level --------------------------------------------------------------
    def _alloc(self) -> int:
        if self.free:
            b = self.free.pop()
        elif self.lru:
            b = self._evict()
        else:
            raise OutOfBlocks()
        self.refcnt[b] = 1
        return b

    def _release(self, b: int, idle: list) -> None:
        """Drop one reference; an unregistered block at zero goes back on the free list, a
        registered one is collected in ``idle`` for the LRU."""
        self.refcnt[b] -= 1
        if self.refcnt[b] == 0:
            (idle if self._registered(b) else self.free).append(b)

    def _registered(self, b: int) -> bool:
        return any(b in blocks for blocks in self.entries.values())

    def _evict(self) -> int:
        b = self.lru.pop(0)
        for key in [k for k, blocks in self.entries.items() if b in blocks]:
            del self.entries[key]
        for x in list(self.lru):
            if not self._registered(x):
                self.lru.remove(x)
                self.free.append(x)
        return b

    # ---- sequence level -----------------------------------------------------------
    def _check(self, seq: int) -> None:
        if seq not in self.tables:
            raise InvalidOp(f"unknown sequence {seq}")

    def _new_id(self) -> int:
        i = 0
        while i in self.tables:
            i += 1
        return i

    def new_seq(self) -> int:
        s = self._new_id()
        self.tables[s] = []
        self.lens[s] = 0
        return s

    def fork(self, parent: int) -> int:
        self._check(parent)
        child = self._new_id()
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.refcnt[b] += 1
        return child

    def blocks_needed(self, seq: int, n: int) -> int:
        """Fresh blocks an append of ``n`` tokens takes: one per position that starts a
        block, plus one copy-on-write block when the first write hits a shared partial block."""
        self._check(seq)
        if n < 0:
            raise InvalidOp("negative token count")
        start = self.lens[seq]
        bs = self.block_size
        need = sum(1 for pos in range(start, start + n) if pos % bs == 0)
        if n > 0 and start % bs != 0 and self.refcnt[self.tables[seq][-1]] > 1:
            need += 1
        return need

    def append(self, seq: int, n: int):
        """Reserve slots for ``n`` tokens.  Returns (slots, cow_pairs)."""
        need = self.blocks_needed(seq, n)
        if need > len(self.free) + len(self.lru):
            raise OutOfBlocks()
        table = self.tables[seq]
        bs = self.block_size
        slots, cow = [], []
        for _ in range(n):
            pos = self.lens[seq]
            if pos % bs == 0:
                table.append(self._alloc())
            elif self.refcnt[table[-1]] > 1:
                old = table[-1]
                new = self._alloc()
                self.refcnt[old] -= 1
                cow.append((old, new))
                table[-1] = new
            slots.append(table[pos // bs] * bs + pos % bs)
            self.lens[seq] = pos + 1
        return slots, cow

    def free_seq(self, seq: int) -> None:
        self._check(seq)
        idle: list[int] = []
        for b in self.tables[seq]:
            self._release(b, idle)
        self.lru.extend(reversed(idle))
        del self.tables[seq]
        del self.lens[seq]

    # ---- prefix cache ([Serving] The Build, Step 8) ------------------------------------
    def prefix_lookup(self, tokens):
        """New sequence holding the longest registered block-aligned prefix of ``tokens``.
        Returns (seq, matched token count).  The prefix grows one block at a time; every
        registered one replaces the previous hit, so the last hit is the longest."""
        s = self.new_seq()
        bs = self.block_size
        hit, blocks = 0, []
        prefix: tuple = ()
        for k in range(len(tokens) // bs):
            prefix = prefix + tuple(int(t) for t in tokens[k * bs:(k + 1) * bs])
            chain = self.entries.get(prefix)
            if chain is not None:
                hit, blocks = len(prefix), chain
        for b in blocks:
            if self.refcnt[b] == 0:
                self.lru.remove(b)
            self.refcnt[b] += 1
        self.tables[s] = list(blocks)
        self.lens[s] = hit
        return s, hit

    def prefix_insert(self, seq: int, tokens) -> int:
        """Register seq's full blocks under their token prefixes.  Returns how many of seq's
        blocks were newly registered."""
        self._check(seq)
        bs = self.block_size
        nfull = min(len(tokens), self.lens[seq]) // bs
        chain: list[int] = []
        added = 0
        for k in range(1, nfull + 1):
            key = tuple(int(t) for t in tokens[: k * bs])
            if key in self.entries:
                chain = list(self.entries[key])
                continue
            b = self.tables[seq][k - 1]
            if self._registered(b):
                break
            chain = chain + [b]
            self.entries[key] = chain
            added += 1
        return added

    def num_evictable(self) -> int:
        return len(self.lru)

    def num_registered(self) -> int:
        return len({b for blocks in self.entries.values() for b in blocks})

    # ---- builders -----------------------------------------------------------------
    def slot(self, seq: int, pos: int) -> int:
        self._check(seq)
        if not 0 <= pos < self.lens[seq]:
            raise InvalidOp("position out of range")
        t = self.tables[seq]
        return t[pos // self.block_size] * self.block_size + pos % self.block_size

    def block_tables(self, seqs, max_blocks: int):
        """Row b = physical blocks of seqs[b] in logical order, padded with -1; lens = tokens."""
        rows, lens = [], []
        for s in seqs:
            self._check(s)
            t = self.tables[s]
            if len(t) > max_blocks:
                raise InvalidOp("max_blocks too small")
            rows.append(list(t) + [-1] * (max_blocks - len(t)))
            lens.append(self.lens[s])
        return rows, lens

    def num_free(self) -> int:
        return len(self.free)

    def live(self):
        return sorted(self.tables)
