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

    # ---- block level --------------------------------------------------------------
    def _alloc(self) -> int:
        if not self.free:
            raise OutOfBlocks()
        b = self.free.pop()
        self.refcnt[b] = 1
        return b

    def _release(self, b: int) -> None:
        self.refcnt[b] -= 1
        if self.refcnt[b] == 0:
            self.free.append(b)

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
        if need > len(self.free):
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
        for b in self.tables[seq]:
            self._release(b)
        del self.tables[seq]
        del self.lens[seq]

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
