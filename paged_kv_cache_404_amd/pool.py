"""Python handle over the C++ host block pool (pkv_pool_* / pkv_seq_* / pkv_build_*).

Argument marshalling only: allocation, copy-on-write and the builders run in libpagedkv.
"""
from __future__ import annotations

import ctypes as C

import numpy as np

from ._lib import check, lib


def _ptr(a: np.ndarray) -> int:
    # the raw address (the C declarations take void*): a quarter of the cost of ctypes.data_as
    return a.ctypes.data


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


class BlockPool:
    def __init__(self, num_blocks: int, block_size: int = 16, free_order=None):
        h = C.c_void_p()
        fo = None if free_order is None else _i32(free_order)
        if fo is not None and fo.size != num_blocks:
            raise ValueError("free_order must have num_blocks entries")
        check(lib.pkv_pool_create(int(num_blocks), int(block_size), None if fo is None else _ptr(fo), C.byref(h)))
        self._h = h
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            lib.pkv_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _out(self, fn, *args) -> int:
        o = C.c_int32()
        check(fn(self._h, *args, C.byref(o)))
        return o.value

    def num_free(self) -> int:
        return self._out(lib.pkv_pool_num_free)

    def free_list(self) -> np.ndarray:
        n = self.num_free()
        buf = np.zeros(max(n, 1), dtype=np.int32)
        got = C.c_int32()
        check(lib.pkv_pool_free_list(self._h, _ptr(buf), buf.size, C.byref(got)))
        return buf[: got.value].copy()

    def refcount(self, block: int) -> int:
        return self._out(lib.pkv_pool_refcount, int(block))

    def new_seq(self) -> int:
        return self._out(lib.pkv_seq_new)

    def fork(self, parent: int) -> int:
        return self._out(lib.pkv_seq_fork, int(parent))

    def blocks_needed(self, seq: int, n: int) -> int:
        return self._out(lib.pkv_seq_blocks_needed, int(seq), int(n))

    def seq_len(self, seq: int) -> int:
        return self._out(lib.pkv_seq_len, int(seq))

    def seq_num_blocks(self, seq: int) -> int:
        return self._out(lib.pkv_seq_num_blocks, int(seq))

    def append(self, seq: int, n: int):
        """Returns (slots int32[n], cow pairs list[(src, dst)])."""
        slots = np.zeros(max(int(n), 1), dtype=np.int32)
        cow = np.zeros(2, dtype=np.int32)
        ncow = C.c_int32()
        check(lib.pkv_seq_append(self._h, int(seq), int(n), _ptr(slots), _ptr(cow), C.byref(ncow)))
        return slots[: int(n)], ([(int(cow[0]), int(cow[1]))] if ncow.value else [])

    def append_many(self, seqs, counts):
        """Batched append in order.  Returns (status, done, slots, cow_pairs [n_cow, 2]); on an
        error the slots of the sequences not appended are -1."""
        s, c = _i32(seqs), _i32(counts)
        total = int(c.sum()) if c.size else 0
        slots = np.empty(max(total, 1), dtype=np.int32)
        cow = np.empty((max(len(s), 1), 2), dtype=np.int32)
        ncow, done = C.c_int32(), C.c_int32()
        st = lib.pkv_seqs_append(self._h, _ptr(s), _ptr(c), len(s), _ptr(slots), _ptr(cow), C.byref(ncow),
                                 C.byref(done))
        if st != 0:
            slots[int(c[: done.value].sum()) if done.value else 0:] = -1
        return st, done.value, slots[:total], cow[: ncow.value]

    def free(self, seq: int) -> None:
        check(lib.pkv_seq_free(self._h, int(seq)))

    def block_tables(self, seqs, max_blocks: int):
        """(tables int32 [n][max_blocks], -1 padded; lens int32 [n]); the C builder writes every entry."""
        s = _i32(seqs)
        n, mb = len(s), int(max_blocks)
        tables = np.empty((max(n, 1), max(mb, 1)), dtype=np.int32)
        lens = np.empty(max(n, 1), dtype=np.int32)
        check(lib.pkv_build_block_tables(self._h, _ptr(s), n, mb, _ptr(tables), _ptr(lens)))
        if n >= 1 and mb >= 1:
            return tables, lens
        return np.full((n, mb), -1, dtype=np.int32), lens[:n].copy()

    def slot_mapping(self, seqs, starts, counts) -> np.ndarray:
        s, st, c = _i32(seqs), _i32(starts), _i32(counts)
        total = int(c.sum()) if c.size else 0
        out = np.zeros(max(total, 1), dtype=np.int32)
        check(lib.pkv_build_slot_mapping(self._h, _ptr(s), _ptr(st), _ptr(c), len(s), _ptr(out)))
        return out[:total].copy()

    # ---- prefix cache ----
    def prefix_insert(self, seq: int, tokens) -> int:
        """Register seq's full blocks under the prefixes of ``tokens``; returns how many."""
        t = _i32(tokens)
        n = C.c_int32()
        check(lib.pkv_prefix_insert(self._h, int(seq), _ptr(t) if t.size else None, int(t.size), C.byref(n)))
        return n.value

    def prefix_lookup(self, tokens):
        """New sequence holding the longest registered block-aligned prefix: (seq, n_matched)."""
        t = _i32(tokens)
        s, n = C.c_int32(), C.c_int32()
        check(lib.pkv_prefix_lookup(self._h, _ptr(t) if t.size else None, int(t.size), C.byref(s), C.byref(n)))
        return s.value, n.value

    def evictable(self) -> np.ndarray:
        """Registered blocks without references, next to evict first."""
        got = C.c_int32()
        buf = np.zeros(max(self.num_blocks, 1), dtype=np.int32)
        check(lib.pkv_prefix_evictable(self._h, _ptr(buf), buf.size, C.byref(got)))
        return buf[: got.value].copy()

    def num_registered(self) -> int:
        return self._out(lib.pkv_prefix_num_registered)
