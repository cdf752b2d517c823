"""Binding of the library's host block manager (block_manager.h).

Keeps the free list, a reference count and last-access stamp per physical
block, each sequence's block table, copy-on-write planning, the prefix cache
and LRU eviction -- all in the native library; this class maps hashable
sequence keys to the library's int64 ids and marshals arrays.  It follows the
pages' block manager ("vLLM 与 KV Cache", how-it-works points 1-4; "vLLM KV
Cache 实现机制" §3.1-3.2 and §4.2 prefix caching; "vLLM — 把操作系统的分页
搬进 GPU KV cache", core mechanism 3 and case 2).

Blocks leave the free list from its front and come back at its end;
forked sequences share blocks until one of them writes into a shared block,
which first gets a fresh copy.
"""
from __future__ import annotations

import ctypes
from typing import Dict, Hashable, Iterable, List, Optional, Sequence, Tuple

import numpy as np

_STAT_FIELDS = ("num_blocks", "free_blocks", "cached_blocks", "used_blocks", "num_sequences", "tokens",
                "table_entries", "prefix_queries", "prefix_hits", "evictions", "cow_copies", "allocations")


class _Stats(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int64) for f in _STAT_FIELDS]


class PoolExhausted(RuntimeError):
    """No free or evictable block is left; the caller must preempt a sequence."""


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, free_order: Optional[Iterable[int]] = None,
                 prefix_caching: bool = False):
        from . import _check, lib
        self._lib, self._check_status = lib(), _check
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = None if free_order is None else np.ascontiguousarray(np.fromiter(free_order, dtype=np.int64))
        if order is not None:
            if order.shape[0] != self.num_blocks or order.min(initial=0) < 0 or order.max(initial=0) >= self.num_blocks:
                raise ValueError("free_order must be a permutation of all block ids")
            order = order.astype(np.int32)
        h = ctypes.c_void_p()
        st = self._lib.bm_create(self.num_blocks, self.block_size, _ptr(order), int(bool(prefix_caching)),
                                 ctypes.byref(h))
        if st == 1:
            raise ValueError("free_order must be a permutation of all block ids (or bad sizes)")
        self._call(st, "bm_create")
        self._h = h
        self._ids: Dict[Hashable, int] = {}
        self._next_id = 0

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.bm_destroy(h)
            self._h = None

    def _call(self, status: int, call: str) -> None:
        from . import KV_ERR_NO_BLOCKS
        if status == KV_ERR_NO_BLOCKS:
            raise PoolExhausted(f"{call}: all {self.num_blocks} blocks are in use")
        self._check_status(status, call)

    def _id(self, seq) -> int:
        if seq not in self._ids:
            raise KeyError(f"unknown sequence {seq!r}")
        return self._ids[seq]

    def _new_id(self, seq) -> int:
        if seq in self._ids:
            raise KeyError(f"sequence {seq!r} exists")
        self._ids[seq] = self._next_id
        self._next_id += 1
        return self._ids[seq]

    # ------------------------------------------------------------ accounting
    def num_free_blocks(self) -> int:
        n = ctypes.c_int64()
        self._call(self._lib.bm_num_free_blocks(self._h, ctypes.byref(n)), "bm_num_free_blocks")
        return n.value

    def ref_count(self, block: int) -> int:
        r = ctypes.c_int32()
        self._call(self._lib.bm_ref_count(self._h, int(block), ctypes.byref(r)), "bm_ref_count")
        return r.value

    def _info(self, seq) -> Tuple[int, int]:
        ln, nb = ctypes.c_int32(), ctypes.c_int32()
        self._call(self._lib.bm_sequence_info(self._h, self._id(seq), ctypes.byref(ln), ctypes.byref(nb)),
                   "bm_sequence_info")
        return ln.value, nb.value

    def table(self, seq) -> List[int]:
        _, nb = self._info(seq)
        out = np.empty(max(nb, 1), dtype=np.int32)
        self._call(self._lib.bm_block_table(self._h, self._id(seq), _ptr(out), nb), "bm_block_table")
        return out[:nb].tolist()

    def length(self, seq) -> int:
        return self._info(seq)[0]

    def waste(self, seq) -> int:
        """Unused token slots in the sequence's last block."""
        ln, nb = self._info(seq)
        return nb * self.block_size - ln

    def stats(self) -> dict:
        s = _Stats()
        self._call(self._lib.bm_stats(self._h, ctypes.byref(s)), "bm_stats")
        return {f: getattr(s, f) for f in _STAT_FIELDS}

    # ------------------------------------------------------------ allocation
    def add_sequence(self, seq, num_tokens: int, tokens: Optional[Sequence[int]] = None,
                     extra_hash: int = 0) -> np.ndarray:
        """Register a sequence and reserve slots for its first num_tokens
        tokens; returns their slots (int64).  With token ids (and prefix
        caching on), leading full blocks already cached are shared; see
        add_sequence_cached for how many."""
        return self.add_sequence_cached(seq, num_tokens, tokens, extra_hash)[0]

    def add_sequence_cached(self, seq, num_tokens: int, tokens: Optional[Sequence[int]] = None,
                            extra_hash: int = 0) -> Tuple[np.ndarray, int]:
        tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
        if tok is not None and tok.shape[0] != num_tokens:
            raise ValueError("tokens must hold num_tokens ids")
        slots = np.empty(max(int(num_tokens), 1), dtype=np.int64)
        cached = ctypes.c_int32()
        sid = self._new_id(seq)
        st = self._lib.bm_add_sequence(self._h, sid, _ptr(tok), int(num_tokens), ctypes.c_uint64(extra_hash & (2**64 - 1)),
                                       _ptr(slots), ctypes.byref(cached))
        if st != 0:
            del self._ids[seq]
        self._call(st, "bm_add_sequence")
        return slots[:num_tokens], cached.value

    def fork(self, parent, children: Sequence[Hashable]) -> None:
        """Children start as copies of the parent's table and share its blocks."""
        pid = self._id(parent)
        for c in children:
            if c in self._ids:
                raise KeyError(f"sequence {c!r} exists")
        if len(set(children)) != len(children):
            raise KeyError("children repeat")
        ids = np.array([self._next_id + i for i in range(len(children))], dtype=np.int64)
        self._call(self._lib.bm_fork(self._h, pid, _ptr(ids), len(children)), "bm_fork")
        for c, i in zip(children, ids):
            self._ids[c] = int(i)
        self._next_id += len(children)

    def free(self, seq) -> None:
        self._call(self._lib.bm_free(self._h, self._id(seq)), "bm_free")
        del self._ids[seq]

    def append_slots(self, seq, count: int, tokens: Optional[Sequence[int]] = None
                     ) -> Tuple[np.ndarray, Optional[Tuple[int, int]]]:
        """Reserve the slots of the sequence's next `count` tokens.  Returns
        (slots, pair): pair = (src, dst) is a block copy that must run before
        the writes (copy-on-write of a shared last block), or None."""
        tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
        if tok is not None and tok.shape[0] != count:
            raise ValueError("tokens must hold count ids")
        slots = np.empty(max(int(count), 1), dtype=np.int64)
        pair = np.empty(2, dtype=np.int32)
        npairs = ctypes.c_int32()
        self._call(self._lib.bm_append_slots(self._h, self._id(seq), _ptr(tok), int(count), _ptr(slots), _ptr(pair),
                                             ctypes.byref(npairs)), "bm_append_slots")
        return slots[:count], (int(pair[0]), int(pair[1])) if npairs.value else None

    def append_batch(self, seqs: Sequence[Hashable], counts: Optional[Sequence[int]] = None,
                     tokens: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
        """One step for a batch, all or nothing: counts[i] (default 1) slots
        for seqs[i] in list order.  Returns (slots int64 [sum(counts)], copy
        pairs int32 [P][2] in the order they arise)."""
        ids = np.array([self._id(s) for s in seqs], dtype=np.int64)
        cnt = np.ones(len(seqs), dtype=np.int32) if counts is None else np.ascontiguousarray(counts, dtype=np.int32)
        total = int(cnt.sum())
        tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
        if tok is not None and tok.shape[0] != total:
            raise ValueError("tokens must hold sum(counts) ids")
        slots = np.empty(max(total, 1), dtype=np.int64)
        pairs = np.empty((max(len(seqs), 1), 2), dtype=np.int32)
        npairs = ctypes.c_int32()
        st = self._lib.bm_append_batch(self._h, _ptr(ids), _ptr(cnt), len(seqs), _ptr(tok), _ptr(slots), _ptr(pairs),
                                       ctypes.byref(npairs))
        if st == 1:
            raise ValueError("a sequence repeats or a count is negative")
        self._call(st, "bm_append_batch")
        return slots[:total], pairs[:npairs.value]

    def ids(self, seqs: Sequence[Hashable]) -> np.ndarray:
        """The library's int64 ids of the given sequences (for reserve_step)."""
        return np.array([self._id(s) for s in seqs], dtype=np.int64)

    def reserve_step(self, ids: np.ndarray, counts: np.ndarray, slots: np.ndarray, pairs: np.ndarray) -> int:
        """append_batch on caller-prepared buffers (ids from ids(), int32
        counts, int64 slots of sum(counts), int32 pairs [len(ids)][2]), for
        loops that reserve every step: no per-call allocation or key lookup.
        Returns the number of copy pairs written."""
        n = ids.shape[0]
        if (ids.dtype != np.int64 or counts.dtype != np.int32 or slots.dtype != np.int64 or pairs.dtype != np.int32
                or counts.shape != (n,) or pairs.shape[0] < n or pairs.shape[1:] != (2,)
                or not all(a.flags.c_contiguous for a in (ids, counts, slots, pairs))
                or slots.shape[0] < int(counts.sum())):
            raise ValueError("reserve_step: ids int64 [n], counts int32 [n], slots int64 [>= sum(counts)], "
                             "pairs int32 [>= n][2], all contiguous")
        npairs = ctypes.c_int32()
        st = self._lib.bm_append_batch(self._h, ids.ctypes.data, counts.ctypes.data, n, None,
                                       slots.ctypes.data, pairs.ctypes.data, ctypes.byref(npairs))
        self._call(st, "bm_append_batch")
        return npairs.value

    def append_slot(self, seq, token: Optional[int] = None) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Reserve the slot of the sequence's next token: (slot, pair)."""
        slots, pair = self.append_slots(seq, 1, None if token is None else [token])
        return int(slots[0]), pair

    # ------------------------------------------------------------ device views
    def block_tables(self, seqs: Sequence[Hashable], max_blocks: Optional[int] = None) -> np.ndarray:
        """int32 [len(seqs)][max_blocks], -1 where a sequence has no block."""
        ids = np.array([self._id(s) for s in seqs], dtype=np.int64)
        if max_blocks is None:
            max_blocks = max([1] + [self._info(s)[1] for s in seqs])
        out = np.empty((len(seqs), max_blocks), dtype=np.int32)
        st = self._lib.bm_block_tables(self._h, _ptr(ids), len(seqs), int(max_blocks), _ptr(out), None)
        if st == 1:
            raise ValueError(f"a sequence has more than max_blocks={max_blocks} blocks")
        self._call(st, "bm_block_tables")
        return out

    def context_lens(self, seqs: Sequence[Hashable]) -> np.ndarray:
        return np.asarray([self._info(s)[0] for s in seqs], dtype=np.int32)
