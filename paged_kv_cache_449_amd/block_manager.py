"""Host-side KV block manager for one pool.

Keeps the free list, a reference count per physical block and each
sequence's block table; hands out the slot of every token written and plans
copy-on-write.  Follows the pages' block manager: blocks are taken from a
free pool only when a token needs one and returned as soon as nothing uses
them ("vLLM 与 KV Cache", how-it-works points 1-4; "vLLM KV Cache 实现机制"
§3.1 data structures and §3.2 allocation); shared blocks carry a reference
count and are copied before the first write into them ("vLLM — 把操作系统的
分页搬进 GPU KV cache", core mechanism 3, case 2).

Order of allocation is deterministic: blocks leave the free list from its
front and come back at its end.
"""
from __future__ import annotations

import collections
from typing import Dict, Hashable, Iterable, List, Optional, Sequence, Tuple

import numpy as np


class PoolExhausted(RuntimeError):
    """No free block is left; the caller must preempt a sequence."""


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, free_order: Optional[Iterable[int]] = None):
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = range(self.num_blocks) if free_order is None else free_order
        self._free = collections.deque(int(b) for b in order)
        if len(self._free) != self.num_blocks or len(set(self._free)) != self.num_blocks:
            raise ValueError("free_order must be a permutation of all block ids")
        self._refs = np.zeros(self.num_blocks, dtype=np.int32)
        self._tables: Dict[Hashable, List[int]] = {}
        self._lens: Dict[Hashable, int] = {}

    # ------------------------------------------------------------ accounting
    def num_free_blocks(self) -> int:
        return len(self._free)

    def ref_count(self, block: int) -> int:
        return int(self._refs[block])

    def table(self, seq) -> List[int]:
        return list(self._tables[seq])

    def length(self, seq) -> int:
        return self._lens[seq]

    def waste(self, seq) -> int:
        """Unused token slots in the sequence's last block."""
        return len(self._tables[seq]) * self.block_size - self._lens[seq]

    # ------------------------------------------------------------ allocation
    def _take(self) -> int:
        if not self._free:
            raise PoolExhausted(f"all {self.num_blocks} blocks are in use")
        b = self._free.popleft()
        self._refs[b] = 1
        return b

    def _drop(self, b: int) -> None:
        self._refs[b] -= 1
        if self._refs[b] == 0:
            self._free.append(b)

    def _slot(self, table: Sequence[int], pos: int) -> int:
        return table[pos // self.block_size] * self.block_size + pos % self.block_size

    def add_sequence(self, seq, num_tokens: int) -> np.ndarray:
        """Register a sequence and reserve slots for its first num_tokens
        tokens; returns their slots (int64)."""
        if seq in self._tables:
            raise KeyError(f"sequence {seq!r} exists")
        self._tables[seq], self._lens[seq] = [], 0
        slots = np.empty(num_tokens, dtype=np.int64)
        for i in range(num_tokens):
            slot, pair = self.append_slot(seq)
            assert pair is None
            slots[i] = slot
        return slots

    def fork(self, parent, children: Sequence[Hashable]) -> None:
        """Children start as copies of the parent's table and share its blocks."""
        t = self._tables[parent]
        for c in children:
            if c in self._tables:
                raise KeyError(f"sequence {c!r} exists")
            self._tables[c] = list(t)
            self._lens[c] = self._lens[parent]
            for b in t:
                self._refs[b] += 1

    def free(self, seq) -> None:
        for b in self._tables.pop(seq):
            self._drop(b)
        del self._lens[seq]

    def append_slot(self, seq) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Reserve the slot of the sequence's next token.  Returns (slot, pair)
        where pair = (src, dst) is a block copy that must run before the write
        (copy-on-write of a shared last block), or None."""
        t = self._tables[seq]
        pos = self._lens[seq]
        pair = None
        if pos % self.block_size == 0:
            t.append(self._take())
        elif self._refs[t[-1]] > 1:
            fresh = self._take()
            pair = (t[-1], fresh)
            self._refs[t[-1]] -= 1
            t[-1] = fresh
        self._lens[seq] = pos + 1
        return self._slot(t, pos), pair

    # ------------------------------------------------------------ device views
    def block_tables(self, seqs: Sequence[Hashable], max_blocks: Optional[int] = None) -> np.ndarray:
        """int32 [len(seqs)][max_blocks], -1 where a sequence has no block."""
        mb = max_blocks or max(1, max(len(self._tables[s]) for s in seqs))
        out = np.full((len(seqs), mb), -1, dtype=np.int32)
        for i, s in enumerate(seqs):
            t = self._tables[s]
            if len(t) > mb:
                raise ValueError(f"sequence {s!r} has {len(t)} blocks > max_blocks {mb}")
            out[i, :len(t)] = t
        return out

    def context_lens(self, seqs: Sequence[Hashable]) -> np.ndarray:
        return np.asarray([self._lens[s] for s in seqs], dtype=np.int32)
