"""The oracle's model of the KV block manager with prefix caching and LRU
eviction -- TEST INFRASTRUCTURE (tests only; the library never imports it).

Written from the pages, independently of the library's C++ manager; the
tests drive both with the same operations and compare every output (slots,
copy pairs, cached-token counts, tables, reference counts, free counts,
hit/eviction/copy counters) for equality.

What it follows:
  * A preallocated pool of equal blocks; a block is taken only when a token
    needs a slot and returned when nothing references it.  Page "vLLM 与 KV
    Cache", how-it-works points 1-4; page "vLLM KV Cache 实现机制" §3.2 step 1.
  * Block record with a reference count and a last-access time; shared blocks
    are copied before the first write (copy-on-write) and never evicted while
    referenced.  Same page §3.1 and §3.2 point 3; page "vLLM — 把操作系统的分页
    搬进 GPU KV cache", core mechanism 3 and case 2.
  * Prefix caching: a full block is found again by its parent block, its exact
    tokens and an extra per-request value.  Page "vLLM KV Cache 实现机制" §4.2.
    Here the lookup key IS that triple (a Python tuple): there is no hash
    value, so no collision handling is needed.
  * LRU: unreferenced cached blocks are evicted least recently used first,
    only when no plain free block is left.  Same page §3.2.

Choices where the pages are open (the same readings the library documents):
  plain free blocks leave from the front of the free list and return at its
  back; a freed sequence releases its blocks last to first; a block's parent
  identity is the registration (a counter) of the parent block; a full block
  is registered when its last slot is reserved, only if the sequence's tokens
  are known and its previous block is registered, and only if no registered
  block has the same key; every matching leading full block is reused.
"""
from __future__ import annotations

import collections
from typing import Dict, List, Optional, Sequence, Tuple


class NoBlocks(RuntimeError):
    pass


class _Seq:
    def __init__(self):
        self.table: List[int] = []
        self.length = 0
        self.extra = 0
        self.track = False
        self.pending: List[int] = []

    def copy(self) -> "_Seq":
        c = _Seq()
        c.table, c.length, c.extra, c.track, c.pending = list(self.table), self.length, self.extra, self.track, list(self.pending)
        return c


class AllocatorModel:
    def __init__(self, num_blocks: int, block_size: int, free_order: Optional[Sequence[int]] = None,
                 prefix_caching: bool = False):
        self.bs = block_size
        self.num_blocks = num_blocks
        self.prefix = prefix_caching
        self.free = collections.deque(range(num_blocks) if free_order is None else [int(b) for b in free_order])
        self.lru: List[int] = []                 # unreferenced cached blocks, oldest release first
        self.ref = [0] * num_blocks
        self.registration = [0] * num_blocks     # 0 = holds no cached prefix
        self.key_of: Dict[int, tuple] = {}       # block -> (parent registration, extra, tokens)
        self.cache: Dict[tuple, int] = {}        # key -> block
        self.next_registration = 1
        self.seqs: Dict[int, _Seq] = {}
        self.hits = self.queries = self.evictions = self.copies = self.allocations = 0

    # ------------------------------------------------------------ primitives
    def available(self) -> int:
        return len(self.free) + len(self.lru)

    def _take(self) -> int:
        if self.free:
            b = self.free.popleft()
        else:
            b = self.lru.pop(0)
            del self.cache[self.key_of.pop(b)]
            self.registration[b] = 0
            self.evictions += 1
        self.ref[b] = 1
        self.allocations += 1
        return b

    def _release(self, b: int) -> None:
        self.ref[b] -= 1
        if self.ref[b] == 0:
            if self.registration[b]:
                self.lru.append(b)
            else:
                self.free.append(b)

    def _share(self, b: int) -> None:
        if b in self.lru:
            self.lru.remove(b)
        self.ref[b] += 1

    def _register_last(self, s: _Seq) -> None:
        """The sequence's last block has just become full."""
        if not (self.prefix and s.track):
            return
        parent = 0
        if len(s.table) >= 2:
            parent = self.registration[s.table[-2]]
            if parent == 0:
                s.track = False
                return
        key = (parent, s.extra, tuple(s.pending))
        if key in self.cache:
            s.track = False
            return
        b = s.table[-1]
        self.registration[b] = self.next_registration
        self.next_registration += 1
        self.key_of[b] = key
        self.cache[key] = b

    def _append_one(self, s: _Seq, token: Optional[int]) -> Tuple[int, Optional[Tuple[int, int]]]:
        pos = s.length
        pair = None
        if pos % self.bs == 0:
            s.table.append(self._take())
            s.pending = []
        elif self.ref[s.table[-1]] > 1:
            fresh = self._take()
            pair = (s.table[-1], fresh)
            self.ref[s.table[-1]] -= 1
            s.table[-1] = fresh
            self.copies += 1
        s.length = pos + 1
        slot = s.table[-1] * self.bs + pos % self.bs
        if s.track:
            if token is None:
                s.track = False
            else:
                s.pending.append(int(token))
                if pos % self.bs == self.bs - 1:
                    self._register_last(s)
        return slot, pair

    # ------------------------------------------------------------ operations
    def add_sequence(self, sid: int, num_tokens: int, tokens: Optional[Sequence[int]] = None, extra: int = 0):
        """(slots, number of leading tokens found in the prefix cache)."""
        if sid in self.seqs:
            raise KeyError(sid)
        bs = self.bs
        track = self.prefix and tokens is not None
        hits: List[int] = []
        queries = 0
        if track:
            parent = 0
            for k in range(num_tokens // bs):
                queries += 1
                key = (parent, extra, tuple(int(t) for t in tokens[k * bs:(k + 1) * bs]))
                if key not in self.cache:
                    break
                hits.append(self.cache[key])
                parent = self.registration[self.cache[key]]
        cached = len(hits) * bs
        need = -(-(num_tokens - cached) // bs)
        if need > self.available() - sum(1 for b in hits if b in self.lru):
            raise NoBlocks("add_sequence")
        s = _Seq()
        s.extra, s.track = extra, track
        for b in hits:
            self._share(b)
            s.table.append(b)
        s.length = cached
        slots = [s.table[i // bs] * bs + i % bs for i in range(cached)]
        for i in range(cached, num_tokens):
            slots.append(self._append_one(s, None if tokens is None else tokens[i])[0])
        self.seqs[sid] = s
        self.queries += queries
        self.hits += len(hits)
        return slots, cached

    def fork(self, parent: int, children: Sequence[int]) -> None:
        src = self.seqs[parent]
        for c in children:
            if c in self.seqs:
                raise KeyError(c)
        for c in children:
            self.seqs[c] = src.copy()
            for b in src.table:
                self.ref[b] += 1

    def append(self, sid: int, count: int, tokens: Optional[Sequence[int]] = None):
        """(slots, copy pair or None) for the sequence's next count tokens."""
        s = self.seqs[sid]
        need = sum(1 for p in range(s.length, s.length + count) if p % self.bs == 0)
        if count > 0 and s.length % self.bs != 0 and self.ref[s.table[-1]] > 1:
            need += 1
        if need > self.available():
            raise NoBlocks("append")
        slots, pair = [], None
        for i in range(count):
            slot, p = self._append_one(s, None if tokens is None else tokens[i])
            slots.append(slot)
            pair = pair or p
        return slots, pair

    def release(self, sid: int) -> None:
        s = self.seqs.pop(sid)
        for b in reversed(s.table):
            self._release(b)

    # ------------------------------------------------------------ views
    def table(self, sid: int) -> List[int]:
        return list(self.seqs[sid].table)

    def length(self, sid: int) -> int:
        return self.seqs[sid].length

    def stats(self) -> dict:
        return {"num_blocks": self.num_blocks, "free_blocks": len(self.free), "cached_blocks": len(self.lru),
                "used_blocks": self.num_blocks - len(self.free) - len(self.lru), "num_sequences": len(self.seqs),
                "tokens": sum(s.length for s in self.seqs.values()),
                "table_entries": sum(len(s.table) for s in self.seqs.values()),
                "prefix_queries": self.queries, "prefix_hits": self.hits, "evictions": self.evictions,
                "cow_copies": self.copies, "allocations": self.allocations}
