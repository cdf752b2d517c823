"""The oracle's own emulation of the KV block manager -- TEST INFRASTRUCTURE.

Written from the pages' description, independently of the library's host
manager; the tests compare the two outputs (block tables, slots, copy pairs)
for equality.

What it follows:
  * Fixed-size blocks; a block is allocated only when a token needs a slot in
    it; blocks come from a free list and may be anywhere in the pool.  Page
    "vLLM 与 KV Cache", how-it-works points 1-3; page "vLLM KV Cache 实现机制",
    §3.2 step 1 (allocation from the free pool).
  * Block record with a reference count, shared by several sequences.  Page
    "vLLM KV Cache 实现机制", §3.1 data structures; page "vLLM — 把操作系统的分页
    搬进 GPU KV cache", core mechanism 3 and case 2 (n candidates share the
    prompt's blocks with ref_count n; writing into a shared block first copies
    it).
  * Slot of token position pos: offset pos mod B inside the physical block that
    the table maps logical block floor(pos / B) to.  Same page 3, core
    mechanisms (table lookup then offset).

Procedure (the harness's fixed choice where the pages leave an order open):
  1. Prompts are cached in prompt order; each token position that starts a new
     logical block takes the next block from the front of the free list.
  2. Every candidate of a prompt starts with a copy of the prompt's table; each
     prompt block's reference count is the number of candidates.
  3. The step appends each sequence's new tokens, in sequence order.  If
     the position starts a new logical block a fresh block is taken.  Else if
     the last block is shared (count > 1) a fresh block is taken, the pair
     (shared, fresh) is recorded for copying, the shared count drops by one and
     the candidate's table points at the fresh block.  The last candidate to
     write finds the count at 1 and writes in place.
"""
from __future__ import annotations

import collections
from typing import Dict, List

import numpy as np


class PoolExhausted(RuntimeError):
    pass


class PagingEmulator:
    def __init__(self, free_order, block_size: int):
        self.free = collections.deque(int(b) for b in free_order)
        self.block_size = block_size
        self.refcount: Dict[int, int] = {}

    def take(self) -> int:
        if not self.free:
            raise PoolExhausted("no free block left")
        b = self.free.popleft()
        self.refcount[b] = 1
        return b

    def give_back(self, b: int) -> None:
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            del self.refcount[b]
            self.free.append(b)

    def slot(self, table: List[int], pos: int) -> int:
        return table[pos // self.block_size] * self.block_size + pos % self.block_size


def plan(wl, free_order) -> dict:
    """Emulate the block manager for a workload.

    Returns a dict with
      prompt_slots: list over prompts of int64 arrays (slot of each cached token)
      tables:       int32 [S][max_blocks], -1 where unused
      new_slots:    int64 [total_q], slots of the tokens the sequences append (sequence order)
      pairs:        int32 [P][2] (src, dst) blocks to copy before the append
      refcount:     dict block -> count after the step
      free_left:    number of blocks still free
    """
    bs = wl.block_size
    em = PagingEmulator(free_order, bs)
    prompt_tables: List[List[int]] = []
    prompt_slots = []
    for L in wl.prompt_lens:
        table: List[int] = []
        slots = np.empty(L, dtype=np.int64)
        for pos in range(L):
            if pos % bs == 0:
                table.append(em.take())
            slots[pos] = em.slot(table, pos)
        prompt_tables.append(table)
        prompt_slots.append(slots)

    # fork: candidates share the prompt's blocks
    seq_tables = [list(prompt_tables[p]) for p in wl.parent]
    ncand = collections.Counter(wl.parent)
    for p, table in enumerate(prompt_tables):
        for b in table:
            em.refcount[b] = ncand[p]
        if ncand[p] == 0:
            for b in table:
                em.give_back(b)

    qn = wl.q_lens
    new_slots = np.empty(int(qn.sum()), dtype=np.int64)
    pairs = []
    i = 0
    for s, p in enumerate(wl.parent):
        table = seq_tables[s]
        for k in range(int(qn[s])):
            pos = wl.prompt_lens[p] + k
            if pos % bs == 0:
                table.append(em.take())
            else:
                last = table[-1]
                if em.refcount[last] > 1:
                    fresh = em.take()
                    pairs.append((last, fresh))
                    em.refcount[last] -= 1
                    table[-1] = fresh
            new_slots[i] = em.slot(table, pos)
            i += 1

    max_blocks = max(len(t) for t in seq_tables)
    tables = np.full((wl.num_seqs, max(max_blocks, 1)), -1, dtype=np.int32)
    for s, t in enumerate(seq_tables):
        tables[s, :len(t)] = t
    return {
        "prompt_slots": prompt_slots,
        "tables": tables,
        "new_slots": new_slots,
        "pairs": np.asarray(pairs, dtype=np.int32).reshape(-1, 2),
        "refcount": dict(em.refcount),
        "free_left": len(em.free),
    }


def internal_waste(context_lens, block_size: int) -> int:
    """Unused token slots in the last block of every sequence (tokens held in
    allocated blocks minus tokens stored)."""
    return int(sum(-(-int(n) // block_size) * block_size - int(n) for n in context_lens))
