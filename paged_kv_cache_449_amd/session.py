"""A batch of sequences decoding over one KV pool.

Host side: a BlockManager (free list, reference counts, tables, slots and
copy-on-write plan).  Device side: the pool, plus the per-step slot mapping,
copy pairs, block tables and context lengths.  A decode step enqueues, on the
current stream:
    copy_blocks(pairs)                      copy-on-write of shared blocks
    reshape_and_cache(k_new, v_new, slots)  append each sequence's new token
    paged_attention_decode(q, ...)          attend over the whole context
(the order a serving engine runs them in once the new token's K/V exist:
"vLLM 与 KV Cache", why a KV cache; "vLLM — 把操作系统的分页搬进 GPU KV cache",
core mechanisms and case 2).
"""
from __future__ import annotations

from typing import Hashable, List, Optional, Sequence

import numpy as np
import torch

from . import (KVPool, copy_blocks, paged_attention_decode, paged_attention_decode_grouped,
               paged_attention_prefill, reshape_and_cache, shared_prefix_groups)
from .block_manager import BlockManager


class DecodeSession:
    def __init__(self, pool: KVPool, manager: BlockManager, num_q_heads: int):
        if manager.num_blocks != pool.num_blocks or manager.block_size != pool.block_size:
            raise ValueError("manager and pool disagree on the block layout")
        self.pool, self.manager, self.num_q_heads = pool, manager, num_q_heads
        self.seqs: List[Hashable] = []
        self.slot_mapping: Optional[torch.Tensor] = None
        self.pairs: Optional[torch.Tensor] = None
        self.block_tables: Optional[torch.Tensor] = None
        self.context_lens: Optional[torch.Tensor] = None
        self.query_start: Optional[torch.Tensor] = None
        self.group_start: Optional[torch.Tensor] = None
        self.group_shared: Optional[torch.Tensor] = None
        self.shared_blocks = 0

    def _dev(self, a: np.ndarray) -> torch.Tensor:
        return torch.from_numpy(np.ascontiguousarray(a)).to(self.pool.device, non_blocking=False)

    def cache_prompts(self, items: Sequence) -> None:
        """items: (seq, k, v) with k/v [L][Hkv][D] (host or device); registers
        each sequence and writes its tokens with one reshape_and_cache call."""
        slots, ks, vs = [], [], []
        for seq, k, v in items:
            slots.append(self.manager.add_sequence(seq, k.shape[0]))
            ks.append(k)
            vs.append(v)
        if not ks or sum(k.shape[0] for k in ks) == 0:
            return
        k = torch.cat(ks).to(self.pool.device)
        v = torch.cat(vs).to(self.pool.device)
        reshape_and_cache(self.pool, k, v, self._dev(np.concatenate(slots)))

    def fork(self, parent: Hashable, children: Sequence[Hashable]) -> None:
        self.manager.fork(parent, children)

    def free(self, seq: Hashable) -> None:
        self.manager.free(seq)

    def prepare_step(self, seqs: Sequence[Hashable], max_blocks: Optional[int] = None,
                     counts: Optional[Sequence[int]] = None) -> None:
        """Reserve the step's new slots -- one per sequence, or counts[i] for
        sequence i -- planning copy-on-write, and upload the step's slot
        mapping, copy pairs, block tables, lengths and query row offsets."""
        self.seqs = list(seqs)
        counts = [1] * len(self.seqs) if counts is None else [int(c) for c in counts]
        slots, pairs = self.manager.append_batch(self.seqs, counts)
        self.slot_mapping = self._dev(slots)
        self.pairs = self._dev(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
        tables = self.manager.block_tables(self.seqs, max_blocks)
        lens = self.manager.context_lens(self.seqs)
        self.block_tables = self._dev(tables)
        self.context_lens = self._dev(lens)
        self.query_start = self._dev(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32))
        # groups of sequences sharing leading blocks (forked candidates), for
        # the grouped decode; at most 16 query rows per group and kv head
        group = max(1, self.num_q_heads // self.pool.num_kv_heads)
        gs, gsh = shared_prefix_groups(tables, lens, max(1, 16 // group))
        self.group_start, self.group_shared = self._dev(gs), self._dev(gsh)
        self.shared_blocks = int(gsh.sum())

    def step_multi(self, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                   out: Optional[torch.Tensor] = None, scale: Optional[float] = None) -> torch.Tensor:
        """Enqueue one multi-token step: copy-on-write copies, the cache write
        of every new token, then causal attention of the new tokens."""
        scale = (1.0 / self.pool.head_dim ** 0.5) if scale is None else scale
        copy_blocks(self.pool, self.pairs)
        reshape_and_cache(self.pool, k_new, v_new, self.slot_mapping)
        return paged_attention_prefill(self.pool, q, self.block_tables, self.context_lens, self.query_start, scale,
                                       out=out)

    def step(self, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, out: Optional[torch.Tensor] = None,
             partition_tokens: int = 0, scale: Optional[float] = None, grouped: bool = False) -> torch.Tensor:
        """Enqueue one decode step; re-running it after the same prepare_step
        rewrites the same bytes and recomputes the same outputs.  grouped:
        read each shared prefix once per group of forked sequences."""
        scale = (1.0 / self.pool.head_dim ** 0.5) if scale is None else scale
        copy_blocks(self.pool, self.pairs)
        reshape_and_cache(self.pool, k_new, v_new, self.slot_mapping)
        return self.attend(q, out=out, partition_tokens=partition_tokens, scale=scale, grouped=grouped)

    def attend(self, q: torch.Tensor, out: Optional[torch.Tensor] = None, partition_tokens: int = 0,
               scale: Optional[float] = None, grouped: bool = False) -> torch.Tensor:
        """Decode attention alone, over the prepared step's tables."""
        scale = (1.0 / self.pool.head_dim ** 0.5) if scale is None else scale
        if grouped:
            return paged_attention_decode_grouped(self.pool, q, self.block_tables, self.context_lens, scale,
                                                  self.group_start, self.group_shared, out=out)
        return paged_attention_decode(self.pool, q, self.block_tables, self.context_lens, scale, out=out,
                                      partition_tokens=partition_tokens)
