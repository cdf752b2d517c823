"""Drive the oracle through a whole decode-step workload -- TEST INFRASTRUCTURE.

Steps, mirroring what a serving engine does for one decode iteration after
its prompts are cached:
  1. cache every prompt token's K/V into its slot (the oracle's own write),
  2. copy the blocks the copy-on-write plan lists,
  3. cache the token each sequence appends,
  4. decode attention for each sequence's query over its whole context.
All inputs come from ``workloads``; slots/tables/pairs from ``oracle.paging``.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

import workloads
from . import HostPool
from .paging import plan


class OracleRun:
    def __init__(self, wl, prompts: Optional[Sequence[int]] = None, scales=None, prompt_kv=None,
                 free_order=None, threads: int = 1):
        """prompts: restrict the prompt writes to these prompts (sampled checks);
        scales: precomputed (k_scale, v_scale) for fp8 pools;
        prompt_kv: optional dict prompt -> (k, v) already drawn;
        free_order: override the workload's free-list order (placement tests);
        threads: host threads for the prompt writes (each prompt's tokens go
        to slots no other prompt owns, so the writes are independent)."""
        self.wl = wl
        order = workloads.free_list_order(wl) if free_order is None else free_order
        self.plan = plan(wl, order)
        ks, vs = scales if scales is not None else workloads.fp8_scales(wl, threads=max(threads, 8))
        self.k_scale, self.v_scale = ks, vs
        hs = workloads.fp8_head_scales(wl) if wl.head_scales else None
        self.head_scales = hs
        self.pool = HostPool(wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim, wl.kv_dtype, ks, vs,
                             head_scales=hs)
        todo = [p for p in (range(wl.num_prompts) if prompts is None else prompts) if wl.prompt_lens[p] > 0]

        def write(p):
            k, v = prompt_kv[p] if prompt_kv is not None and p in prompt_kv else workloads.prompt_kv(wl, p)
            self.pool.reshape_and_cache(k, v, wl.src_dtype, self.plan["prompt_slots"][p])

        if threads > 1 and len(todo) > 1:
            from concurrent.futures import ThreadPoolExecutor
            with ThreadPoolExecutor(min(threads, len(todo))) as ex:
                list(ex.map(write, todo))
        else:
            for p in todo:
                write(p)
        self.pool.copy_blocks(self.plan["pairs"])
        kn, vn = workloads.new_kv(wl)
        slots = self.plan["new_slots"]
        if prompts is not None:
            keep = np.isin(np.repeat(np.asarray(wl.parent), wl.q_lens), np.asarray(list(prompts)))
            slots = np.where(keep, slots, -1)
        self.pool.reshape_and_cache(kn, vn, wl.src_dtype, slots)
        self.q = workloads.q_values(wl)

    @property
    def tables(self) -> np.ndarray:
        return self.plan["tables"]

    def decode(self, seqs: Optional[Sequence[int]] = None) -> np.ndarray:
        wl = self.wl
        return self.pool.decode(self.q, wl.q_dtype, self.tables, wl.context_lens, wl.scale, wl.num_q_heads, seqs)

    def decode_parallel(self, threads: int) -> np.ndarray:
        """decode() of every sequence, the sequences dealt (longest first) to
        `threads` host threads; each thread's call computes its own rows."""
        wl = self.wl
        n = wl.context_lens
        order = sorted(range(wl.num_seqs), key=lambda s: -int(n[s]))
        parts = [p for p in (order[i::threads] for i in range(max(1, threads))) if p]
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(len(parts)) as ex:
            outs = list(ex.map(self.decode, parts))
        out = outs[0]
        for part, o in zip(parts[1:], outs[1:]):
            out[part] = o[part]
        return out

    def prefill(self, seqs: Optional[Sequence[int]] = None) -> np.ndarray:
        """Causal attention of every sequence's new tokens ([total_q][Hq][D]);
        with `seqs`, only those sequences' rows are computed (others NaN)."""
        wl = self.wl
        qs = wl.query_start
        if seqs is None:
            return self.pool.prefill(self.q, wl.q_dtype, self.tables, wl.context_lens, qs, wl.scale, wl.num_q_heads)
        sel = sorted(seqs)
        sub_qs = np.concatenate([[0], np.cumsum([qs[s + 1] - qs[s] for s in sel])]).astype(np.int32)
        rows = np.concatenate([np.arange(qs[s], qs[s + 1]) for s in sel])
        q = self.q[torch.as_tensor(rows, dtype=torch.long)].contiguous()
        got = self.pool.prefill(q, wl.q_dtype, self.tables[sel], wl.context_lens[sel], sub_qs, wl.scale,
                                wl.num_q_heads)
        out = np.full((wl.total_q, wl.num_q_heads, wl.head_dim), np.nan)
        out[rows] = got
        return out

    def prefill_rows(self, s: int, a: int, b: int) -> np.ndarray:
        """Rows a..b-1 of sequence s's new tokens ([b - a][Hq][D]).  Row i
        sits at position n - m + i and sees only the tokens up to it, so the
        rows are those of a call whose context ends at row b - 1."""
        wl = self.wl
        qs = wl.query_start
        n, m = int(wl.context_lens[s]), int(qs[s + 1] - qs[s])
        assert 0 <= a < b <= m
        q = self.q[int(qs[s]) + a:int(qs[s]) + b].contiguous()
        ctx = np.array([n - m + b], dtype=np.int32)
        return self.pool.prefill(q, wl.q_dtype, self.tables[s:s + 1], ctx, np.array([0, b - a], dtype=np.int32),
                                 wl.scale, wl.num_q_heads)


def tolerance(kv_dtype: str):
    """(atol, rtol) of the elementwise bound |gpu - oracle| <= atol + rtol*|oracle|."""
    return (2e-3, 5e-2) if kv_dtype == "fp8e4m3" else (2e-3, 1e-2)


def check_close(got: np.ndarray, want: np.ndarray, kv_dtype: str) -> None:
    atol, rtol = tolerance(kv_dtype)
    got = np.asarray(got, dtype=np.float64)
    bad = ~(np.abs(got - want) <= atol + rtol * np.abs(want))
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{int(bad.sum())} of {bad.size} elements out of tolerance; first {idx.tolist()}: "
                             f"got {got[tuple(idx.T)]}, want {want[tuple(idx.T)]}")
