"""Trace-driven accounting of the host block manager (no GPU work).

Replays request traces through the library's native BlockManager and
reports what the pages use to argue for paging:

  * utilisation: stored tokens over reserved slots, paged (whole blocks of
    each live sequence) against a contiguous allocator that reserves every
    request's maximum length up front ("vLLM 与 KV Cache", the memory problem
    and how-it-works; "vLLM — 把操作系统的分页搬进 GPU KV cache", what it is:
    utilisation figures);
  * parallel sampling: blocks held by n candidates sharing one prompt against
    n private copies ("vLLM — 把操作系统的分页搬进 GPU KV cache", case 2);
  * prefix caching: prompt tokens whose KV is found in the cache, blocks
    evicted under pool pressure ("vLLM KV Cache 实现机制" §4.2-4.3);
  * the manager's own speed: batched decode-step slot reservations per
    second.

Traces are plain data (prompt/output lengths, optional token ids); the seeded
generators live beside the other synthetic inputs.
"""
from __future__ import annotations

import time
from typing import Optional, Sequence

import numpy as np

from .block_manager import BlockManager, PoolExhausted


def _blocks(n: int, bs: int) -> int:
    return -(-int(n) // bs)


def utilisation(prompt_lens: Sequence[int], output_lens: Sequence[int], max_new_tokens: int,
                block_size: int = 16) -> dict:
    """Admit every request, decode one token per live request per step until
    each has produced its output, freeing finished requests.  At each step
    the paged pool holds (used blocks) * block_size slots and a contiguous
    allocator would hold sum(prompt + max_new_tokens) over live requests;
    both are compared with the tokens actually stored.  Ratios are
    step-weighted sums: sum(tokens) / sum(slots)."""
    bs = block_size
    p = np.asarray(prompt_lens, dtype=np.int64)
    o = np.asarray(output_lens, dtype=np.int64)
    need = int(sum(_blocks(a + b, bs) for a, b in zip(p, o)))
    m = BlockManager(need, bs)
    for i, n in enumerate(p):
        m.add_sequence(i, int(n))
    live = list(range(len(p)))
    done = np.zeros(len(p), dtype=np.int64)
    tok_sum = paged_sum = contig_sum = 0
    peak_used = 0
    worst_waste = 0
    steps = 0
    while live:
        st = m.stats()
        tok_sum += st["tokens"]
        paged_sum += st["used_blocks"] * bs
        contig_sum += int(sum(p[i] + max_new_tokens for i in live))
        peak_used = max(peak_used, st["used_blocks"])
        worst_waste = max(worst_waste, max(m.waste(i) for i in live))
        m.append_batch(live)
        steps += 1
        done[live] += 1
        fin = [i for i in live if done[i] >= o[i]]
        for i in fin:
            m.free(i)
        live = [i for i in live if done[i] < o[i]]
    return {"requests": int(len(p)), "steps": steps, "block_size": bs, "max_new_tokens": int(max_new_tokens),
            "paged_utilisation": tok_sum / paged_sum, "contiguous_utilisation": tok_sum / contig_sum,
            "paged_waste_slots_per_seq_max": int(worst_waste), "peak_blocks": int(peak_used),
            "contiguous_peak_slots": int(sum(p + max_new_tokens))}


def parallel_sampling(prompt_len: int, n: int, gen_len: int, block_size: int = 16) -> dict:
    """One prompt, n candidates forked from it, gen_len decode steps.  Blocks
    held at the end against n private copies of prompt + output."""
    bs = block_size
    m = BlockManager(_blocks(prompt_len + gen_len, bs) * n + 1, bs)
    m.add_sequence("prompt", prompt_len)
    kids = [("cand", i) for i in range(n)]
    m.fork("prompt", kids)
    m.free("prompt")
    copies = 0
    for _ in range(gen_len):
        _, pairs = m.append_batch(kids)
        copies += len(pairs)
    paged = m.stats()["used_blocks"]
    private = n * _blocks(prompt_len + gen_len, bs)
    return {"prompt_len": prompt_len, "n": n, "gen_len": gen_len, "block_size": bs, "paged_blocks": paged,
            "private_blocks": private, "saving": 1.0 - paged / private, "copies": copies}


def prefix_caching(tokens: Sequence[Sequence[int]], output_lens: Sequence[int], num_blocks: int,
                   concurrency: int, block_size: int = 16) -> dict:
    """Requests arrive in order; each is added with its prompt tokens (its
    cached leading blocks are shared), produces its output tokens, and is
    freed once `concurrency` newer requests are live.  Pool pressure evicts
    cached blocks least recently used first."""
    bs = block_size
    m = BlockManager(num_blocks, bs, prefix_caching=True)
    live = []
    prompt_tokens = reused = 0
    for i, (t, out) in enumerate(zip(tokens, output_lens)):
        while True:
            try:
                _, cached = m.add_sequence_cached(i, len(t), t)
                break
            except PoolExhausted:
                if not live:
                    raise
                m.free(live.pop(0))
        prompt_tokens += len(t)
        reused += cached
        live.append(i)
        while True:
            try:
                m.append_slots(i, int(out))
                break
            except PoolExhausted:
                if len(live) == 1:
                    raise
                m.free(live.pop(0))
        if len(live) > concurrency:
            m.free(live.pop(0))
    st = m.stats()
    return {"requests": len(tokens), "num_blocks": num_blocks, "concurrency": concurrency, "block_size": bs,
            "prompt_tokens": prompt_tokens, "reused_tokens": reused, "reused_fraction": reused / prompt_tokens,
            "block_hit_rate": st["prefix_hits"] / max(st["prefix_queries"], 1), "evictions": st["evictions"],
            "prefix_queries": st["prefix_queries"], "prefix_hits": st["prefix_hits"]}


def manager_speed(num_seqs: int = 256, steps: int = 512, prompt_len: int = 512, block_size: int = 16) -> dict:
    """Batched decode-step reservations: num_seqs sequences, `steps` calls
    of one slot each (one bm_append_batch call per step, on prepared
    buffers as a serving loop would hold them)."""
    bs = block_size
    m = BlockManager(num_seqs * (_blocks(prompt_len + steps, bs) + 1), bs)
    seqs = list(range(num_seqs))
    for s in seqs:
        m.add_sequence(s, prompt_len)
    ids = m.ids(seqs)
    counts = np.ones(num_seqs, dtype=np.int32)
    slots = np.empty(num_seqs, dtype=np.int64)
    pairs = np.empty((num_seqs, 2), dtype=np.int32)
    t = time.perf_counter()
    for _ in range(steps):
        m.reserve_step(ids, counts, slots, pairs)
    dt = time.perf_counter() - t
    return {"num_seqs": num_seqs, "steps": steps, "seconds": dt, "slots_per_s": num_seqs * steps / dt,
            "us_per_step": dt / steps * 1e6}


def main(argv: Optional[Sequence[str]] = None) -> int:
    import json
    import sys
    sys.path.insert(0, ".")
    import workloads as W   # synthetic traces (run from the repository root)

    tr = W.serving_trace()
    res = {"utilisation": utilisation(tr.prompt_lens, tr.output_lens, tr.max_new_tokens, tr.block_size)}
    res["parallel_sampling"] = [parallel_sampling(P, 4, g) for P, g in ((1023, 64), (1023, 256), (256, 64),
                                                                         (4096, 64))]
    pt = W.prefix_trace()
    res["prefix_caching"] = prefix_caching(pt.tokens, pt.output_lens, num_blocks=4096, concurrency=64,
                                           block_size=pt.block_size)
    res["manager_speed"] = manager_speed()
    print(json.dumps(res, indent=1))
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
