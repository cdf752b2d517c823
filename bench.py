#!/usr/bin/env python
"""Paged decode attention benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one decode iteration of the whole hot path for a batch resident in
HBM: copy_blocks (copy-on-write pairs, none for workloads without sharing),
reshape_and_cache (the new token of every sequence) and paged_attention_decode.
Prints one JSON line.  `value` is KV bytes read per step / wall time per step
(GB/s), from K steps run back to back between two synchronisations; `roofline`
is the decode kernel's algorithmic bytes over its own duration, from HIP events
around each launch in K further steps, against the MI355X HBM peak;
`cpu_baseline` is the fp64 CPU oracle timed on a bounded sample of the same
workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

import workloads as W

METRIC = "paged decode attention: achieved KV HBM GB/s (% of peak) + µs/step, batch 256"
METRIC_MULTI = "paged multi-token causal attention: achieved TFLOP/s or KV GB/s (roofline bound) + µs/step"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0   # dense bf16/f16 matrix cores (fp8 KV is widened to bf16/f16)
DEFAULT_WORKLOAD = "c3_llama7b_bf16_bs16"


def get_workload(name: str) -> W.Workload:
    allw = {**W.full_configs(), **W.small_configs(), **W.multi_token_configs(), **W.small_multi_token_configs(),
            **W.variant_configs(), **W.small_variant_configs()}
    if name not in allw:
        raise SystemExit(f"unknown workload {name}; choose from {sorted(allw)}")
    return allw[name]


def build_session(wl: W.Workload, device, prompt_batch: int = 16, free_order=None):
    """Pool + block manager + cached prompts + one planned step for a workload.
    Returns (session, q, k_new, v_new) with the step's inputs on the device."""
    import paged_kv_cache_449_amd as pk
    from paged_kv_cache_449_amd.session import DecodeSession

    ks, vs = W.fp8_scales(wl)
    pool = pk.KVPool(wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim, W.TORCH_DTYPE[wl.kv_dtype],
                     device, ks, vs)
    if wl.head_scales:
        pk.kv_pool_set_head_scales(pool, *W.fp8_head_scales(wl))
    # every slot starts as all-ones bytes (NaN in every KV dtype)
    pool.k_cache.view(torch.uint8).fill_(W.POISON_BYTE)
    pool.v_cache.view(torch.uint8).fill_(W.POISON_BYTE)
    mgr = pk.BlockManager(wl.num_blocks, wl.block_size,
                          W.free_list_order(wl) if free_order is None else free_order)
    sess = DecodeSession(pool, mgr, wl.num_q_heads)
    for b0 in range(0, wl.num_prompts, prompt_batch):
        ps = list(range(b0, min(b0 + prompt_batch, wl.num_prompts)))
        kvs = W.all_prompt_kv(wl, ps)
        sess.cache_prompts([(("p", p), k, v) for p, (k, v) in zip(ps, kvs)])
    children = {}
    for s, p in enumerate(wl.parent):
        children.setdefault(p, []).append(("s", s))
    for p in range(wl.num_prompts):
        sess.fork(("p", p), children.get(p, []))
        sess.free(("p", p))
    sess.prepare_step([("s", s) for s in range(wl.num_seqs)], counts=wl.q_lens.tolist())
    q = W.q_values(wl).to(device)
    kn, vn = W.new_kv(wl)
    torch.cuda.synchronize(device)
    return sess, q, kn.to(device), vn.to(device)


def decode_bytes(wl: W.Workload) -> dict:
    """Algorithmic bytes of one decode launch: every cached token's K and V
    row of every kv head (2 * Hkv * D * elem bytes per token), q and out, the
    table entries of the blocks in use and the lengths."""
    n = wl.context_lens.astype(np.int64)
    eb = W.ELEM_BYTES[wl.kv_dtype]
    qb = W.ELEM_BYTES[wl.q_dtype]
    kv = int(n.sum()) * 2 * wl.num_kv_heads * wl.head_dim * eb
    qo = 2 * wl.num_seqs * wl.num_q_heads * wl.head_dim * qb
    tables = int((-(-n // wl.block_size)).sum()) * 4 + wl.num_seqs * 4
    return {"kv": kv, "total": kv + qo + tables, "tokens": int(n.sum())}


def prefill_cost(wl: W.Workload) -> dict:
    """Algorithmic work of one multi-token launch.  flops: 4 * D per
    (query row, query head, visible token) -- QK^T and PV, 2 * D each --
    with row i of a sequence seeing n - m + i + 1 tokens.  bytes: every cached
    token's K and V row of every kv head once, q and out, the table entries in
    use, the lengths and the row offsets."""
    n = wl.context_lens.astype(np.int64)
    m = wl.q_lens.astype(np.int64)
    pairs = int((m * (n - m) + m * (m + 1) // 2).sum())
    flops = 4 * wl.head_dim * wl.num_q_heads * pairs
    kv = int(n.sum()) * 2 * wl.num_kv_heads * wl.head_dim * W.ELEM_BYTES[wl.kv_dtype]
    qo = 2 * wl.total_q * wl.num_q_heads * wl.head_dim * W.ELEM_BYTES[wl.q_dtype]
    tables = int((-(-n // wl.block_size)).sum()) * 4 + wl.num_seqs * 4 + (wl.num_seqs + 1) * 4
    return {"flops": flops, "kv": kv, "total": kv + qo + tables, "tokens": int(n.sum()), "row_token_pairs": pairs}


def cpu_baseline_prefill(wl: W.Workload, target_s: float = 12.0):
    """The fp64 oracle on one host core over the first sequences of a
    multi-token workload, sized to about target_s seconds, in the unit of the
    workload's roofline bound; then the same sample on the host's cores.
    Returns (one core, all cores)."""
    from oracle.run import OracleRun

    n = wl.context_lens.astype(np.int64)
    m = wl.q_lens.astype(np.int64)
    pairs = m * (n - m) + m * (m + 1) // 2
    run = OracleRun(wl)
    t = time.perf_counter()
    run.prefill_rows(0, 0, min(int(m[0]), 4)) if m[0] > 0 else None
    probe_pairs = sum(int(n[0] - m[0]) + i + 1 for i in range(min(int(m[0]), 4)))
    rate = probe_pairs / max(time.perf_counter() - t, 1e-6)
    k = int(np.searchsorted(np.cumsum(pairs), rate * target_s)) + 1
    k = max(1, min(k, wl.num_seqs))
    t = time.perf_counter()
    run.prefill(list(range(k)))
    dt = time.perf_counter() - t
    cost = prefill_cost(wl)
    done = int(pairs[:k].sum())
    if cost["flops"] / (MFMA_PEAK_TFLOPS * 1e12) >= cost["total"] / (HBM_PEAK_GBS * 1e9):
        value, unit = 4 * wl.head_dim * wl.num_q_heads * done / dt / 1e12, "TFLOP/s"
    else:
        toks = int(n[:k].sum())
        value, unit = toks * 2 * wl.num_kv_heads * wl.head_dim * W.ELEM_BYTES[wl.kv_dtype] / dt / 1e9, "GB/s"
    res = {"value": round(value, 6), "unit": unit, "cores": 1, "kind": "oracle",
           "sample": f"sequences 0..{k - 1} of {wl.num_seqs} ({done} of {int(pairs.sum())} (row, token) pairs), "
                     f"{dt:.1f} s single-threaded fp64"}
    # the same sample on the host's cores: sequences dealt to threads, one
    # unchanged oracle call per thread
    from concurrent.futures import ThreadPoolExecutor
    threads = host_threads()
    order = sorted(range(k), key=lambda s: -int(pairs[s]))
    parts = [p for p in (order[i::threads] for i in range(threads)) if p]
    t = time.perf_counter()
    with ThreadPoolExecutor(len(parts)) as ex:
        list(ex.map(run.prefill, parts))
    dtp = time.perf_counter() - t
    par = {"value": round(value * dt / dtp, 6), "unit": unit, "cores": len(parts), "kind": "oracle",
           "sample": f"the single-core sample ({k} sequences), sequences dealt to {len(parts)} threads, "
                     f"{dtp:.2f} s fp64"}
    return res, par


def unique_bytes(wl: W.Workload, sess) -> dict:
    """HBM lower bound of one decode when sequences share blocks: every
    physical block read once, up to the furthest token any sequence uses in
    it, plus q, out, the table entries and the lengths."""
    return _unique_from_tables(wl, sess.block_tables.cpu().numpy())


def _unique_from_tables(wl: W.Workload, tables: np.ndarray) -> dict:
    n = wl.context_lens.astype(np.int64)
    bs = wl.block_size
    used = {}
    for s in range(tables.shape[0]):
        for i in range(int(-(-n[s] // bs))):
            blk = int(tables[s, i])
            used[blk] = max(used.get(blk, 0), int(min(bs, n[s] - i * bs)))
    tokens = sum(used.values())
    base = decode_bytes(wl)
    kv = tokens * 2 * wl.num_kv_heads * wl.head_dim * W.ELEM_BYTES[wl.kv_dtype]
    return {"kv": kv, "total": base["total"] - base["kv"] + kv, "tokens": tokens}


def grouped_bytes(wl: W.Workload, sess) -> dict:
    """Algorithmic bytes of one grouped decode: each group's shared prefix
    (whole blocks, as the library cuts it) once per kv head, every
    sequence's remaining tokens, q and out, and the table entries read."""
    return _grouped_from_tables(wl, sess.block_tables.cpu().numpy())


def _grouped_from_tables(wl: W.Workload, tables: np.ndarray) -> dict:
    from paged_kv_cache_449_amd import shared_prefix_groups
    n = wl.context_lens.astype(np.int64)
    bs = wl.block_size
    limit = max(1, 16 // wl.group)
    gs, gsh = shared_prefix_groups(tables, n, limit)
    shared = np.zeros_like(n)
    unique_tokens = 0
    for g in range(gsh.shape[0]):
        a, b = int(gs[g]), min(int(gs[g + 1]), int(gs[g]) + limit)
        sh = (min(int(gsh[g]) * bs, int(n[a:b].min())) // bs) * bs if b > a else 0
        shared[a:b] = sh
        unique_tokens += sh
    unique_tokens += int((n - shared).sum())
    per_tok = 2 * wl.num_kv_heads * wl.head_dim * W.ELEM_BYTES[wl.kv_dtype]
    qb = W.ELEM_BYTES[wl.q_dtype]
    kv = unique_tokens * per_tok
    qo = 2 * wl.num_seqs * wl.num_q_heads * wl.head_dim * qb
    tables = int((-(-n // bs)).sum()) * 4 + wl.num_seqs * 4
    return {"kv": kv, "total": kv + qo + tables, "tokens": unique_tokens}


def cpu_baseline(wl: W.Workload, target_s: float = 12.0):
    """The fp64 oracle on one host core over the first sequences of the
    workload, sized to about target_s seconds of CPU work.  Returns the
    result, the oracle run and the sampled sequences."""
    from oracle.run import OracleRun

    n = wl.context_lens.astype(np.int64)
    per_tok = 2 * wl.num_kv_heads * wl.head_dim * W.ELEM_BYTES[wl.kv_dtype]
    # calibrate on a few sequences, then size the sample
    probe = list(range(min(4, wl.num_seqs)))
    prompts = sorted({wl.parent[s] for s in probe})
    run = OracleRun(wl, prompts=prompts)
    t = time.perf_counter()
    run.decode(probe)
    dt = time.perf_counter() - t
    rate = float(n[probe].sum()) / max(dt, 1e-6)     # tokens per second
    want = rate * target_s
    k = int(np.searchsorted(np.cumsum(n), want)) + 1
    k = max(1, min(k, wl.num_seqs))
    seqs = list(range(k))
    prompts = sorted({wl.parent[s] for s in seqs})
    run = OracleRun(wl, prompts=prompts, scales=(run.k_scale, run.v_scale))
    t = time.perf_counter()
    run.decode(seqs)
    dt = time.perf_counter() - t
    toks = int(n[seqs].sum())
    return {"value": round(toks * per_tok / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"sequences 0..{k - 1} of {wl.num_seqs} ({toks} of {int(n.sum())} cached tokens), "
                      f"{dt:.1f} s single-threaded fp64"}, run, seqs


# Host threads of the all-cores oracle leg: at most the CPU share one GPU's
# job is given on the measurement host (16 cores), whatever the machine has.
HOST_THREAD_CAP = 16


def host_threads(limit: int = HOST_THREAD_CAP) -> int:
    """Host cores this process may use, at most `limit`."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, limit))


def host_facts() -> dict:
    """What the oracle timings ran on: the machine's logical CPU count, the
    cores this process may use, the thread cap of the all-cores leg, and the
    CPU model."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"os_cpu_count": os.cpu_count(), "usable_cores": usable, "thread_cap": HOST_THREAD_CAP,
            "cpu_model": model}


def cpu_baseline_parallel(wl: W.Workload, run, seqs, threads: int) -> dict:
    """The same oracle on the same sample, its sequences dealt (longest first)
    to `threads` host threads; each thread's call runs the unchanged oracle on
    its own sequences."""
    from concurrent.futures import ThreadPoolExecutor

    n = wl.context_lens.astype(np.int64)
    per_tok = 2 * wl.num_kv_heads * wl.head_dim * W.ELEM_BYTES[wl.kv_dtype]
    order = sorted(seqs, key=lambda s: -int(n[s]))
    parts = [order[i::threads] for i in range(threads)]
    parts = [p for p in parts if p]
    t = time.perf_counter()
    with ThreadPoolExecutor(len(parts)) as ex:
        list(ex.map(run.decode, parts))
    dt = time.perf_counter() - t
    toks = int(n[seqs].sum())
    return {"value": round(toks * per_tok / dt / 1e9, 4), "unit": "GB/s", "cores": len(parts), "kind": "oracle",
            "sample": f"the single-core sample ({len(seqs)} sequences, {toks} cached tokens), sequences dealt to "
                      f"{len(parts)} threads, {dt:.2f} s fp64"}


_CSRC = "paged_kv_cache_449_amd/csrc/"
KERNEL_SOURCES = {
    "decode": tuple(_CSRC + f for f in ("common.h", "decode_plan.h", "decode_kernel.h", "decode_mfma.h",
                                        "decode_items.h", "decode.hip", "decode_grouped.h", "decode_grouped.hip")),
    "prefill": tuple(_CSRC + f for f in ("common.h", "decode_plan.h", "decode_kernel.h", "decode_mfma.h",
                                         "decode_items.h", "prefill_kernel.h", "prefill.hip")),
}
_PROFILES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")
TRAFFIC_FILES = {"decode": os.path.join(_PROFILES, "decode_traffic.json"),
                 "prefill": os.path.join(_PROFILES, "prefill_traffic.json")}


def kernel_source_digest(kind: str = "decode") -> str:
    """sha256 over a kernel's sources: counters taken on other sources do not
    describe this kernel."""
    import hashlib
    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(root, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(wl_name: str, kind: str = "decode"):
    """HBM bytes per launch of the decode or multi-token kernel from the
    committed rocprofv3 counter summary, if it was taken on this workload and
    on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILES[kind]) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get("workloads", {}).get(wl_name)
    if not entry or rec.get("kernel_source_sha256") != kernel_source_digest(kind):
        return None
    return entry.get("traffic_bytes_per_launch")


def achievable_read(dev, gib: int = 2, tile_bytes: int = 4096, reps: int = 5) -> dict:
    """HBM read rate of a plain streaming kernel of the decode kernel's load
    form (kv_stream_read): gib GiB of tile_bytes tiles in a seeded random
    order, mean of reps launches timed with HIP events."""
    import paged_kv_cache_449_amd as pk
    buf = torch.empty(gib << 30, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    n = buf.numel() // tile_bytes
    tiles = torch.randperm(n, generator=torch.Generator().manual_seed(449)).to(torch.int32).to(dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(2):
        pk.kv_stream_read(buf, tile_bytes, tiles, sink)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, e in ev:
        a.record()
        pk.kv_stream_read(buf, tile_bytes, tiles, sink)
        e.record()
    torch.cuda.synchronize(dev)
    us = float(np.mean([a.elapsed_time(e) for a, e in ev])) * 1e3
    del buf
    return {"kernel": "kv_stream_read", "value": round(n * tile_bytes / us / 1e3, 1), "unit": "GB/s",
            "tile_bytes": tile_bytes, "bytes": n * tile_bytes, "order": "random", "us": round(us, 1)}


def write_kernels(wl: W.Workload, sess, pool, wevs) -> dict:
    """The step's two writes from the HIP events around them: copy_blocks
    (each pair reads and writes one block of K and one of V) and
    reshape_and_cache (each new token's K and V rows read in the source dtype,
    written in the pool dtype, plus its slot).  Median over the steps."""
    P = int(sess.pairs.shape[0])
    T = int(sess.slot_mapping.shape[0])
    row = wl.num_kv_heads * wl.head_dim
    res = {}
    if P > 0:
        us = float(np.median([w[0].elapsed_time(w[1]) for w in wevs])) * 1e3
        nbytes = P * 2 * 2 * pool.block_bytes
        res["copy_blocks"] = {"pairs": P, "us": round(us, 2), "bytes": nbytes, "GBs": round(nbytes / us / 1e3, 1)}
    us = float(np.median([w[1].elapsed_time(w[2]) for w in wevs])) * 1e3
    nbytes = T * (2 * row * (W.ELEM_BYTES[wl.src_dtype] + W.ELEM_BYTES[wl.kv_dtype]) + 8)
    res["reshape_and_cache"] = {"tokens": T, "us": round(us, 2), "bytes": nbytes, "GBs": round(nbytes / us / 1e3, 1)}
    return res


def swap_measurement(pool, n: int, reps: int = 5) -> dict:
    """swap_blocks of n pool blocks (K and V) to pinned host memory and back
    into the same blocks (their contents are unchanged), HIP-event timed."""
    import paged_kv_cache_449_amd as pk
    dev = pool.device
    area = pk.HostSwapArea(pool, n)
    ids = torch.arange(n, dtype=torch.int32, device=dev)
    pairs = torch.stack([ids, ids], 1).contiguous()
    nbytes = 2 * n * pool.block_bytes
    res = {"blocks": n, "bytes": nbytes}
    for name, direction in (("out", pk.KV_SWAP_OUT), ("in", pk.KV_SWAP_IN)):
        pk.swap_blocks(pool, area, pairs, direction)
        torch.cuda.synchronize(dev)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in evs:
            a.record()
            pk.swap_blocks(pool, area, pairs, direction)
            b.record()
        torch.cuda.synchronize(dev)
        us = float(np.median([a.elapsed_time(b) for a, b in evs])) * 1e3
        res[f"{name}_us"] = round(us, 1)
        res[f"{name}_GBs"] = round(nbytes / us / 1e3, 2)
    return res


def multi_token_result(wl: W.Workload, args, kern_ms: np.ndarray, step_ms: float) -> dict:
    """JSON line of a multi-token workload: the roofline is the matrix cores
    when the launch's flops take longer at peak than its bytes, else HBM."""
    c = prefill_cost(wl)
    kern_s = float(kern_ms.mean()) / 1e3
    mfma = c["flops"] / (MFMA_PEAK_TFLOPS * 1e12) >= c["total"] / (HBM_PEAK_GBS * 1e9)
    if mfma:
        achieved, peak, unit = c["flops"] / kern_s / 1e12, MFMA_PEAK_TFLOPS, "TFLOP/s"
        value = c["flops"] / (step_ms / 1e3) / 1e12
    else:
        achieved, peak, unit = c["total"] / kern_s / 1e9, HBM_PEAK_GBS, "GB/s"
        value = c["kv"] / (step_ms / 1e3) / 1e9
    print(f"[bench] prefill kernel mean {kern_ms.mean() * 1e3:.1f} us; step {step_ms * 1e3:.1f} us; "
          f"{c['flops'] / kern_s / 1e12:.1f} TFLOP/s, {c['total'] / kern_s / 1e9:.1f} GB/s", file=sys.stderr,
          flush=True)
    return {
        "metric": METRIC_MULTI,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "us_per_step": round(step_ms * 1e3, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "num_seqs": wl.num_seqs, "total_q": wl.total_q,
                   "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
                   "block_size": wl.block_size, "kv_dtype": wl.kv_dtype, "q_dtype": wl.q_dtype,
                   "cached_tokens": c["tokens"], "row_token_pairs": c["row_token_pairs"],
                   "flops_per_launch": c["flops"], "bytes_per_launch": c["total"], "placement": args.placement,
                   "flush": args.flush, "graph": args.graph, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma" if mfma else "hbm", "achieved": round(achieved, 2), "peak": peak,
                     "unit": unit, "frac": round(achieved / peak, 4), "traffic": measured_traffic(wl.name, "prefill"),
                     "kernel": "paged_prefill_kernel", "kernel_us": round(float(kern_ms.mean()) * 1e3, 2),
                     "tflops": round(c["flops"] / kern_s / 1e12, 2),
                     "kv_gbs": round(c["total"] / kern_s / 1e9, 1)},
    }


def block_manager_result(steps: int = 512, num_seqs: int = 256) -> dict:
    """Host block manager: batched decode-step slot reservations per second
    through the library, with the oracle's allocator model timed on the same
    loop, and the simulator's accounting on the synthetic traces."""
    from paged_kv_cache_449_amd import simulate
    from oracle.allocator import AllocatorModel

    speed = simulate.manager_speed(num_seqs=num_seqs, steps=steps)
    bs, P = 16, 512
    m = AllocatorModel(num_seqs * (-(-(P + steps) // bs) + 1), bs)
    for s in range(num_seqs):
        m.add_sequence(s, P)
    t = time.perf_counter()
    for _ in range(steps):
        for s in range(num_seqs):
            m.append(s, 1)
    dt = time.perf_counter() - t
    tr = W.serving_trace()
    pt = W.prefix_trace()
    return {
        "metric": "host block manager: decode-step slot reservations per second (batched, 256 sequences)",
        "value": round(speed["slots_per_s"], 1), "unit": "slots/s", "n_gpus": 0, "steps": steps, "warmup": 0,
        "ms_per_step": round(speed["us_per_step"] / 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int64", "data": "synthetic",
        "config": {"workload": "block_manager_decode_steps", "num_seqs": num_seqs, "prompt_len": P,
                   "block_size": bs, "parallelism": "host"},
        "cpu_baseline": {"value": round(num_seqs * steps / dt, 1), "unit": "slots/s", "cores": 1, "kind": "oracle",
                         "sample": f"the same {steps} steps x {num_seqs} sequences through the oracle's model"},
        "simulation": {
            "utilisation": simulate.utilisation(tr.prompt_lens, tr.output_lens, tr.max_new_tokens, tr.block_size),
            "parallel_sampling": [simulate.parallel_sampling(P_, 4, g) for P_, g in ((1023, 64), (1023, 256),
                                                                                     (4096, 64))],
            "prefix_caching": simulate.prefix_caching(pt.tokens, pt.output_lens, num_blocks=4096, concurrency=64,
                                                      block_size=pt.block_size)},
    }


def _pmc_rows(csv_path: str):
    import csv
    with open(csv_path) as f:
        return sorted(csv.DictReader(f), key=lambda r: int(r["Dispatch_Id"]))


def summarise_pmc(fetch_csv: str, write_csv: str, kernel_match, calib_match=("bitwise_not", "BitwiseNot")) -> dict:
    """HBM bytes per launch from two rocprofv3 --pmc runs (FETCH_SIZE, then
    WRITE_SIZE; counter_collection.csv, KiB per dispatch).  Each counter is
    scaled by what it read for the calibration kernel of --calibrate-copy,
    which reads 1 GiB and writes 1 GiB.  kernel_match: substrings of the
    kernel names that make up one launch of the call (several kernels of one
    call are summed in dispatch order; a launch ends at the last name in
    kernel_match)."""
    out = {}
    for ctr, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _pmc_rows(path)
        cal = [float(r["Counter_Value"]) for r in rows if any(c in r["Kernel_Name"] for c in calib_match)]
        seq = [(r["Kernel_Name"], float(r["Counter_Value"])) for r in rows
               if any(k in r["Kernel_Name"] for k in kernel_match)]
        launches, cur = [], 0.0
        for name, v in seq:
            cur += v
            if kernel_match[-1] in name:
                launches.append(cur)
                cur = 0.0
        if not cal or not launches:
            raise SystemExit(f"{path}: no calibration or no {kernel_match} dispatches")
        out[ctr] = (float(np.mean(launches)), len(launches), cal[0])
    f_kib, nd, f_cal = out["FETCH_SIZE"]
    w_kib, _, w_cal = out["WRITE_SIZE"]
    fetch_scale, write_scale = 1048576.0 / f_cal, 1048576.0 / w_cal
    fb = int(round(f_kib * 1024 * fetch_scale))
    wb = int(round(w_kib * 1024 * write_scale))
    return {"kernels": list(kernel_match), "dispatches": nd, "FETCH_SIZE_KiB_per_dispatch": round(f_kib, 6),
            "WRITE_SIZE_KiB_per_dispatch": round(w_kib, 6), "calibration_FETCH_SIZE_KiB": f_cal,
            "calibration_WRITE_SIZE_KiB": w_cal, "fetch_scale": round(fetch_scale, 6),
            "write_scale": round(write_scale, 6), "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
            "traffic_bytes_per_launch": fb + wb}


def record_traffic(kind: str, key: str, entry: dict, algorithmic: int, commands) -> None:
    """Merge one workload's counter summary into profiles/<kind>_traffic.json,
    stamped with the current kernel sources' digest (entries taken on other
    sources are dropped)."""
    path = TRAFFIC_FILES[kind]
    digest = kernel_source_digest(kind)
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    if rec.get("kernel_source_sha256") != digest:
        rec = {"what": f"HBM bytes per {kind} launch from rocprofv3 counters, scaled by a plain elementwise kernel "
                       "that reads 1 GiB and writes 1 GiB (bench.py --calibrate-copy) in the same run",
               "kernel_source_sha256": digest, "kernel_sources": list(KERNEL_SOURCES[kind]), "workloads": {}}
    entry = dict(entry, algorithmic_bytes_per_launch=int(algorithmic), commands=list(commands))
    entry["traffic_over_algorithmic"] = round(entry["traffic_bytes_per_launch"] / algorithmic, 4)
    rec["workloads"][key] = entry
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps({key: entry}), flush=True)


def decode_summary(name: str, dev, steps: int, warmup: int) -> dict:
    """One more decode workload in the same run: build it, warm up, then time
    `steps` whole steps back to back (step time) and `steps` more with HIP
    events around each decode launch (kernel time), as for the main line.
    Shared blocks are counted once (the HBM lower bound)."""
    import paged_kv_cache_449_amd as pk
    name, _, pt_text = name.partition(":")   # "workload:tokens" overrides its partition size
    wl = get_workload(name)
    print(f"[bench] building {wl.name}", file=sys.stderr, flush=True)
    sess, q, kn, vn = build_session(wl, dev)
    out = torch.empty_like(q)
    pool = sess.pool
    pt = int(pt_text) if pt_text else wl.partition_tokens

    def one_step(ev=None):
        pk.copy_blocks(pool, sess.pairs)
        pk.reshape_and_cache(pool, kn, vn, sess.slot_mapping)
        if ev is None:
            pk.paged_attention_decode(pool, q, sess.block_tables, sess.context_lens, wl.scale, out=out,
                                      partition_tokens=pt)
            return
        ev[0].record()
        ws = pk.paged_attention_plan(pool, q, sess.block_tables, sess.context_lens, partition_tokens=pt)
        ev[1].record()
        pk.paged_attention_decode_planned(pool, q, sess.block_tables, sess.context_lens, wl.scale, ws, out=out,
                                          partition_tokens=pt)
        ev[2].record()

    for _ in range(warmup):
        one_step()
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for _ in range(steps):
        one_step()
    torch.cuda.synchronize(dev)
    step_us = (time.perf_counter() - t0) * 1e6 / steps
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(steps)]
    for e in evs:
        one_step(e)
    torch.cuda.synchronize(dev)
    us = np.array([b.elapsed_time(c) for a, b, c in evs]) * 1e3
    plan_us = np.array([a.elapsed_time(b) for a, b, c in evs]) * 1e3
    nb = unique_bytes(wl, sess) if sess.shared_blocks > 0 else decode_bytes(wl)
    logical = decode_bytes(wl)
    achieved = nb["total"] / (float(us.mean()) / 1e6) / 1e9
    res = {"workload": wl.name, "num_seqs": wl.num_seqs, "block_size": wl.block_size, "kv_dtype": wl.kv_dtype,
           "partition_tokens": pt, "kernel_us": round(float(us.mean()), 2),
           "kernel_us_p10_median_p90": [round(float(x), 1) for x in np.percentile(us, [10, 50, 90])],
           "us_per_step": round(step_us, 1), "bytes_per_launch": nb["total"],
           "bytes_counted": "unique (each shared block once)" if sess.shared_blocks > 0 else "algorithmic",
           "achieved": round(achieved, 1), "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
           "kv_gbs_per_step": round(nb["kv"] / (step_us / 1e6) / 1e9, 1),
           "logical_gbs": round(logical["total"] / (float(us.mean()) / 1e6) / 1e9, 1),
           "plan_us": round(float(plan_us.mean()), 2),
           "call_us": round(float((plan_us + us).mean()), 2),
           "call_frac": round(nb["total"] / (float((plan_us + us).mean()) / 1e6) / 1e9 / HBM_PEAK_GBS, 4)}
    print(f"[bench] {wl.name}: decode kernel {us.mean():.1f} us, frac {res['frac']}; plan kernel "
          f"{plan_us.mean():.1f} us, call frac {res['call_frac']}", file=sys.stderr, flush=True)
    del sess, q, kn, vn, out, pool
    torch.cuda.empty_cache()
    return res


# The batch-256 workloads of the headline metric besides the default one:
# the LLaMA-7B shape at block size 32, and parallel sampling (64 prompts x 4
# candidates sharing their prompt's blocks).
ALSO_DEFAULT = ("c3_llama7b_bf16_bs32", "c4_parallel_sampling_f16_p1023")


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one plain 1 GiB device copy before the timed steps: under rocprofv3 --pmc its "
                         "FETCH_SIZE/WRITE_SIZE give the counters' scale against bytes known to move")
    ap.add_argument("--swap-blocks", type=int, default=0,
                    help="also time swap_blocks moving this many pool blocks to pinned host memory and back "
                         "(reported under 'swap'; not part of the step)")
    ap.add_argument("--placement", choices=["shuffled", "sequential"], default="shuffled",
                    help="shuffled: blocks from a seeded random free list (the workload); sequential: "
                         "the free list in id order, so each sequence's blocks are contiguous (the "
                         "paged-vs-contiguous comparison)")
    ap.add_argument("--partition-tokens", type=int, default=None,
                    help="context split of paged_attention_decode: 0 lets the library size it, k*block_size fixes "
                         "the chunk length (default: the workload's own setting)")
    ap.add_argument("--flush", choices=["none", "read", "write"], default="none",
                    help="before every step, outside its events, read (read) or write (write) a 512 MiB buffer: "
                         "read evicts the Infinity Cache and L2 of the KV data, write also leaves dirty lines that "
                         "drain during the next kernels; ms_per_step is then the mean of the steps' own event "
                         "intervals")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step (its copy_blocks, cache write and decode launches) in a HIP graph and "
                         "time replays of it for ms_per_step; the kernel time still comes from eager steps")
    ap.add_argument("--grouped", action="store_true",
                    help="decode with paged_attention_decode_grouped: each shared prefix (forked candidates) is "
                         "read once per group")
    ap.add_argument("--block-manager", action="store_true",
                    help="host block manager only (no GPU): reservation rate, oracle beside it, trace accounting")
    ap.add_argument("--also", default=None,
                    help="comma-separated decode workloads timed after the main one and reported under 'also' "
                         "(default: the other batch-256 headline workloads when the main one is the default; "
                         "'none' for none; 'name:tokens' overrides a workload's partition size)")
    ap.add_argument("--summarise-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"), default=None,
                    help="no GPU work: turn the counter_collection.csv files of a rocprofv3 --pmc FETCH_SIZE run "
                         "and a --pmc WRITE_SIZE run of this same command line (with --calibrate-copy) into HBM "
                         "bytes per launch, and record them in profiles/<kind>_traffic.json")
    ap.add_argument("--summarise-sq", nargs="+", default=None, metavar="PMC_CSV",
                    help="print markdown rows of shader (SQ) counters per dispatch of the attention kernels, "
                         "one rocprofv3 --pmc pass per CSV, with the ratios between them")
    ap.add_argument("--summarise-l2", default=None, metavar="PMC_CSV",
                    help="no GPU work: the counter_collection.csv of a rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum run "
                         "of this same command line -> one markdown row per decode kernel (L2 hits and misses per "
                         "dispatch, hit rate, misses in bytes)")
    ap.add_argument("--summarise-trace", nargs=2, metavar=("TRACE_DIR", "BENCH_LOG"), default=None,
                    help="no GPU work: turn a rocprofv3 --kernel-trace --stats run of this same command line "
                         "(its output directory, prefix kt, and the run's stderr) into "
                         "profiles/<kind>_<workload>_kernel_trace.md")
    args = ap.parse_args(argv)
    if args.summarise_l2:
        return summarise_l2_main(args)
    if args.summarise_sq:
        return summarise_sq_main(args)
    if args.summarise_trace:
        return summarise_trace_main(args, argv)
    if args.block_manager:
        print(json.dumps(block_manager_result()), flush=True)
        return 0
    if args.summarise_pmc:
        return summarise_main(args, argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build runs the decode path on a single MI355X "
              "(sharding across GPUs is a design note only); run with --gpus 1", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2

    import paged_kv_cache_449_amd as pk

    wl = get_workload(args.workload)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    print(f"[bench] building {wl.name}", file=sys.stderr, flush=True)
    order = None if args.placement == "shuffled" else np.arange(wl.num_blocks, dtype=np.int32)
    sess, q, kn, vn = build_session(wl, dev, free_order=order)
    out = torch.empty_like(q)
    pool = sess.pool
    pt = wl.partition_tokens if args.partition_tokens is None else args.partition_tokens
    # counters taken at the workload's own split describe only that split
    traffic_key = wl.name + (":grouped" if args.grouped else "") + ("" if pt == wl.partition_tokens else f":pt{pt}")

    multi = wl.multi_token

    def one_step(ev=None, wev=None):
        if wev is not None:
            wev[0].record()
        pk.copy_blocks(pool, sess.pairs)
        if wev is not None:
            wev[1].record()
        pk.reshape_and_cache(pool, kn, vn, sess.slot_mapping)
        if wev is not None:
            wev[2].record()
        if ev is not None:
            ev[0].record()
        if multi:
            pk.paged_attention_prefill(pool, q, sess.block_tables, sess.context_lens, sess.query_start, wl.scale,
                                       out=out)
        elif args.grouped:
            pk.paged_attention_decode_grouped(pool, q, sess.block_tables, sess.context_lens, wl.scale,
                                              sess.group_start, sess.group_shared, out=out)
        elif ev is not None and len(ev) == 3:
            # the two halves of the call, so the decode kernel is timed on its
            # own: ev[0]..ev[1] the plan kernel, ev[1]..ev[2] the decode kernel
            ws = pk.paged_attention_plan(pool, q, sess.block_tables, sess.context_lens, partition_tokens=pt)
            ev[1].record()
            pk.paged_attention_decode_planned(pool, q, sess.block_tables, sess.context_lens, wl.scale, ws, out=out,
                                              partition_tokens=pt)
        else:
            pk.paged_attention_decode(pool, q, sess.block_tables, sess.context_lens, wl.scale, out=out,
                                      partition_tokens=pt)
        if ev is not None:
            ev[-1].record()

    if args.calibrate_copy:
        # an elementwise kernel that reads 1 GiB and writes 1 GiB (a plain
        # same-dtype copy may go to a DMA engine, which the counters miss)
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize(dev)
        del src, dst
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if args.flush != "none" else None

    def flush():
        if args.flush == "read":
            scratch.max()
        elif args.flush == "write":
            scratch.zero_()

    for _ in range(args.warmup):
        flush()
        one_step()
    torch.cuda.synchronize(dev)
    step = one_step
    if args.graph:
        # out and the workspace exist after the warm-up, so the captured
        # launches allocate nothing and record no memset
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            one_step()
        torch.cuda.synchronize(dev)
        step = graph.replay
        for _ in range(2):
            step()
        torch.cuda.synchronize(dev)

    # 1. The step time: K steps back to back between two synchronisations,
    #    with no event inside (each event record is a packet of its own on
    #    the queue, about 5 us apart from the kernels).  With a flush, the
    #    steps' own event intervals leave it out.
    sevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for i in range(args.steps):
        flush()
        if scratch is not None:
            sevs[i][0].record()
        step()
        if scratch is not None:
            sevs[i][1].record()
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    step_ms = wall * 1e3 / args.steps if scratch is None else float(np.mean([a.elapsed_time(b) for a, b in sevs]))

    # 2. The kernel time: K more steps with HIP events around each launch,
    #    recorded on the stream the library launches on.
    split = not (multi or args.grouped)   # flat decode: plan and decode kernels timed apart
    nev = 3 if split else 2
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(nev)) for _ in range(args.steps)]
    wevs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize(dev)
    for i in range(args.steps):
        flush()
        one_step(evs[i], wevs[i])
    torch.cuda.synchronize(dev)
    dec_ms = np.array([e[-2].elapsed_time(e[-1]) for e in evs])
    plan_ms = np.array([e[0].elapsed_time(e[1]) for e in evs]) if split else None
    writes = write_kernels(wl, sess, pool, wevs)
    if multi:
        res = multi_token_result(wl, args, dec_ms, step_ms)
        res["writes"] = writes
        res["achievable"] = achievable_read(dev)
        if res["roofline"]["unit"] == "GB/s":
            res["roofline"]["frac_of_achievable"] = round(res["roofline"]["achieved"] / res["achievable"]["value"], 4)
        if not args.no_cpu_baseline:
            print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
            res["cpu_baseline"], res["cpu_baseline_parallel"] = cpu_baseline_prefill(wl)
        print(json.dumps(res), flush=True)
        return 0
    nb = decode_bytes(wl)
    dec_mean_s = float(dec_ms.mean()) / 1e3
    logical = nb
    if args.grouped:
        nb = grouped_bytes(wl, sess)
    elif sess.shared_blocks > 0:
        # candidates read shared blocks once each; the roofline and the
        # headline rate count each block once (the HBM lower bound), so
        # cache hits cannot lift them past the peak
        nb = unique_bytes(wl, sess)
    logical_total = logical["total"]
    achieved = nb["total"] / dec_mean_s / 1e9
    print(f"[bench] decode kernel mean {dec_ms.mean() * 1e3:.1f} us (min {dec_ms.min() * 1e3:.1f}, "
          f"max {dec_ms.max() * 1e3:.1f}); step {step_ms * 1e3:.1f} us"
          + (f"; plan kernel {plan_ms.mean() * 1e3:.1f} us" if split else ""), file=sys.stderr, flush=True)

    res = {
        "metric": METRIC,
        "value": round(nb["kv"] / (step_ms / 1e3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "us_per_step": round(step_ms * 1e3, 1),
        "pct_of_hbm_peak": round(100 * nb["kv"] / (step_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "num_seqs": wl.num_seqs, "num_q_heads": wl.num_q_heads,
                   "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim, "block_size": wl.block_size,
                   "kv_dtype": wl.kv_dtype, "q_dtype": wl.q_dtype, "cached_tokens": nb["tokens"],
                   "kv_bytes_per_step": nb["kv"], "kv_bytes_logical": logical["kv"], "partition_tokens": pt,
                   "placement": args.placement,
                   "flush": args.flush, "graph": args.graph,
                   "decode": "grouped" if args.grouped else "flat",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(traffic_key),
                     "kernel": ("paged_decode_shared_kernel + paged_decode_suffix_kernel" if args.grouped
                                else "paged_decode_kernel"),
                     "kernel_us": round(float(dec_ms.mean()) * 1e3, 2),
                     "kernel_us_p10_median_p90": [round(float(x) * 1e3, 1)
                                                  for x in np.percentile(dec_ms, [10, 50, 90])],
                     "bytes_per_launch": nb["total"],
                     "logical_gbs": round(logical_total / dec_mean_s / 1e9, 1)},
    }
    if split:
        # the whole paged_attention_decode call: the plan kernel, then the
        # decode kernel (a serving step plans once for all its layers)
        call_s = float((plan_ms + dec_ms).mean()) / 1e3
        res["roofline"]["plan_kernel"] = "paged_decode_plan_kernel"
        res["roofline"]["plan_us"] = round(float(plan_ms.mean()) * 1e3, 2)
        res["roofline"]["call_us"] = round(call_s * 1e6, 2)
        res["roofline"]["call_frac"] = round(nb["total"] / call_s / 1e9 / HBM_PEAK_GBS, 4)
    if args.flush == "none" and not args.graph:
        # 3. The serving-realistic cache state: a 512 MiB write before each
        #    step (the layer's own projections write just before decode), so
        #    dirty lines drain while the decode kernel reads.
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        fevs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(nev)) for _ in range(args.steps)]
        torch.cuda.synchronize(dev)
        for i in range(args.steps):
            scratch.zero_()
            one_step(fevs[i])
        torch.cuda.synchronize(dev)
        fus = np.array([e[-2].elapsed_time(e[-1]) for e in fevs]) * 1e3
        fach = nb["total"] / (float(fus.mean()) / 1e6) / 1e9
        res["roofline"]["flush_write"] = {"what": "512 MiB written before every step, outside the events",
                                          "kernel_us": round(float(fus.mean()), 2),
                                          "achieved": round(fach, 1), "frac": round(fach / HBM_PEAK_GBS, 4)}
        del scratch
    if args.swap_blocks > 0:
        res["swap"] = swap_measurement(pool, min(args.swap_blocks, wl.num_blocks))
    res["writes"] = writes
    res["achievable"] = achievable_read(dev)
    res["roofline"]["frac_of_achievable"] = round(achieved / res["achievable"]["value"], 4)
    also = args.also
    if also is None:
        also = ",".join(ALSO_DEFAULT) if wl.name == DEFAULT_WORKLOAD and not (args.grouped or args.graph) else "none"
    if also != "none":
        del sess, q, kn, vn, out, pool
        torch.cuda.empty_cache()
        res["also"] = [decode_summary(n, dev, args.steps, args.warmup) for n in also.split(",") if n]
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        res["cpu_baseline"], run, seqs = cpu_baseline(wl)
        res["cpu_baseline_parallel"] = cpu_baseline_parallel(wl, run, seqs, host_threads())
        res["cpu_baseline"]["host"] = res["cpu_baseline_parallel"]["host"] = host_facts()
    print(json.dumps(res), flush=True)
    return 0


def summarise_main(args, argv) -> int:
    """--summarise-pmc: the counter files of one workload's two --pmc runs
    into its entry of profiles/<kind>_traffic.json."""
    wl = get_workload(args.workload)
    kind = "prefill" if wl.multi_token else "decode"
    pt = wl.partition_tokens if args.partition_tokens is None else args.partition_tokens
    key = wl.name + (":grouped" if args.grouped else "") + ("" if pt == wl.partition_tokens else f":pt{pt}")
    if wl.multi_token:
        match = ("paged_prefill",)
        algorithmic = prefill_cost(wl)["total"]
    else:
        from oracle.paging import plan
        tables = plan(wl, W.free_list_order(wl))["tables"]
        if args.grouped:
            match = ("paged_decode_shared_kernel", "paged_decode_suffix_kernel")
            algorithmic = _grouped_from_tables(wl, tables)["total"]
        else:
            match = ("paged_decode_kernel",)   # the decode kernel alone (the plan kernel is timed apart)
            shared = bool(np.any((tables[1:, 0] >= 0) & (tables[1:, 0] == tables[:-1, 0])))
            algorithmic = (_unique_from_tables(wl, tables) if shared else decode_bytes(wl))["total"]
    entry = summarise_pmc(args.summarise_pmc[0], args.summarise_pmc[1], match)
    rest = [a for a in (argv if argv is not None else sys.argv[1:])]
    i = rest.index("--summarise-pmc")
    base = " ".join(rest[:i] + rest[i + 3:])
    cmds = [f"rocprofv3 --pmc {c} --output-format csv -d <dir> -o pmc -- python3 bench.py {base} --calibrate-copy"
            for c in ("FETCH_SIZE", "WRITE_SIZE")]
    record_traffic(kind, key, entry, algorithmic, cmds)
    return 0


def summarise_sq_main(args) -> int:
    """--summarise-sq: shader counters of the attention kernels, summed over
    the GPU per dispatch and averaged over the dispatches of each pass, then
    the ratios between them.  Wave-cycle counters share one unit, so their
    ratios are shares of the waves' lifetime; the matrix-core busy cycles are
    set against 1024 SIMDs x the dispatch time at 2.4 GHz."""
    vals, durs = {}, {}
    name = None
    for path in args.summarise_sq:
        per = {}
        for r in _pmc_rows(path):
            if "paged_decode_kernel" not in r["Kernel_Name"] and "paged_prefill" not in r["Kernel_Name"]:
                continue
            name = r["Kernel_Name"].split("(")[0].replace("void ", "").replace("pkv::", "")
            d = per.setdefault(r["Dispatch_Id"], {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            durs.setdefault(path, {})[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        for c in {c for d in per.values() for c in d}:
            vals[c] = float(np.mean([d[c] for d in per.values() if c in d]))
    us = float(np.mean([u for d in durs.values() for u in d.values()]))
    wl = get_workload(args.workload)
    print(f"| {wl.name} | `{name}` | {us:.1f} | " + "; ".join(f"{c} {v:.4g}" for c, v in sorted(vals.items())) + " |")
    wc = vals.get("SQ_WAVE_CYCLES")
    out = []
    for c in ("SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS", "SQ_WAIT_ANY"):
        if wc and c in vals:
            out.append(f"{c} / SQ_WAVE_CYCLES {vals[c] / wc:.3f}")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in vals:
        out.append(f"matrix-core busy {vals['SQ_VALU_MFMA_BUSY_CYCLES'] / (1024 * us * 2400):.3f} of 1024 SIMDs")
    if "SQ_LDS_BANK_CONFLICT" in vals and vals.get("SQ_LDS_IDX_ACTIVE"):
        out.append(f"LDS bank conflicts / LDS active {vals['SQ_LDS_BANK_CONFLICT'] / vals['SQ_LDS_IDX_ACTIVE']:.3f}")
    if "SQ_INSTS_MFMA" in vals:
        for c in ("SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_LDS"):
            if c in vals:
                out.append(f"{c} per MFMA {vals[c] / vals['SQ_INSTS_MFMA']:.2f}")
    print("| | | | " + "; ".join(out) + " |")
    return 0


def summarise_l2_main(args) -> int:
    """--summarise-l2: L2 (TCC) hits and misses per dispatch of the attention
    kernels of one run, averaged over its dispatches; one request is one
    128-byte line."""
    rows = _pmc_rows(args.summarise_l2)
    per = {}
    for r in rows:
        name = r["Kernel_Name"]
        if not any(k in name for k in ("paged_decode", "paged_prefill")):
            continue
        d = per.setdefault(name, {}).setdefault(r["Dispatch_Id"], {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    wl = get_workload(args.workload)
    for name, disp in per.items():
        hits = float(np.mean([d.get("TCC_HIT_sum", 0.0) for d in disp.values()]))
        miss = float(np.mean([d.get("TCC_MISS_sum", 0.0) for d in disp.values()]))
        rate = hits / (hits + miss) if hits + miss else 0.0
        short = name.split("(")[0].replace("void ", "").replace("pkv::", "")
        print(f"| {wl.name} | `{short}` | {len(disp)} | {hits:,.0f} | {miss:,.0f} | {rate:.3f} | "
              f"{miss * 128 / 1e9:.3f} GB |")
    return 0


def summarise_trace_main(args, argv) -> int:
    """--summarise-trace: a kernel trace of one bench.py run -> a short
    markdown summary under profiles/: the per-kernel statistics and, for the
    dominant kernel, the average over each timed region of the run (warm-up,
    back-to-back steps, HIP-event steps, and steps after a 512 MiB write)."""
    import csv
    tdir, log = args.summarise_trace
    wl = get_workload(args.workload)
    kind = "prefill" if wl.multi_token else "decode"
    stats = list(csv.DictReader(open(os.path.join(tdir, "kt_kernel_stats.csv"))))
    trace = sorted(csv.DictReader(open(os.path.join(tdir, "kt_kernel_trace.csv"))),
                   key=lambda r: int(r["Start_Timestamp"]))
    main_name = "paged_prefill" if wl.multi_token else "paged_decode_kernel"
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace if main_name in r["Kernel_Name"]]
    plan = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace
            if "paged_decode_plan_kernel" in r["Kernel_Name"]]
    W, K = args.warmup, args.steps
    names = ["warm-up", "steps back to back", "steps with HIP events", "steps after a 512 MiB write"]
    bounds = [0, W, W + K, W + 2 * K, W + 3 * K]
    rows = []
    for i, nm in enumerate(names):
        seg = durs[bounds[i]:bounds[i + 1]]
        if seg:
            rows.append(f"| {nm} | {len(seg)} | {np.mean(seg):.1f} | {np.min(seg):.1f} | {np.max(seg):.1f} |")
    rest = list(argv if argv is not None else sys.argv[1:])
    i = rest.index("--summarise-trace")
    base = " ".join(rest[:i] + rest[i + 3:])
    bench_lines = [ln.strip() for ln in open(log) if ln.startswith("[bench]") and ("kernel" in ln or "step" in ln)]
    out = [f"# Kernel trace: {wl.name}", "",
           "Command (from the repository root, on one MI355X):", "", "```",
           f"rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o kt -- python3 bench.py {base}",
           "```", "", "| kernel | calls | average (µs) | min (µs) | max (µs) | share of GPU time |",
           "|---|---|---|---|---|---|"]
    for r in stats[:8]:
        out.append(f"| `{r['Name'][:110]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    out += ["", f"`{main_name}` by region of the run (launches in dispatch order):", "",
            "| region | launches | average (µs) | min (µs) | max (µs) |", "|---|---|---|---|---|", *rows]
    if plan:
        out += ["", f"`paged_decode_plan_kernel`: {len(plan)} launches, average {np.mean(plan):.1f} µs "
                    f"(min {np.min(plan):.1f}, max {np.max(plan):.1f})."]
    if bench_lines:
        out += ["", "bench.py's own timing in the same run:", "", *[f"    {ln}" for ln in bench_lines]]
    tag = wl.name + ("" if args.partition_tokens is None or args.partition_tokens == wl.partition_tokens
                     else f"_pt{args.partition_tokens}")
    path = os.path.join(_PROFILES, f"{kind}_{tag}_kernel_trace.md")
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")
    print(path)
    return 0


if __name__ == "__main__":
    sys.exit(main())
