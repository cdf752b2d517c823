"""Shared GPU-side helpers for the parity tests: run a workload's decode step
through the library (C ABI via the binding) and bring pools and outputs back
to the host for comparison with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import bench
import workloads as W


def device():
    return torch.device("cuda", 0)


def announce(msg: str) -> None:
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


def run_gpu(wl, partition_tokens=None, free_order=None, repeat: int = 1, grouped: bool = False):
    """Build the workload on the GPU and run `repeat` decode steps.
    Returns a dict with host copies of the pools (raw bytes), the output of
    each step (float64) and the session's step inputs."""
    announce(f"{wl.name} partition={partition_tokens if partition_tokens is not None else wl.partition_tokens}"
             f"{' grouped' if grouped else ''}")
    dev = device()
    sess, q, kn, vn = bench.build_session(wl, dev, free_order=free_order)
    pt = wl.partition_tokens if partition_tokens is None else partition_tokens
    outs = []
    for _ in range(repeat):
        out = sess.step(q, kn, vn, partition_tokens=pt, scale=wl.scale, grouped=grouped)
        torch.cuda.synchronize(dev)
        outs.append(out.float().cpu().double().numpy())
    pool = sess.pool
    return {
        "session": sess,
        "k": pool.k_cache.view(torch.uint8).cpu().numpy().reshape(-1),
        "v": pool.v_cache.view(torch.uint8).cpu().numpy().reshape(-1),
        "out": outs[0],
        "outs": outs,
        "tables": sess.block_tables.cpu().numpy(),
        "pairs": sess.pairs.cpu().numpy(),
        "slots": sess.slot_mapping.cpu().numpy(),
        "q": q,
    }


def run_gpu_prefill(wl, repeat: int = 1):
    """Build a multi-token workload on the GPU and run `repeat` steps (cache
    writes of every new token, then causal attention of the new rows)."""
    announce(f"{wl.name} prefill total_q={wl.total_q}")
    dev = device()
    sess, q, kn, vn = bench.build_session(wl, dev)
    outs = []
    for _ in range(repeat):
        out = sess.step_multi(q, kn, vn, scale=wl.scale)
        torch.cuda.synchronize(dev)
        outs.append(out.float().cpu().double().numpy())
    pool = sess.pool
    return {
        "session": sess,
        "k": pool.k_cache.view(torch.uint8).cpu().numpy().reshape(-1),
        "v": pool.v_cache.view(torch.uint8).cpu().numpy().reshape(-1),
        "out": outs[0],
        "outs": outs,
        "tables": sess.block_tables.cpu().numpy(),
        "slots": sess.slot_mapping.cpu().numpy(),
        "q": q,
    }
