"""CPU oracle for paged decode attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The library (``paged_kv_cache_449_amd``) never does, and this
package never imports the library: the two share no code.  Inputs come from
the seeded generators in ``workloads`` (which hold no paged-attention
arithmetic) and expected values come from here.

Contents:
  * ``liboracle.so`` (built from ``oracle.c`` with gcc): fp64 decode attention
    over a paged pool, the cache write (with its own E4M3FN encoder) and the
    block copy, plus number-format decoders written from their definitions.
  * ``paging``: the oracle's own block manager emulation (free list, sharing,
    copy-on-write plan, slot of each written token).
  * ``run``: drives both for a whole workload, producing the pools and the
    expected outputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

DT_CODE = {"f32": 0, "f16": 1, "bf16": 2, "fp8e4m3": 3}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8e4m3": 1}


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (plain -O2, no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64, f32, f64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_double
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f64.restype = f64
        L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f64.restype = f64
        L.oracle_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_to_f64.restype = f64
        L.oracle_f32_to_e4m3_sat.argtypes = [f32]
        L.oracle_f32_to_e4m3_sat.restype = ctypes.c_uint8
        L.oracle_reshape_and_cache.argtypes = [vp, vp, i32, i64, i32, i32, i32, f32, f32, vp, vp, i32, vp, i64, vp,
                                               vp]
        L.oracle_reshape_and_cache.restype = i32
        L.oracle_copy_blocks.argtypes = [vp, vp, i64, i64, vp, i64]
        L.oracle_copy_blocks.restype = i32
        L.oracle_decode.argtypes = [vp, vp, i32, i64, i32, i32, i32, f64, f64, vp, i32, i32, i32,
                                    vp, i32, vp, f64, vp, i32, vp, vp, vp]
        L.oracle_decode.restype = i32
        L.oracle_swap_blocks.argtypes = [vp, vp, i64, vp, vp, i64, i64, vp, i64, i32]
        L.oracle_swap_blocks.restype = i32
        L.oracle_prefill.argtypes = [vp, vp, i32, i64, i32, i32, i32, f64, f64, vp, i32, i32, i32,
                                     vp, i32, vp, vp, f64, vp, vp, vp]
        L.oracle_prefill.restype = i32
        L.oracle_kv_footprint_bytes.argtypes = [i32, i32, i32, i64, i32]
        L.oracle_kv_footprint_bytes.restype = f64
        _lib = L
    return _lib


class OracleError(RuntimeError):
    pass


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _raw(t) -> np.ndarray:
    """A CPU torch tensor or numpy array as a C-contiguous numpy view of its bytes."""
    if isinstance(t, np.ndarray):
        return np.ascontiguousarray(t)
    t = t.contiguous()
    return t.view(dtype=_torch_int_view(t)).numpy()


def _torch_int_view(t):
    import torch
    return {1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}[t.element_size()]


# ---------------------------------------------------------------- scalar codecs

def f16_to_f64(bits: int) -> float:
    return lib().oracle_f16_to_f64(bits)


def bf16_to_f64(bits: int) -> float:
    return lib().oracle_bf16_to_f64(bits)


def e4m3_to_f64(code: int) -> float:
    return lib().oracle_e4m3_to_f64(code)


def f32_to_e4m3(x: float) -> int:
    return lib().oracle_f32_to_e4m3_sat(x)


def kv_footprint_bytes(layers: int, heads: int, head_dim: int, tokens: int, dtype_bytes: int) -> float:
    return lib().oracle_kv_footprint_bytes(layers, heads, head_dim, tokens, dtype_bytes)


# ---------------------------------------------------------------- pool emulation

def _opt(a):
    return None if a is None else _ptr(a)


class HostPool:
    """Host copy of the K and V pools, laid out [num_blocks][H][B][D] of the
    pool dtype, stored as raw bytes.  New pools are filled with 0xFF (NaN in
    every supported dtype) so that any read of an unowned slot shows up.
    fp8 pools use one scale per tensor, or one per kv head when head_scales
    = (k [H], v [H]) fp32 arrays are given."""

    def __init__(self, num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int, dtype: str,
                 k_scale: float = 1.0, v_scale: float = 1.0, fill: int = 0xFF, head_scales=None):
        self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim = num_blocks, block_size, num_kv_heads, head_dim
        self.dtype, self.k_scale, self.v_scale = dtype, float(k_scale), float(v_scale)
        self.k_head = self.v_head = None
        if head_scales is not None:
            self.k_head = np.ascontiguousarray(head_scales[0], dtype=np.float32)
            self.v_head = np.ascontiguousarray(head_scales[1], dtype=np.float32)
            assert self.k_head.shape == (num_kv_heads,) and self.v_head.shape == (num_kv_heads,)
        self.block_bytes = num_kv_heads * block_size * head_dim * ELEM_BYTES[dtype]
        self.k = np.full(num_blocks * self.block_bytes, fill, dtype=np.uint8)
        self.v = np.full(num_blocks * self.block_bytes, fill, dtype=np.uint8)

    def reshape_and_cache(self, k, v, src_dtype: str, slots: np.ndarray) -> None:
        kr, vr = _raw(k), _raw(v)
        slots = np.ascontiguousarray(slots, dtype=np.int64)
        T = slots.shape[0]
        rc = lib().oracle_reshape_and_cache(_ptr(self.k), _ptr(self.v), DT_CODE[self.dtype], self.num_blocks,
                                           self.block_size, self.num_kv_heads, self.head_dim,
                                           self.k_scale, self.v_scale, _ptr(kr), _ptr(vr), DT_CODE[src_dtype],
                                           _ptr(slots), T, _opt(self.k_head), _opt(self.v_head))
        if rc:
            raise OracleError(f"oracle_reshape_and_cache rc={rc}")

    def copy_blocks(self, pairs: np.ndarray) -> None:
        pairs = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
        rc = lib().oracle_copy_blocks(_ptr(self.k), _ptr(self.v), self.block_bytes, self.num_blocks,
                                     _ptr(pairs), pairs.shape[0])
        if rc:
            raise OracleError(f"oracle_copy_blocks rc={rc}")

    def swap(self, host_k: np.ndarray, host_v: np.ndarray, pairs: np.ndarray, out: bool) -> None:
        """Move whole blocks to (out) or from a host swap area held as uint8
        arrays of host_blocks * block_bytes each."""
        pairs = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
        assert host_k.dtype == np.uint8 and host_k.size % self.block_bytes == 0 and host_k.size == host_v.size
        rc = lib().oracle_swap_blocks(_ptr(self.k), _ptr(self.v), self.num_blocks, _ptr(host_k), _ptr(host_v),
                                     host_k.size // self.block_bytes, self.block_bytes, _ptr(pairs), pairs.shape[0],
                                     1 if out else 0)
        if rc:
            raise OracleError(f"oracle_swap_blocks rc={rc}")

    def prefill(self, q, q_dtype: str, block_tables: np.ndarray, context_lens: np.ndarray,
                query_start: np.ndarray, scale: float, num_q_heads: int) -> np.ndarray:
        """Causal attention of each sequence's new query rows (the last
        query_start[s+1] - query_start[s] of its context) over its paged
        context; q [total_q][Hq][D] -> fp64 [total_q][Hq][D]."""
        qr = _raw(q)
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        cl = np.ascontiguousarray(context_lens, dtype=np.int32)
        qs = np.ascontiguousarray(query_start, dtype=np.int32)
        S, max_blocks = bt.shape
        total_q = int(qs[-1])
        out = np.full((total_q, num_q_heads, self.head_dim), np.nan, dtype=np.float64)
        rc = lib().oracle_prefill(_ptr(self.k), _ptr(self.v), DT_CODE[self.dtype], self.num_blocks, self.block_size,
                                  self.num_kv_heads, self.head_dim, self.k_scale, self.v_scale, _ptr(qr),
                                  DT_CODE[q_dtype], S, num_q_heads, _ptr(bt), max_blocks, _ptr(cl), _ptr(qs),
                                  float(scale), _ptr(out), _opt(self.k_head), _opt(self.v_head))
        if rc:
            raise OracleError(f"oracle_prefill rc={rc}")
        return out

    def decode(self, q, q_dtype: str, block_tables: np.ndarray, context_lens: np.ndarray, scale: float,
               num_q_heads: int, seqs: Optional[Sequence[int]] = None) -> np.ndarray:
        qr = _raw(q)
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        cl = np.ascontiguousarray(context_lens, dtype=np.int32)
        S, max_blocks = bt.shape
        out = np.full((S, num_q_heads, self.head_dim), np.nan, dtype=np.float64)
        sel = None if seqs is None else np.ascontiguousarray(seqs, dtype=np.int32)
        rc = lib().oracle_decode(_ptr(self.k), _ptr(self.v), DT_CODE[self.dtype], self.num_blocks, self.block_size,
                                 self.num_kv_heads, self.head_dim, self.k_scale, self.v_scale, _ptr(qr),
                                 DT_CODE[q_dtype], S, num_q_heads, _ptr(bt), max_blocks, _ptr(cl), float(scale),
                                 None if sel is None else _ptr(sel), 0 if sel is None else sel.shape[0],
                                 _ptr(out), _opt(self.k_head), _opt(self.v_head))
        if rc:
            raise OracleError(f"oracle_decode rc={rc}")
        return out
