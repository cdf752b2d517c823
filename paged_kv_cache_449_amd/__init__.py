"""Python binding of libpagedkv.so (paged KV-cache pool + decode attention for
MI355X / gfx950).

The functions carry the C ABI's names and only marshal arguments: torch
tensors supply device memory and the current HIP stream; every step of the
path runs in the library's HIP kernels.  There is no fallback: if the shared
library is missing or fails to load, every call raises.

    pool = KVPool(num_blocks, block_size, num_kv_heads, head_dim, torch.bfloat16)
    reshape_and_cache(pool, k_new, v_new, slot_mapping)
    copy_blocks(pool, pairs)
    out = paged_attention_decode(pool, q, block_tables, context_lens, scale)
    swap_blocks(pool, HostSwapArea(pool, n), pairs, KV_SWAP_OUT)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

from .block_manager import BlockManager, PoolExhausted  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")

KV_OK, KV_ERR_INVALID_ARG, KV_ERR_UNSUPPORTED, KV_ERR_OOM, KV_ERR_HIP, KV_ERR_WORKSPACE, KV_ERR_NO_BLOCKS = range(7)
KV_F32, KV_F16, KV_BF16, KV_FP8_E4M3FN = range(4)
KV_SWAP_OUT, KV_SWAP_IN = range(2)

DTYPE_CODE = {torch.float32: KV_F32, torch.float16: KV_F16, torch.bfloat16: KV_BF16,
              torch.float8_e4m3fn: KV_FP8_E4M3FN}

_lib_handle: Optional[ctypes.CDLL] = None


class PagedKVError(RuntimeError):
    def __init__(self, status: int, call: str):
        super().__init__(f"{call}: {status_string(status)} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libpagedkv.so; raises if it has not been built."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m paged_kv_cache_449_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, vp, sz, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float
        pp = ctypes.POINTER(ctypes.c_void_p)
        L.kv_pool_create.argtypes = [i32, i32, i32, i32, ctypes.c_int, pp]
        L.kv_pool_create_from.argtypes = [i32, i32, i32, i32, ctypes.c_int, vp, vp, sz, pp]
        L.kv_pool_destroy.argtypes = [vp]
        L.kv_pool_info.argtypes = [vp, pp, pp, ctypes.POINTER(sz), ctypes.POINTER(i64)]
        L.kv_pool_set_scales.argtypes = [vp, f32, f32]
        L.kv_pool_set_head_scales.argtypes = [vp, vp, vp, vp]
        L.reshape_and_cache.argtypes = [vp, vp, vp, ctypes.c_int, vp, i32, vp]
        L.paged_attention_decode.argtypes = [vp, vp, ctypes.c_int, vp, vp, i32, vp, i32, i32, f32, i32, vp, sz, vp]
        L.paged_attention_workspace_size.argtypes = [vp, i32, i32, i32, i32, ctypes.POINTER(sz)]
        L.paged_attention_decode_noalloc.argtypes = [vp, vp, ctypes.c_int, vp, vp, i32, vp, i32, i32, f32, i32, vp]
        L.paged_attention_plan.argtypes = [vp, ctypes.c_int, vp, i32, vp, i32, i32, i32, vp, sz, vp]
        L.paged_attention_decode_planned.argtypes = [vp, vp, ctypes.c_int, vp, vp, i32, vp, i32, i32, f32, i32, vp,
                                                     sz, vp]
        L.copy_blocks.argtypes = [vp, vp, i32, vp]
        L.swap_blocks.argtypes = [vp, vp, vp, i64, vp, i32, ctypes.c_int, vp]
        L.paged_attention_prefill.argtypes = [vp, vp, ctypes.c_int, vp, vp, i32, vp, vp, i32, i32, i32, f32, vp,
                                              sz, vp]
        L.paged_attention_prefill_workspace_size.argtypes = [vp, i32, ctypes.POINTER(sz)]
        L.paged_attention_decode_grouped.argtypes = [vp, vp, ctypes.c_int, vp, vp, i32, vp, i32, i32, f32, vp, vp,
                                                     i32, vp, sz, vp]
        L.paged_attention_decode_grouped_workspace_size.argtypes = [vp, i32, i32, ctypes.POINTER(sz)]
        L.kv_stream_read.argtypes = [vp, sz, i32, vp, i32, vp, vp]
        L.kv_status_string.argtypes = [ctypes.c_int]
        L.kv_status_string.restype = ctypes.c_char_p
        # host block manager (block_manager.h)
        u64 = ctypes.c_uint64
        L.bm_create.argtypes = [i64, i32, vp, i32, pp]
        L.bm_destroy.argtypes = [vp]
        L.bm_destroy.restype = None
        L.bm_add_sequence.argtypes = [vp, i64, vp, i32, u64, vp, vp]
        L.bm_fork.argtypes = [vp, i64, vp, i32]
        L.bm_append_slots.argtypes = [vp, i64, vp, i32, vp, vp, vp]
        L.bm_append_batch.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp]
        L.bm_free.argtypes = [vp, i64]
        L.bm_num_free_blocks.argtypes = [vp, vp]
        L.bm_sequence_info.argtypes = [vp, i64, vp, vp]
        L.bm_block_table.argtypes = [vp, i64, vp, i32]
        L.bm_block_tables.argtypes = [vp, vp, i32, i32, vp, vp]
        L.bm_ref_count.argtypes = [vp, i32, vp]
        L.bm_stats.argtypes = [vp, vp]
        for fn in ("bm_create", "bm_add_sequence", "bm_fork", "bm_append_slots", "bm_append_batch", "bm_free", "bm_num_free_blocks",
                   "bm_sequence_info", "bm_block_table", "bm_block_tables", "bm_ref_count", "bm_stats"):
            getattr(L, fn).restype = ctypes.c_int
        for fn in ("kv_pool_create", "kv_pool_create_from", "kv_pool_destroy", "kv_pool_info", "kv_pool_set_scales",
                   "kv_pool_set_head_scales",
                   "reshape_and_cache", "paged_attention_decode", "paged_attention_workspace_size", "copy_blocks",
                   "paged_attention_decode_noalloc", "paged_attention_plan", "paged_attention_decode_planned",
                   "swap_blocks", "paged_attention_prefill", "paged_attention_prefill_workspace_size",
                   "paged_attention_decode_grouped", "paged_attention_decode_grouped_workspace_size",
                   "kv_stream_read"):
            getattr(L, fn).restype = ctypes.c_int
        _lib_handle = L
    return _lib_handle


def status_string(status: int) -> str:
    return lib().kv_status_string(status).decode()


def _check(status: int, call: str) -> None:
    if status != KV_OK:
        raise PagedKVError(status, call)


def _stream(device: torch.device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream)


def _dev_ptr(t: torch.Tensor, name: str, device: torch.device) -> int:
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


class KVPool:
    """K and V pools, each a device tensor [num_blocks][num_kv_heads][block_size][head_dim],
    described to the library with kv_pool_create_from (torch owns the memory)."""

    def __init__(self, num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int, dtype: torch.dtype,
                 device=None, k_scale: float = 1.0, v_scale: float = 1.0):
        if dtype not in DTYPE_CODE:
            raise ValueError(f"unsupported KV dtype {dtype}")
        self.device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim = num_blocks, block_size, num_kv_heads, head_dim
        self.dtype = dtype
        shape = (num_blocks, num_kv_heads, block_size, head_dim)
        self.k_cache = torch.empty(shape, dtype=dtype, device=self.device)
        self.v_cache = torch.empty(shape, dtype=dtype, device=self.device)
        h = ctypes.c_void_p()
        nbytes = self.k_cache.numel() * self.k_cache.element_size()
        with torch.cuda.device(self.device):
            _check(lib().kv_pool_create_from(num_blocks, block_size, num_kv_heads, head_dim, DTYPE_CODE[dtype],
                                             self.k_cache.data_ptr(), self.v_cache.data_ptr(), nbytes,
                                             ctypes.byref(h)), "kv_pool_create_from")
        self.handle = h
        self.k_scale, self.v_scale = 1.0, 1.0
        self.head_scales = None
        if dtype == torch.float8_e4m3fn:
            kv_pool_set_scales(self, k_scale, v_scale)
        self._workspace: Optional[torch.Tensor] = None

    @property
    def block_bytes(self) -> int:
        return self.num_kv_heads * self.block_size * self.head_dim * self.k_cache.element_size()

    def workspace(self, nbytes: int) -> torch.Tensor:
        """A zero-initialised device workspace of at least nbytes, reused across calls."""
        if self._workspace is None or self._workspace.numel() < nbytes:
            self._workspace = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return self._workspace

    def close(self) -> None:
        if getattr(self, "handle", None) is not None and self.handle.value:
            lib().kv_pool_destroy(self.handle)
            self.handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def kv_pool_set_scales(pool: KVPool, k_scale: float, v_scale: float) -> None:
    _check(lib().kv_pool_set_scales(pool.handle, float(k_scale), float(v_scale)), "kv_pool_set_scales")
    pool.k_scale, pool.v_scale = float(k_scale), float(v_scale)
    pool.head_scales = None


def kv_pool_set_head_scales(pool: KVPool, k_scales, v_scales, stream=None) -> None:
    """fp8 pools: one scale per kv head (sequences of num_kv_heads floats,
    each finite and > 0); None, None returns to the per-tensor scales.  The
    values are uploaded to a device tensor that the library copies, in stream
    order, into the pool's own scale table."""
    import numpy as np
    d = pool.device
    if k_scales is None and v_scales is None:
        _check(lib().kv_pool_set_head_scales(pool.handle, None, None, _stream(d, stream)), "kv_pool_set_head_scales")
        pool.head_scales = None
        return
    k = np.ascontiguousarray(k_scales, dtype=np.float32)
    v = np.ascontiguousarray(v_scales, dtype=np.float32)
    if k.shape != (pool.num_kv_heads,) or v.shape != (pool.num_kv_heads,):
        raise ValueError(f"need {pool.num_kv_heads} scales each")
    if not (np.all(np.isfinite(k)) and np.all(np.isfinite(v)) and np.all(k > 0) and np.all(v > 0)):
        raise ValueError("scales must be finite and > 0")
    dev = torch.from_numpy(np.concatenate([k, v])).to(d)
    _check(lib().kv_pool_set_head_scales(pool.handle, dev.data_ptr(), dev.data_ptr() + 4 * pool.num_kv_heads,
                                         _stream(d, stream)), "kv_pool_set_head_scales")
    pool._head_scale_src = dev   # alive until the stream copy has run
    pool.head_scales = (k.copy(), v.copy())


def kv_pool_info(pool: KVPool):
    k, v = ctypes.c_void_p(), ctypes.c_void_p()
    nbytes = ctypes.c_size_t()
    strides = (ctypes.c_int64 * 4)()
    _check(lib().kv_pool_info(pool.handle, ctypes.byref(k), ctypes.byref(v), ctypes.byref(nbytes), strides),
           "kv_pool_info")
    return k.value, v.value, nbytes.value, tuple(strides)


class LibraryPool:
    """A pool whose memory the library allocates (kv_pool_create) and frees."""

    def __init__(self, num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int, dtype: torch.dtype):
        h = ctypes.c_void_p()
        _check(lib().kv_pool_create(num_blocks, block_size, num_kv_heads, head_dim, DTYPE_CODE[dtype],
                                    ctypes.byref(h)), "kv_pool_create")
        self.handle = h

    def close(self) -> None:
        if self.handle.value:
            _check(lib().kv_pool_destroy(self.handle), "kv_pool_destroy")
            self.handle = ctypes.c_void_p()


def kv_pool_create(num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int,
                   dtype: torch.dtype) -> LibraryPool:
    return LibraryPool(num_blocks, block_size, num_kv_heads, head_dim, dtype)


def reshape_and_cache(pool: KVPool, k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                      stream=None) -> None:
    """Store k/v [T][Hkv][D] into the pool at slot_mapping (int64 [T], <0 skips)."""
    if k.shape != v.shape or k.dim() != 3 or k.shape[1:] != (pool.num_kv_heads, pool.head_dim):
        raise ValueError(f"k/v must be [T][{pool.num_kv_heads}][{pool.head_dim}], got {tuple(k.shape)}")
    if k.dtype != v.dtype or k.dtype not in DTYPE_CODE:
        raise ValueError("k and v must share a supported dtype")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (k.shape[0],):
        raise ValueError("slot_mapping must be int64 [T]")
    d = pool.device
    _check(lib().reshape_and_cache(pool.handle, _dev_ptr(k, "k", d), _dev_ptr(v, "v", d), DTYPE_CODE[k.dtype],
                                   _dev_ptr(slot_mapping, "slot_mapping", d), k.shape[0], _stream(d, stream)),
           "reshape_and_cache")


def copy_blocks(pool: KVPool, pairs: torch.Tensor, stream=None) -> None:
    """Copy whole blocks for each (src, dst) row of pairs (int32 [P][2])."""
    if pairs.dtype != torch.int32 or pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be int32 [P][2]")
    if pairs.shape[0] == 0:
        return
    d = pool.device
    _check(lib().copy_blocks(pool.handle, _dev_ptr(pairs, "pairs", d), pairs.shape[0], _stream(d, stream)),
           "copy_blocks")


class HostSwapArea:
    """Pinned host memory for swapped-out blocks: K and V, each
    [num_blocks][num_kv_heads][block_size][head_dim] of the pool dtype."""

    def __init__(self, pool: KVPool, num_blocks: int):
        shape = (num_blocks, pool.num_kv_heads, pool.block_size, pool.head_dim)
        self.num_blocks = num_blocks
        self.k_cache = torch.empty(shape, dtype=pool.dtype, pin_memory=True)
        self.v_cache = torch.empty(shape, dtype=pool.dtype, pin_memory=True)


def swap_blocks(pool: KVPool, area: HostSwapArea, pairs: torch.Tensor, direction: int, stream=None) -> None:
    """KV_SWAP_OUT: pool block src -> host block dst; KV_SWAP_IN: host block src
    -> pool block dst, for each (src, dst) row of pairs (device int32 [P][2])."""
    if pairs.dtype != torch.int32 or pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be int32 [P][2]")
    if area.k_cache.dtype != pool.dtype or area.k_cache.shape[1:] != pool.k_cache.shape[1:]:
        raise ValueError("swap area and pool disagree on the block layout")
    if pairs.shape[0] == 0:
        return
    d = pool.device
    _check(lib().swap_blocks(pool.handle, area.k_cache.data_ptr(), area.v_cache.data_ptr(), area.num_blocks,
                             _dev_ptr(pairs, "pairs", d), pairs.shape[0], int(direction), _stream(d, stream)),
           "swap_blocks")


def paged_attention_workspace_size(pool: KVPool, num_seqs: int, num_q_heads: int, max_blocks: int,
                                   partition_tokens: int = 0) -> int:
    n = ctypes.c_size_t()
    _check(lib().paged_attention_workspace_size(pool.handle, num_seqs, num_q_heads, max_blocks, partition_tokens,
                                                ctypes.byref(n)), "paged_attention_workspace_size")
    return n.value


def paged_attention_prefill(pool: KVPool, q: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                            query_start: torch.Tensor, scale: float, out: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Causal attention of each sequence's new query rows q [total_q][Hq][D]
    (sequence s owns rows query_start[s]:query_start[s+1], the last tokens of
    its context) over its paged context."""
    if q.dim() != 3 or q.shape[2] != pool.head_dim or q.dtype not in DTYPE_CODE:
        raise ValueError(f"q must be [total_q][Hq][{pool.head_dim}] of a supported dtype")
    S = block_tables.shape[0]
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2:
        raise ValueError("block_tables must be int32 [S][max_blocks]")
    if context_lens.dtype != torch.int32 or context_lens.shape != (S,):
        raise ValueError("context_lens must be int32 [S]")
    if query_start.dtype != torch.int32 or query_start.shape != (S + 1,):
        raise ValueError("query_start must be int32 [S + 1]")
    total_q, Hq = q.shape[0], q.shape[1]
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    n = ctypes.c_size_t()
    _check(lib().paged_attention_prefill_workspace_size(pool.handle, Hq, ctypes.byref(n)),
           "paged_attention_prefill_workspace_size")
    if workspace is None:
        workspace = pool.workspace(n.value)
    d = pool.device
    _check(lib().paged_attention_prefill(pool.handle, _dev_ptr(q, "q", d), DTYPE_CODE[q.dtype], _dev_ptr(out, "out", d),
                                         _dev_ptr(block_tables, "block_tables", d), block_tables.shape[1],
                                         _dev_ptr(context_lens, "context_lens", d),
                                         _dev_ptr(query_start, "query_start", d), S, total_q, Hq, float(scale),
                                         _dev_ptr(workspace, "workspace", d),
                                         workspace.numel() * workspace.element_size(), _stream(d, stream)),
           "paged_attention_prefill")
    return out


def shared_prefix_groups(block_tables, context_lens, group_size_limit: int):
    """Groups of consecutive sequences that share their leading blocks (host
    arrays in, numpy int32 arrays out): (group_start [num_groups + 1],
    group_shared [num_groups]).  A group is a run of sequences whose first
    table entry is the same physical block, cut to at most group_size_limit
    members; its shared length is the number of leading entries every member
    holds in common (the library cuts it to whole blocks within every
    member's context).  Sequences that share nothing form groups of one with
    shared length 0, so the groups cover the batch."""
    import numpy as np
    bt = np.asarray(block_tables)
    cl = np.asarray(context_lens)
    S = bt.shape[0]
    starts, shared = [], []
    s = 0
    while s < S:
        e = s + 1
        while e < S and e - s < group_size_limit and bt[e, 0] >= 0 and bt[e, 0] == bt[s, 0]:
            e += 1
        k = 0
        if e - s > 1:
            rows = bt[s:e]
            same = np.all(rows == rows[0], axis=0)
            k = int(np.argmin(same)) if not same.all() else bt.shape[1]
        starts.append(s)
        shared.append(k)
        s = e
    return np.asarray(starts + [S], dtype=np.int32), np.asarray(shared, dtype=np.int32)


def paged_attention_decode_grouped(pool: KVPool, q: torch.Tensor, block_tables: torch.Tensor,
                                   context_lens: torch.Tensor, scale: float, group_start: torch.Tensor,
                                   group_shared: torch.Tensor, out: Optional[torch.Tensor] = None,
                                   workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Decode attention with the shared prefix of each group of sequences read
    once per group (group_start [G + 1], group_shared [G]: device int32)."""
    if q.dim() != 3 or q.shape[2] != pool.head_dim or q.dtype not in DTYPE_CODE:
        raise ValueError(f"q must be [S][Hq][{pool.head_dim}] of a supported dtype")
    S, Hq = q.shape[0], q.shape[1]
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must be int32 [S][max_blocks]")
    if context_lens.dtype != torch.int32 or context_lens.shape != (S,):
        raise ValueError("context_lens must be int32 [S]")
    ng = group_shared.shape[0]
    if group_start.dtype != torch.int32 or group_shared.dtype != torch.int32 or group_start.shape != (ng + 1,):
        raise ValueError("group_start must be int32 [G + 1] and group_shared int32 [G]")
    if out is None:
        out = torch.empty_like(q)
    n = ctypes.c_size_t()
    _check(lib().paged_attention_decode_grouped_workspace_size(pool.handle, S, Hq, ctypes.byref(n)),
           "paged_attention_decode_grouped_workspace_size")
    if workspace is None:
        workspace = pool.workspace(n.value)
    d = pool.device
    _check(lib().paged_attention_decode_grouped(pool.handle, _dev_ptr(q, "q", d), DTYPE_CODE[q.dtype],
                                                _dev_ptr(out, "out", d), _dev_ptr(block_tables, "block_tables", d),
                                                block_tables.shape[1], _dev_ptr(context_lens, "context_lens", d), S,
                                                Hq, float(scale), _dev_ptr(group_start, "group_start", d),
                                                _dev_ptr(group_shared, "group_shared", d) if ng else None, ng,
                                                _dev_ptr(workspace, "workspace", d),
                                                workspace.numel() * workspace.element_size(), _stream(d, stream)),
           "paged_attention_decode_grouped")
    return out


def kv_stream_read(buf: torch.Tensor, tile_bytes: int, tiles: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Measurement primitive: read the tiles of buf (tile_bytes each) listed
    in tiles (int32, device) with the decode kernel's load form; sink is a
    device int32/uint32 tensor of at least one element."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    if tiles.dtype != torch.int32 or tiles.dim() != 1:
        raise ValueError("tiles must be int32 [num_tiles]")
    if sink.numel() < 1 or sink.element_size() != 4:
        raise ValueError("sink must hold at least one 32-bit element")
    d = buf.device
    with torch.cuda.device(d):   # the call runs on the current device
        _check(lib().kv_stream_read(_dev_ptr(buf, "buf", d), buf.numel() * buf.element_size(), int(tile_bytes),
                                    _dev_ptr(tiles, "tiles", d), tiles.numel(), _dev_ptr(sink, "sink", d),
                                    _stream(d, stream)), "kv_stream_read")


def paged_attention_decode(pool: KVPool, q: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                           scale: float, out: Optional[torch.Tensor] = None, partition_tokens: int = 0,
                           workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Decode attention of q [S][Hq][D] over each sequence's paged context."""
    if q.dim() != 3 or q.shape[2] != pool.head_dim or q.dtype not in DTYPE_CODE:
        raise ValueError(f"q must be [S][Hq][{pool.head_dim}] of a supported dtype")
    S, Hq = q.shape[0], q.shape[1]
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must be int32 [S][max_blocks]")
    if context_lens.dtype != torch.int32 or context_lens.shape != (S,):
        raise ValueError("context_lens must be int32 [S]")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    max_blocks = block_tables.shape[1]
    need = paged_attention_workspace_size(pool, S, Hq, max_blocks, partition_tokens)
    if workspace is None:
        workspace = pool.workspace(need)
    d = pool.device
    _check(lib().paged_attention_decode(pool.handle, _dev_ptr(q, "q", d), DTYPE_CODE[q.dtype],
                                        _dev_ptr(out, "out", d), _dev_ptr(block_tables, "block_tables", d), max_blocks,
                                        _dev_ptr(context_lens, "context_lens", d), S, Hq, float(scale),
                                        partition_tokens, _dev_ptr(workspace, "workspace", d),
                                        workspace.numel() * workspace.element_size(), _stream(d, stream)),
           "paged_attention_decode")
    return out


DECODE_SCRATCH_BYTES = 64 << 20   # PAGEDKV_DECODE_SCRATCH_BYTES


def paged_attention_decode_noalloc(pool: KVPool, q: torch.Tensor, block_tables: torch.Tensor,
                                   context_lens: torch.Tensor, scale: float, out: torch.Tensor,
                                   partition_tokens: int = 0, stream=None) -> torch.Tensor:
    """paged_attention_decode with the library's fixed device scratch area in
    place of a workspace: the call allocates nothing (out is the caller's).
    Calls that overlap in time on one device race."""
    if q.dim() != 3 or q.shape[2] != pool.head_dim or q.dtype not in DTYPE_CODE:
        raise ValueError(f"q must be [S][Hq][{pool.head_dim}] of a supported dtype")
    S, Hq = q.shape[0], q.shape[1]
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must be int32 [S][max_blocks]")
    if context_lens.dtype != torch.int32 or context_lens.shape != (S,):
        raise ValueError("context_lens must be int32 [S]")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    d = pool.device
    _check(lib().paged_attention_decode_noalloc(pool.handle, _dev_ptr(q, "q", d), DTYPE_CODE[q.dtype],
                                                _dev_ptr(out, "out", d), _dev_ptr(block_tables, "block_tables", d),
                                                block_tables.shape[1], _dev_ptr(context_lens, "context_lens", d), S,
                                                Hq, float(scale), partition_tokens, _stream(d, stream)),
           "paged_attention_decode_noalloc")
    return out


def _decode_args(pool: KVPool, q, block_tables, context_lens):
    if q.dim() != 3 or q.shape[2] != pool.head_dim or q.dtype not in DTYPE_CODE:
        raise ValueError(f"q must be [S][Hq][{pool.head_dim}] of a supported dtype")
    S = q.shape[0]
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must be int32 [S][max_blocks]")
    if context_lens.dtype != torch.int32 or context_lens.shape != (S,):
        raise ValueError("context_lens must be int32 [S]")


def paged_attention_plan(pool: KVPool, q: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                         partition_tokens: int = 0, workspace: Optional[torch.Tensor] = None,
                         stream=None) -> torch.Tensor:
    """Write the launch plan of a decode over these tables into `workspace`
    (returned); q supplies only the shape and dtype."""
    _decode_args(pool, q, block_tables, context_lens)
    S, Hq = q.shape[0], q.shape[1]
    need = paged_attention_workspace_size(pool, S, Hq, block_tables.shape[1], partition_tokens)
    if workspace is None:
        workspace = pool.workspace(need)
    d = pool.device
    _check(lib().paged_attention_plan(pool.handle, DTYPE_CODE[q.dtype], _dev_ptr(block_tables, "block_tables", d),
                                      block_tables.shape[1], _dev_ptr(context_lens, "context_lens", d), S, Hq,
                                      partition_tokens, _dev_ptr(workspace, "workspace", d),
                                      workspace.numel() * workspace.element_size(), _stream(d, stream)),
           "paged_attention_plan")
    return workspace


def paged_attention_decode_planned(pool: KVPool, q: torch.Tensor, block_tables: torch.Tensor,
                                   context_lens: torch.Tensor, scale: float, workspace: torch.Tensor,
                                   out: Optional[torch.Tensor] = None, partition_tokens: int = 0,
                                   stream=None) -> torch.Tensor:
    """The decode kernel alone, over the plan paged_attention_plan wrote into
    `workspace` for the same tables, lengths, shapes and split."""
    _decode_args(pool, q, block_tables, context_lens)
    S, Hq = q.shape[0], q.shape[1]
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    d = pool.device
    _check(lib().paged_attention_decode_planned(pool.handle, _dev_ptr(q, "q", d), DTYPE_CODE[q.dtype],
                                                _dev_ptr(out, "out", d), _dev_ptr(block_tables, "block_tables", d),
                                                block_tables.shape[1], _dev_ptr(context_lens, "context_lens", d), S,
                                                Hq, float(scale), partition_tokens,
                                                _dev_ptr(workspace, "workspace", d),
                                                workspace.numel() * workspace.element_size(), _stream(d, stream)),
           "paged_attention_decode_planned")
    return out
