"""Seeded synthetic inputs for paged decode attention.

This module only *draws* inputs: configuration shapes, context lengths, the
order of the free-block list (which fixes where blocks land in the pool), and
the values of q and of every token's K/V.  It contains none of the paged
attention arithmetic (no slot/offset math, no block allocation, no attention,
no quantisation), so both the HIP path and the CPU oracle can consume it
without sharing any of the method's code.

Shapes follow the workloads the pages describe:
  * LLaMA-13B-like head shapes (40 heads x 128) -- page "vLLM KV Cache 实现机制",
    §2.2 (capacity estimate).
  * LLaMA-7B-like heads (32 x 128) at max_num_seqs 256 -- same page, §5.1
    (launch flags) and page "vLLM — 把操作系统的分页搬进 GPU KV cache", case 1.
  * Parallel sampling with n = 4 candidates sharing a prompt -- the latter
    page, case 2.
  * block_size 16 by default, 32 as the alternative -- page "vLLM 与 KV Cache",
    how-it-works point 1, and "vLLM KV Cache 实现机制" §2.3 table.
  * fp8 KV cache dtype -- "vLLM KV Cache 实现机制" §2.3 table.

Every random stream comes from numpy's SeedSequence with entropy
449000 + config index and a spawn key naming the stream, so any piece (one
sequence's K/V, the q tensor, the lengths) can be regenerated on its own.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

# dtype names used across the repository (the C ABI uses the same order)
DTYPES = ("f32", "f16", "bf16", "fp8e4m3")
TORCH_DTYPE = {
    "f32": torch.float32,
    "f16": torch.float16,
    "bf16": torch.bfloat16,
    "fp8e4m3": torch.float8_e4m3fn,
}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8e4m3": 1}

# spawn-key streams
_STREAM_LENS, _STREAM_PLACE, _STREAM_Q, _STREAM_PROMPT_KV, _STREAM_NEW_KV = 0, 1, 2, 3, 4

POISON_BYTE = 0xFF  # NaN bit pattern in every supported KV dtype


@dataclasses.dataclass(frozen=True)
class Workload:
    """One decode-step workload.

    Sequences are grouped under prompts: sequence ``s`` continues prompt
    ``parent[s]`` (prompt_len tokens already cached) with one new token, so its
    context length after the step is ``prompt_lens[parent[s]] + 1``.  When
    several sequences share a parent they are parallel-sampling candidates that
    share the prompt's blocks.
    """

    name: str
    index: int                # seed index
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    kv_dtype: str             # pool dtype
    q_dtype: str              # dtype of q and of the output
    src_dtype: str            # dtype of K/V handed to the cache write
    block_size: int
    prompt_lens: Tuple[int, ...]
    parent: Tuple[int, ...]
    num_blocks: int           # pool size in blocks
    partition_tokens: int = 0  # 0 = library chooses the context split
    same_candidates: bool = False  # candidates of a prompt get identical q / new K/V
    query_lens: Tuple[int, ...] = ()  # new tokens per sequence; empty = one each (decode)
    head_scales: bool = False  # fp8: one scale per kv head; K/V of head h drawn with gain HEAD_GAINS[h % 4]

    @property
    def num_seqs(self) -> int:
        return len(self.parent)

    @property
    def num_prompts(self) -> int:
        return len(self.prompt_lens)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def q_lens(self) -> np.ndarray:
        """New tokens (query rows) of each sequence in the step."""
        if not self.query_lens:
            return np.ones(self.num_seqs, dtype=np.int32)
        return np.asarray(self.query_lens, dtype=np.int32)

    @property
    def total_q(self) -> int:
        return int(self.q_lens.sum())

    @property
    def query_start(self) -> np.ndarray:
        """int32 [S + 1]: sequence s owns query rows query_start[s]:query_start[s+1]."""
        return np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int32)

    @property
    def multi_token(self) -> bool:
        return bool(self.query_lens)

    @property
    def context_lens(self) -> np.ndarray:
        pl = np.asarray(self.prompt_lens, dtype=np.int64)
        return (pl[np.asarray(self.parent, dtype=np.int64)] + self.q_lens).astype(np.int32)

    @property
    def max_blocks_per_seq(self) -> int:
        return max(1, -(-int(self.context_lens.max()) // self.block_size))

    def seed(self, stream: int, key: int = 0) -> np.random.SeedSequence:
        return np.random.SeedSequence(entropy=449_000 + self.index, spawn_key=(stream, key))


def _rng(wl: Workload, stream: int, key: int = 0) -> np.random.Generator:
    return np.random.default_rng(wl.seed(stream, key))


# --------------------------------------------------------------------------
# configurations


def _pool_blocks(prompt_lens: Sequence[int], parent: Sequence[int], bs: int, query_lens=None) -> int:
    """Pool sizing recipe: 1.2 x an upper bound of the blocks the step needs.

    Upper bound per prompt: its cached tokens rounded up to whole blocks, plus,
    per candidate, one fresh block more than its new tokens fill.
    """
    cands = np.bincount(np.asarray(parent), minlength=len(prompt_lens))
    need = sum(-(-int(L) // bs) for L in prompt_lens)
    if query_lens:
        need += sum(-(-int(q) // bs) + 1 for q in query_lens)
    else:
        need += int(cands.sum())
    return int(math.ceil(1.2 * need))


def _make(name, index, hq, hkv, d, kv, q, bs, ctx_lens=None, prompt_lens=None, parent=None,
          num_blocks=None, src=None, partition_tokens=0, same_candidates=False, query_lens=None,
          head_scales=False) -> Workload:
    """ctx_lens are context lengths after the step (cached + new tokens)."""
    if prompt_lens is None:
        ctx = [int(x) for x in ctx_lens]
        qn = [1] * len(ctx) if query_lens is None else [int(x) for x in query_lens]
        prompt_lens = [c - k for c, k in zip(ctx, qn)]
        parent = list(range(len(ctx)))
    if num_blocks is None:
        num_blocks = _pool_blocks(prompt_lens, parent, bs, query_lens)
    if src is None:
        src = "bf16" if kv == "fp8e4m3" else kv
    return Workload(name=name, index=index, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                    kv_dtype=kv, q_dtype=q, src_dtype=src, block_size=bs,
                    prompt_lens=tuple(int(x) for x in prompt_lens), parent=tuple(int(p) for p in parent),
                    num_blocks=int(num_blocks), partition_tokens=partition_tokens,
                    same_candidates=same_candidates,
                    query_lens=tuple(int(x) for x in query_lens) if query_lens is not None else (),
                    head_scales=bool(head_scales))


def _lens_uniform(index: int, n: int, lo: int, hi: int) -> np.ndarray:
    rng = np.random.default_rng(np.random.SeedSequence(449_000 + index, spawn_key=(_STREAM_LENS, 0)))
    return rng.integers(lo, hi, size=n, endpoint=True)


def _lens_lognormal(index: int, n: int, median: float, sigma: float, lo: int, hi: int) -> np.ndarray:
    rng = np.random.default_rng(np.random.SeedSequence(449_000 + index, spawn_key=(_STREAM_LENS, 0)))
    x = rng.lognormal(mean=math.log(median), sigma=sigma, size=n)
    return np.clip(np.rint(x), lo, hi).astype(np.int64)


def config_c1() -> Workload:
    """Tiny: 4 MHA heads x 64, fp32, bs 16, pool 32 blocks, lengths {1,15,16,33}."""
    return _make("c1_tiny_f32", 1, 4, 4, 64, "f32", "f32", 16, ctx_lens=[1, 15, 16, 33], num_blocks=32)


def config_c2(num_seqs=64, lo=128, hi=2048, heads=40, index=2, name="c2_llama13b_f16") -> Workload:
    """LLaMA-13B-shaped layer: 40 MHA heads x 128, fp16, bs 16, lengths U[128, 2048]."""
    return _make(name, index, heads, heads, 128, "f16", "f16", 16,
                 ctx_lens=_lens_uniform(index, num_seqs, lo, hi))


def config_c3(block_size=16, num_seqs=256, heads=32, lo=16, hi=4096, index=3, name=None) -> Workload:
    """LLaMA-7B-shaped: 32 MHA heads x 128, bf16, 256 seqs, lognormal(512, 0.8) clipped [16, 4096]."""
    name = name or f"c3_llama7b_bf16_bs{block_size}"
    return _make(name, index, heads, heads, 128, "bf16", "bf16", block_size,
                 ctx_lens=_lens_lognormal(index, num_seqs, 512.0, 0.8, lo, hi))


def config_c4(num_prompts=64, n=4, prompt_len=1023, heads=32, same_candidates=False, index=4,
              name=None) -> Workload:
    """Parallel sampling: prompts shared by n candidates (ref_count n), fp16, bs 16.

    prompt_len 1023 puts the appended token in the last slot of a partly
    filled shared block, so the step copies that block for all but one
    candidate; prompt_len 1024 is the block-aligned variant (no copy).
    """
    name = name or f"c4_parallel_sampling_f16_p{prompt_len}"
    parent = [p for p in range(num_prompts) for _ in range(n)]
    return _make(name, index, heads, heads, 128, "f16", "f16", 16,
                 prompt_lens=[prompt_len] * num_prompts, parent=parent, same_candidates=same_candidates)


def config_c5(kv="fp8e4m3", num_seqs=128, lo=2048, hi=8192, hq=32, hkv=8, partition_tokens=512,
              index=5, name=None, head_scales=False, q="bf16") -> Workload:
    """GQA long context: 32 q heads / 8 KV heads x 128, bf16 q, fp8 (or bf16) KV, U[2048, 8192]."""
    name = name or f"c5_gqa_long_{kv}"
    return _make(name, index, hq, hkv, 128, kv, q, 16,
                 ctx_lens=_lens_uniform(index, num_seqs, lo, hi), partition_tokens=partition_tokens,
                 head_scales=head_scales)


def config_prefill_chunk(num_seqs=16, chunk=512, lo=0, hi=3072, heads=32, index=6, name="p1_chunked_prefill_bf16",
                         kv="bf16", q="bf16", hkv=None) -> Workload:
    """Chunked prefill: each sequence appends a chunk of `chunk` prompt tokens
    after U[lo, hi] cached ones and attends to them causally (LLaMA-7B-shaped
    heads, bf16, bs 16)."""
    cached = _lens_uniform(index, num_seqs, lo, hi)
    return _make(name, index, heads, hkv or heads, 128, kv, q, 16, ctx_lens=cached + chunk,
                 query_lens=[chunk] * num_seqs)


def config_spec_verify(num_seqs=256, draft=4, heads=32, index=7, name="p2_spec_verify_bf16", lo=16,
                       hi=4096) -> Workload:
    """Speculative verification: the LLaMA-7B-shaped high-concurrency batch,
    each sequence checking `draft` proposed tokens at once (lognormal cached
    lengths as in the decode workload)."""
    cached = _lens_lognormal(index, num_seqs, 512.0, 0.8, lo, hi)
    return _make(name, index, heads, heads, 128, "bf16", "bf16", 16, ctx_lens=cached + draft,
                 query_lens=[draft] * num_seqs)


def config_prefill_gqa(num_seqs=32, chunk=128, lo=1024, hi=4096, index=8, name="p3_gqa_chunk_fp8", kv="fp8e4m3",
                       hq=32, hkv=8) -> Workload:
    """GQA (32 query / 8 KV heads) chunk of `chunk` new tokens over U[lo, hi]
    cached ones, fp8 KV with bf16 queries."""
    cached = _lens_uniform(index, num_seqs, lo, hi)
    return _make(name, index, hq, hkv, 128, kv, "bf16", 16, ctx_lens=cached + chunk, query_lens=[chunk] * num_seqs)


def multi_token_configs() -> Dict[str, Workload]:
    """Multi-token (causal) attention workloads at their stated sizes."""
    ws = [config_prefill_chunk(), config_spec_verify(), config_prefill_gqa()]
    return {w.name: w for w in ws}


def small_multi_token_configs() -> Dict[str, Workload]:
    """Reduced multi-token workloads the oracle finishes in seconds: tiles that
    span blocks, partial tiles, chunks starting mid-block, empty cached
    prefixes, and every query-group size."""
    ws = [
        config_prefill_chunk(num_seqs=3, chunk=37, lo=0, hi=90, heads=2, name="p1s_bf16"),
        config_spec_verify(num_seqs=9, draft=4, heads=3, hi=300, name="p2s_bf16"),
        config_prefill_gqa(num_seqs=3, chunk=21, lo=30, hi=200, hq=8, hkv=2, name="p3s_fp8"),
        config_prefill_gqa(num_seqs=4, chunk=9, lo=0, hi=70, hq=8, hkv=2, kv="bf16", name="p3s_bf16"),
        _make("p4s_f16_g16", 9, 16, 1, 64, "f16", "f16", 32, ctx_lens=[40, 77], query_lens=[40, 5]),
        _make("p5s_fp8_f16_g8", 10, 16, 2, 256, "fp8e4m3", "f16", 16, ctx_lens=[33, 100, 18],
              query_lens=[16, 3, 18]),
    ]
    return {w.name: w for w in ws}


def full_configs() -> Dict[str, Workload]:
    """The five workloads at their stated sizes (c3 at both block sizes, c5 in fp8 and bf16)."""
    ws = [config_c1(), config_c2(), config_c3(16), config_c3(32), config_c4(), config_c4(prompt_len=1024),
          config_c5("fp8e4m3"), config_c5("bf16")]
    return {w.name: w for w in ws}


def small_configs() -> Dict[str, Workload]:
    """Reduced versions the oracle finishes in seconds; they still span several
    blocks per sequence, several work splits and ragged last blocks."""
    ws = [
        config_c1(),
        config_c2(num_seqs=6, lo=40, hi=700, heads=4, name="c2s_f16"),
        config_c3(16, num_seqs=12, heads=3, lo=16, hi=900, name="c3s_bf16_bs16"),
        config_c3(32, num_seqs=12, heads=3, lo=16, hi=900, name="c3s_bf16_bs32"),
        config_c4(num_prompts=3, n=4, prompt_len=95, heads=2, name="c4s_cow_f16"),
        config_c4(num_prompts=2, n=4, prompt_len=96, heads=2, name="c4s_aligned_f16"),
        config_c4(num_prompts=2, n=4, prompt_len=47, heads=2, same_candidates=True, name="c4s_same_f16"),
        config_c5("fp8e4m3", num_seqs=5, lo=300, hi=1500, hq=8, hkv=2, name="c5s_fp8"),
        config_c5("bf16", num_seqs=5, lo=300, hi=1500, hq=8, hkv=2, name="c5s_bf16"),
    ]
    return {w.name: w for w in ws}


def variant_configs() -> Dict[str, Workload]:
    """Variants of the decode workloads at full size: block sizes 8 and 64
    for the LLaMA-7B shape, an 8:1 query group (32 q / 4 KV heads) in fp8 and
    bf16, per-head fp8 scales on the GQA long-context batch, and the LLaMA-7B
    shape at 1024 and 2048 sequences (the batch past which a decode launch's
    fixed cost would show)."""
    ws = [config_c3(8), config_c3(64),
          config_c5("fp8e4m3", hkv=4, name="c5_gqa8_long_fp8e4m3"), config_c5("bf16", hkv=4, name="c5_gqa8_long_bf16"),
          config_c5("fp8e4m3", head_scales=True, name="c5_gqa_long_fp8_headscale"),
          config_c3(16, num_seqs=1024, index=16, name="c3_llama7b_bf16_bs16_s1024"),
          config_c3(16, num_seqs=2048, index=17, name="c3_llama7b_bf16_bs16_s2048")]
    return {w.name: w for w in ws}


def small_variant_configs() -> Dict[str, Workload]:
    """Reduced variants for parity: block sizes 8 and 64, 8:1 and 16:1
    groups, per-head fp8 scales with bf16 and f16 queries, and per-head scales
    in a multi-token step."""
    ws = [
        config_c3(8, num_seqs=10, heads=3, lo=16, hi=500, name="c3s_bf16_bs8"),
        config_c3(64, num_seqs=10, heads=3, lo=16, hi=900, name="c3s_bf16_bs64"),
        config_c5("fp8e4m3", num_seqs=5, lo=300, hi=1500, hq=16, hkv=2, name="c5s_gqa8_fp8"),
        config_c5("fp8e4m3", num_seqs=5, lo=300, hi=1500, hq=8, hkv=4, head_scales=True, name="c5s_fp8_headscale"),
        config_c5("fp8e4m3", num_seqs=4, lo=20, hi=600, hq=4, hkv=4, head_scales=True, q="f16",
                  name="c5s_fp8_headscale_mha_f16"),
        _make("p6s_fp8_headscale", 15, 8, 4, 128, "fp8e4m3", "bf16", 16, ctx_lens=[60, 37, 130],
              query_lens=[20, 37, 9], head_scales=True),
        config_c5("bf16", num_seqs=4, lo=100, hi=700, hq=16, hkv=1, name="c5s_gqa16_bf16"),
        config_c5("fp8e4m3", num_seqs=4, lo=100, hi=700, hq=32, hkv=2, q="f16", name="c5s_gqa16_fp8_f16"),
    ]
    return {w.name: w for w in ws}


def custom(name, hq, hkv, d, kv, q, bs, ctx_lens, num_blocks=None, index=90, partition_tokens=0,
           src=None) -> Workload:
    """Free-form workload for edge-case tests."""
    return _make(name, index, hq, hkv, d, kv, q, bs, ctx_lens=ctx_lens, num_blocks=num_blocks,
                 partition_tokens=partition_tokens, src=src)


# --------------------------------------------------------------------------
# draws


def free_list_order(wl: Workload) -> np.ndarray:
    """Seeded permutation of all physical block ids: the order in which the
    free list hands blocks out (random physical placement)."""
    return _rng(wl, _STREAM_PLACE).permutation(wl.num_blocks).astype(np.int32)


def _normal(rng: np.random.Generator, shape, dtype: str) -> torch.Tensor:
    x = torch.from_numpy(rng.standard_normal(size=shape, dtype=np.float32))
    return x if dtype == "f32" else x.to(TORCH_DTYPE[dtype])


def q_values(wl: Workload) -> torch.Tensor:
    """q [total_q][Hq][d] ~ N(0,1), rounded (RNE) to the q dtype (total_q = S
    for decode: one query token per sequence)."""
    if wl.same_candidates:
        per_prompt = _normal(_rng(wl, _STREAM_Q), (wl.num_prompts, wl.num_q_heads, wl.head_dim), wl.q_dtype)
        return per_prompt[torch.as_tensor(wl.parent, dtype=torch.long)].contiguous()
    return _normal(_rng(wl, _STREAM_Q), (wl.total_q, wl.num_q_heads, wl.head_dim), wl.q_dtype)


HEAD_GAINS = (0.25, 1.0, 4.0, 0.5)   # powers of two: exact in every source dtype


def _head_gain(wl: Workload, x: torch.Tensor) -> torch.Tensor:
    """Per-head magnitudes for per-head-scale workloads: head h scaled by
    HEAD_GAINS[h % 4] (exact), so heads need different fp8 scales."""
    if not wl.head_scales:
        return x
    g = torch.tensor([HEAD_GAINS[h % 4] for h in range(wl.num_kv_heads)], dtype=torch.float32)
    return (x.float() * g[None, :, None]).to(x.dtype)


def prompt_kv(wl: Workload, p: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """K and V of prompt p's cached tokens: each [prompt_len][Hkv][d] in src dtype."""
    rng = _rng(wl, _STREAM_PROMPT_KV, p)
    shape = (wl.prompt_lens[p], wl.num_kv_heads, wl.head_dim)
    k = _normal(rng, shape, wl.src_dtype)
    v = _normal(rng, shape, wl.src_dtype)
    return _head_gain(wl, k), _head_gain(wl, v)


def all_prompt_kv(wl: Workload, prompts: Optional[Sequence[int]] = None, threads: int = 8):
    prompts = range(wl.num_prompts) if prompts is None else prompts
    with ThreadPoolExecutor(threads) as ex:
        return list(ex.map(lambda p: prompt_kv(wl, p), prompts))


def new_kv(wl: Workload) -> Tuple[torch.Tensor, torch.Tensor]:
    """K and V of the tokens the sequences append in the step, in sequence
    order: [total_q][Hkv][d] in src dtype."""
    rng = _rng(wl, _STREAM_NEW_KV)
    n = wl.num_prompts if wl.same_candidates else wl.total_q
    shape = (n, wl.num_kv_heads, wl.head_dim)
    k = _head_gain(wl, _normal(rng, shape, wl.src_dtype))
    v = _head_gain(wl, _normal(rng, shape, wl.src_dtype))
    if wl.same_candidates:
        idx = torch.as_tensor(wl.parent, dtype=torch.long)
        k, v = k[idx].contiguous(), v[idx].contiguous()
    return k, v


def fp8_scales(wl: Workload, threads: int = 8) -> Tuple[float, float]:
    """Per-tensor fp8 scales (recipe; the pages fix none): amax(|x|) / 448 over
    every K (resp. V) value of the workload, computed in fp32.  1.0 for non-fp8
    pools."""
    if wl.kv_dtype != "fp8e4m3":
        return 1.0, 1.0

    def amax(p):
        k, v = prompt_kv(wl, p)
        return float(k.float().abs().max()) if k.numel() else 0.0, float(v.float().abs().max()) if v.numel() else 0.0

    with ThreadPoolExecutor(threads) as ex:
        mx = list(ex.map(amax, range(wl.num_prompts)))
    kn, vn = new_kv(wl)
    km = max([m[0] for m in mx] + [float(kn.float().abs().max())])
    vm = max([m[1] for m in mx] + [float(vn.float().abs().max())])
    ks = float(np.float32(km) / np.float32(448.0))
    vs = float(np.float32(vm) / np.float32(448.0))
    return ks, vs


def fp8_head_scales(wl: Workload, threads: int = 8) -> Tuple[np.ndarray, np.ndarray]:
    """Per-kv-head fp8 scales (recipe): amax(|x|) / 448 over every K (resp.
    V) value of head h in the workload, in fp32.  Arrays of num_kv_heads."""
    H = wl.num_kv_heads

    def amax(p):
        k, v = prompt_kv(wl, p)
        z = np.zeros(H, dtype=np.float32)
        if not k.numel():
            return z, z
        return (k.float().abs().amax(dim=(0, 2)).numpy(), v.float().abs().amax(dim=(0, 2)).numpy())

    with ThreadPoolExecutor(threads) as ex:
        mx = list(ex.map(amax, range(wl.num_prompts)))
    kn, vn = new_kv(wl)
    km = np.max(np.stack([m[0] for m in mx] + [kn.float().abs().amax(dim=(0, 2)).numpy()]), axis=0)
    vm = np.max(np.stack([m[1] for m in mx] + [vn.float().abs().amax(dim=(0, 2)).numpy()]), axis=0)
    return (km.astype(np.float32) / np.float32(448.0)).astype(np.float32), \
        (vm.astype(np.float32) / np.float32(448.0)).astype(np.float32)


# --------------------------------------------------------------------------
# request traces for the host block manager's simulator

_STREAM_TRACE = 5


def _trace_rng(index: int, key: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(449_000 + index, spawn_key=(_STREAM_TRACE, key)))


@dataclasses.dataclass(frozen=True)
class RequestTrace:
    """Requests admitted together: prompt and output lengths per request, the
    length a contiguous allocator would reserve for each (prompt +
    max_new_tokens), and optional prompt token ids."""
    name: str
    prompt_lens: Tuple[int, ...]
    output_lens: Tuple[int, ...]
    max_new_tokens: int
    block_size: int = 16
    tokens: Tuple[Tuple[int, ...], ...] = ()


def serving_trace(num_requests: int = 256, index: int = 20, block_size: int = 16, max_new_tokens: int = 2048,
                  name: str = "serving_lognormal") -> RequestTrace:
    """Prompts lognormal(ln 512, 0.8) clipped to [16, 4096] (the LLaMA-7B
    decode law); outputs lognormal(ln 128, 1.0) clipped to [1, max_new_tokens]
    -- chat-like length mixes standing in for the ShareGPT traces the pages
    mention."""
    rng = _trace_rng(index)
    p = np.clip(np.rint(rng.lognormal(math.log(512), 0.8, num_requests)), 16, 4096).astype(int)
    o = np.clip(np.rint(rng.lognormal(math.log(128), 1.0, num_requests)), 1, max_new_tokens).astype(int)
    return RequestTrace(name, tuple(p.tolist()), tuple(o.tolist()), max_new_tokens, block_size)


def prefix_trace(num_requests: int = 512, num_templates: int = 8, index: int = 21, block_size: int = 16,
                 vocab: int = 32000, name: str = "shared_system_prompts") -> RequestTrace:
    """Requests that open with one of `num_templates` system prompts (lengths
    U[64, 1024], picked with Zipf-like weights 1/(k+1)) followed by a user
    part of U[16, 512] tokens; token ids uniform over the vocabulary; outputs
    lognormal(ln 128, 1.0) clipped to [1, 1024]."""
    rng = _trace_rng(index)
    templates = [rng.integers(0, vocab, size=int(rng.integers(64, 1025))) for _ in range(num_templates)]
    w = 1.0 / np.arange(1, num_templates + 1)
    pick = rng.choice(num_templates, size=num_requests, p=w / w.sum())
    toks, plens = [], []
    for t in pick:
        user = rng.integers(0, vocab, size=int(rng.integers(16, 513)))
        seq = np.concatenate([templates[t], user]).astype(int)
        toks.append(tuple(seq.tolist()))
        plens.append(len(seq))
    o = np.clip(np.rint(rng.lognormal(math.log(128), 1.0, num_requests)), 1, 1024).astype(int)
    return RequestTrace(name, tuple(plens), tuple(o.tolist()), 1024, block_size, tuple(toks))
