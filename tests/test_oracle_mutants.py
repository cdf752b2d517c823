"""The pins bite: plant plausible mistakes in a copy of the oracle's C source
(on the CPU, in a temporary directory), and check that the pinned checks
reject every mutant while accepting the unmodified source."""
import ctypes
import os
import subprocess
import tempfile

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle.run import OracleRun

MUTANTS = {
    "dropped_scale": ("sc[t] = scale * acc;", "sc[t] = acc;"),
    "softmax_sign": ("sc[t] = exp(sc[t] - m);", "sc[t] = exp(m - sc[t]);"),
    "causal_off_by_one": ("int seen = n - m + i + 1;", "int seen = n - m + i;"),
    "causal_ignored": ("attend(qd, Kc, Vc, seen, D,", "attend(qd, Kc, Vc, n, D,"),
    "query_row": ("size_t qoff = ((size_t)(q0 + i) * Hq + hq) * D;", "size_t qoff = ((size_t)(q0 + i) * Hq + gi) * D;"),
    "no_normalise": ("o[j] = acc / l;", "o[j] = acc;"),
    "block_index": ("block_tables[(size_t)s * max_blocks + t / B]", "block_tables[(size_t)s * max_blocks + t % B]"),
    "slot_offset": ("int o = t % B;", "int o = t / B;"),
    "gqa_mapping": ("int hq = hk * g + gi;", "int hq = gi * H + hk;"),
    "layout_transposed": ("size_t base = ((size_t)((int64_t)blk * H + hk) * B + o) * D;",
                          "size_t base = ((size_t)((int64_t)blk * B + o) * H + hk) * D;"),
    "fp8_exponent": ("v = ldexp((double)(8 + m), e - 10);", "v = ldexp((double)(8 + m), e - 11);"),
    "fp8_scale_missing": ("Kc[(size_t)t * D + j] = fp8 ? kv * k_scale : kv;", "Kc[(size_t)t * D + j] = kv;"),
    "f16_subnormal": ("v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);"),
    "tie_to_odd": ("else c = (lo % 2 == 0) ? lo : hi;", "else c = (lo % 2 == 0) ? hi : lo;"),
    "write_slot": ("int64_t b = s / B, o = s % B;", "int64_t b = s / B, o = (s + 1) % B;"),
    "head_scale_read": ("if (k_head) k_scale = k_head[hk];", "if (k_head) k_scale = k_head[0];"),
    "head_scale_write": ("const float ks = k_head ? k_head[h] : k_scale,", "const float ks = k_head ? k_head[0] : k_scale,"),
}


def _build_variant(tmp, name, edit, occurrence=0):
    """Copy of the oracle source with the `occurrence`-th instance of the
    edit's text replaced (every instance is planted on its own)."""
    src = open(oracle._SRC).read()
    if edit is not None:
        old, new = edit
        at = -1
        for _ in range(occurrence + 1):
            at = src.index(old, at + 1)
        src = src[:at] + new + src[at + len(old):]
    c = os.path.join(tmp, f"{name}.c")
    so = os.path.join(tmp, f"lib{name}.so")
    open(c, "w").write(src)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-o", so, c, "-lm"])
    return so


def _load(so):
    good = oracle.lib()
    L = ctypes.CDLL(so)
    for fn in ["oracle_f16_to_f64", "oracle_bf16_to_f64", "oracle_e4m3_to_f64", "oracle_f32_to_e4m3_sat",
               "oracle_reshape_and_cache", "oracle_copy_blocks", "oracle_decode", "oracle_prefill",
               "oracle_kv_footprint_bytes"]:
        getattr(L, fn).argtypes = getattr(good, fn).argtypes
        getattr(L, fn).restype = getattr(good, fn).restype
    return L


def _pins_pass() -> bool:
    """A compact subset of the pins: formats exhaustively, decode vs the
    library routine on an MHA fp16, a GQA bf16 and a GQA fp8 workload."""
    from test_oracle_decode import _sdpa_expected
    from test_oracle_prefill import _sdpa_causal
    from test_oracle_variants import _sdpa as _sdpa_variant
    from test_oracle_formats import _same
    try:
        ref16 = np.arange(65536, dtype=np.uint16).view(np.float16).astype(np.float64)
        if not all(_same(oracle.f16_to_f64(c), float(ref16[c])) for c in range(65536)):
            return False
        ref8 = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
        if not all(_same(oracle.e4m3_to_f64(c), float(ref8[c])) for c in range(256)):
            return False
        g = sorted({float(ref8[c]) for c in range(0x7F)})
        mids = [(a + b) / 2 for a, b in zip(g[:-1], g[1:])]
        want = torch.tensor(mids, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).tolist()
        if [oracle.f32_to_e4m3(x) for x in mids] != want:
            return False
        for name in ["c2s_f16", "c5s_bf16", "c5s_fp8"]:
            wl = W.small_configs()[name]
            run = OracleRun(wl)
            np.testing.assert_allclose(run.decode(), _sdpa_expected(wl, run), rtol=1e-10, atol=1e-12)
        for name in ["p1s_bf16", "p3s_fp8"]:
            wl = W.small_multi_token_configs()[name]
            run = OracleRun(wl)
            np.testing.assert_allclose(run.prefill(), _sdpa_causal(wl, run), rtol=1e-10, atol=1e-12)
        wl = W.small_variant_configs()["c5s_fp8_headscale"]
        run = OracleRun(wl)
        np.testing.assert_allclose(run.decode(), _sdpa_variant(wl, run), rtol=1e-10, atol=1e-12)
    except (AssertionError, oracle.OracleError):
        return False
    return True


def test_pins_accept_original_and_reject_every_mutant():
    saved = oracle._lib
    try:
        with tempfile.TemporaryDirectory() as tmp:
            oracle._lib = _load(_build_variant(tmp, "original", None))
            assert _pins_pass(), "pins reject the unmodified oracle"
            survivors = []
            src = open(oracle._SRC).read()
            for name, edit in MUTANTS.items():
                count = src.count(edit[0])
                assert count >= 1, name
                for k in range(count):
                    oracle._lib = _load(_build_variant(tmp, f"{name}_{k}", edit, k))
                    if _pins_pass():
                        survivors.append(f"{name}[{k}]")
            assert not survivors, f"mutants not caught by the pins: {survivors}"
    finally:
        oracle._lib = saved
