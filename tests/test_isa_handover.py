"""The hand-over between split decode workers, checked in the gfx950
assembly the compiler makes of one decode unit (no GPU needed).

A worker publishes its partial record with write-through stores (cache
policy sc1), waits for every vector memory operation to complete, then
counts itself in with a relaxed device-scope atomic add; the worker that
completes the count reads the records with sc1 loads.  These tests fail if
a toolchain change drops the policy bits or the wait, which would let a
merger read stale records without any error.  They also check that no
scalar-cache write-back or invalidate is emitted."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    import paged_kv_cache_449_amd.build as B
    out = tmp_path_factory.mktemp("isa") / "decode_bf16_bf16.s"
    src = os.path.join(B.CSRC, "decode_bf16_bf16.hip")
    cmd = [B.HIPCC, *B.CFLAGS, "-S", "--cuda-device-only", src, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _kernel_bodies(text):
    """(name, lines) of every decode kernel in the assembly."""
    bodies = []
    for m in re.finditer(r"^(_ZN3pkv19paged_decode_kernel\w+):.*$", text, re.M):
        end = text.index(".Lfunc_end", m.end())
        bodies.append((m.group(1), text[m.end():end].splitlines()))
    return bodies


def test_every_arrival_follows_a_full_vector_memory_wait(asm):
    bodies = _kernel_bodies(asm)
    assert len(bodies) >= 10
    checked = 0
    for name, lines in bodies:
        for i, line in enumerate(lines):
            if "global_atomic_add" not in line or "sc0" not in line:   # returning adds: arrivals
                continue
            # walking back: a full vmcnt wait comes before any vector memory
            # instruction (the arrival's block and the ones that lead to it)
            ok = False
            for x in reversed(lines[max(0, i - 80):i]):
                x = x.strip()
                if x.startswith("s_waitcnt") and "vmcnt(0)" in x:
                    ok = True
                    break
                if re.match(r"(buffer|global|flat)_(load|store|atomic)", x):
                    break
            assert ok, (name, i)
            checked += 1
    assert checked >= len(bodies)


def test_records_move_with_write_through_policy(asm):
    for name, lines in _kernel_bodies(asm):
        stores = [x for x in lines if "buffer_store_dwordx4" in x]
        loads_sc1 = [x for x in lines if "buffer_load_dwordx4" in x and "sc1" in x]
        assert stores and all("sc1" in x for x in stores), name
        assert loads_sc1, name


def test_no_scalar_cache_writes(asm):
    assert not re.search(r"\bs_(dcache_wb|dcache_inv|store|buffer_store|atomic|scratch_store)", asm)
