"""CPU model of the decode launch's work plan, work split and merge bookkeeping.

Replays, in Python and with the device code's integer formulas, what the
plan kernel writes (items, per-sequence entries, worker descriptors, record
rows) and what each worker wavefront then does with it: which blocks it
streams, which partial records it writes, which arrival counters it bumps and
which records the merging worker reads.  For many length mixes, tables with
and without shared prefixes, splits and grid sizes it checks that every index
stays inside its buffer, every block of every (kv head, sequence) is
streamed exactly once (a group's shared prefix once for all its members),
every output is written exactly once, and every merge reads exactly the
records its output's pieces wrote.  This is the host-side check of the grid
and indexes before they run on the device.
"""
import numpy as np
import pytest

COUNTER_SLOTS = 65536
SHARED_SPLIT = 4


def host_plan(S, hkv, max_blocks, bs, G, pt, num_cus=256, waves_per_cu=8, groupable=True):
    """make_plan in decode.hip: split, descriptor rounds, grouping limits."""
    units = S * hkv * max_blocks
    if pt > 0:
        chunk = pt // bs
        min_chunk = (units + COUNTER_SLOTS - 9) // (COUNTER_SLOTS - 8)
        chunk = max(chunk, min_chunk)
        workers = -(-units // chunk)
    else:
        chunk = 0
        workers = min(num_cus * waves_per_cu, units)
    workers = max(workers, 1)
    workers = (workers + 7) & ~7
    desc_rounds = 1 if pt > 0 else SHARED_SPLIT
    assert workers * desc_rounds <= COUNTER_SLOTS
    grouping = groupable and G <= 8 and bs >= 16 and hkv * S <= COUNTER_SLOTS
    return {"chunk": chunk, "workers": workers, "desc_rounds": desc_rounds,
            "max_members": 16 // G if grouping else 0,
            "grec_rows": (4 * hkv * S * G + 16 * min(workers, 8192)) if grouping else 0,
            "flat_rows": 2 * workers * desc_rounds * G}


def device_plan(tables, lens, hkv, bs, num_blocks, G, hp):
    """paged_decode_plan_kernel, sequentially (its scans give the same values)."""
    S, max_blocks = tables.shape
    max_len = max_blocks * bs
    n = np.clip(lens, 0, max_len).astype(np.int64)
    eq = np.zeros(S, bool)
    for s in range(1, S):
        b0, bp = int(tables[s, 0]), int(tables[s - 1, 0])
        eq[s] = n[s] > 0 and n[s - 1] > 0 and 0 <= b0 < num_blocks and b0 == bp
    M = hp["max_members"]
    grouped = bool(eq.any()) and M >= 2 and hkv * S <= COUNTER_SLOTS
    c = np.zeros(S, np.int64)
    gid = np.arange(S)
    groups = {}
    if grouped:
        for s in range(S):
            if not eq[s]:
                continue
            cap = min(n[s], n[s - 1]) // bs
            k = 0
            while k < cap and tables[s, k] == tables[s - 1, k]:
                k += 1
            c[s] = k
        run_start, g = 0, -1
        for s in range(S):
            if c[s] < 1:
                run_start = s
            lead = (s - run_start) % M == 0
            g += 1 if lead else 0
            gid[s] = g
        for s in range(S):
            if s > 0 and gid[s - 1] == gid[s]:
                continue
            k, m = 2**31 - 1, 1
            for j in range(1, M):
                if s + j >= S or gid[s + j] != gid[s]:
                    break
                k = min(k, int(c[s + j]))
                m += 1
            groups[int(gid[s])] = {"k": k, "m": m, "first": s}
        grouped = any(gr["m"] >= 2 and gr["k"] >= 1 for gr in groups.values())

    def real(s):
        gr = groups.get(int(gid[s]))
        return grouped and gr is not None and gr["m"] >= 2 and gr["k"] >= 1

    def lay_out(grouped_now):
        items, seqs, pos = [], [], 0
        for s in range(S):
            q = {"s_item": -1}
            if n[s] > 0:
                nb = -(-int(n[s]) // bs)
                k = groups[int(gid[s])]["k"] if (grouped_now and real(s)) else 0
                if k and groups[int(gid[s])]["first"] == s:
                    gr = groups[int(gid[s])]
                    gr["item"] = len(items)
                    items.append({"s": s, "off": 0, "len": k, "n": k * bs, "pos": pos, "m": gr["m"]})
                    pos += k
                if nb - k > 0:
                    q["s_item"] = len(items)
                    items.append({"s": s, "off": k, "len": nb - k, "n": int(n[s]), "pos": pos, "m": 0,
                                  "g_len": 0})
                    pos += nb - k
            seqs.append(q)
        return items, seqs, pos

    flags, RH = 0, 0
    for attempt in range(2):
        items, seqs, TB = lay_out(grouped)
        T = TB * hkv
        flags = 2 if grouped else (1 if eq.any() else 0)
        rounds = SHARED_SPLIT if (hp["chunk"] == 0 and flags & 1) else 1
        workers = hp["workers"] * rounds
        chunk = hp["chunk"] if hp["chunk"] > 0 else max(1, -(-T // workers))
        if not grouped:
            break
        RH = 0
        for s in range(S):
            q = seqs[s]
            if n[s] == 0:
                continue
            gr = groups[int(gid[s])]
            lead = real(s) and gr["first"] == s
            gp = ((gr["k"] + chunk - 1) // chunk + 1) * gr["m"] * G if lead else 0
            if lead:
                items[gr["item"]]["rbase"] = RH
            if q["s_item"] >= 0:
                it = items[q["s_item"]]
                it["rbase"] = RH + gp
                RH += gp + ((it["len"] + chunk - 1) // chunk + 1) * G
            else:
                RH += gp
        for s in range(S):
            q = seqs[s]
            if q["s_item"] >= 0 and real(s):
                gr = groups[int(gid[s])]
                gi = items[gr["item"]]
                si = items[q["s_item"]]
                si.update(member=s - gr["first"], g_pos=gi["pos"], g_len=gi["len"], g_rbase=gi["rbase"],
                          g_m=gi["m"])
        if RH * hkv <= hp["grec_rows"]:
            break
        grouped = False
    nv = -(-T // chunk)
    per_round = ((nv + 7) & ~7) if rounds == 1 else hp["workers"]
    W = hp["workers"]
    assert rounds <= hp["desc_rounds"]
    desc = {}
    q8 = per_round >> 3
    for i, it in enumerate(items):
        for h in range(hkv):
            a = h * TB + it["pos"]
            e = a + it["len"]
            v = (a + chunk - 1) // chunk
            while v * chunk < e:
                rd, u = divmod(v, per_round)
                wg = (u % q8) * 8 + u // q8
                assert 0 <= rd < rounds and 0 <= wg < W
                assert (rd, wg) not in desc
                desc[(rd, wg)] = {"v": v, "h": h, "i": i, "off": v * chunk - a}
                v += 1
    assert len(desc) == nv
    assert walk_descs(items, TB, hkv, chunk, rounds, hp["workers"]) == desc
    return {"items": items, "seqs": seqs, "desc": desc, "T": T, "TB": TB, "NI": len(items), "chunk": chunk,
            "rounds": rounds, "flags": flags, "RH": RH, "n": n, "groups": groups, "gid": gid,
            "grouped": grouped}


def walk_descs(items, TB, hkv, C, rounds, W, threads=1024):
    """plan_write_descs: each thread takes a contiguous range of chunk ids,
    binary-searches the first one's item and walks forward."""
    pos = [it["pos"] for it in items]
    NI = len(items)
    T = TB * hkv
    nv = -(-T // C)
    per_round = ((nv + 7) & ~7) if rounds == 1 else W
    q8 = per_round >> 3

    def find(r):
        lo, hi = 0, NI
        while hi - lo > 1:
            mid = (lo + hi) >> 1
            if pos[mid] <= r:
                lo = mid
            else:
                hi = mid
        return lo

    out = {}
    per = -(-nv // threads)
    for t in range(threads):
        v = t * per
        vend = min(v + per, nv)
        if v >= vend:
            continue
        start = v * C
        h, r = divmod(start, TB)
        i = find(r)
        rd, u = divmod(v, per_round)
        uq, ur = divmod(u, q8)
        while True:
            while i + 1 < NI and pos[i + 1] <= r:
                i += 1
            key = (rd, ur * 8 + uq)
            assert key not in out
            out[key] = {"v": v, "h": h, "i": i, "off": r - pos[i]}
            v += 1
            if v >= vend:
                break
            r += C
            if r >= TB:
                while r >= TB:
                    r -= TB
                    h += 1
                i = find(r)
            ur += 1
            if ur == q8:
                ur = 0
                uq += 1
                if uq == 8:
                    uq, rd = 0, rd + 1
    return out


def walk(pl, hkv, bs, G, hp, max_blocks):
    """Every worker's chunks (decode_chunk / grouped_chunk) and merges."""
    items, T, TB, NI, C = pl["items"], pl["T"], pl["TB"], pl["NI"], pl["chunk"]
    n = pl["n"]
    S = len(n)
    nb = -(-n // bs)
    streamed = np.zeros((hkv, S, max(max_blocks, 1)), np.int32)
    shared_reads = {}
    written = np.zeros((hkv, S), np.int32)
    counters = {}
    recs = {}
    grouped = pl["flags"] & 2
    cap_rows = max(hp["grec_rows"], hp["flat_rows"])

    def pieces(h, ipos, ilen):
        a = h * TB + ipos
        return (a + ilen - 1) // C - a // C + 1

    order = sorted(pl["desc"].items(), key=lambda kv: np.random.default_rng(kv[1]["v"]).random())
    for (rd, wg), d in order:
        start, end = d["v"] * C, min(d["v"] * C + C, T)
        h, i, off, pos = d["h"], d["i"], d["off"], start
        while True:
            it = items[i]
            ln = min(it["len"] - off, end - pos)
            assert ln >= 1 and 0 <= h < hkv
            s = it["s"]
            blocks = range(it["off"] + off, it["off"] + off + ln)
            assert blocks.stop <= nb[s] <= max_blocks
            if it["m"] > 0:   # G-item piece: members' rows
                assert grouped and it["m"] * G <= 16
                for b in blocks:
                    for j in range(it["m"]):
                        assert b < n[s + j] // bs   # inside every member's full blocks
                        shared_reads[(h, s + j, b)] = shared_reads.get((h, s + j, b), 0) + 1
                pg = pieces(h, it["pos"], it["len"])
                k = d["v"] - (h * TB + it["pos"]) // C
                assert 0 <= k < pg <= -(-it["len"] // C) + 1
                rows = it["m"] * G
                row0 = h * pl["RH"] + it["rbase"] + k * rows
                for j in range(it["m"]):
                    for r in range(G):
                        key = row0 + j * G + r
                        assert key not in recs and 0 <= key < hkv * pl["RH"] <= cap_rows
                        recs[key] = (h, s + j, "g", k)
                for j in range(it["m"]):
                    counters[(h, s + j)] = counters.get((h, s + j), 0) + 1
            else:
                for b in blocks:
                    streamed[h, s, b] += 1
                ps = pieces(h, it["pos"], it["len"])
                pg = pieces(h, it["g_pos"], it["g_len"]) if grouped and it.get("g_len", 0) > 0 else 0
                whole = ps + pg == 1
                if not grouped:
                    whole = off == 0 and off + ln == it["len"]
                if whole:
                    written[h, s] += 1
                elif grouped:
                    k = d["v"] - (h * TB + it["pos"]) // C
                    row0 = h * pl["RH"] + it["rbase"] + k * G
                    for r in range(G):
                        key = row0 + r
                        assert key not in recs and 0 <= key < hkv * pl["RH"] <= cap_rows
                        recs[key] = (h, s, "s", k)
                    counters[(h, s)] = counters.get((h, s), 0) + 1
                else:   # flat: slot 0/1 of the worker, counter of the run's first worker
                    kk = 0 if pos == start else 1
                    key = ("flat", 2 * d["v"] + kk)
                    assert key not in recs and 2 * d["v"] + kk < 2 * hp["workers"] * hp["desc_rounds"]
                    recs[key] = (h, s)
                    seg = pos - off
                    fw, lw = seg // C, (seg + it["len"] - 1) // C
                    assert fw < lw and fw < COUNTER_SLOTS
                    counters[("flat", fw)] = counters.get(("flat", fw), 0) + 1
                    if counters[("flat", fw)] == lw - fw + 1:
                        for v in range(fw, lw + 1):
                            kk2 = 0 if v * C >= seg else 1
                            assert recs.get(("flat", 2 * v + kk2)) == (h, s)
                        written[h, s] += 1
                        counters[("flat", fw)] = 0
            pos += ln
            if pos >= end:
                break
            i += 1
            if i == NI:
                i, h = 0, h + 1
            off = 0
    if grouped:   # merges: each output's records, G-item pieces then S-item pieces
        for (h, s), got in counters.items():
            it_s = items[pl["seqs"][s]["s_item"]] if pl["seqs"][s]["s_item"] >= 0 else None
            gr = pl["groups"].get(int(pl["gid"][s]))
            pg = pieces(h, items[gr["item"]]["pos"], items[gr["item"]]["len"]) if (
                gr and "item" in gr and gr["m"] >= 2 and gr["k"] >= 1) else 0
            ps = pieces(h, it_s["pos"], it_s["len"]) if it_s else 0
            assert got == pg + ps and h * S + s < COUNTER_SLOTS
            for c in range(pg):
                gi = items[gr["item"]]
                mem = s - gr["first"]
                for r in range(G):
                    key = h * pl["RH"] + gi["rbase"] + c * gi["m"] * G + mem * G + r
                    assert recs[key] == (h, s, "g", c)
            for c in range(ps):
                for r in range(G):
                    key = h * pl["RH"] + it_s["rbase"] + c * G + r
                    assert recs[key] == (h, s, "s", c)
            written[h, s] += 1
    else:
        assert all(v == 0 for v in counters.values())
    # every block of every (kv head, sequence) is read exactly once: by the
    # sequence's own items, or by its group's G-item for all members
    for h in range(hkv):
        for s in range(S):
            for b in range(nb[s]):
                assert streamed[h, s, b] + shared_reads.get((h, s, b), 0) == 1, (h, s, b)
            assert not streamed[h, s, nb[s]:].any()
            assert written[h, s] == (1 if nb[s] > 0 else 0), (h, s)


def replay(tables, lens, hkv, bs, pt, G=1, num_blocks=None, **kw):
    tables = np.asarray(tables, np.int64)
    S, mb = tables.shape
    num_blocks = num_blocks if num_blocks is not None else int(tables.max(initial=0)) + 1
    hp = host_plan(S, hkv, mb, bs, G, pt, **kw)
    pl = device_plan(tables, np.asarray(lens), hkv, bs, num_blocks, G, hp)
    walk(pl, hkv, bs, G, hp, mb)
    return pl


def private_tables(lens, bs, mb, rng):
    """Tables with every sequence on its own blocks, in random places."""
    S = len(lens)
    ids = rng.permutation(S * mb)
    t = -np.ones((S, mb), np.int64)
    for s in range(S):
        k = -(-int(min(lens[s], mb * bs)) // bs)
        t[s, :k] = ids[s * mb:s * mb + k]
    return t


def forked_tables(prompt_lens, n, extra, bs, rng, mb=None):
    """n candidates per prompt sharing its full blocks; the partial last block
    and `extra` further tokens on blocks of their own (copy-on-write)."""
    S = len(prompt_lens) * n
    lens = np.array([p + extra for p in prompt_lens for _ in range(n)])
    mb = mb or int(max(-(-lens // bs)))
    t = -np.ones((S, mb), np.int64)
    nxt = 0
    for pi, p in enumerate(prompt_lens):
        full = p // bs
        shared_ids = list(range(nxt, nxt + full))
        nxt += full
        for j in range(n):
            s = pi * n + j
            t[s, :full] = shared_ids
            k = -(-int(lens[s]) // bs)
            for b in range(full, k):
                t[s, b] = nxt
                nxt += 1
    perm = rng.permutation(nxt)
    return np.where(t >= 0, perm[np.maximum(t, 0)], -1), lens


CASES = [
    ([1, 15, 16, 33], 4, 3, 16, 0),
    ([1, 15, 16, 33], 4, 3, 16, 16),
    ([700, 5, 2048, 130, 0, 64], 3, 128, 16, 0),
    ([700, 5, 2048, 130, 0, 64], 3, 128, 16, 16),
    ([700, 5, 2048, 130, 0, 64], 3, 128, 16, 48),
    ([4096] * 3 + [16] * 40, 2, 256, 16, 0),
    ([9000, 3], 1, 64, 16, 0),              # length above the table: clamped
    ([0, 0, 0], 2, 4, 16, 0),
]


@pytest.mark.parametrize("case", CASES)
def test_flat_bookkeeping(case):
    lens, hkv, mb, bs, pt = case
    t = private_tables(lens, bs, mb, np.random.default_rng(1))
    pl = replay(t, lens, hkv, bs, pt)
    assert pl["flags"] == 0


@pytest.mark.parametrize("G", [1, 4, 8])
@pytest.mark.parametrize("pt", [0, 16, 64])
@pytest.mark.parametrize("shape", [([1023] * 3, 4, 1), ([95, 80, 130], 4, 5), ([1024] * 2, 4, 1),
                                   ([47], 4, 1), ([200, 31], 8, 40), ([16, 16], 3, 0)])
def test_grouped_bookkeeping(shape, pt, G):
    prompts, n, extra = shape
    rng = np.random.default_rng(7)
    t, lens = forked_tables(prompts, n, extra, 16, rng)
    pl = replay(t, lens, 2, 16, pt, G=G)
    if G <= 8 and min(prompts) >= 16:
        assert pl["flags"] == 2, "forked candidates should be grouped"


def test_shared_first_block_without_a_full_shared_block_stays_flat():
    """Candidates that share only a partial first block have nothing to read
    once: the plan stays flat (the L2-sharing mode)."""
    t = np.array([[5, -1]] * 4 + [[7, 8]] * 2, np.int64)   # 10 tokens on one shared block; 20 on two
    lens = np.array([10, 10, 10, 10, 20, 20])
    t[5, 0] = 9
    pl = replay(t, lens, 2, 16, 0, num_blocks=10)
    assert pl["flags"] == 1


def test_grouping_is_off_for_small_blocks_and_wide_groups():
    t, lens = forked_tables([100, 64], 4, 3, 8, np.random.default_rng(4))
    assert replay(t, lens, 2, 8, 0)["flags"] == 1           # block size 8: no 16-token tiles
    t, lens = forked_tables([100, 64], 4, 3, 16, np.random.default_rng(4))
    assert replay(t, lens, 1, 16, 0, G=16)["flags"] == 1    # 16 query rows: one member per group


def test_group_records_fall_back_to_flat_when_short():
    t, lens = forked_tables([400] * 4, 4, 2, 16, np.random.default_rng(5))
    hp = host_plan(t.shape[0], 2, t.shape[1], 16, 1, 0)
    hp["grec_rows"] = 3   # far too few rows: the plan is laid out flat
    pl = device_plan(t, lens, 2, 16, int(t.max()) + 1, 1, hp)
    assert pl["flags"] == 1
    walk(pl, 2, 16, 1, hp, t.shape[1])


@pytest.mark.parametrize("seed", range(10))
@pytest.mark.parametrize("cus", [4, 256])
def test_random_bookkeeping(seed, cus):
    rng = np.random.default_rng(seed)
    bs = int(rng.choice([8, 16, 32, 64]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    hkv = int(rng.integers(1, 9))
    if seed % 2:
        prompts = rng.integers(0, 300, size=int(rng.integers(1, 40))).tolist()
        t, lens = forked_tables(prompts, int(rng.integers(1, 9)), int(rng.integers(0, 40)), bs, rng)
        # shuffle some rows so runs of candidates are broken up
        if seed % 3 == 0:
            perm = rng.permutation(len(lens))
            t, lens = t[perm], lens[perm]
    else:
        S = int(rng.integers(1, 300))
        mb = int(rng.integers(1, 80))
        lens = rng.integers(0, mb * bs + 1, size=S)
        t = private_tables(lens, bs, mb, rng)
    pt = int(rng.choice([0, bs, 3 * bs, 32 * bs]))
    replay(t, lens, hkv, bs, pt, G=G, num_cus=cus, waves_per_cu=int(rng.integers(1, 20)))


def test_workload_shapes_fit():
    import workloads as W
    from oracle.paging import plan
    for wl in W.full_configs().values():
        tables = plan(wl, W.free_list_order(wl))["tables"]
        pl = replay(tables, wl.context_lens, wl.num_kv_heads, wl.block_size, wl.partition_tokens,
                    G=wl.group, num_blocks=wl.num_blocks)
        shared = len(set(wl.parent)) < wl.num_seqs
        assert bool(pl["flags"] & 2) == shared, wl.name
