"""The grouped GEMM's tile scheduler, restated on the CPU: every (slot, M tile, N tile) listed once,
and the per-XCD lists fit the sizes the host allocates.

`gemm::schedule_kernel` (csrc/gemm.hip) turns the slot offsets of a permuted batch into eight
per-XCD tile lists.  Units of up to four 128-row M tiles of one slot (with all their N tiles) are
sorted by key (largest first: full units, then the last unit of each slot by its row blocks),
dealt serpentine over the eight XCDs (sorted position i goes to XCD i % 8, or 7 - i % 8 on odd
rounds), and each XCD's list takes its units alternately from its larger and its smaller half.
The host sizes each list for an eighth of the tile bound plus one unit (`gemm_tile_slots`); if a
list would overflow, the kernel falls back to contiguous runs.  This test mirrors that arithmetic
step for step on seeded routings (the bench workloads' own, and random skewed, uniform and
one-expert batches) and checks coverage, disjointness and capacity, and that the balanced order
never needs the fallback on them.  The device kernel itself is exercised by every GPU test that
takes the matrix-core path (`tests/test_gpu_tile_order.py` compares both orders bit for bit).
"""
import numpy as np
import pytest

BM = 128
UNIT_M = 4
KEYS = UNIT_M * (BM // 32 + 4) + 1  # unit keys 0 .. 32
LDS_MAX = 150 * 1024


def tiles_max(R, S, nt):
    return (R // BM + min(R, S)) * nt


def tile_slots(R, S, nt):
    m = tiles_max(R, S, nt)
    return 0 if m == 0 else ((m + 7) // 8 + UNIT_M * nt) * 8


def schedule(counts, cap, nt_gu, nt_dn):
    """Returns ('balanced', {gemm: {x: [(s, m_tile, n)] in list order}}) or ('fallback', None)."""
    S = len(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    mt, nu, klast = [], [], []
    for s in range(S):
        lo = min(max(off[s], 0), cap)
        hi = min(max(off[s + 1], lo), cap)
        n = hi - lo
        m = (n + BM - 1) // BM
        mt.append(m)
        if m > 0:
            u = (m + UNIT_M - 1) // UNIT_M
            mtl = m - UNIT_M * (u - 1)            # M tiles of the slot's last unit
            rl = n - BM * (m - 1)                  # rows of the slot's last M tile
            klast.append((BM // 32 + 4) * (mtl - 1) + (rl + 31) // 32 + 4)
        else:
            u = 0
            klast.append(0)
        nu.append(u)
    umax = tiles_max(cap, S, 1)
    # full units (key KEYS-1) first, in slot order; then the other last units by key, descending,
    # slot order within a key
    useq, keyq = [], []
    for s in range(S):
        nf = (nu[s] - 1) + (1 if klast[s] == KEYS - 1 else 0) if nu[s] > 0 else 0
        for i in range(nf):
            useq.append((i, s))
            keyq.append(KEYS - 1)
    for key in range(KEYS - 2, -1, -1):
        for s in range(S):
            if nu[s] > 0 and klast[s] == key:
                useq.append((nu[s] - 1, s))
                keyq.append(key)
    U = len(useq)
    need = 4 * (S + 1) + 4 * (4 * umax)  # slot bases; per unit two words, per M tile two
    if not (umax > 0 and U <= umax and need <= LDS_MAX):
        return "fallback", None
    cap_gu, cap_dn = tile_slots(cap, S, nt_gu) // 8, tile_slots(cap, S, nt_dn) // 8
    lists = {}
    xcnt = [0] * 8
    order = {}
    for x in range(8):
        jl = U >> 3
        J = jl + (1 if 8 * jl + ((7 - x) if (jl & 1) else x) < U else 0)
        JH, JC = (J + 1) >> 1, J >> 1
        seq = []
        for p in range(J):
            if (x & 1) == 0:
                j = JH + (p >> 1) if (p & 1) else (p >> 1)
            else:
                j = (p >> 1) if (p & 1) else (JH + (p >> 1) if (p >> 1) < JC else (p >> 1))
            seq.append(8 * j + ((7 - x) if (j & 1) else x))
        assert sorted(seq) == [i for i in range(U) if (i % 8 == x if (i // 8) % 2 == 0 else 7 - i % 8 == x)]
        order[x] = seq
        xcnt[x] = sum(min(UNIT_M, mt[useq[i][1]] - UNIT_M * useq[i][0]) for i in seq)
    if any(xcnt[x] * nt_gu > cap_gu or xcnt[x] * nt_dn > cap_dn for x in range(8)):
        return "fallback", None
    for g, nt, cx in (("gate_up", nt_gu, cap_gu), ("down", nt_dn, cap_dn)):
        lists[g] = {}
        for x in range(8):
            entries = []
            for i in order[x]:
                ui, s = useq[i]
                for mm in range(min(UNIT_M, mt[s] - UNIT_M * ui)):
                    for n in range(nt):
                        entries.append((s, UNIT_M * ui + mm, n))
            assert len(entries) == xcnt[x] * nt <= cx
            lists[g][x] = entries
    return "balanced", lists


def check(counts, cap, nt_gu=8, nt_dn=16):
    kind, lists = schedule(counts, cap, nt_gu, nt_dn)
    assert kind == "balanced"
    mt = [(min(c, cap) + BM - 1) // BM for c in counts]
    for g, nt in (("gate_up", nt_gu), ("down", nt_dn)):
        got = [e for x in range(8) for e in lists[g][x]]
        want = {(s, m, n) for s in range(len(counts)) for m in range(mt[s]) for n in range(nt)}
        assert len(got) == len(set(got)), "a tile listed twice"
        assert set(got) == want, "a tile missing"
    return lists


def test_random_routings_balanced_and_covered():
    rng = np.random.default_rng(0)
    for _ in range(120):
        S = int(rng.choice([1, 2, 7, 8, 64, 110, 384, 1024]))
        k = int(rng.choice([1, 2, 8]))
        T = int(rng.choice([1, 5, 16, 300, 4096]))
        R = T * k
        p = rng.zipf(1.3, size=S).astype(float) if rng.random() < 0.5 else rng.random(S)
        p /= p.sum()
        c = rng.multinomial(R, p)
        if rng.random() < 0.2:
            c[:] = 0
            c[0] = R
        check(list(c), R)


@pytest.mark.parametrize("name,T", [("prefill_fp8_zipf", 4096), ("compact_mxfp4", 4096), ("decode_fp8", 512)])
def test_bench_workload_routings(name, T):
    from synth import gen
    cfg = gen.config(name, T=T)
    lg = gen.make_logits(cfg, batch=0)
    idx = np.argsort(-lg, axis=1, kind="stable")[:, :cfg.k]
    c = np.bincount(idx.ravel(), minlength=cfg.E)
    if cfg.resident:
        sm, _ = gen.make_slot_map(cfg)
        c = np.array([c[np.nonzero(sm == s)[0][0]] for s in range(cfg.S)])
    lists = check(list(c), T * cfg.k)
    # the serpentine deal keeps the XCDs' tile counts within a few units of each other
    ntiles = [len(lists["gate_up"][x]) for x in range(8)]
    assert max(ntiles) - min(ntiles) <= 3 * UNIT_M * 8


def test_empty_and_single_row():
    # no rows: the host launches no GEMM (zero list slots); the kernel would take the fallback
    assert tile_slots(0, 16, 8) == 0 and schedule([0] * 16, 0, 8, 16)[0] == "fallback"
    check([1] + [0] * 15, 1)
    check([0] * 383 + [8], 8)
