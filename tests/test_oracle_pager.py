"""Pins of the slot-miss path's replacement rule (CPU only), and the
library's native pager (host logic, no GPU) against it."""
import os

import numpy as np
import pytest

import oracle
from golden_io import lines


def _golden():
    for ln in lines("lru_tiny.txt"):
        need, fills, table = [f.strip() for f in ln.split("|")]
        need = [int(v) for v in need.split()]
        fills = [] if fills == "-" else [tuple(int(a) for a in f.split(":")) for f in fills.split()]
        yield need, fills, [int(v) for v in table.split()]


def test_lru_hand_case():
    lru = oracle.LRUSlots(6, 3)
    for need, fills, table in _golden():
        t, f = lru.plan(need)
        assert f == fills and t == table
    assert (lru.hits, lru.misses) == (5, 7)


def test_lru_invariants_under_zipf_reuse():
    rng = np.random.default_rng(1)
    E, S = 64, 20
    p = (np.arange(E) + 1.0) ** -1.1
    p /= p.sum()
    lru = oracle.LRUSlots(E, S)
    for _ in range(200):
        need = rng.choice(E, rng.integers(1, 12), replace=False, p=p)
        before = list(lru.slot_of)
        t, fills = lru.plan(need)
        assert all(t[e] >= 0 for e in need)                              # everything needed is resident
        assert sorted(e for e, _ in fills) == sorted(e for e in set(need.tolist()) if before[e] < 0)
        occupied = [s for s in t if s >= 0]
        assert len(occupied) == len(set(occupied)) <= S                 # one expert per slot
        for e in range(E):                                               # hits never move
            if before[e] >= 0 and t[e] >= 0:
                assert t[e] == before[e]
    assert lru.hits > lru.misses                                         # the skew gives reuse
    with pytest.raises(ValueError):
        lru.plan(list(range(S + 1)))


def test_native_pager_matches_oracle():
    import moe_expert_layer_topk_amd as moe
    if not os.path.exists(moe.LIB_PATH):
        pytest.skip("library not built")
    for need, fills, table in _golden():
        pass
    pg = moe.Pager(2, 6, 3)
    for need, fills, table in _golden():
        t, fe, fs = pg.plan(0, need)
        assert t.tolist() == table and list(zip(fe.tolist(), fs.tolist())) == fills
    assert pg.stats(0) == (5, 7) and pg.stats(1) == (0, 0)
    rng = np.random.default_rng(7)
    E, S = 256, 102
    p = (rng.permutation(E) + 1.0) ** -1.1
    p /= p.sum()
    pg = moe.Pager(3, E, S)
    ref = [oracle.LRUSlots(E, S) for _ in range(3)]
    for step in range(60):
        for layer in range(3):
            need = rng.choice(E, 8 * int(rng.integers(1, 9)), p=p)       # duplicates allowed
            t, fe, fs = pg.plan(layer, need)
            rt, rf = ref[layer].plan(need)
            assert t.tolist() == rt and list(zip(fe.tolist(), fs.tolist())) == rf
    assert pg.stats() == (sum(r.hits for r in ref), sum(r.misses for r in ref))
    with pytest.raises(moe.MoeError):
        pg.plan(0, np.arange(S + 1))
