"""Pins for the oracle's routing and align steps (CPU only)."""
import numpy as np
import pytest

import oracle
from golden_io import lines, closed_form, kv


def test_route_hand_cases():
    for ln in lines("route_tiny.txt"):
        head, lg, mk, ids, ws, err = [f.strip() for f in ln.split("|")]
        E, k = map(int, head.split())
        logits = np.array([[float(v) for v in lg.split()]], dtype=np.float32)
        mask = None if mk == "-" else np.array([int(v) for v in mk.split()], dtype=np.uint8)
        got_ids, got_w, got_err = oracle.route(logits, mask, k)
        assert got_ids[0].tolist() == [int(v) for v in ids.split()], ln
        want_w = [closed_form(v) for v in ws.split()]
        assert np.allclose(got_w[0], want_w, rtol=0, atol=1e-15), ln
        assert got_err == int(err), ln


def _random_logits(rng, T, E, ties=False):
    lg = rng.standard_normal((T, E)).astype(np.float32)
    if ties:  # coarse values so equal logits are common, and signed zeros
        lg = np.round(lg * 2).astype(np.float32) / 2
        lg[lg == 0] = np.where(rng.random((lg == 0).sum()) < 0.5, -0.0, 0.0)
    return lg


@pytest.mark.parametrize("ties", [False, True])
def test_route_matches_brute_force_sort(ties):
    rng = np.random.default_rng(11)
    T, E, k = 64, 40, 6
    lg = _random_logits(rng, T, E, ties)
    ids, w, err = oracle.route(lg, None, k)
    assert err == 0
    for t in range(T):
        # brute force: Python's sort of (-logit, id); -0.0 == 0.0 compare equal
        order = sorted(range(E), key=lambda e: (-float(lg[t, e]), e))[:k]
        assert ids[t].tolist() == order
        z = np.exp(lg[t, order].astype(np.float64) - lg[t, order].max())
        assert np.allclose(w[t], z / z.sum(), rtol=1e-14, atol=0)


def test_route_invariants():
    rng = np.random.default_rng(5)
    lg = _random_logits(rng, 200, 256) * 3
    ids, w, err = oracle.route(lg, None, 8)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(np.diff(w, axis=1) <= 0)                     # best first
    assert all(len(set(r)) == 8 for r in ids.tolist())         # distinct experts
    # chosen logits dominate every unchosen one
    for t in range(200):
        rest = np.setdiff1d(np.arange(256), ids[t])
        assert lg[t, ids[t]].min() >= lg[t, rest].max()


def test_route_mask_excludes_experts():
    rng = np.random.default_rng(9)
    lg = _random_logits(rng, 50, 64)
    mask = (rng.random(64) < 0.3).astype(np.uint8)
    ids, w, err = oracle.route(lg, mask, 4)
    assert err == 0
    assert np.all(mask[ids] == 1)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-12)


def test_align_hand_case():
    g = kv("align_tiny.txt")
    T, k, E, bm = (int(g[n][0]) for n in ("T", "k", "E", "block_m"))
    ids = np.array([int(v) for v in g["ids"]], dtype=np.int32).reshape(T, k)
    soe = np.array([int(v) for v in g["slot_of_expert"]], dtype=np.int32)
    al = oracle.align(ids, E, bm, soe)
    for name in ("counts", "seg_offset", "sorted_pair", "block_slot"):
        assert al[name].tolist() == [int(v) for v in g[name]], name
    assert al["n_padded"] == int(g["n_padded"][0])
    assert al["err"] == int(g["err"][0])


@pytest.mark.parametrize("T,k,E,bm", [(1, 8, 256, 16), (37, 3, 10, 4), (300, 8, 64, 32), (64, 2, 8, 128)])
def test_align_matches_brute_force(T, k, E, bm):
    rng = np.random.default_rng(T * 1000 + E)
    p = rng.random(E) ** 3
    ids = np.stack([rng.choice(E, k, replace=False, p=p / p.sum()) for _ in range(T)]).astype(np.int32)
    soe = rng.permutation(E).astype(np.int32)
    al = oracle.align(ids, E, bm, soe)
    # brute force: sort pair indices by (expert, pair index), then pad each segment
    flat = ids.reshape(-1)
    order = sorted(range(T * k), key=lambda q: (flat[q], q))
    want, want_bs = [], []
    for e in range(E):
        seg = [q for q in order if flat[q] == e]
        if seg:
            nb = -(-len(seg) // bm)
            want += seg + [T * k] * (nb * bm - len(seg))
            want_bs += [soe[e]] * nb
    assert al["sorted_pair"].tolist() == want
    assert al["block_slot"].tolist() == want_bs
    # invariants
    real = al["sorted_pair"][al["sorted_pair"] != T * k]
    assert np.array_equal(np.sort(real), np.arange(T * k))      # every pair exactly once
    assert np.all(np.bincount(real // k, minlength=T) == k)    # each token k times
    assert al["counts"].sum() == T * k
    assert np.all(np.diff(al["seg_offset"]) % bm == 0)
    for e in range(E):
        seg = al["sorted_pair"][al["seg_offset"][e]:al["seg_offset"][e + 1]]
        r = seg[seg != T * k]
        assert np.all(flat[r] == e)
        assert np.all(seg[:r.size] == r)                        # padding only at the tail
    assert al["n_padded"] <= oracle.align_capacity(T, k, E, bm)
    assert al["err"] == 0


def test_align_capacity_bound_is_tight():
    # every expert gets one pair more than a multiple of block_m -> worst padding
    T, k, E, bm = 20, 1, 4, 4
    ids = (np.arange(T) % E).astype(np.int32).reshape(T, 1)    # 5 pairs per expert
    al = oracle.align(ids, E, bm, np.arange(E, dtype=np.int32))
    assert al["n_padded"] == E * 8 == oracle.align_capacity(T, k, E, bm)


def test_align_counts_invalid_and_nonresident():
    ids = np.array([[0, -1], [1, 0]], dtype=np.int32)
    al = oracle.align(ids, 2, 2, np.array([0, -1], dtype=np.int32))
    assert al["counts"].tolist() == [2, 1]
    assert al["sorted_pair"].tolist() == [0, 3, 2, 4]
    assert al["block_slot"].tolist() == [0, -1]
    assert al["err"] == 2          # one invalid id, one pair on a non-resident expert
