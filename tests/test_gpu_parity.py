"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Integer outputs (route ids, every align output) must be bit-exact; route
weights within 1e-6; layer outputs within max|out - ref| <= 2e-2 * max|ref|
against the fp64 oracle in the same activation mode.
"""
import numpy as np
import pytest

import oracle
import moe_expert_layer_topk_amd as moe
from gen import CONFIGS, make_layer, make_bank
from gen.configs import Config
from harness import device_pool, device_inputs, oracle_layer, rel_max_err, bank_on_device

pytestmark = pytest.mark.gpu

OUT_TOL = 2e-2
W_TOL = 1e-6


def _say(*a):
    print(*a, flush=True)


def check_route(logits_np, mask_np, k, ids, w, err):
    oi, ow, oe = oracle.route(logits_np, mask_np, k)
    assert np.array_equal(ids.cpu().numpy(), oi), "route ids differ"
    assert np.abs(w.cpu().numpy().astype(np.float64) - ow).max() <= W_TOL
    assert int(err.item()) == oe


def check_align(al, ref, block_m):
    n = int(al["n_padded"].item())
    assert n == ref["n_padded"]
    assert np.array_equal(al["sorted_pair"][:n].cpu().numpy(), ref["sorted_pair"])
    assert np.array_equal(al["block_slot"][:n // block_m].cpu().numpy(), ref["block_slot"])
    assert np.array_equal(al["counts"].cpu().numpy(), ref["counts"])
    assert np.array_equal(al["seg_offset"].cpu().numpy(), ref["seg_offset"])
    assert int(al["err"].item()) == ref["err"]


def run_layer(li, bank, dev, block_m, act_mode, sample=None, bank_dev=None, cache=None, fused=False):
    c = li.cfg
    _say(f"[layer] {c.name} T={li.T} layer={li.layer} block_m={block_m} act={act_mode} fused={fused}")
    pool = device_pool(li, bank, dev, bank_dev)
    x, logits, soe, mask = device_inputs(li, dev)
    out, (ids, w, rerr), al = moe.layer(pool, x, logits, c.k, soe, block_m, act_mode, mask=mask, fused=fused)
    import torch
    torch.cuda.synchronize()
    ref = oracle_layer(li, bank, block_m, act_mode, token_subset=sample, cache=cache)
    if sample is None:
        check_route(li.logits, li.mask, c.k, ids, w, rerr)
    else:
        oi, ow, _ = oracle.route(li.logits[sample], li.mask, c.k)
        assert np.array_equal(ids.cpu().numpy()[sample], oi)
        assert np.abs(w.cpu().numpy()[sample].astype(np.float64) - ow).max() <= W_TOL
    check_align(al, ref, block_m)
    rows = None if sample is None else np.asarray(sample)
    e = rel_max_err(out, ref["out"], rows)
    _say(f"    rel max err {e:.3e}")
    assert e <= OUT_TOL
    return out, ref


# ---------------------------------------------------------------- route
def test_route_c0(gpu):
    li = make_layer(CONFIGS["C0"], 16, 0)
    x, logits, soe, mask = device_inputs(li, gpu)
    ids, w, err = moe.route(logits, 2)
    check_route(li.logits, None, 2, ids, w, err)


def test_route_ties_signed_zero_and_masks(gpu):
    import torch
    rng = np.random.default_rng(0)
    T, E, k = 200, 64, 6
    lg = (np.round(rng.standard_normal((T, E)) * 2) / 2).astype(np.float32)
    lg[lg == 0] = np.where(rng.random((lg == 0).sum()) < 0.5, -0.0, 0.0).astype(np.float32)
    ids, w, err = moe.route(torch.from_numpy(lg).to(gpu), k)
    check_route(lg, None, k, ids, w, err)
    mask = (rng.random(E) < 0.5).astype(np.uint8)
    ids, w, err = moe.route(torch.from_numpy(lg).to(gpu), k, mask=torch.from_numpy(mask).to(gpu))
    check_route(lg, mask, k, ids, w, err)
    few = np.zeros(E, np.uint8)
    few[[3, 17, 40]] = 1                       # fewer than k allowed experts
    ids, w, err = moe.route(torch.from_numpy(lg).to(gpu), k, mask=torch.from_numpy(few).to(gpu))
    check_route(lg, few, k, ids, w, err)
    assert int(err.item()) == T


@pytest.mark.parametrize("name,T", [("C1", 32), ("C2", 16384), ("C3", 32), ("C3", 4096)])
def test_route_full_size(gpu, name, T):
    c = CONFIGS[name]
    li = make_layer(c, T, 0)
    x, logits, soe, mask = device_inputs(li, gpu)
    ids, w, err = moe.route(logits, c.k, mask=mask)
    check_route(li.logits, li.mask, c.k, ids, w, err)


def test_route_e1024_k32(gpu):
    import torch
    rng = np.random.default_rng(4)
    lg = rng.standard_normal((37, 1024)).astype(np.float32)
    ids, w, err = moe.route(torch.from_numpy(lg).to(gpu), 32)
    check_route(lg, None, 32, ids, w, err)


# ---------------------------------------------------------------- align
def _rand_ids(rng, T, k, E, skew=3.0):
    p = rng.random(E) ** skew
    p /= p.sum()
    return np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T,k,E,block_m", [(1, 8, 256, 16), (32, 8, 256, 16), (37, 3, 10, 64), (300, 8, 64, 32),
                                           (1024, 8, 256, 256), (1025, 8, 256, 128), (4096, 10, 512, 128),
                                           (16384, 8, 256, 128), (5000, 2, 1000, 16)])
def test_align_matches_oracle(gpu, T, k, E, block_m):
    import torch
    rng = np.random.default_rng(T + E)
    ids = _rand_ids(rng, T, k, E)
    soe = rng.permutation(E).astype(np.int32)
    soe[rng.random(E) < 0.05] = -1             # some experts not resident
    _say(f"[align] T={T} k={k} E={E} bm={block_m} NP={T * k}")
    al = moe.align(torch.from_numpy(ids).to(gpu), E, block_m, torch.from_numpy(soe).to(gpu))
    ref = oracle.align(ids, E, block_m, soe)
    check_align(al, ref, block_m)
    al2 = moe.align(torch.from_numpy(ids).to(gpu), E, block_m, torch.from_numpy(soe).to(gpu))
    n = ref["n_padded"]
    assert torch.equal(al["sorted_pair"][:n], al2["sorted_pair"][:n])   # run-to-run identical


@pytest.mark.parametrize("name,T,block_m", [("C0", 16, 16), ("C1", 1, 16), ("C1", 32, 16), ("C3", 32, 32),
                                            ("C1", 128, 64), ("C2", 2048, 128)])
def test_route_align_fused(gpu, name, T, block_m):
    """moe_route_align equals moe_route followed by moe_align (one kernel
    when T*k <= 1024, the two-kernel path above that)."""
    c = CONFIGS[name]
    li = make_layer(c, T, 1)
    x, logits, soe, mask = device_inputs(li, gpu)
    ids, w, al = moe.route_align(logits, c.k, block_m, soe, mask=mask)
    oi, ow, oe = oracle.route(li.logits, li.mask, c.k)
    assert np.array_equal(ids.cpu().numpy(), oi)
    assert np.abs(w.cpu().numpy().astype(np.float64) - ow).max() <= W_TOL
    ref = oracle.align(oi, c.E, block_m, li.slot_of_expert)
    err = al.pop("err").cpu().numpy()
    assert err[0] == oe
    al["err"] = torch_scalar(err[1])
    check_align(al, ref, block_m)


def torch_scalar(v):
    import torch
    return torch.tensor([int(v)], dtype=torch.int32)


def test_route_align_fused_shortfall(gpu):
    """Tokens with fewer than k allowed experts: -1 entries are left out of
    align and counted in both error words."""
    import torch
    rng = np.random.default_rng(3)
    T, E, k = 20, 64, 6
    lg = rng.standard_normal((T, E)).astype(np.float32)
    mask = np.zeros(E, np.uint8)
    mask[[1, 5, 9, 30]] = 1
    soe = rng.permutation(E).astype(np.int32)
    ids, w, al = moe.route_align(torch.from_numpy(lg).to(gpu), k, 16, torch.from_numpy(soe).to(gpu),
                                 mask=torch.from_numpy(mask).to(gpu))
    oi, ow, oe = oracle.route(lg, mask, k)
    assert np.array_equal(ids.cpu().numpy(), oi)
    ref = oracle.align(oi, E, 16, soe)
    err = al.pop("err").cpu().numpy()
    assert err[0] == oe == T
    al["err"] = torch_scalar(err[1])
    check_align(al, ref, 16)


def test_align_duplicate_ids_in_a_token(gpu):
    """An id listed twice by one token (moe_align takes any ids): still the
    stable counting sort of the oracle."""
    import torch
    rng = np.random.default_rng(8)
    for T in (3, 40, 200):
        ids = rng.integers(0, 6, size=(T, 4)).astype(np.int32)
        ids[0] = [2, 2, 5, 2]
        soe = np.arange(6, dtype=np.int32)
        al = moe.align(torch.from_numpy(ids).to(gpu), 6, 16, torch.from_numpy(soe).to(gpu))
        check_align(al, oracle.align(ids, 6, 16, soe), 16)


def test_align_invalid_ids(gpu):
    import torch
    ids = np.array([[0, -1], [1, 0], [5, 2]], dtype=np.int32)    # -1 and 5 are outside [0, E)
    soe = np.array([0, 1, 2], dtype=np.int32)
    al = moe.align(torch.from_numpy(ids).to(gpu), 3, 16, torch.from_numpy(soe).to(gpu))
    check_align(al, oracle.align(ids, 3, 16, soe), 16)
    big = np.random.default_rng(1).integers(-2, 260, size=(2000, 8)).astype(np.int32)   # multi-block path
    soe = np.arange(256, dtype=np.int32)
    al = moe.align(torch.from_numpy(big).to(gpu), 256, 64, torch.from_numpy(soe).to(gpu))
    check_align(al, oracle.align(big, 256, 64, soe), 64)


# ---------------------------------------------------------------- expert FFN / whole layer
@pytest.mark.parametrize("act_mode,block_m", [(0, 16), (0, 32), (0, 64), (1, 64), (1, 128)])
def test_layer_c0(gpu, act_mode, block_m):
    c = CONFIGS["C0"]
    run_layer(make_layer(c, 16, 0), make_bank(c), gpu, block_m, act_mode)


MID = Config("mid", 70, (300, 50), 256, 128, 16, 4, 1, 0.1, True, slots=0)
MIX = Config("mix", 71, (200, 40), 256, 128, 16, 4, 1, 0.1, True, slots=0, int4_frac=0.4, resident_all_at=1)
# several K steps in both products (H / 128 = 4, I / 128 = 3), ragged blocks, int4 mixed in
WIDE = Config("wide", 72, (700,), 512, 384, 24, 6, 1, 0.1, True, slots=0, int4_frac=0.25, resident_all_at=1)
# inter 640: the decode down kernel's 12-chunk variant (FP8 and int4 slots), five int4 groups along K
LONGI = Config("longi", 73, (40, 200), 256, 640, 16, 4, 1, 0.1, True, slots=0, int4_frac=0.4, resident_all_at=1)


@pytest.mark.parametrize("cfg,T,act_mode,block_m", [(MID, 300, 1, 64), (MID, 300, 1, 128), (MID, 50, 0, 16),
                                                    (MID, 50, 0, 64), (MID, 50, 1, 64), (MIX, 200, 1, 128),
                                                    (MIX, 40, 0, 16), (MIX, 40, 0, 32), (MIX, 40, 1, 64),
                                                    (WIDE, 700, 1, 128), (WIDE, 700, 1, 64), (LONGI, 40, 0, 16),
                                                    (LONGI, 200, 1, 128)])
def test_layer_mid_sizes(gpu, cfg, T, act_mode, block_m):
    run_layer(make_layer(cfg, T, 0), make_bank(cfg), gpu, block_m, act_mode)


def test_layer_single_token(gpu):
    c = CONFIGS["C1"]
    bank = make_bank(c)
    run_layer(make_layer(c, 1, 3), bank, gpu, 16, 0)
    run_layer(make_layer(c, 1, 3), bank, gpu, 64, 1)


def test_nonresident_expert_contributes_zero(gpu):
    c = CONFIGS["C0"]
    li = make_layer(c, 16, 0)
    ids, _, _ = oracle.route(li.logits, None, c.k)
    li.slot_of_expert[int(ids[0, 0])] = -1
    for act, bm in ((0, 16), (1, 64)):
        out, ref = run_layer(li, make_bank(c), gpu, bm, act)
        assert ref["err"] > 0


def test_nonresident_expert_contributes_zero_fp8_tiles(gpu):
    li = make_layer(WIDE, 700, 1)
    ids, _, _ = oracle.route(li.logits, None, WIDE.k)
    for e in (int(ids[0, 0]), int(ids[5, 2])):
        li.slot_of_expert[e] = -1
    out, ref = run_layer(li, make_bank(WIDE), gpu, 128, 1)
    assert ref["err"] > 0


@pytest.mark.parametrize("T", [1, 8, 32])
def test_layer_c1_decode(gpu, T):
    c = CONFIGS["C1"]
    bank = make_bank(c)
    li = make_layer(c, T, 7)
    run_layer(li, bank, gpu, 16, 0, fused=True)
    run_layer(li, bank, gpu, 32, 0)


def test_layer_c3_masked_decode(gpu):
    c = CONFIGS["C3"]
    run_layer(make_layer(c, 32, 5), make_bank(c), gpu, 16, 0)


def test_layer_c4_mixed_decode(gpu):
    c = CONFIGS["C4"]
    li = make_layer(c, 8, 2)
    assert (li.slot_fmt == 1).any()
    run_layer(li, make_bank(c), gpu, 16, 0)
    run_layer(li, make_bank(c), gpu, 64, 1)


# ---------------------------------------------------------------- whole layer in one call (moe_layer)
# E = 1024 experts: the widest router the kernels take (16 logits per lane)
WIDEE = Config("widee", 74, (12, 40), 128, 64, 1024, 8, 1, 0.1, True, slots=0)


def run_layer_call(li, bank, dev, block_m=16, act_mode=0):
    """moe_layer against the oracle, and bit-identical to the separate calls
    (route, align, expert FFN) on the same inputs."""
    import torch
    out, ref = run_layer(li, bank, dev, block_m, act_mode, fused="layer")
    out2, _, _ = moe.layer(device_pool(li, bank, dev), *_layer_args(li, dev), block_m, act_mode,
                           mask=device_inputs(li, dev)[3])
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), "moe_layer differs from the separate calls"
    return out, ref


def _layer_args(li, dev):
    x, logits, soe, _ = device_inputs(li, dev)
    return x, logits, li.cfg.k, soe


@pytest.mark.parametrize("T", [1, 8, 16, 17, 32, 64])
def test_layer_call_c1(gpu, T):
    """Route inside the gate/up kernel up to 16 tokens, the route kernel
    above; the pairs sorted in every workgroup; T = 64 is the largest
    decode batch (512 pairs)."""
    c = CONFIGS["C1"]
    run_layer_call(make_layer(c, T, 4), make_bank(c), gpu)


@pytest.mark.parametrize("T", [16, 32])
def test_layer_call_c3_masked(gpu, T):
    c = CONFIGS["C3"]
    run_layer_call(make_layer(c, T, 2), make_bank(c), gpu)


def test_layer_call_c4_mixed(gpu):
    c = CONFIGS["C4"]
    li = make_layer(c, 8, 3)
    assert (li.slot_fmt == 1).any()
    run_layer_call(li, make_bank(c), gpu)


@pytest.mark.parametrize("cfg,T", [(WIDEE, 12), (WIDEE, 40), (LONGI, 40), (MIX, 40), (CONFIGS["C0"], 16)])
def test_layer_call_shapes(gpu, cfg, T):
    run_layer_call(make_layer(cfg, T, 0), make_bank(cfg), gpu)


def test_layer_call_shortfall(gpu):
    """One allowed expert for k = 2: every token is short by one; the -1
    entries are counted by route and align and left out of the FFN."""
    c = CONFIGS["C0"]
    li = make_layer(c, 16, 0)
    li.mask = np.zeros(c.E, np.uint8)
    li.mask[5] = 1
    out, ref = run_layer_call(li, make_bank(c), gpu)
    assert ref["err"] == 16


def test_layer_call_nonresident(gpu):
    """A routed expert without a slot contributes nothing and is counted."""
    c = CONFIGS["C1"]
    li = make_layer(c, 8, 1)
    ids, _, _ = oracle.route(li.logits, li.mask, c.k)
    for e in (int(ids[0, 0]), int(ids[3, 4])):
        li.slot_of_expert[e] = -1
    out, ref = run_layer_call(li, make_bank(c), gpu)
    assert ref["err"] > 0


def test_layer_call_batched_falls_back(gpu):
    """Shapes outside the decode path run the separate calls' kernels."""
    run_layer_call(make_layer(MID, 300, 0), make_bank(MID), gpu, 64, 1)


def block_complete_tokens(li, block_m):
    """Tokens whose rows cover every align block of the layer: for each block,
    the tokens of its first and its last real row (a segment's last, partial
    block included), taken from the oracle's own route and align."""
    c = li.cfg
    ids, _, _ = oracle.route(li.logits, li.mask, c.k)
    al = oracle.align(ids, c.E, block_m, li.slot_of_expert)
    NP, sp = li.T * c.k, al["sorted_pair"]
    toks = set()
    for b in range(al["n_padded"] // block_m):
        rows = sp[b * block_m:(b + 1) * block_m]
        real = rows[rows < NP]
        if real.size:
            toks.update((int(real[0]) // c.k, int(real[-1]) // c.k))
    return np.array(sorted(toks)), al["n_padded"] // block_m


@pytest.mark.parametrize("name,T,block_m", [("C2", 16384, 128), ("C4", 8192, 128), ("C3", 4096, 128)])
def test_layer_batched_full_size_every_block(gpu, name, T, block_m):
    """Full-size batched layers in the launch configuration the benchmark
    times, compared on every element of a token set that reaches every
    128-row block (first and last real row of each), so every tile, every
    segment's partial last block and every int4 block is checked."""
    from harness import BoundedCache
    c = CONFIGS[name]
    bank = make_bank(c)
    _say(f"[bank] {name}: generating {bank.n} experts")
    bdev = bank_on_device(bank, gpu)
    li = make_layer(c, T, 0)
    sample, n_blocks = block_complete_tokens(li, block_m)
    _say(f"    {sample.size} of {T} tokens cover all {n_blocks} blocks")
    run_layer(li, bank, gpu, block_m, 1, sample=sample, bank_dev=bdev, cache=BoundedCache())


# ---------------------------------------------------------------- dequant
@pytest.mark.parametrize("fmt", [0, 1])
def test_dequant_slot(gpu, fmt):
    import torch
    c = CONFIGS["C4"]
    bank = make_bank(c)
    li = make_layer(c, 8, 0)
    pool = device_pool(li, bank, gpu)
    s = int(np.nonzero(li.slot_fmt == fmt)[0][0])
    w13, w2 = moe.dequant_slot(pool, s)
    torch.cuda.synchronize()
    R13, R2 = oracle.dequant_slot(bank.slot(li.slot_src[s], fmt), fmt, c.H, c.I)
    for got, ref in ((w13, R13), (w2, R2)):
        g = got.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(g - ref) <= np.abs(ref) * 2.0 ** -23)
