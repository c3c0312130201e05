"""Device-side robustness of the boundary: unusable slots, pool validation
and the workspace-poisoning debug mode (through the C ABI).

A slot-table entry outside the pool, a slot whose tag is not a format, and
an FP8 slot in a pool whose stride holds only int4 slots must all behave like
a non-resident expert (its pairs add zero): the GPU output is compared with
the oracle run on the same table with those entries set to -1. moe_layer
counts such pairs in its align error word. With poisoning on, every FFN
call must give bit-identical outputs (no workspace data is read before it is
written).
"""
import numpy as np
import pytest

import oracle
import moe_expert_layer_topk_amd as moe
from gen import CONFIGS, make_layer, make_bank, slot_bytes
from gen.configs import Config
from harness import device_pool, device_inputs, oracle_layer, rel_max_err, SlotPool_from_host

pytestmark = pytest.mark.gpu

MIX = Config("mix", 71, (200, 40), 256, 128, 16, 4, 1, 0.1, True, slots=0, int4_frac=0.4, resident_all_at=1)


def _say(*a):
    print(*a, flush=True)


def _layer_vs_oracle(li, bank, pool, dev, block_m, act_mode, soe_gpu, soe_oracle, fused):
    import torch
    x, logits, _, mask = device_inputs(li, dev)
    out, (ids, w, rerr), al = moe.layer(pool, x, logits, li.cfg.k, torch.from_numpy(soe_gpu).to(dev), block_m,
                                        act_mode, mask=mask, fused=fused)
    torch.cuda.synchronize()
    li2 = type(li)(**{**li.__dict__, "slot_of_expert": soe_oracle})
    ref = oracle_layer(li2, bank, block_m, act_mode)
    e = rel_max_err(out, ref["out"])
    _say(f"    rel max err {e:.3e}, align err {int(al['err'].item())} (oracle {ref['err']})")
    assert e <= 2e-2
    return out, al, ref


@pytest.mark.parametrize("act_mode,block_m,fused", [(0, 16, "layer"), (0, 16, False), (1, 128, "layer"),
                                                    (1, 64, False)])
def test_slot_table_entry_past_the_pool(gpu, act_mode, block_m, fused):
    c = CONFIGS["C0"] if act_mode == 0 else MIX
    T = 16 if act_mode == 0 else 200
    li = make_layer(c, T, 0)
    bank = make_bank(c)
    ids, _, _ = oracle.route(li.logits, li.mask, c.k)
    bad = sorted({int(ids[0, 0]), int(ids[3, 1])})
    soe_gpu = li.slot_of_expert.copy()
    soe_orc = li.slot_of_expert.copy()
    soe_gpu[bad[0]] = li.n_slots                          # one past the last slot
    if len(bad) > 1:
        soe_gpu[bad[1]] = li.n_slots + 1000
    soe_orc[bad] = -1
    _say(f"[slots] {c.name} T={T} act={act_mode} bm={block_m} fused={fused}: experts {bad} outside the pool")
    pool = device_pool(li, bank, gpu)
    out, al, ref = _layer_vs_oracle(li, bank, pool, gpu, block_m, act_mode, soe_gpu, soe_orc, fused)
    if fused == "layer":                                  # moe_layer checks the table against the pool
        n = ref["n_padded"]
        assert np.array_equal(al["block_slot"][:n // block_m].cpu().numpy(), ref["block_slot"])
        assert int(al["err"].item()) == ref["err"] > 0


@pytest.mark.parametrize("act_mode,block_m,fused", [(0, 16, "layer"), (0, 32, False), (1, 128, False),
                                                    (1, 128, "layer"), (1, 64, False)])
def test_fp8_slots_in_an_int4_stride_pool(gpu, act_mode, block_m, fused):
    """Stride = the int4 slot size exactly (its 16 spare tail bytes included):
    int4 slots are usable, FP8 slots are not (their layout does not fit), and
    the last slot's reads stay inside the pool."""
    import torch
    T = 40 if act_mode == 0 else 200
    li = make_layer(MIX, T, 0)
    bank = make_bank(MIX)
    # put an int4 expert in the last slot: its tail reads are the ones at the pool's end
    s4, last = int(np.nonzero(li.slot_fmt == 1)[0][0]), li.n_slots - 1
    for arr in (li.slot_src, li.slot_fmt):
        arr[[s4, last]] = arr[[last, s4]]
    e4, el = int(np.nonzero(li.slot_of_expert == s4)[0][0]), int(np.nonzero(li.slot_of_expert == last)[0][0])
    li.slot_of_expert[e4], li.slot_of_expert[el] = last, s4
    assert li.slot_fmt[last] == 1
    stride = slot_bytes(MIX.H, MIX.I, 1)
    assert moe.slot_bytes(MIX.H, MIX.I, 1) == stride
    host = np.zeros((li.n_slots, stride), dtype=np.uint8)
    for s in range(li.n_slots):
        b = bank.slot(li.slot_src[s], li.slot_fmt[s])
        host[s] = b[:stride] if b.size >= stride else np.pad(b, (0, stride - b.size))
    pool = SlotPool_from_host(host, li.slot_fmt, MIX.H, MIX.I, gpu)
    soe_orc = li.slot_of_expert.copy()
    soe_orc[[e for e in range(MIX.E) if soe_orc[e] >= 0 and li.slot_fmt[soe_orc[e]] == 0]] = -1
    _say(f"[int4 stride] T={T} act={act_mode} bm={block_m} fused={fused}")
    _layer_vs_oracle(li, bank, pool, gpu, block_m, act_mode, li.slot_of_expert.copy(), soe_orc, fused)
    err, status = moe.pool_check(pool)
    torch.cuda.synchronize()
    want = np.where(li.slot_fmt == 0, 2, 0)
    assert np.array_equal(status.cpu().numpy(), want)
    assert int(err.item()) == int((want != 0).sum())


def test_unknown_format_tag(gpu):
    import torch
    c = CONFIGS["C0"]
    li = make_layer(c, 16, 0)
    bank = make_bank(c)
    ids, _, _ = oracle.route(li.logits, li.mask, c.k)
    e = int(ids[2, 0])
    pool = device_pool(li, bank, gpu)
    pool.fmt[int(li.slot_of_expert[e])] = 7
    soe_orc = li.slot_of_expert.copy()
    soe_orc[e] = -1
    for act, bm, fused in ((0, 16, "layer"), (1, 64, False)):
        _layer_vs_oracle(li, bank, pool, gpu, bm, act, li.slot_of_expert.copy(), soe_orc, fused)
    w13, w2 = moe.dequant_slot(pool, int(li.slot_of_expert[e]))
    torch.cuda.synchronize()
    assert torch.isnan(w13).all() and torch.isnan(w2).all()


def test_pool_check_statuses(gpu):
    import torch
    li = make_layer(MIX, 40, 0)
    bank = make_bank(MIX)
    pool = device_pool(li, bank, gpu)
    S = li.n_slots
    fp8 = [s for s in range(S) if li.slot_fmt[s] == 0]
    i4 = [s for s in range(S) if li.slot_fmt[s] == 1]
    want = np.zeros(S, dtype=np.uint8)
    pool.fmt[fp8[0]] = 9
    want[fp8[0]] = 1
    # an int4 group with zero 7.5, another with an infinite scale
    off = moe.slot_part_offset(MIX.H, MIX.I, 1, 1)
    sz = pool.data[i4[0], off:off + 4].clone().view(torch.float16)
    sz[1] = 7.5
    pool.data[i4[0], off:off + 4] = sz.view(torch.uint8)
    want[i4[0]] = 3
    off3 = moe.slot_part_offset(MIX.H, MIX.I, 1, 3)
    sz = pool.data[i4[1], off3 + 8:off3 + 12].clone().view(torch.float16)
    sz[0] = float("inf")
    pool.data[i4[1], off3 + 8:off3 + 12] = sz.view(torch.uint8)
    want[i4[1]] = 3
    # an FP8 row scale that is NaN (last w2 row)
    o = moe.slot_part_offset(MIX.H, MIX.I, 0, 3) + 4 * (MIX.H - 1)
    pool.data[fp8[1], o:o + 4] = torch.tensor([float("nan")], dtype=torch.float32, device=gpu).view(torch.uint8)
    want[fp8[1]] = 4
    err, status = moe.pool_check(pool)
    torch.cuda.synchronize()
    assert np.array_equal(status.cpu().numpy(), want)
    assert int(err.item()) == 4


def test_poisoned_workspace_changes_nothing(gpu):
    import torch
    cases = [(CONFIGS["C0"], 16, 0, 16, "layer"), (CONFIGS["C0"], 16, 1, 64, False), (MIX, 40, 0, 16, "layer"),
             (MIX, 40, 0, 32, False), (MIX, 200, 1, 128, False), (MIX, 200, 1, 64, False),
             (CONFIGS["C1"], 8, 0, 16, "layer"), (CONFIGS["C1"], 32, 0, 16, "layer")]
    try:
        for c, T, act, bm, fused in cases:
            li = make_layer(c, T, 1)
            bank = make_bank(c)
            pool = device_pool(li, bank, gpu)
            x, logits, soe, mask = device_inputs(li, gpu)
            _say(f"[poison] {c.name} T={T} act={act} bm={bm} fused={fused}")
            moe.debug_poison(False)
            ref, _, _ = moe.layer(pool, x, logits, c.k, soe, bm, act, mask=mask, fused=fused)
            moe.debug_poison(True)
            out, _, _ = moe.layer(pool, x, logits, c.k, soe, bm, act, mask=mask, fused=fused)
            torch.cuda.synchronize()
            assert not torch.isnan(out.float()).any()
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    finally:
        moe.debug_poison(False)
