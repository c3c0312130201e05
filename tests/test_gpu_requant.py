"""moe_requant_slot against the oracle's requantization (bit for bit), and
a layer whose least-routed experts were switched to int4 by the plan."""
import numpy as np
import pytest

import oracle
import moe_expert_layer_topk_amd as moe
from gen import CONFIGS, make_layer, make_bank
from gen.configs import Config
from harness import device_pool, device_inputs, rel_max_err

pytestmark = pytest.mark.gpu


def _int4_arrays(buf, H, I):
    offs, sizes, _ = oracle.slot_offsets(H, I, 1)
    return [np.asarray(buf[o:o + n]) for o, n in zip(offs, sizes)]


@pytest.mark.parametrize("name", ["C1", "C3"])
def test_requant_slot_bit_exact(gpu, name):
    import torch
    c = CONFIGS[name]
    if c.I % 128:
        pytest.skip("int4 needs inter % 128 == 0")
    li = make_layer(c, 8, 0)
    bank = make_bank(c)
    pool = device_pool(li, bank, gpu)
    S = li.n_slots
    src, dst = 0, S - 1
    assert li.slot_fmt[src] == 0
    err = torch.zeros(1, dtype=torch.int32, device=gpu)
    moe.requant_slot(pool, src, dst, err=err)
    torch.cuda.synchronize()
    want = oracle.requant_slot(bank.slot(li.slot_src[src], 0), c.H, c.I)
    got = pool.data[dst].cpu().numpy()
    for g, w in zip(_int4_arrays(got, c.H, c.I), _int4_arrays(want, c.H, c.I)):
        assert np.array_equal(g, w)
    assert int(pool.fmt[dst].item()) == 1 and int(err.item()) == 0
    # a source that is not an FP8 slot: nothing written, counted
    before = pool.data[1].clone()
    moe.requant_slot(pool, dst, 1, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 1 and torch.equal(pool.data[1], before)


MIDR = Config("midr", 76, (40, 400), 512, 256, 32, 4, 1, 0.1, True, slots=0)


@pytest.mark.parametrize("T,act_mode,block_m", [(40, 0, 16), (400, 1, 128)])
def test_layer_with_planned_int4_experts(gpu, T, act_mode, block_m):
    """Route and align once, take the 10 least-routed experts from the align
    counts, requantize each into a spare slot, point the slot table there and
    run the layer: the output matches the oracle run on the oracle's own
    requantized bytes."""
    import torch
    c = MIDR
    li = make_layer(c, T, 0)
    bank = make_bank(c)
    x, logits, soe, mask = device_inputs(li, gpu)
    _, _, al = moe.route_align(logits, c.k, block_m, soe)
    counts = al["counts"].cpu().numpy()
    plan = moe.bitwidth_plan(counts, 10)
    assert np.array_equal(plan, oracle.bitwidth_plan(counts, 10))
    low = np.nonzero(plan == 1)[0]
    # the pool gets one spare slot per planned expert
    S = li.n_slots
    host = np.zeros((S + low.size, bank.stride), dtype=np.uint8)
    for s in range(S):
        b = bank.slot(li.slot_src[s], li.slot_fmt[s])
        host[s, :b.size] = b
    fmt = np.concatenate([li.slot_fmt, np.zeros(low.size, np.uint8)])
    pool = moe.SlotPool(torch.from_numpy(host).to(gpu), torch.from_numpy(fmt).to(gpu), c.H, c.I)
    soe_new = li.slot_of_expert.copy()
    ref_pool = host.copy()
    ref_fmt = fmt.copy()
    for i, e in enumerate(low):
        moe.requant_slot(pool, int(li.slot_of_expert[e]), S + i)
        soe_new[e] = S + i
        r = oracle.requant_slot(host[li.slot_of_expert[e]], c.H, c.I)
        ref_pool[S + i, :r.size] = r
        ref_fmt[S + i] = 1
    out, _, _ = moe.layer(pool, x, logits, c.k, torch.from_numpy(soe_new).to(gpu), block_m, act_mode)
    torch.cuda.synchronize()
    assert np.array_equal(pool.fmt.cpu().numpy(), ref_fmt)
    ref = oracle.layer_forward(li.logits, None, c.k, soe_new, ref_pool, ref_fmt, c.H, c.I, li.x_bits, block_m,
                               act_mode)
    e = rel_max_err(out, ref["out"])
    print(f"    rel max err {e:.3e}", flush=True)
    assert e <= 2e-2
