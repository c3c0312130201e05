"""moe_layer_noalloc (the whole-layer call with the library's built-in
scratch as its workspace) gives exactly what moe_layer gives with a caller
workspace, on two calls in a row, the second with a smaller input, in the
decode path and in the FP8 matrix-core path; an oversized layer is refused
before anything runs."""
import numpy as np
import pytest

import moe_expert_layer_topk_amd as moe
from gen import CONFIGS, make_layer, make_bank
from gen.configs import Config
from harness import device_pool, device_inputs

pytestmark = pytest.mark.gpu

MIX = Config("mix", 71, (200, 40), 256, 128, 16, 4, 1, 0.1, True, slots=0, int4_frac=0.4, resident_all_at=1)


def _same(a, b):
    import torch
    assert a.dtype == b.dtype and a.shape == b.shape
    assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.uint8) if b.dtype == torch.bfloat16 else b)


def _compare(li, bank, dev, block_m, act_mode):
    import torch
    c = li.cfg
    print(f"[noalloc] {c.name} T={li.T} block_m={block_m} act={act_mode}", flush=True)
    pool = device_pool(li, bank, dev)
    x, logits, soe, mask = device_inputs(li, dev)
    out0, ids0, w0, al0 = moe.layer_call(pool, x, logits, c.k, soe, block_m, act_mode, mask=mask)
    out1, ids1, w1, al1 = moe.layer_call_noalloc(pool, x, logits, c.k, soe, block_m, act_mode, mask=mask)
    torch.cuda.synchronize()
    _same(out1, out0)
    _same(ids1, ids0)
    _same(w1, w0)
    n = int(al0["n_padded"].item())
    assert int(al1["n_padded"].item()) == n
    _same(al1["sorted_pair"][:n], al0["sorted_pair"][:n])
    _same(al1["block_slot"][:n // block_m], al0["block_slot"][:n // block_m])
    for key in ("counts", "seg_offset", "err"):
        _same(al1[key], al0[key])


@pytest.mark.parametrize("first,second", [(("C1", 32, 16, 0), ("C1", 8, 16, 0)),
                                          (("mix", 200, 128, 1), ("mix", 40, 64, 1)),
                                          (("C3", 32, 16, 0), ("C0", 16, 16, 0))])
def test_noalloc_matches_moe_layer(gpu, first, second):
    for name, T, bm, act in (first, second):
        c = MIX if name == "mix" else CONFIGS[name]
        _compare(make_layer(c, T, 2), make_bank(c), gpu, bm, act)


def test_noalloc_refuses_oversized_layer(gpu):
    import torch
    c = CONFIGS["C2"]
    T = 4096                                       # FP8 workspace far above the scratch size
    assert moe.layer_workspace_bytes(T, c.k, c.E, c.H, c.I, 128, 1) > (32 << 20)
    li = make_layer(CONFIGS["C0"], 16, 0)
    pool = device_pool(li, make_bank(CONFIGS["C0"]), gpu)
    x = torch.zeros((T, c.H), dtype=torch.bfloat16, device=gpu)
    logits = torch.zeros((T, c.E), dtype=torch.float32, device=gpu)
    soe = torch.zeros(c.E, dtype=torch.int32, device=gpu)
    big = moe.SlotPool(pool.data, pool.fmt, c.H, c.I)
    with pytest.raises(moe.MoeError, match="scratch"):
        moe.layer_call_noalloc(big, x, logits, c.k, soe, 128, 1)
