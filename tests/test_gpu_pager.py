"""The slot-miss path on the GPU: resident-first passes (moe_expert_ffn_pass)
and the pager's fills from page-locked host memory on a copy stream.

Two passes over one workspace, the first deferring some experts' blocks and
the second deferring the rest, must write exactly what one moe_expert_ffn
call writes. A decode loop that starts from an empty VRAM pool, plans each
step with the pager, fills the misses on a copy stream while the resident
experts' pass runs, then runs the filled experts' pass, must match the oracle
run on the pool the plan describes, with the oracle LRU's hits and misses.
"""
import numpy as np
import pytest

import oracle
import moe_expert_layer_topk_amd as moe
from gen import CONFIGS, make_layer, make_bank, step_tokens
from gen.configs import Config
from harness import device_pool, device_inputs, rel_max_err

pytestmark = pytest.mark.gpu

MIX = Config("mix", 71, (200, 40), 256, 128, 16, 4, 1, 0.1, True, slots=0, int4_frac=0.4, resident_all_at=1)


def _bits(t):
    import torch
    return t.view(torch.int16)


@pytest.mark.parametrize("name,T,act_mode,block_m", [("C1", 8, 0, 16), ("C1", 32, 0, 32), ("mix", 200, 1, 128),
                                                     ("mix", 200, 1, 64), ("mix", 40, 0, 16)])
def test_two_passes_equal_one_call(gpu, name, T, act_mode, block_m):
    import torch
    c = MIX if name == "mix" else CONFIGS[name]
    li = make_layer(c, T, 1)
    pool = device_pool(li, make_bank(c), gpu)
    x, logits, soe, mask = device_inputs(li, gpu)
    ids, w, _ = moe.route(logits, c.k, mask=mask)
    E = c.E
    one = moe.expert_ffn(pool, x, c.k, E, w, moe.align(ids, E, block_m, soe), block_m, act_mode)
    rng = np.random.default_rng(T)
    deferred = rng.random(E) < 0.4
    soe_h = li.slot_of_expert
    t1 = np.where(deferred, moe.SLOT_DEFERRED, soe_h).astype(np.int32)
    t2 = np.where(deferred, soe_h, moe.SLOT_DEFERRED).astype(np.int32)
    need = moe.ffn_workspace_bytes(T, c.k, E, c.H, c.I, block_m, act_mode)
    ws = torch.empty(need, dtype=torch.uint8, device=gpu)
    out = torch.empty_like(one)
    a1 = moe.align(ids, E, block_m, torch.from_numpy(t1).to(gpu))
    moe.expert_ffn_pass(pool, x, c.k, E, w, a1, block_m, act_mode, False, out, ws)
    a2 = moe.align(ids, E, block_m, torch.from_numpy(t2).to(gpu))
    moe.expert_ffn_pass(pool, x, c.k, E, w, a2, block_m, act_mode, True, out, ws)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(one))
    ref_err = oracle.align(ids.cpu().numpy(), E, block_m, soe_h)["err"]
    assert int(a1["err"].item()) + int(a2["err"].item()) <= ref_err   # deferred entries are not errors


def test_slot_miss_path_decode_loop(gpu):
    import torch
    c = CONFIGS["C1"]
    T, S, L = 8, 64, 2
    bank = make_bank(c)
    host = torch.from_numpy(bank.materialize(0)).pin_memory()          # expert e of every layer = bank row e
    host_fmt = torch.zeros(c.E, dtype=torch.uint8).pin_memory()
    pools = [moe.SlotPool(torch.zeros((S, bank.stride), dtype=torch.uint8, device=gpu),
                         torch.zeros(S, dtype=torch.uint8, device=gpu), c.H, c.I) for _ in range(L)]
    pager = moe.Pager(L, c.E, S)
    refs = [oracle.LRUSlots(c.E, S) for _ in range(L)]
    copy = torch.cuda.Stream()
    comp = torch.cuda.current_stream()
    need = moe.ffn_workspace_bytes(T, c.k, c.E, c.H, c.I, 16, 0)
    ws = torch.empty(need, dtype=torch.uint8, device=gpu)
    for step in range(4):
        for layer in range(L):
            xb, lg = step_tokens(c, T, layer, step)
            x = torch.from_numpy(xb.view(np.int16).copy()).to(gpu).view(torch.bfloat16)
            logits = torch.from_numpy(lg).to(gpu)
            ids, w, _ = moe.route(logits, c.k)
            ids_h = ids.cpu().numpy()                                   # (synchronises)
            table, fe, fs = pager.plan(layer, ids_h)
            rt, rf = refs[layer].plan(ids_h.reshape(-1))
            assert table.tolist() == rt and list(zip(fe.tolist(), fs.tolist())) == rf
            copy.wait_stream(comp)
            moe.pager_fill(pools[layer], host, host_fmt, fe, fs, copy)
            filled = torch.cuda.Event()
            filled.record(copy)
            miss = np.zeros(c.E, bool)
            miss[fe] = True
            t1 = np.where(miss, moe.SLOT_DEFERRED, table).astype(np.int32)
            t2 = np.where(miss, table, moe.SLOT_DEFERRED).astype(np.int32)
            out = torch.empty((T, c.H), dtype=torch.bfloat16, device=gpu)
            a1 = moe.align(ids, c.E, 16, torch.from_numpy(t1).to(gpu))
            moe.expert_ffn_pass(pools[layer], x, c.k, c.E, w, a1, 16, 0, False, out, ws)   # hits, during the fill
            comp.wait_event(filled)
            a2 = moe.align(ids, c.E, 16, torch.from_numpy(t2).to(gpu))
            moe.expert_ffn_pass(pools[layer], x, c.k, c.E, w, a2, 16, 0, True, out, ws)
            torch.cuda.synchronize()
            # the oracle on the pool the plan describes (slot s holds bank row owner[s])
            pool_h = np.zeros((S, bank.stride), dtype=np.uint8)
            for e in range(c.E):
                if table[e] >= 0:
                    b = bank.slot(e, 0)
                    pool_h[table[e], :b.size] = b
            ref = oracle.layer_forward(lg, None, c.k, table, pool_h, np.zeros(S, np.uint8), c.H, c.I, xb, 16, 0)
            assert np.array_equal(ids_h, ref["ids"])
            e_rel = rel_max_err(out, ref["out"])
            print(f"[pager] step {step} layer {layer}: {fe.size} misses, rel max err {e_rel:.3e}", flush=True)
            assert e_rel <= 2e-2
    h, m = pager.stats()
    assert (h, m) == (sum(r.hits for r in refs), sum(r.misses for r in refs)) and h > 0
