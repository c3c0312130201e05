"""The compressed host tier on the GPU: moe_fp8_unpack expands packed slots
(per-row Huffman codes of FP8 exponents, packed by the library's host packer,
whose bytes equal the oracle's) back into the FP8 slot bit for bit, and the
slot-miss path fills from a packed host bank."""
import numpy as np
import pytest

import oracle
import moe_expert_layer_topk_amd as moe
from gen import CONFIGS, make_bank, step_tokens
from harness import rel_max_err

pytestmark = pytest.mark.gpu


def _fp8_parts(buf, H, I):
    offs, sizes, _ = oracle.slot_offsets(H, I, 0)
    return [np.asarray(buf[o:o + n]) for o, n in zip(offs, sizes)]


@pytest.mark.parametrize("case", ["C1", "C3", "skewed"])
def test_unpack_bit_exact(gpu, case):
    import torch
    if case == "skewed":
        from test_oracle_huffman import _skewed_slot
        H, I = 512, 256
        slots = [_skewed_slot(H, I, 9)]
    else:
        c = CONFIGS[case]
        H, I = c.H, c.I
        bank = make_bank(c)
        slots = [bank.slot(b, 0) for b in (0, 5, 77)]
    stride = moe.slot_bytes(H, I, 0)
    pool = moe.SlotPool(torch.full((len(slots) + 1, stride), 0xAB, dtype=torch.uint8, device=gpu),
                        torch.full((len(slots) + 1,), 7, dtype=torch.uint8, device=gpu), H, I)
    err = torch.zeros(1, dtype=torch.int32, device=gpu)
    sizes = []
    for i, s in enumerate(slots):
        packed = moe.fp8_pack(s, H, I)
        sizes.append(packed.size / s.size)
        moe.fp8_unpack(pool, torch.from_numpy(packed).to(gpu), i + 1, err=err)
    torch.cuda.synchronize()
    print(f"    packed size / FP8 slot size: {np.round(sizes, 4).tolist()}", flush=True)
    got = pool.data.cpu().numpy()
    for i, s in enumerate(slots):
        for g, w in zip(_fp8_parts(got[i + 1], H, I), _fp8_parts(s, H, I)):
            assert np.array_equal(g, w)
    assert pool.fmt.cpu().numpy().tolist() == [7] + [0] * len(slots)
    assert int(err.item()) == 0
    # a header for another shape: nothing written, one error
    bad = moe.fp8_pack(slots[0], H, I)
    bad[4:8] = np.array([H + 256], dtype="<u4").view(np.uint8)
    before = pool.data[0].clone()
    moe.fp8_unpack(pool, torch.from_numpy(bad).to(gpu), 0, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 1 and torch.equal(pool.data[0], before) and int(pool.fmt[0].item()) == 7


def test_slot_miss_path_from_packed_bank(gpu):
    import torch
    c = CONFIGS["C1"]
    T, S = 8, 64
    bank = make_bank(c)
    packed = [moe.fp8_pack(bank.slot(e, 0), c.H, c.I) for e in range(c.E)]
    sizes = np.array([p.size for p in packed], dtype=np.uint64)
    offsets = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.uint64)
    host = torch.from_numpy(np.concatenate(packed)).pin_memory()
    print(f"    packed bank {host.numel() / (c.E * moe.slot_bytes(c.H, c.I, 0)):.4f} of the FP8 bank", flush=True)
    staging = torch.empty(int(S * (sizes.max() + 16)), dtype=torch.uint8, device=gpu)
    pool = moe.SlotPool(torch.zeros((S, moe.slot_bytes(c.H, c.I, 0)), dtype=torch.uint8, device=gpu),
                        torch.zeros(S, dtype=torch.uint8, device=gpu), c.H, c.I)
    pager = moe.Pager(1, c.E, S)
    copy = torch.cuda.Stream()
    comp = torch.cuda.current_stream()
    err = torch.zeros(1, dtype=torch.int32, device=gpu)
    ws = torch.empty(moe.ffn_workspace_bytes(T, c.k, c.E, c.H, c.I, 16, 0), dtype=torch.uint8, device=gpu)
    for step in range(3):
        xb, lg = step_tokens(c, T, 0, step)
        x = torch.from_numpy(xb.view(np.int16).copy()).to(gpu).view(torch.bfloat16)
        ids, w, _ = moe.route(torch.from_numpy(lg).to(gpu), c.k)
        ids_h = ids.cpu().numpy()
        table, fe, fs = pager.plan(0, ids_h)
        copy.wait_stream(comp)
        moe.pager_fill_packed(pool, host, offsets, sizes, fe, fs, staging, copy, err=err)
        comp.wait_stream(copy)
        al = moe.align(ids, c.E, 16, torch.from_numpy(table).to(gpu))
        out = moe.expert_ffn(pool, x, c.k, c.E, w, al, 16, 0, ws=ws)
        torch.cuda.synchronize()
        pool_h = np.zeros((S, moe.slot_bytes(c.H, c.I, 0)), dtype=np.uint8)
        for e in range(c.E):
            if table[e] >= 0:
                pool_h[table[e]] = bank.slot(e, 0)
        ref = oracle.layer_forward(lg, None, c.k, table, pool_h, np.zeros(S, np.uint8), c.H, c.I, xb, 16, 0)
        e_rel = rel_max_err(out, ref["out"])
        print(f"[packed pager] step {step}: {fe.size} misses, rel max err {e_rel:.3e}", flush=True)
        assert e_rel <= 2e-2 and int(err.item()) == 0
