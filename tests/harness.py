"""Shared plumbing for the GPU tests and the benchmark: move generator
inputs to the device and drive the oracle on the same inputs. Holds no layer
arithmetic of its own."""
import numpy as np

import oracle
from gen import FMT_FP8_E4M3_ROW, FMT_INT4_G128


def device_pool(li, bank, dev, bank_dev=None):
    """The layer's slot pool on the device. bank_dev: optional {fmt: uint8
    device tensor [n_bank, stride]} to copy slots from (large configs)."""
    import torch
    from moe_expert_layer_topk_amd import SlotPool
    c = li.cfg
    S = li.n_slots
    if bank_dev is None:
        host = np.zeros((S, bank.stride), dtype=np.uint8)
        for s in range(S):
            b = bank.slot(li.slot_src[s], li.slot_fmt[s])
            host[s, :b.size] = b
        data = torch.from_numpy(host).to(dev)
    else:
        data = torch.empty((S, bank.stride), dtype=torch.uint8, device=dev)
        for f in (FMT_FP8_E4M3_ROW, FMT_INT4_G128):
            idx = np.nonzero(li.slot_fmt == f)[0]
            if idx.size:
                src = torch.from_numpy(li.slot_src[idx].astype(np.int64)).to(dev)
                data[torch.from_numpy(idx).to(dev)] = bank_dev[f].index_select(0, src)
    fmt = torch.from_numpy(li.slot_fmt.copy()).to(dev)
    return SlotPool(data, fmt, c.H, c.I)


def SlotPool_from_host(host, slot_fmt, hidden, inter, dev):
    """A pool from host bytes uint8 [n_slots, stride] and per-slot tags."""
    import torch
    from moe_expert_layer_topk_amd import SlotPool
    return SlotPool(torch.from_numpy(np.ascontiguousarray(host)).to(dev), torch.from_numpy(slot_fmt.copy()).to(dev),
                    hidden, inter)


def bank_on_device(bank, dev):
    import torch
    return {f: torch.from_numpy(bank.materialize(f)).to(dev) for f in bank.fmts}


def device_inputs(li, dev):
    import torch
    x = torch.from_numpy(li.x_bits.view(np.int16).copy()).to(dev).view(torch.bfloat16)
    logits = torch.from_numpy(li.logits.copy()).to(dev)
    soe = torch.from_numpy(li.slot_of_expert.copy()).to(dev)
    mask = None if li.mask is None else torch.from_numpy(li.mask.copy()).to(dev)
    return x, logits, soe, mask


class BoundedCache(dict):
    """A dict that keeps only its `size` most recent entries (the oracle walks
    blocks in ascending expert order, so one decoded expert at a time is
    enough and keeps host memory bounded at full-size layers)."""

    def __init__(self, size=2):
        super().__init__()
        self.size = size

    def __setitem__(self, key, value):
        while len(self) >= self.size:
            del self[next(iter(self))]
        super().__setitem__(key, value)


class OracleSlots:
    """weights_of_slot for the oracle: decode each bank expert once."""

    def __init__(self, li, bank, cache=None):
        self.li, self.bank = li, bank
        self.cache = {} if cache is None else cache

    def __call__(self, s):
        key = (int(self.li.slot_src[s]), int(self.li.slot_fmt[s]))
        if key not in self.cache:
            c = self.li.cfg
            self.cache[key] = oracle.dequant_slot(self.bank.slot(*key), key[1], c.H, c.I)
        return self.cache[key]


def oracle_layer(li, bank, block_m, act_mode, token_subset=None, cache=None):
    c = li.cfg
    return oracle.layer_forward(li.logits, li.mask, c.k, li.slot_of_expert, None, li.slot_fmt, c.H, c.I,
                                li.x_bits, block_m, act_mode, weights_of_slot=OracleSlots(li, bank, cache),
                                token_subset=token_subset)


def rel_max_err(out_bf16, ref, rows=None):
    """max|out - ref| / max|ref| over the given rows (all by default)."""
    o = out_bf16.float().cpu().numpy().astype(np.float64)
    if rows is not None:
        o, ref = o[rows], ref[rows]
    den = np.abs(ref).max()
    return float(np.abs(o - ref).max() / (den if den > 0 else 1.0))
