"""Pins of the bit-width plan and the FP8 -> int4-g128 requantization
(CPU only), and the library's host-side plan against the oracle's."""
import os

import numpy as np
import pytest

import oracle
import moe_expert_layer_topk_amd as moe
from gen import encode_slot, slot_layout


def _fp8_slot_from_codes(H, I, c13, s13, c2, s2):
    lay = slot_layout(H, I, 0)
    buf = np.zeros(lay["total"][1], dtype=np.uint8)
    for name, arr in (("w13", c13), ("w13_scale", s13), ("w2", c2), ("w2_scale", s2)):
        off, n = lay[name]
        raw = np.ascontiguousarray(arr).view(np.uint8).reshape(-1)
        buf[off:off + n] = raw
    return buf


def _e4m3_codes_of(v):
    import torch
    return torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_plan_least_routed_ties_to_lower_id():
    counts = np.array([5, 0, 3, 3, 9, 0, 1])
    fmt = oracle.bitwidth_plan(counts, 3)
    assert fmt.tolist() == [0, 1, 0, 0, 0, 1, 1]        # ids 1 and 5 (count 0), then 6 (count 1)
    assert oracle.bitwidth_plan(counts, 4).tolist() == [0, 1, 1, 0, 0, 1, 1]   # 2 before 3
    assert oracle.bitwidth_plan(counts, 0).sum() == 0
    assert oracle.bitwidth_plan(counts, 99).tolist() == [1] * 7


def test_library_plan_matches_oracle():
    if not os.path.exists(moe.LIB_PATH):
        pytest.skip("library not built")
    rng = np.random.default_rng(2)
    for E, n in ((8, 3), (256, 77), (512, 0), (1000, 999)):
        counts = rng.integers(0, 6, E).astype(np.int32)      # many ties
        assert np.array_equal(moe.bitwidth_plan(counts, n), oracle.bitwidth_plan(counts, n))


def test_requant_reproduces_a_grid_exact_slot():
    """Rows whose decoded values are (d - 7) / 16 with d in 0..15 and both
    ends present in every group: s = 1/16, zero = 7, q = d exactly, so the
    int4 slot decodes to the same matrices as the FP8 one."""
    H, I = 256, 128
    rng = np.random.default_rng(4)

    def grid(rows, cols):
        d = rng.integers(0, 16, (rows, cols))
        d[:, 0::128] = 0
        d[:, 1::128] = 15
        return (d - 7).astype(np.float32)

    v13, v2 = grid(2 * I, H), grid(H, I)
    fp8 = _fp8_slot_from_codes(H, I, _e4m3_codes_of(v13), np.full(2 * I, 1 / 16, np.float32),
                               _e4m3_codes_of(v2), np.full(H, 1 / 16, np.float32))
    W13, W2 = oracle.dequant_slot(fp8, 0, H, I)
    R13, R2 = oracle.dequant_slot(oracle.requant_slot(fp8, H, I), 1, H, I)
    assert np.array_equal(R13, W13) and np.array_equal(R2, W2)


def test_requant_error_bound_and_ranges():
    H, I = 256, 128
    rng = np.random.default_rng(5)
    w13 = rng.standard_normal((2 * I, H)) * 0.02
    w2 = rng.standard_normal((H, I)) * 0.02
    fp8 = encode_slot(w13, w2, 0)
    W13, W2 = oracle.dequant_slot(fp8, 0, H, I)
    r = oracle.requant_slot(fp8, H, I)
    R13, R2 = oracle.dequant_slot(r, 1, H, I)
    offs, sizes, _ = oracle.slot_offsets(H, I, 1)
    for (W, R, o) in ((W13, R13, 1), (W2, R2, 3)):
        sz = r[offs[o]:offs[o] + sizes[o]].view(np.float16).astype(np.float64).reshape(W.shape[0], -1, 2)
        s, z = sz[..., 0], sz[..., 1]
        assert np.all((z == np.rint(z)) & (z >= 0) & (z <= 15))
        # one step of the group's grid at most (half a step where nothing clips)
        step = np.repeat(s, 128, axis=1)
        assert np.all(np.abs(R - W) <= step * (1 + 1e-6))
        assert np.mean(np.abs(R - W) <= step / 2 * (1 + 1e-6)) > 0.99
