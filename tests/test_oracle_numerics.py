"""Pins for the oracle's number formats (CPU only)."""
import math

import numpy as np
import pytest

import oracle
from oracle.numerics import pow2_scale_exponent
from golden_io import lines


def test_e4m3_hand_values():
    for ln in lines("e4m3_decode.txt"):
        code, val = ln.split()
        got = oracle.E4M3_TABLE[int(code, 16)]
        want = float(val)
        if math.isnan(want):
            assert math.isnan(got), code
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), code


def test_e4m3_table_matches_torch_library_decode():
    torch = pytest.importorskip("torch")
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    lib = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = oracle.E4M3_TABLE
    nan = np.isnan(lib)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(lib[~nan], ours[~nan])
    assert np.array_equal(np.signbit(lib[~nan]), np.signbit(ours[~nan]))


def test_e4m3_rne_hand_values():
    for ln in lines("e4m3_rne.txt"):
        val, code = ln.split()
        got = int(oracle.e4m3_encode_rne(np.array([float(val)]))[0])
        assert got == int(code, 16), (val, hex(got))


def test_e4m3_rne_matches_torch_cast():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.uniform(-448, 448, 20000),
                        rng.standard_normal(20000) * 0.01,
                        oracle.E4M3_TABLE[:0x7F],                       # exact codes
                        (oracle.E4M3_TABLE[:0x7E] + oracle.E4M3_TABLE[1:0x7F]) / 2])  # every midpoint
    ours = oracle.e4m3_encode_rne(v)
    lib = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch keeps the sign of values that round to zero as well
    assert np.array_equal(ours, lib)


def test_e4m3_rne_rejects_out_of_range():
    with pytest.raises(ValueError):
        oracle.e4m3_encode_rne(np.array([449.0]))


def test_pow2_exponent_definition():
    # smallest s with amax <= 448 * 2**s
    amax = np.array([0.0, 448.0, 448.0001, 449.0, 224.0, 224.1, 0.5, 1e-30, 3.0e4, 2.0 ** -140])
    s = pow2_scale_exponent(amax)
    assert s[0] == 0
    assert list(s[1:7]) == [0, 1, 1, -1, 0, -9]
    nz = amax > 0
    assert np.all(amax[nz] <= np.ldexp(448.0, s[nz]))
    assert np.all(amax[nz] > np.ldexp(448.0, s[nz] - 1))


def test_act_quant_properties():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((5, 300)) * np.array([[1e-3], [1], [50], [1e4], [0]])
    codes, exps, deq = oracle.act_quant_pow2(v)
    assert exps.shape == (5, 3)                       # groups of 128, 128, 44
    assert np.all(exps[4] == 0) and np.all(deq[4] == 0)
    # every group's largest magnitude maps into (224, 448]
    for r in range(4):
        for g in range(3):
            blk = v[r, g * 128:(g + 1) * 128]
            m = np.abs(blk).max() / 2.0 ** exps[r, g]
            assert 224 < m <= 448
    # relative error of E4M3 (3 mantissa bits) is at most 2**-4 for normals
    rel = np.abs(deq - v) / np.maximum(np.abs(v), 1e-300)
    big = np.abs(v) > np.ldexp(2.0 ** -6, np.repeat(exps, 128, axis=1)[:, :300])
    assert np.all(rel[big] <= 2.0 ** -4 + 1e-15)


def test_act_quant_exact_for_representable_rows():
    # values that are E4M3 codes times a power of two come back unchanged
    row = np.array([[448.0, -3.5, 0.015625, 1.0] * 32]) * 2.0 ** -5
    _, exps, deq = oracle.act_quant_pow2(row)
    assert exps[0, 0] == -5
    assert np.array_equal(deq, row)


def test_bf16_and_f16_decode():
    assert oracle.bf16_decode(np.array([0x3F80, 0xC000, 0x3F81], dtype=np.uint16)).tolist() == \
        [1.0, -2.0, 1.0078125]
    assert oracle.f16_decode(np.array([0x3C00, 0x3800, 0xC400], dtype=np.uint16)).tolist() == \
        [1.0, 0.5, -4.0]


def test_silu_values():
    z = np.array([0.0, 1.0, -1.0, 20.0, -800.0])
    got = oracle.silu(z)
    assert got[0] == 0.0
    assert abs(got[1] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
    assert abs(got[2] + 1.0 / (1.0 + math.e)) < 1e-15
    assert abs(got[3] - 20.0) < 1e-7
    assert got[4] == 0.0
