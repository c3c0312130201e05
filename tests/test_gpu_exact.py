"""Bit-exact parity of the HIP path on integer-valued layers (gen/exact.py),
and of the activation quantization's codes and exponents.

On an integer-valued layer every intermediate of either activation mode is
exact (gate pre-activations large enough that silu(z) = z in fp32, h with
at most four significant bits, y a multiple of 16 below 2^11, route weights
1/4), so the layer output before its final rounding is the same number on
both sides: the GPU's bf16 output must equal the oracle's fp64 output rounded
to bf16, bit for bit. This catches layout and indexing slips a relative
tolerance could hide. Paths covered: the decode kernels (one moe_layer call,
and the separate calls with 32-pair blocks), the FP8 matrix-core kernels with
int4 tiles beside them (128-pair blocks), and the simple tile kernels
(64-pair blocks); FP8 and int4 slots in every pool.
"""
import numpy as np
import pytest

import oracle
import moe_expert_layer_topk_amd as moe
from gen import make_integer_layer, bf16_round
from harness import device_pool, device_inputs, oracle_layer

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _bits(out):
    import torch
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("H,I,T,act_mode,block_m,fused", [
    (2048, 512, 8, 0, 16, "layer"), (2048, 512, 32, 0, 16, "layer"), (2048, 512, 8, 0, 32, False),
    (256, 640, 40, 0, 16, "layer"), (2048, 512, 700, 1, 128, False), (2048, 512, 300, 1, 64, False),
    (256, 640, 400, 1, 128, False), (2048, 512, 40, 1, 128, "layer")])
def test_integer_layer_bit_exact(gpu, H, I, T, act_mode, block_m, fused):
    import torch
    li, bank, _ = make_integer_layer(H, I, 16, 4, T)
    assert (li.slot_fmt == 1).any() and (li.slot_fmt == 0).any()
    _say(f"[exact] H={H} I={I} T={T} act={act_mode} block_m={block_m} fused={fused}")
    pool = device_pool(li, bank, gpu)
    x, logits, soe, mask = device_inputs(li, gpu)
    out, (ids, w, rerr), al = moe.layer(pool, x, logits, 4, soe, block_m, act_mode, fused=fused)
    torch.cuda.synchronize()
    ref = oracle_layer(li, bank, block_m, act_mode)
    assert np.array_equal(ids.cpu().numpy(), ref["ids"])
    assert np.all(w.cpu().numpy() == 0.25)
    n = ref["n_padded"]
    assert np.array_equal(al["sorted_pair"][:n].cpu().numpy(), ref["sorted_pair"])
    want = bf16_round(ref["out"].astype(np.float32))      # exact values: one rounding, same on both sides
    assert np.array_equal(ref["out"].astype(np.float32).astype(np.float64), ref["out"])
    got = _bits(out)
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, f"{bad[0].size} outputs differ, first at token {bad[0][0]} column {bad[1][0]}"


def _bf16_rows(rng, R, C):
    """bf16 rows mixing magnitudes, exact zeros, negative zeros, e4m3 rounding
    midpoints and all-zero groups."""
    v = rng.standard_normal((R, C)).astype(np.float32)
    scale = np.float32(2.0) ** rng.integers(-20, 20, (R, C // 128)).astype(np.float32)
    v *= np.repeat(scale, 128, axis=1)
    v[rng.random((R, C)) < 0.03] = 0.0
    v[rng.random((R, C)) < 0.03] = -0.0
    # midpoints between e4m3 neighbours (1 + m/8 + 1/16) 2^e: ties to even
    mid = rng.random((R, C)) < 0.05
    m = rng.integers(0, 8, (R, C)).astype(np.float32)
    e = rng.integers(-6, 8, (R, C)).astype(np.float32)
    v = np.where(mid, (1 + m / 8 + 1 / 16) * np.float32(2.0) ** e, v).astype(np.float32)
    v[0, :128] = 0.0                                       # an all-zero group
    v[1, 128:256] = 448.0                                  # amax exactly 448 * 2^0
    v[2, :128] = np.float32(480.0)                         # above 448: the next exponent
    return bf16_round(v)


@pytest.mark.parametrize("R,C", [(5, 256), (300, 2048), (4096, 2048)])
def test_quant_act_codes_bit_exact(gpu, R, C):
    import torch
    rng = np.random.default_rng(R + C)
    xb = _bf16_rows(rng, R, C)
    x = torch.from_numpy(xb.view(np.int16)).to(gpu).view(torch.bfloat16)
    codes, exps = moe.quant_act(x)
    torch.cuda.synchronize()
    rc, re, _ = oracle.act_quant_pow2(oracle.bf16_decode(xb))
    assert np.array_equal(exps.cpu().numpy().astype(np.int64) - 127, re)
    assert np.array_equal(codes.cpu().numpy(), rc)
