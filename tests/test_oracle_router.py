"""Pins of the router-gate oracle (CPU only): a case worked by hand, a
brute-force sum per logit, and the error bound it states for fp32 sums."""
import math

import numpy as np

import oracle
from gen import bf16_round, CONFIGS, make_layer, router_inputs
from golden_io import kv


def test_router_hand_case():
    g = kv("router_tiny.txt")
    f = lambda key: [float(v) for v in g[key]]
    x = np.array([f("x0"), f("x1")], dtype=np.float32)
    W = np.array([f("w0"), f("w1"), f("w2")], dtype=np.float32)
    out = oracle.router_logits(bf16_round(x), W, np.array(f("bias"), dtype=np.float32))
    assert out.tolist() == [f("out0"), f("out1")]
    no_bias = oracle.router_logits(bf16_round(x), W)
    assert no_bias.tolist() == [[-1.5, 3.5, 4.0], [-4.25, -0.5, 8.0]]


def test_router_brute_force_sums():
    rng = np.random.default_rng(5)
    T, H, E = 6, 256, 10
    xb = bf16_round(rng.standard_normal((T, H)).astype(np.float32))
    W = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    out = oracle.router_logits(xb, W, b)
    x = oracle.bf16_decode(xb)
    for t in range(T):
        for e in range(E):
            want = math.fsum([float(x[t, h]) * float(W[e, h]) for h in range(H)] + [float(b[e])])
            assert abs(out[t, e] - want) <= 1e-13 * (1 + abs(want))


def test_router_matches_generator_logits():
    """The generator draws each layer's logits from the same gate in fp64
    (before rounding W_g to fp32): the two differ only by that rounding."""
    c = CONFIGS["C1"]
    li = make_layer(c, 32, 3)
    W, b = router_inputs(c, 32, 3)
    out = oracle.router_logits(li.x_bits, W, b)
    assert np.abs(out - li.logits.astype(np.float64)).max() < 1e-4


def test_fp32_sum_bound_holds_for_float32_sums():
    """numpy's float32 matmul (one summation order among many) stays inside
    the stated bound."""
    rng = np.random.default_rng(6)
    xb = bf16_round(rng.standard_normal((64, 2048)).astype(np.float32))
    W = (rng.standard_normal((256, 2048)) * 0.05).astype(np.float32)
    exact = oracle.router_logits(xb, W)
    f32 = oracle.bf16_decode(xb).astype(np.float32) @ W.T
    bound = oracle.fp32_sum_bound(xb, W, 2048)
    assert np.all(np.abs(f32.astype(np.float64) - exact) <= bound)
