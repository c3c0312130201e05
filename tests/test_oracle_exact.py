"""Pins of the oracle on integer-valued layers (CPU only).

On these inputs (gen/exact.py) every step of the layer is exact: the gate
pre-activation is large enough that silu(z) = z in fp64, and the activation
quantization of either mode reproduces its input. The oracle's output must
then equal the layer evaluated in plain int64 arithmetic from the integer
weights, with no slot decode, no align and no activation step: per token,
sum over its chosen experts of w2 (gate * up), divided by k.
"""
import numpy as np
import pytest

import oracle
from gen import make_integer_layer
from harness import oracle_layer


def integer_reference(li, bank, x_int):
    c = li.cfg
    out = np.zeros((li.T, c.H), dtype=np.int64)
    for t in range(li.T):
        chosen = np.nonzero(li.logits[t] == 1.0)[0]
        assert chosen.size == c.k
        for e in chosen:
            w13, w2 = bank.weights(int(e))
            g = w13[:c.I] @ x_int[t]
            u = w13[c.I:] @ x_int[t]
            out[t] += w2 @ (g * u)
    return out.astype(np.float64) / c.k


@pytest.mark.parametrize("H,I,T", [(256, 128, 40), (256, 640, 24)])
@pytest.mark.parametrize("act_mode", [oracle.ACT_BF16, oracle.ACT_FP8_G128_POW2])
def test_oracle_equals_integer_arithmetic(H, I, T, act_mode):
    li, bank, x_int = make_integer_layer(H, I, 8, 4, T)
    ref = oracle_layer(li, bank, 16, act_mode)
    want = integer_reference(li, bank, x_int)
    assert np.array_equal(ref["out"], want)
    assert np.all(ref["w"] == 0.25)


def test_integer_layer_stays_in_the_exact_range():
    li, bank, x_int = make_integer_layer(256, 128, 8, 4, 40)
    c = li.cfg
    for e in range(c.E):
        w13, w2 = bank.weights(e)
        g = x_int @ w13[:c.I].T
        u = x_int @ w13[c.I:].T
        assert g.min() >= 48 and g.max() <= 128        # silu(z) == z in fp64 from z >= 38
        assert np.abs(u).max() <= 4
        h = g * u
        odd = np.abs(h[h != 0])
        while np.any(odd % 2 == 0):
            odd = np.where(odd % 2 == 0, odd // 2, odd)
        assert odd.max() <= 15                          # four significant bits: exact in e4m3
        y = h @ w2.T
        assert np.all(y % 16 == 0) and np.abs(y).max() < 2 ** 12
    # both slot formats decode to the same integer matrices
    for e in range(c.E):
        w13, w2 = bank.weights(e)
        for fmt in (0, 1):
            W13, W2 = oracle.dequant_slot(bank.slot(e, fmt), fmt, c.H, c.I)
            assert np.array_equal(W13, w13) and np.array_equal(W2, w2)
