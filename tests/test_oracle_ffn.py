"""Pins for the oracle's slot decode, expert FFN and whole layer (CPU only)."""
import numpy as np
import pytest

import oracle
from golden_io import kv, closed_form
from gen import CONFIGS, make_layer, make_bank, layer_pool_bytes, encode_slot


def _fp8_slot(H, I, w13_codes, w13_scale, w2_codes, w2_scale):
    offs, sizes, total = oracle.slot_offsets(H, I, 0)
    buf = np.zeros(total, dtype=np.uint8)
    parts = [np.array(w13_codes, dtype=np.uint8), np.array(w13_scale, dtype=np.float32),
             np.array(w2_codes, dtype=np.uint8), np.array(w2_scale, dtype=np.float32)]
    for o, n, a in zip(offs, sizes, parts):
        raw = a.view(np.uint8).reshape(-1)
        assert raw.size == n
        buf[o:o + n] = raw
    return buf


def tiny_case(mod=oracle):
    g = kv("ffn_tiny.txt")
    h = lambda key: [int(v, 16) for v in g[key]]
    f = lambda key: [float(v) for v in g[key]]
    H, I = 2, 1
    offs, sizes, total = mod.slot_offsets(H, I, 0)
    pool = np.stack([_fp8_slot(H, I, h("slot0_w13"), f("slot0_w13_scale"), h("slot0_w2"), f("slot0_w2_scale")),
                     _fp8_slot(H, I, h("slot1_w13"), f("slot1_w13_scale"), h("slot1_w2"), f("slot1_w2_scale"))])
    x = np.array(f("x"), dtype=np.float32).reshape(2, 2)
    x_bits = (x.view(np.uint32) >> 16).astype(np.uint16)          # exact in bf16
    logits = np.array(f("logits"), dtype=np.float32).reshape(2, 2)
    want = np.array([[closed_form(v) for v in g["out0"]], [closed_form(v) for v in g["out1"]]])
    return pool, x_bits, logits, want


def test_ffn_hand_case():
    pool, x_bits, logits, want = tiny_case()
    r = oracle.layer_forward(logits, None, 1, np.array([1, 0], dtype=np.int32), pool,
                             np.zeros(2, np.uint8), 2, 1, x_bits, 2, oracle.ACT_BF16)
    assert r["ids"].tolist() == [[0], [1]]
    assert np.allclose(r["out"], want, rtol=1e-14, atol=0)


def test_int4_slot_hand_case():
    H = I = 128
    offs, sizes, total = oracle.slot_offsets(H, I, 1)
    buf = np.zeros(total, dtype=np.uint8)
    q = np.arange(H) % 16
    buf[offs[0]:offs[0] + H // 2] = (q[0::2] | (q[1::2] << 4)).astype(np.uint8)  # w13 row 0
    sz = np.zeros((2 * I, H // 128, 2), dtype=np.float16)
    sz[:, :, 0] = 1.0
    sz[0, 0] = [0.5, 8.0]
    buf[offs[1]:offs[1] + sizes[1]] = sz.view(np.uint8).reshape(-1)
    sz2 = np.ones((H, I // 128, 2), dtype=np.float16)
    buf[offs[3]:offs[3] + sizes[3]] = sz2.view(np.uint8).reshape(-1)
    W13, W2 = oracle.dequant_slot(buf, 1, H, I)
    assert W13[0].tolist() == [((c % 16) - 8) * 0.5 for c in range(H)]   # -4.0 ... 3.5
    assert np.all(W13[1:] == 0)
    assert np.all(W2 == -1.0)                                            # (0 - 1) * 1


@pytest.mark.parametrize("fmt", [0, 1])
def test_slot_decode_matches_generator_weights(fmt):
    """The generator quantizes known float weights with its own code; the
    oracle's decode of those bytes must give them back within the format's
    rounding error, which fails for any wrong offset, transposition, nibble
    order or scale index."""
    rng = np.random.default_rng(1)
    H, I = 256, 128
    w13 = rng.standard_normal((2 * I, H)) * 0.02
    w2 = rng.standard_normal((H, I)) * 0.02
    W13, W2 = oracle.dequant_slot(encode_slot(w13, w2, fmt), fmt, H, I)
    if fmt == 0:   # half an E4M3 step of the row max, relative 2**-4
        tol13 = np.abs(w13).max(axis=1, keepdims=True) * 2.0 ** -4
        tol2 = np.abs(w2).max(axis=1, keepdims=True) * 2.0 ** -4
    else:          # half an int4 step of each group's range, plus fp16 scale rounding
        tol13 = (np.ptp(w13.reshape(2 * I, -1, 128), axis=2) / 15 * 0.51 + 1e-4).repeat(128, axis=1)
        tol2 = (np.ptp(w2.reshape(H, -1, 128), axis=2) / 15 * 0.51 + 1e-4).repeat(128, axis=1)
    assert np.all(np.abs(W13 - w13) <= tol13)
    assert np.all(np.abs(W2 - w2) <= tol2)


def _dense_per_token(li, pool, k, H, I, act_mode):
    """Brute force: each token through its k experts one at a time, no align,
    routing from a plain stable argsort."""
    T = li.x_bits.shape[0]
    lg = li.logits.astype(np.float64)
    if li.mask is not None:
        lg = np.where(li.mask[None, :] != 0, lg, -np.inf)
    out = np.zeros((T, H))
    for t in range(T):
        top = np.argsort(-lg[t], kind="stable")[:k]
        z = np.exp(lg[t, top] - lg[t, top].max())
        w = z / z.sum()
        x = oracle.bf16_decode(li.x_bits[t])
        if act_mode == 1:
            x = oracle.act_quant_pow2(x[None, :])[2][0]
        for j, e in enumerate(top):
            s = li.slot_of_expert[e]
            W13, W2 = oracle.dequant_slot(pool[s], int(li.slot_fmt[s]), H, I)
            g, u = W13[:I] @ x, W13[I:] @ x
            h = g / (1 + np.exp(-g)) * u
            if act_mode == 1:
                h = oracle.act_quant_pow2(h[None, :])[2][0]
            out[t] += w[j] * (W2 @ h)
    return out


@pytest.mark.parametrize("act_mode", [0, 1])
@pytest.mark.parametrize("block_m", [1, 16, 64])
def test_layer_matches_dense_per_token_C0(act_mode, block_m):
    c = CONFIGS["C0"]
    li = make_layer(c, 16, 0)
    pool = layer_pool_bytes(li, make_bank(c))
    r = oracle.layer_forward(li.logits, li.mask, c.k, li.slot_of_expert, pool, li.slot_fmt,
                             c.H, c.I, li.x_bits, block_m, act_mode)
    want = _dense_per_token(li, pool, c.k, c.H, c.I, act_mode)
    assert np.allclose(r["out"], want, rtol=0, atol=1e-12 * np.abs(want).max())


def test_layer_matches_dense_mixed_int4_small():
    from gen.configs import Config
    c = Config("mix", 90, (12,), 256, 128, 6, 3, 1, 0.1, True, slots=6, int4_frac=0.5)
    li = make_layer(c, 12, 0)
    assert set(li.slot_fmt.tolist()) == {0, 1}
    pool = layer_pool_bytes(li, make_bank(c))
    r = oracle.layer_forward(li.logits, li.mask, c.k, li.slot_of_expert, pool, li.slot_fmt,
                             c.H, c.I, li.x_bits, 8, 0)
    want = _dense_per_token(li, pool, c.k, c.H, c.I, 0)
    assert np.allclose(r["out"], want, rtol=0, atol=1e-12 * np.abs(want).max())


def test_single_expert_is_a_dense_swiglu_mlp():
    """E=1, k=1: every weight is 1 and the layer is a plain SwiGLU MLP."""
    rng = np.random.default_rng(2)
    T, H, I = 9, 128, 64
    w13 = rng.standard_normal((2 * I, H)) * 0.05
    w2 = rng.standard_normal((H, I)) * 0.05
    slot = encode_slot(w13, w2, 0)
    W13, W2 = oracle.dequant_slot(slot, 0, H, I)
    x = rng.standard_normal((T, H)).astype(np.float32)
    x_bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    xv = (x_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    r = oracle.layer_forward(np.zeros((T, 1), np.float32), None, 1, np.zeros(1, np.int32),
                             slot[None, :], np.zeros(1, np.uint8), H, I, x_bits, 4, 0)
    G = xv @ W13[:I].T
    U = xv @ W13[I:].T
    want = (G * (1 / (1 + np.exp(-G))) * U) @ W2.T
    assert np.allclose(r["w"], 1.0)
    assert np.allclose(r["out"], want, rtol=0, atol=1e-13)


def test_token_subset_changes_nothing_else():
    c = CONFIGS["C0"]
    li = make_layer(c, 16, 0)
    pool = layer_pool_bytes(li, make_bank(c))
    full = oracle.layer_forward(li.logits, None, c.k, li.slot_of_expert, pool, li.slot_fmt,
                                c.H, c.I, li.x_bits, 16, 1)
    sub = oracle.layer_forward(li.logits, None, c.k, li.slot_of_expert, pool, li.slot_fmt,
                               c.H, c.I, li.x_bits, 16, 1, token_subset=[3, 7])
    assert np.array_equal(sub["out"][[3, 7]], full["out"][[3, 7]])
    assert np.all(sub["out"][[0, 1, 2]] == 0)


def test_nonresident_expert_contributes_zero():
    c = CONFIGS["C0"]
    li = make_layer(c, 16, 0)
    pool = layer_pool_bytes(li, make_bank(c))
    soe = li.slot_of_expert.copy()
    ids, w, _ = oracle.route(li.logits, None, c.k)
    e = int(ids[0, 0])
    soe[e] = -1
    r = oracle.layer_forward(li.logits, None, c.k, soe, pool, li.slot_fmt, c.H, c.I, li.x_bits, 4, 0)
    assert r["err"] == int((ids == e).sum())
    full = oracle.layer_forward(li.logits, None, c.k, li.slot_of_expert, pool, li.slot_fmt,
                                c.H, c.I, li.x_bits, 4, 0)
    # removing expert e's contribution by hand
    W13, W2 = oracle.dequant_slot(pool[li.slot_of_expert[e]], 0, c.H, c.I)
    diff = np.zeros_like(full["out"])
    for t, j in zip(*np.nonzero(ids == e)):
        x = oracle.bf16_decode(li.x_bits[t])
        g, u = W13[:c.I] @ x, W13[c.I:] @ x
        diff[t] = w[t, j] * (W2 @ (oracle.silu(g) * u))
    assert np.allclose(full["out"] - diff, r["out"], rtol=0, atol=1e-12)
