"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins catch every one of them."""
import importlib.util
import math
import os
import shutil
import sys

import numpy as np
import pytest

from golden_io import lines, closed_form, kv
from gen import encode_slot

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")

MUTANTS = {
    "gate_up_swapped": ("ffn.py", "h = silu(gu[:, :I]) * gu[:, I:]", "h = silu(gu[:, I:]) * gu[:, :I]"),
    "route_weight_dropped": ("ffn.py", "topk_w[t[r], j[r]] * y[r]", "y[r]"),
    "silu_sign": ("numerics.py", "z / (1.0 + np.exp(-z))", "z / (1.0 + np.exp(z))"),
    "ties_to_higher_id": ("route.py", "np.lexsort((experts, -v))", "np.lexsort((-experts, -v))"),
    "no_renormalise": ("route.py", "z / z.sum() if take.size else z", "z if take.size else z"),
    "softmax_no_shift_sign": ("route.py", "np.exp(chosen - chosen.max())", "np.exp(chosen.max() - chosen)"),
    "align_unstable": ("align.py", "for p in range(flat.size):", "for p in reversed(range(flat.size)):"),
    "align_no_padding": ("align.py", "padded = -(-counts // block_m) * block_m", "padded = counts"),
    "block_slot_by_block": ("align.py", "block_slot[b0:b1] = slot_of_expert[e]", "block_slot[b0:b1] = e"),
    "e4m3_bias": ("numerics.py", "2.0 ** (e - 7)", "2.0 ** (e - 8)"),
    "e4m3_subnormal": ("numerics.py", "(2.0 ** -6) * (m / 8.0)", "(2.0 ** -7) * (m / 8.0)"),
    "rne_ties_up": ("numerics.py", "((d_lo == d_hi) & (_POS_CODES[lo] % 2 == 0))", "((d_lo == d_hi) & False)"),
    "int4_nibble_order": ("slots.py", "q[:, 0::2] = p & 0x0F\n    q[:, 1::2] = p >> 4",
                          "q[:, 0::2] = p >> 4\n    q[:, 1::2] = p & 0x0F"),
    "int4_zero_sign": ("slots.py", "return (q - zero) * scale", "return (q + zero) * scale"),
    "fp8_scale_missing": ("slots.py", "return c13 * s13[:, None], c2 * s2[:, None]",
                          "return c13, c2 * s2[:, None]"),
    "w2_scale_index": ("slots.py", "c2 * s2[:, None]", "c2 * s2[::-1][:, None]"),
    "pow2_scale_exponent_dropped": ("numerics.py", "deq[:, sl] = np.ldexp(E4M3_TABLE[c], s[:, None])",
                                    "deq[:, sl] = E4M3_TABLE[c]"),
    "pow2_scale_too_large": ("numerics.py", "s[nz] = np.ceil(np.log2(amax[nz] / 448.0)).astype(np.int64)",
                             "s[nz] = np.ceil(np.log2(amax[nz] / 448.0)).astype(np.int64) + 3"),
    "act_group_wrong": ("numerics.py", "ACT_GROUP = 128", "ACT_GROUP = 64"),
    "router_bias_dropped": ("router.py", "out = out + np.asarray(bias", "out = out + 0 * np.asarray(bias"),
    "router_bias_sign": ("router.py", "out = out + np.asarray(bias", "out = out - np.asarray(bias"),
    "router_x_not_decoded": ("router.py", "x = bf16_decode(x_bits)", "x = np.asarray(x_bits, dtype=np.float64)"),
    "requant_divisor_16": ("requant.py", "(mx - mn) / np.float32(15.0)", "(mx - mn) / np.float32(16.0)"),
    "requant_zero_sign": ("requant.py", "np.rint((-mn) / s32)", "np.rint(mn / s32)"),
    "requant_nibble_order": ("requant.py", "(q[:, 0::2] | (q[:, 1::2] << 4))", "(q[:, 1::2] | (q[:, 0::2] << 4))"),
    "plan_ties_to_higher_id": ("requant.py", "key=lambda e: (int(counts[e]), e)", "key=lambda e: (int(counts[e]), -e)"),
    "lru_evicts_most_recent": ("pager.py", "key=lambda v: (self.last[v], v))", "key=lambda v: (-self.last[v], v))"),
    "lru_free_slot_highest": ("pager.py", "slot = free[0]", "slot = free[-1]"),
    "huffman_ties_to_higher_symbol": ("huffman.py", "nodes.sort(key=lambda n: (n[0], n[1]))",
                                      "nodes.sort(key=lambda n: (n[0], -n[1]))"),
    "huffman_no_length_limit": ("huffman.py", "while max(lens) > MAX_LEN:", "while max(lens) > MAX_LEN + 8:"),
    "huffman_floor_not_scaled": ("huffman.py", "floor = (total << k) // 256 + 1", "floor = total // 256 + 1 + k"),
    "huffman_canonical_order": ("huffman.py", "order = sorted((l, s) for s, l in enumerate(lens) if l > 0)",
                                "order = sorted((l, -s) for s, l in enumerate(lens) if l > 0)\n    order = [(l, -s) for l, s in order]"),
    "lru_no_touch_on_hit": ("pager.py", "        for e in want:\n            self.last[e] = self.step",
                            "        for e, _ in fills:\n            self.last[e] = self.step"),
}


def load_variant(tmp_path, name, mutation=None):
    dst = tmp_path / name
    pkg = dst / ("oracle_" + name)
    shutil.copytree(ORACLE_DIR, pkg, ignore=shutil.ignore_patterns("__pycache__"))
    if mutation:
        fname, old, new = mutation
        src = (pkg / fname).read_text()
        assert src.count(old) == 1, (name, old)
        (pkg / fname).write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("oracle_" + name, pkg / "__init__.py",
                                                  submodule_search_locations=[str(pkg)])
    mod = importlib.util.module_from_spec(spec)
    sys.modules["oracle_" + name] = mod
    spec.loader.exec_module(mod)
    return mod


# ---- the pins, written against a module argument
def pin_e4m3(m):
    for ln in lines("e4m3_decode.txt"):
        code, val = ln.split()
        got, want = m.E4M3_TABLE[int(code, 16)], float(val)
        if not (math.isnan(want) and math.isnan(got)) and got != want:
            return False
    for ln in lines("e4m3_rne.txt"):
        val, code = ln.split()
        if int(m.e4m3_encode_rne(np.array([float(val)]))[0]) != int(code, 16):
            return False
    return True


def pin_route(m):
    for ln in lines("route_tiny.txt"):
        head, lg, mk, ids, ws, err = [f.strip() for f in ln.split("|")]
        E, k = map(int, head.split())
        logits = np.array([[float(v) for v in lg.split()]], dtype=np.float32)
        mask = None if mk == "-" else np.array([int(v) for v in mk.split()], dtype=np.uint8)
        gi, gw, ge = m.route(logits, mask, k)
        if gi[0].tolist() != [int(v) for v in ids.split()]:
            return False
        if not np.allclose(gw[0], [closed_form(v) for v in ws.split()], atol=1e-15, rtol=0):
            return False
    return True


def pin_align(m):
    g = kv("align_tiny.txt")
    T, k, E, bm = (int(g[n][0]) for n in ("T", "k", "E", "block_m"))
    ids = np.array([int(v) for v in g["ids"]], dtype=np.int32).reshape(T, k)
    al = m.align(ids, E, bm, np.array([int(v) for v in g["slot_of_expert"]], dtype=np.int32))
    return all(al[n].tolist() == [int(v) for v in g[n]] for n in ("counts", "seg_offset", "sorted_pair", "block_slot"))


def pin_ffn(m):
    from test_oracle_ffn import tiny_case
    pool, x_bits, logits, want = tiny_case(m)
    r = m.layer_forward(logits, None, 1, np.array([1, 0], dtype=np.int32), pool,
                        np.zeros(2, np.uint8), 2, 1, x_bits, 2, 0)
    return np.allclose(r["out"], want, rtol=1e-14, atol=0)


def pin_slots(m):
    rng = np.random.default_rng(1)
    H, I = 256, 128
    w13 = rng.standard_normal((2 * I, H)) * 0.02
    w2 = rng.standard_normal((H, I)) * 0.02
    for fmt in (0, 1):
        W13, W2 = m.dequant_slot(encode_slot(w13, w2, fmt), fmt, H, I)
        for W, w in ((W13, w13), (W2, w2)):
            if fmt == 0:
                tol = np.abs(w).max(axis=1, keepdims=True) * 2.0 ** -4
            else:
                tol = (np.ptp(w.reshape(w.shape[0], -1, 128), axis=2) / 15 * 0.51 + 1e-4).repeat(128, axis=1)
            if np.any(np.abs(W - w) > tol):
                return False
    return True


def pin_act_quant(m):
    rng = np.random.default_rng(3)
    v = rng.standard_normal((4, 256)) * 10
    _, exps, deq = m.act_quant_pow2(v)
    if exps.shape != (4, 2):
        return False
    for r in range(4):
        for g in range(2):
            mx = np.abs(v[r, g * 128:(g + 1) * 128]).max() / 2.0 ** exps[r, g]
            if not 224 < mx <= 448:
                return False
    return np.abs(deq - v).max() <= np.abs(v).max() * 2.0 ** -4


def pin_dense_C0(m):
    """Whole layer against the per-token brute force of test_oracle_ffn."""
    from test_oracle_ffn import _dense_per_token
    from gen import CONFIGS, make_layer, make_bank, layer_pool_bytes
    c = CONFIGS["C0"]
    li = make_layer(c, 16, 0)
    pool = layer_pool_bytes(li, make_bank(c))
    for act in (0, 1):
        r = m.layer_forward(li.logits, li.mask, c.k, li.slot_of_expert, pool, li.slot_fmt,
                            c.H, c.I, li.x_bits, 4, act)
        want = _dense_per_token(li, pool, c.k, c.H, c.I, act)
        if not np.allclose(r["out"], want, rtol=0, atol=1e-12 * np.abs(want).max()):
            return False
    return True


def pin_router(m):
    g = kv("router_tiny.txt")
    f = lambda key: [float(v) for v in g[key]]
    from gen import bf16_round
    x = np.array([f("x0"), f("x1")], dtype=np.float32)
    W = np.array([f("w0"), f("w1"), f("w2")], dtype=np.float32)
    out = m.router_logits(bf16_round(x), W, np.array(f("bias"), dtype=np.float32))
    return out.tolist() == [f("out0"), f("out1")]


def pin_integer_layer(m):
    """The integer-valued layer against int64 arithmetic (test_oracle_exact)."""
    from gen import make_integer_layer
    from test_oracle_exact import integer_reference
    li, bank, x_int = make_integer_layer(256, 128, 8, 4, 24)
    pool = np.zeros((li.n_slots, bank.stride), dtype=np.uint8)
    for s in range(li.n_slots):
        b = bank.slot(li.slot_src[s], li.slot_fmt[s])
        pool[s, :b.size] = b
    want = integer_reference(li, bank, x_int)
    for act in (0, 1):
        r = m.layer_forward(li.logits, None, 4, li.slot_of_expert, pool, li.slot_fmt, 256, 128, li.x_bits, 16, act)
        if not np.array_equal(r["out"], want):
            return False
    return True


def pin_requant(m):
    from test_oracle_requant import test_requant_reproduces_a_grid_exact_slot, test_plan_least_routed_ties_to_lower_id
    import test_oracle_requant as tr
    saved = tr.oracle
    tr.oracle = m
    try:
        test_requant_reproduces_a_grid_exact_slot()
        test_plan_least_routed_ties_to_lower_id()
    finally:
        tr.oracle = saved
    return True


def pin_pager(m):
    import test_oracle_pager as tp
    saved = tp.oracle
    tp.oracle = m
    try:
        tp.test_lru_hand_case()
    finally:
        tp.oracle = saved
    return True


def pin_huffman(m):
    import test_oracle_huffman as th
    saved = th.huffman
    th.huffman = m.huffman
    try:
        th.test_textbook_huffman_lengths()
        th.test_ties_single_symbol_and_flat_fallback()
        # canonical code values of a fixed set of lengths, worked by hand
        codes = m.huffman.canonical_codes([2, 0, 3, 3, 2, 2] + [0] * 10)
        if codes != {0: (0, 2), 4: (1, 2), 5: (2, 2), 2: (6, 3), 3: (7, 3)}:
            return False
    finally:
        th.huffman = saved
    return True


PINS = [pin_e4m3, pin_route, pin_align, pin_ffn, pin_slots, pin_act_quant, pin_dense_C0, pin_router,
        pin_integer_layer, pin_requant, pin_pager, pin_huffman]


def all_pins_pass(m):
    ok = True
    for p in PINS:
        try:
            ok &= bool(p(m))
        except Exception:
            ok = False
    return ok


def test_unmutated_copy_passes_every_pin(tmp_path):
    assert all_pins_pass(load_variant(tmp_path, "clean"))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    assert not all_pins_pass(load_variant(tmp_path, name, MUTANTS[name])), name
