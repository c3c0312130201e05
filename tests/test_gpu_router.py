"""The router gate GEMM (moe_route_gemm) against the oracle.

The logits may differ from the exact values only by the rounding of an fp32
sum of exact products: |gpu - exact| <= gamma_{3H+8} sum |x W| plus a few
roundings of the result. Routing is then checked bit for bit on the GPU's own
logits (the oracle's route on them), and against the oracle's exact logits for
every token whose k + 1 best logits are further apart than twice the token's
largest deviation (closer logits can legitimately swap under fp32 summation).
"""
import numpy as np
import pytest

import oracle
import moe_expert_layer_topk_amd as moe
from gen import CONFIGS, make_layer, router_inputs
from gen.configs import Config

pytestmark = pytest.mark.gpu


def _run(gpu, li, W, b, k, mask=None):
    import torch
    x = torch.from_numpy(li.x_bits.view(np.int16).copy()).to(gpu).view(torch.bfloat16)
    Wd = torch.from_numpy(W).to(gpu)
    bd = None if b is None else torch.from_numpy(b).to(gpu)
    md = None if mask is None else torch.from_numpy(mask).to(gpu)
    logits, ids, w, err = moe.route_gemm(x, Wd, k, bias=bd, mask=md)
    torch.cuda.synchronize()
    ref = oracle.router_logits(li.x_bits, W, b)
    tol = oracle.fp32_sum_bound(li.x_bits, W, 3 * li.cfg.H + 8) + 2.0 ** -22 * (np.abs(ref) + (0 if b is None else np.abs(b)[None, :]))
    got = logits.cpu().numpy().astype(np.float64)
    dev = np.abs(got - ref)
    print(f"    max |logit - exact| {dev.max():.3e} (bound {tol.max():.3e})", flush=True)
    assert np.all(dev <= tol)
    # routing of the GPU's own logits: bit-exact
    oi, ow, oe = oracle.route(logits.cpu().numpy(), mask, k)
    gi = ids.cpu().numpy()
    assert np.array_equal(gi, oi)
    assert np.abs(w.cpu().numpy() - ow).max() <= 1e-6
    assert int(err.item()) == oe
    # against the exact logits wherever the GPU's deviation cannot reorder
    # them: every gap among a token's k + 1 best exact logits wider than
    # twice that token's largest deviation (which the bound above limits)
    ri, _, _ = oracle.route(ref.astype(np.float32), mask, k)
    v = np.where(mask[None, :] != 0, ref, -np.inf) if mask is not None else ref
    srt = -np.sort(-v, axis=1)[:, :k + 1]
    gaps = srt[:, :-1] - srt[:, 1:]
    decided = np.all(gaps > 2 * dev.max(axis=1, keepdims=True), axis=1)
    assert np.array_equal(gi[decided], ri[decided])
    assert decided.mean() > 0.9
    return logits


@pytest.mark.parametrize("name,T", [("C0", 16), ("C1", 1), ("C1", 32), ("C1", 64), ("C2", 16384), ("C3", 4096),
                                    ("C3", 32)])
def test_route_gemm_matches_oracle(gpu, name, T):
    c = CONFIGS[name]
    li = make_layer(c, T, 0)
    W, b = router_inputs(c, T, 0)
    print(f"[router] {name} T={T} E={c.E} H={c.H}", flush=True)
    _run(gpu, li, W, b if c.zipf else None, c.k, li.mask)


def test_route_gemm_wide_and_ragged(gpu):
    """E = 1000 (not a multiple of 16), T = 70 (ragged token tiles), no bias."""
    c = Config("wr", 75, (70,), 512, 128, 1000, 8, 1, 0.05, False)
    li = make_layer(c, 70, 0)
    W, _ = router_inputs(c, 70, 0)
    _run(gpu, li, W, None, 8)


def test_route_gemm_repeats_bit_for_bit(gpu):
    import torch
    c = CONFIGS["C2"]
    li = make_layer(c, 4096, 1)
    W, b = router_inputs(c, 4096, 1)
    x = torch.from_numpy(li.x_bits.view(np.int16).copy()).to(gpu).view(torch.bfloat16)
    Wd, bd = torch.from_numpy(W).to(gpu), torch.from_numpy(b).to(gpu)
    l1, i1, _, _ = moe.route_gemm(x, Wd, c.k, bias=bd)
    l2, i2, _, _ = moe.route_gemm(x, Wd, c.k, bias=bd)
    torch.cuda.synchronize()
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)) and torch.equal(i1, i2)
