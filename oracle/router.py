"""Router gate: the logits the router ranks experts by.

PagedWeight commentary (spectral-agent.com), "technically interesting
points": a router picks, per token, the experts that process it. The pages
give no formula; reading taken (the usual MoE gate, the one the synthetic
workloads are drawn from): a linear map of the token row,
    logits[t, e] = sum_h x[t, h] * W_g[e, h] + bias[e],
with x the bf16 token row, W_g the fp32 gate matrix [E, H] and an optional
fp32 per-expert bias, evaluated exactly (fp64 products and sums of the given
values; the fp32 rounding of the result is left to the caller).
"""
import numpy as np

from .numerics import bf16_decode


def router_logits(x_bits: np.ndarray, W_g: np.ndarray, bias=None) -> np.ndarray:
    """x_bits uint16 [T, H] (bf16), W_g float32 [E, H], bias float32 [E] or None -> fp64 [T, E]."""
    x = bf16_decode(x_bits)
    W = np.asarray(W_g, dtype=np.float32).astype(np.float64)
    out = x @ W.T
    if bias is not None:
        out = out + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]
    return out


def fp32_sum_bound(x_bits: np.ndarray, W_g: np.ndarray, n_terms: int) -> np.ndarray:
    """A bound on |fp32 evaluation - exact| for any order of summing n_terms
    exact products whose absolute values add to sum_h |x W| (the standard
    gamma_n bound, n u / (1 - n u), u = 2^-24), plus one rounding of the
    bias add. fp64 [T, E]."""
    x = np.abs(bf16_decode(x_bits))
    W = np.abs(np.asarray(W_g, dtype=np.float32).astype(np.float64))
    u = 2.0 ** -24
    g = n_terms * u / (1 - n_terms * u)
    return g * (x @ W.T)
