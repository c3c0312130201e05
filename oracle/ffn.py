"""Per-expert SwiGLU FFN over the aligned segments, then the weighted combine.

vllm-expert-pager article (rand.pepabo.com), Table 1 set-up: each expert holds
w13_weight (gate and up fused) and w2_weight (down); section "hierarchical
paging of expert weights": the weights are read from the expert's VRAM slot.
PagedWeight commentary (spectral-agent.com), section "what was released": the
layer output mixes the outputs of the experts the router chose. The pages give
no formula; reading taken (SwiGLU, the usual Qwen-MoE expert):
    gu = W13 a,  h = silu(gu[:I]) * gu[I:],  y = W2 h,
    out[t] = sum_j w[t, j] * y(t, j)      (kept in fp64)
Activation modes (the pages fix no activation precision):
* ACT_BF16: a is the bf16 token row itself and h is kept exact;
* ACT_FP8_G128_POW2: a and h are each quantized to E4M3 with one power-of-two
  scale per (row, 128 consecutive K elements), the operands an FP8 matrix
  instruction consumes; the oracle uses the dequantized values.
"""
import numpy as np

from .numerics import bf16_decode, act_quant_pow2, silu
from .slots import dequant_slot

ACT_BF16 = 0
ACT_FP8_G128_POW2 = 1


def expert_ffn(pool, slot_fmt, H: int, I: int, x_bits: np.ndarray, k: int, topk_w: np.ndarray,
               sorted_pair: np.ndarray, block_slot: np.ndarray, n_padded: int, block_m: int,
               act_mode: int, weights_of_slot=None, token_subset=None) -> np.ndarray:
    """Returns out fp64 [T, H]. pool[s] gives slot s's bytes; slot_fmt[s] its format.

    weights_of_slot(s) -> (W13, W2) may replace the decode of pool[s] (e.g. a
    cache). token_subset restricts the work to those tokens' outputs (rows of
    other tokens stay zero); it changes no arithmetic.
    """
    x_bits = np.asarray(x_bits)
    T = x_bits.shape[0]
    topk_w = np.asarray(topk_w, dtype=np.float64)
    sentinel = T * k
    if weights_of_slot is None:
        cache = {}

        def weights_of_slot(s):
            if s not in cache:
                cache[s] = dequant_slot(pool[s], int(slot_fmt[s]), H, I)
            return cache[s]
    want = None
    if token_subset is not None:
        want = np.zeros(T, dtype=bool)
        want[np.asarray(token_subset)] = True
    out = np.zeros((T, H), dtype=np.float64)
    for b in range(n_padded // block_m):
        s = int(block_slot[b])
        if s < 0:                       # expert not resident: contributes zero
            continue
        rows = np.asarray(sorted_pair[b * block_m:(b + 1) * block_m], dtype=np.int64)
        rows = rows[rows != sentinel]
        if want is not None:
            rows = rows[want[rows // k]]
        if rows.size == 0:
            continue
        t = rows // k
        j = rows % k
        a = bf16_decode(x_bits[t])                      # [n, H]
        if act_mode == ACT_FP8_G128_POW2:
            a = act_quant_pow2(a)[2]
        W13, W2 = weights_of_slot(s)
        gu = a @ W13.T                                  # [n, 2I]
        h = silu(gu[:, :I]) * gu[:, I:]                 # [n, I]
        if act_mode == ACT_FP8_G128_POW2:
            h = act_quant_pow2(h)[2]
        y = h @ W2.T                                    # [n, H]
        for r in range(rows.size):                      # weighted combine
            out[t[r]] += topk_w[t[r], j[r]] * y[r]
    return out
