"""One MoE expert layer end to end: route -> align -> expert FFN + combine.

This is the order of the steps the vllm-expert-pager article (rand.pepabo.com,
section "hierarchical paging of expert weights") walks through for one layer:
the router's choice decides which experts' slots are read, and the MOE-GEN
explainer (aibr.jp, section 3) groups the tokens per expert before running it.
"""
import numpy as np

from .route import route
from .align import align
from .ffn import expert_ffn


def layer_forward(logits, mask, k, slot_of_expert, pool, slot_fmt, H, I, x_bits,
                  block_m, act_mode, weights_of_slot=None, token_subset=None):
    logits = np.asarray(logits, dtype=np.float32)
    E = logits.shape[1]
    ids, w, route_err = route(logits, mask, k)
    al = align(ids, E, block_m, slot_of_expert)
    out = expert_ffn(pool, slot_fmt, H, I, x_bits, k, w, al["sorted_pair"], al["block_slot"],
                     al["n_padded"], block_m, act_mode, weights_of_slot=weights_of_slot,
                     token_subset=token_subset)
    return dict(ids=ids, w=w, route_err=route_err, out=out, **al)
