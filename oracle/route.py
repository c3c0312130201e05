"""Top-k routing of each token from its fp32 router logits.

PagedWeight commentary (spectral-agent.com), sections "what was released" and
"technically interesting points": a router picks, per token, the few experts
that process it. The pages give no formula. Reading taken:
* masked experts (not resident, when a mask is given) count as -inf;
* the k chosen experts are the first k in the order (logit descending, expert
  id ascending), comparing logits by IEEE value so -0.0 equals +0.0;
* their weights are the softmax over the k chosen logits, i.e. the softmax
  over all experts renormalised to the chosen ones, so each token's weights
  sum to 1. Selecting on logits equals selecting on exact probabilities.
A token with fewer than k unmasked experts keeps the ones it has, fills the
rest with id -1 and weight 0, and counts once in the error total.
"""
import numpy as np


def route(logits: np.ndarray, mask, k: int):
    """logits float32 [T, E]; mask uint8 [E] (nonzero = may be routed) or None.

    Returns (ids int32 [T, k], weights fp64 [T, k], err int).
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    vals = logits.astype(np.float64)
    allowed = np.ones(E, dtype=bool) if mask is None else (np.asarray(mask) != 0)
    ids = np.full((T, k), -1, dtype=np.int32)
    w = np.zeros((T, k), dtype=np.float64)
    err = 0
    experts = np.arange(E)
    for t in range(T):
        v = np.where(allowed, vals[t], -np.inf)
        order = np.lexsort((experts, -v))       # primary: -logit, then id
        n_ok = int(allowed.sum())
        take = order[:min(k, n_ok)]
        if n_ok < k:
            err += 1
        chosen = v[take]
        z = np.exp(chosen - chosen.max()) if take.size else chosen
        ids[t, :take.size] = take
        w[t, :take.size] = z / z.sum() if take.size else z
    return ids, w, err
