"""Group token-expert pairs by expert: a stable counting sort into padded
per-expert segments, plus the expert -> slot indirection.

MOE-GEN explainer (aibr.jp), sections 1 and 3: tokens are gathered per expert
module so each expert runs one large batch instead of many tiny ones.
vllm-expert-pager article (rand.pepabo.com), section "hierarchical paging of
expert weights": each layer keeps a table of which experts sit in which VRAM
slot. Reading taken for the layout (the pages fix none): pair p = t*k + j;
segments in ascending expert id; inside a segment pairs keep ascending p; each
segment is padded to a multiple of block_m with the sentinel T*k; an expert
with no pairs has no block; every block records the slot of its expert.
"""
import numpy as np


def align_capacity(T: int, k: int, E: int, block_m: int) -> int:
    """Upper bound on the padded length: T*k pairs plus at most block_m-1
    padding rows for each of the at most min(E, T*k) non-empty segments."""
    n = T * k + min(E, T * k) * (block_m - 1)
    return -(-n // block_m) * block_m


def align(ids: np.ndarray, E: int, block_m: int, slot_of_expert: np.ndarray):
    """ids int32 [T, k] -> dict of int32 arrays and error count.

    sorted_pair [n_padded], block_slot [n_padded // block_m], counts [E],
    seg_offset [E + 1], n_padded, err. Pairs whose id is outside [0, E) take no
    part; pairs routed to an expert with slot -1 keep their place but their
    blocks carry slot -1. err counts both kinds of pair.
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    sentinel = T * k
    valid = (flat >= 0) & (flat < E)
    counts = np.bincount(flat[valid], minlength=E).astype(np.int64)
    padded = -(-counts // block_m) * block_m
    seg_offset = np.zeros(E + 1, dtype=np.int64)
    seg_offset[1:] = np.cumsum(padded)
    n_padded = int(seg_offset[E])
    sorted_pair = np.full(n_padded, sentinel, dtype=np.int64)
    fill = seg_offset[:E].copy()
    for p in range(flat.size):          # ascending p keeps each segment stable
        if valid[p]:
            e = flat[p]
            sorted_pair[fill[e]] = p
            fill[e] += 1
    block_slot = np.empty(n_padded // block_m, dtype=np.int64)
    slot_of_expert = np.asarray(slot_of_expert, dtype=np.int64)
    for e in range(E):
        b0, b1 = seg_offset[e] // block_m, seg_offset[e + 1] // block_m
        block_slot[b0:b1] = slot_of_expert[e]
    nonresident = int(sum(counts[e] for e in range(E) if slot_of_expert[e] < 0))
    err = int((~valid).sum()) + nonresident
    return dict(sorted_pair=sorted_pair.astype(np.int32), block_slot=block_slot.astype(np.int32),
                counts=counts.astype(np.int32), seg_offset=seg_offset.astype(np.int32),
                n_padded=n_padded, err=err)
