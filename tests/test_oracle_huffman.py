"""Pins of the compressed host tier's format (CPU only): per-row canonical
Huffman codes of FP8 exponents, and the library's host packer producing the
oracle's bytes."""
import os

import numpy as np
import pytest

import oracle
from oracle import huffman
from gen import encode_slot


def test_textbook_huffman_lengths():
    """Frequencies a:45 b:13 c:12 d:16 e:9 f:5 (the classic example) give
    lengths a 1, b c d 3, e f 4."""
    counts = [45, 13, 12, 16, 9, 5] + [0] * 10
    assert huffman.code_lengths(counts)[:6] == [1, 3, 3, 3, 4, 4]
    assert huffman.code_lengths(counts)[6:] == [0] * 10


def test_ties_single_symbol_and_flat_fallback():
    # equal weights 1,1,1,1: merges (0,1), then (2,3), then both: all length 2
    assert huffman.code_lengths([1, 1, 1, 1] + [0] * 12)[:4] == [2, 2, 2, 2]
    # weights 1,1,1: the two lower symbols merge first, so symbol 2 gets the short code
    assert huffman.code_lengths([1, 1, 1] + [0] * 13)[:3] == [2, 2, 1]
    # weights 1,1,2: (0,1) first (ties to the lower symbol), then with 2
    assert huffman.code_lengths([1, 1, 2] + [0] * 13)[:3] == [2, 2, 1]
    assert huffman.code_lengths([0] * 7 + [9] + [0] * 8) == [0] * 7 + [1] + [0] * 8
    # Fibonacci weights 1 1 2 3 5 8 13 21 34 55 make a depth-9 tree; with the
    # floor 143 // 256 + 1 = 1 added (k = 0) the weights 2 2 3 4 6 9 14 22 35
    # 56 merge (worked by hand) into lengths 6 6 5 4 4 4 3 3 2 2
    fib = [1, 1, 2, 3, 5, 8, 13, 21, 34, 55] + [0] * 6
    assert max(huffman._huffman_lengths(fib)) == 9
    assert huffman.code_lengths(fib) == [6, 6, 5, 4, 4, 4, 3, 3, 2, 2] + [0] * 6
    # counts 1 1 1 1 1 10 16 26 83 116 162 (total 418): with floor 418 // 256
    # + 1 = 2 symbol 0 still sits at depth 9 (worked by hand); with the k = 1
    # floor 836 // 256 + 1 = 4 the weights 5 5 5 5 5 14 20 30 87 120 166 give
    # lengths 6 6 6 6 5 5 4 4 2 2 2 (worked by hand)
    two = [1, 1, 1, 1, 1, 10, 16, 26, 83, 116, 162] + [0] * 5
    assert huffman.code_lengths(two) == [6, 6, 6, 6, 5, 5, 4, 4, 2, 2, 2] + [0] * 5


def test_canonical_codes_are_prefix_free_and_complete():
    rng = np.random.default_rng(0)
    for _ in range(200):
        counts = rng.integers(0, 50, 16) * (rng.random(16) < 0.7)
        if counts.sum() == 0 or (counts > 0).sum() < 2:
            continue
        lens = huffman.code_lengths(counts)
        codes = huffman.canonical_codes(lens)
        assert sum(2.0 ** -l for l in lens if l) == 1.0                  # Kraft equality: a full tree
        words = [format(c, f"0{l}b") for c, l in codes.values()]
        for a in words:
            for b in words:
                assert a == b or not b.startswith(a)
        assert max(lens) <= huffman.MAX_LEN


def test_round_trip_and_size():
    rng = np.random.default_rng(1)
    H, I = 512, 256
    slot = encode_slot(rng.standard_normal((2 * I, H)) * 0.02, rng.standard_normal((H, I)) * 0.02, 0)
    packed = huffman.pack_slot(slot, H, I)
    assert np.array_equal(huffman.unpack_slot(packed, H, I), slot[:huffman.unpack_slot(packed, H, I).size])
    assert packed.size < 0.95 * slot.size


def _skewed_slot(H, I, seed):
    """FP8 codes with rows of every kind: Gaussian, constant (one exponent),
    heavy-tailed (long codes, the flat fallback) and all-zero."""
    rng = np.random.default_rng(seed)
    slot = encode_slot(rng.standard_normal((2 * I, H)) * 0.02, rng.standard_normal((H, I)) * 0.02, 0)
    offs, sizes, _ = oracle.slot_offsets(H, I, 0)
    w13 = slot[offs[0]:offs[0] + sizes[0]].reshape(2 * I, H)
    w13[0] = 0x38
    w13[1] = 0
    w13[2] = rng.choice(np.arange(256, dtype=np.uint8), H, p=np.r_[np.full(128, 0.5 / 128), np.full(128, 0.5 / 128)])
    fib = np.array([1, 1, 2, 3, 5, 8, 13, 21, 34, 55, 89, 144], float)
    w13[3] = (rng.choice(12, H, p=fib / fib.sum()) << 3).astype(np.uint8) | rng.integers(0, 8, H).astype(np.uint8)
    # exponent counts that need the second floor step (with the rest on exponent 11)
    counts = [1, 1, 1, 1, 1, 10, 16, 26, 83, 116, 162]
    if H >= sum(counts):
        ex = np.concatenate([np.repeat(np.arange(11), counts), np.full(H - sum(counts), 11)])
        w13[4] = (rng.permutation(ex) << 3).astype(np.uint8)
    return slot


@pytest.mark.parametrize("H,I,seed", [(512, 256, 2), (256, 768, 3)])
def test_library_packer_matches_oracle(H, I, seed):
    import moe_expert_layer_topk_amd as moe
    if not os.path.exists(moe.LIB_PATH):
        pytest.skip("library not built")
    slot = _skewed_slot(H, I, seed)
    want = huffman.pack_slot(slot, H, I)
    got = moe.fp8_pack(slot, H, I)
    assert got.size == want.size and np.array_equal(got, want)
    assert np.array_equal(huffman.unpack_slot(want, H, I), slot[:huffman.unpack_slot(want, H, I).size])
