"""Seeded integer-valued layers: inputs on which every step of the layer is
exact, so the GPU result must equal the oracle's bit for bit.

Recipe (seeded PCG64, SeedSequence([90, H, I, E, k, T, tag])):

* x: columns [0, H/2) take values in {12, 16}, columns [H/2, H) in
  {-2, ..., 2} (bf16 and e4m3 hold them exactly; an all-integer row needs no
  rounding under any power-of-two scale).
* Every expert's w13 gate row has one nonzero, in {4, 8}, at a seeded column
  of the first half; every up row has two nonzeros, +-1, at seeded columns of
  the second half; every w2 row has two nonzeros in {+-1, +-2}. So the gate
  pre-activation lies in {48, 64, 96, 128} (large enough that
  z / (1 + exp(-z)) equals z in fp32 and in fp64), the up value in [-4, 4],
  h = gate * up has at most four significant bits (exact in e4m3 under its
  power-of-two group scale, and in bf16), y = w2 h is a multiple of 16 below
  2^11, and with k = 4 equal chosen logits every route weight is 1/4.
* Storage: FP8 slots hold the integer codes with row scale 1.0; int4 slots
  hold q = w + 7 with (scale, zero) = (1.0, 7.0) in every group.
* Routing: each token gets k distinct seeded experts with logit 1.0, every
  other expert logit 0.0 (ties in the chosen set are broken by the router's
  lower-id rule, which leaves the set itself fixed).

This module writes inputs only; the expected values come from the oracle.
"""
import numpy as np

from .configs import Config
from .inputs import (FMT_FP8_E4M3_ROW, FMT_INT4_G128, INT4_GROUP, LayerInputs, bf16_round, pool_stride,
                     slot_layout)

_TAG = {"x": 0, "w": 1, "route": 2, "slots": 3, "fmt": 4}


def _rng(H, I, E, k, T, tag):
    return np.random.default_rng(np.random.SeedSequence([90, H, I, E, k, T, _TAG[tag]]))


def integer_weights(H: int, I: int, e: int, seed_key):
    """Integer w13 [2I, H] and w2 [H, I] of expert e (int64)."""
    rng = np.random.default_rng(np.random.SeedSequence(list(seed_key) + [e]))
    w13 = np.zeros((2 * I, H), dtype=np.int64)
    w2 = np.zeros((H, I), dtype=np.int64)
    half = H // 2
    w13[np.arange(I), rng.integers(0, half, I)] = rng.choice([4, 8], I)
    for r in range(I, 2 * I):
        cols = rng.choice(np.arange(half, H), 2, replace=False)
        w13[r, cols] = rng.choice([-1, 1], 2)
    for r in range(H):
        cols = rng.choice(I, 2, replace=False)
        w2[r, cols] = rng.choice([-2, -1, 1, 2], 2)
    return w13, w2


def _fp8_codes(v: np.ndarray) -> np.ndarray:
    import torch
    return torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def encode_integer_slot(w13: np.ndarray, w2: np.ndarray, fmt: int) -> np.ndarray:
    H, I = w13.shape[1], w2.shape[1]
    lay = slot_layout(H, I, fmt)
    buf = np.zeros(lay["total"][1], dtype=np.uint8)

    def put(name, arr):
        off, n = lay[name]
        raw = np.ascontiguousarray(arr).view(np.uint8).reshape(-1)
        assert raw.size == n, (name, raw.size, n)
        buf[off:off + n] = raw

    if fmt == FMT_FP8_E4M3_ROW:
        put("w13", _fp8_codes(w13)); put("w13_scale", np.ones(2 * I, np.float32))
        put("w2", _fp8_codes(w2)); put("w2_scale", np.ones(H, np.float32))
        return buf

    def pack(w):
        q = (w + 7).astype(np.uint8)
        assert q.max() <= 15
        return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)

    def sz(rows, cols):
        a = np.empty((rows, cols // INT4_GROUP, 2), dtype=np.float16)
        a[:, :, 0] = 1.0
        a[:, :, 1] = 7.0
        return a

    put("w13", pack(w13)); put("w13_sz", sz(2 * I, H))
    put("w2", pack(w2)); put("w2_sz", sz(H, I))
    return buf


class IntegerBank:
    """Slot bytes of the integer experts, in both formats (the ExpertBank
    interface the test harness uses)."""

    def __init__(self, H, I, E, seed_key):
        self.H, self.I, self.n = H, I, E
        self.fmts = (FMT_FP8_E4M3_ROW, FMT_INT4_G128)
        self.stride = pool_stride(H, I, self.fmts)
        self.seed_key = tuple(seed_key)
        self._cache = {}

    def weights(self, e):
        return integer_weights(self.H, self.I, e, self.seed_key)

    def slot(self, e, fmt):
        key = (int(e), int(fmt))
        if key not in self._cache:
            w13, w2 = self.weights(e)
            self._cache[key] = encode_integer_slot(w13, w2, key[1])
        return self._cache[key]

    def materialize(self, fmt):
        out = np.zeros((self.n, self.stride), dtype=np.uint8)
        for e in range(self.n):
            s = self.slot(e, fmt)
            out[e, :s.size] = s
        return out


def make_integer_layer(H: int, I: int, E: int, k: int, T: int, int4_frac: float = 0.3):
    """Returns (LayerInputs, IntegerBank, x_int [T, H] int64)."""
    cfg = Config(f"int{H}x{I}", 90, (T,), H, I, E, k, 1, 0.0, False, slots=0, int4_frac=int4_frac)
    half = H // 2
    rx = _rng(H, I, E, k, T, "x")
    x = np.empty((T, H), dtype=np.int64)
    x[:, :half] = rx.choice([12, 16], (T, half))
    x[:, half:] = rx.integers(-2, 3, (T, H - half))
    x_bits = bf16_round(x.astype(np.float32))
    rr = _rng(H, I, E, k, T, "route")
    logits = np.zeros((T, E), dtype=np.float32)
    for t in range(T):
        logits[t, rr.choice(E, k, replace=False)] = 1.0
    expert_fmt = np.zeros(E, dtype=np.uint8)
    n4 = int(round(int4_frac * E)) if I % INT4_GROUP == 0 and H % INT4_GROUP == 0 else 0
    expert_fmt[_rng(H, I, E, k, T, "fmt").choice(E, n4, replace=False)] = FMT_INT4_G128
    slot_pos = _rng(H, I, E, k, T, "slots").permutation(E).astype(np.int32)
    slot_src = np.empty(E, dtype=np.int32)
    slot_src[slot_pos] = np.arange(E)
    slot_fmt = np.empty(E, dtype=np.uint8)
    slot_fmt[slot_pos] = expert_fmt
    li = LayerInputs(cfg, T, 0, x_bits, logits, None, slot_pos, slot_src, slot_fmt, expert_fmt)
    bank = IntegerBank(H, I, E, (91, H, I, E))
    return li, bank, x
