"""Seeded synthetic inputs: activations, router logits, quantized expert slots.

Recipe (every draw comes from numpy's PCG64 seeded by
SeedSequence([cfg_id, T, layer, tag])):

* x ~ N(0, 1), rounded to bf16 (round to nearest even).
* Router: W_g ~ N(0, wg_std) [E, H]; optional log-Zipf(s=1.1) prior
  bias_e = ln p_e with p_e proportional to (pi_e + 1)^-1.1 for a seeded rank
  permutation pi. The prior gives the skewed, reuse-heavy expert choice the
  vllm-expert-pager article relies on (section on hierarchical paging of
  expert weights: recently chosen experts tend to be chosen again).
  logits = fp32(x @ W_g^T + bias), computed in fp64 and rounded once.
* Expert weights ~ N(0, w_std): w13 [2I, H] (rows [0, I) gate, [I, 2I) up)
  and w2 [H, I], the fused gate+up and down tensors the article names
  w13_weight and w2_weight (Table 1 set-up). They are generated once per
  "bank" expert and copied into each layer's slots.
* FP8 storage: per-row fp32 scale amax/448 and OCP e4m3fn codes (torch's CPU
  float8_e4m3fn cast, round to nearest even). INT4 storage: unsigned 4-bit,
  group 128 along K, fp16 (scale, zero) per group.
* Slot table: which experts are resident and in which slot. For decode-sized
  batches the resident set is every expert some token ranks in its top k
  (numpy stable argsort of the logits; this stands in for the pager's fill of
  missing experts before the layer runs) plus a seeded fill up to the slot
  count; if more experts are needed than there are slots, the pool grows to
  hold them all, the working-buffer rule of the article's paging section.

Nothing here computes routing weights, align, the FFN or the combine.
"""
from dataclasses import dataclass
from typing import Optional, Dict
import numpy as np

from .configs import Config

FMT_FP8_E4M3_ROW = 0
FMT_INT4_G128 = 1
INT4_GROUP = 128
SLOT_ALIGN = 256

_TAGS = {"x": 0, "Wg": 1, "zipf_perm": 2, "slot_perm": 3, "w13": 4, "w2": 5,
         "int4_pick": 6, "fill": 7, "bankmap": 8, "resident": 9}


def _rng(cfg_id: int, T: int, layer: int, tag: str) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg_id, T, layer, _TAGS[tag]]))


def _al(n: int) -> int:
    return (n + SLOT_ALIGN - 1) // SLOT_ALIGN * SLOT_ALIGN


def slot_layout(H: int, I: int, fmt: int) -> Dict[str, tuple]:
    """Byte offset and byte length of each array inside one slot."""
    if fmt == FMT_FP8_E4M3_ROW:
        parts = [("w13", 2 * I * H), ("w13_scale", 2 * I * 4), ("w2", H * I), ("w2_scale", H * 4)]
    elif fmt == FMT_INT4_G128:
        if H % INT4_GROUP or I % INT4_GROUP:
            raise ValueError("int4 slots need hidden and inter multiples of 128")
        parts = [("w13", 2 * I * H // 2), ("w13_sz", 2 * I * (H // INT4_GROUP) * 4),
                 ("w2", H * I // 2), ("w2_sz", H * (I // INT4_GROUP) * 4)]
    else:
        raise ValueError(f"unknown slot format {fmt}")
    # an int4 slot keeps 16 spare bytes after its last array (the library's
    # layout: its kernels read (scale, zero) rows 16 bytes at a time)
    tail = 16 if fmt == FMT_INT4_G128 else 0
    out, off = {}, 0
    for i, (name, n) in enumerate(parts):
        out[name] = (off, n)
        off = _al(off + n + (tail if i == len(parts) - 1 else 0))
    out["total"] = (0, off)
    return out


def slot_bytes(H: int, I: int, fmt: int) -> int:
    return slot_layout(H, I, fmt)["total"][1]


def pool_stride(H: int, I: int, fmts) -> int:
    return max(slot_bytes(H, I, f) for f in set(int(f) for f in fmts))


# ---------------------------------------------------------------- bf16 bits
def bf16_round(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even. No NaN/inf."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    b = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return b.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- quantizers (input preparation)
def _fp8_rows(w: np.ndarray):
    import torch
    w = np.asarray(w, dtype=np.float32)
    amax = np.abs(w).max(axis=1)
    scale = (amax / np.float32(448.0)).astype(np.float32)
    scale[amax == 0] = 1.0
    q = np.clip(w / scale[:, None], -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def _int4_rows(w: np.ndarray):
    w = np.asarray(w, dtype=np.float64)
    R, C = w.shape
    G = C // INT4_GROUP
    wg = w.reshape(R, G, INT4_GROUP)
    mn, mx = wg.min(axis=2), wg.max(axis=2)
    s = ((mx - mn) / 15.0).astype(np.float16)
    s[s == 0] = 1.0
    s64 = s.astype(np.float64)
    z = np.clip(np.rint(-mn / s64), 0, 15).astype(np.float16)
    q = np.clip(np.rint(wg / s64[:, :, None]) + z.astype(np.float64)[:, :, None], 0, 15)
    q = q.astype(np.uint8).reshape(R, C)
    packed = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    sz = np.stack([s, z], axis=2)  # [R, G, 2] fp16
    return packed, sz


def encode_slot(w13: np.ndarray, w2: np.ndarray, fmt: int) -> np.ndarray:
    """Quantize one expert's weights (fp32 or fp64) into the slot byte layout."""
    H = w13.shape[1]
    I = w2.shape[1]
    lay = slot_layout(H, I, fmt)
    buf = np.zeros(lay["total"][1], dtype=np.uint8)

    def put(name, arr):
        off, n = lay[name]
        raw = np.ascontiguousarray(arr).view(np.uint8).reshape(-1)
        assert raw.size == n, (name, raw.size, n)
        buf[off:off + n] = raw

    if fmt == FMT_FP8_E4M3_ROW:
        c13, s13 = _fp8_rows(w13)
        c2, s2 = _fp8_rows(w2)
        put("w13", c13); put("w13_scale", s13); put("w2", c2); put("w2_scale", s2)
    else:
        p13, sz13 = _int4_rows(w13)
        p2, sz2 = _int4_rows(w2)
        put("w13", p13); put("w13_sz", sz13); put("w2", p2); put("w2_sz", sz2)
    return buf


# ---------------------------------------------------------------- expert bank
class ExpertBank:
    """Seeded experts, generated lazily, each stored in every format asked for.

    Bank expert b of config c draws w13 and w2 from SeedSequence([c, 0, b, tag]).
    """

    def __init__(self, cfg: Config, fmts=(FMT_FP8_E4M3_ROW,)):
        self.cfg = cfg
        self.fmts = tuple(sorted(set(fmts)))
        self.n = cfg.E
        self.stride = pool_stride(cfg.H, cfg.I, self.fmts)
        self._cache: Dict[tuple, np.ndarray] = {}

    def weights(self, b: int):
        c = self.cfg
        w13 = _rng(c.cfg_id, 0, b, "w13").standard_normal((2 * c.I, c.H), dtype=np.float32)
        w2 = _rng(c.cfg_id, 0, b, "w2").standard_normal((c.H, c.I), dtype=np.float32)
        w13 *= np.float32(c.w_std)
        w2 *= np.float32(c.w_std)
        return w13, w2

    def slot(self, b: int, fmt: int) -> np.ndarray:
        key = (int(b), int(fmt))
        if key not in self._cache:
            w13, w2 = self.weights(b)
            for f in self.fmts:
                self._cache[(int(b), f)] = encode_slot(w13, w2, f)
        return self._cache[key]

    def materialize(self, fmt: int, workers: int = 8) -> np.ndarray:
        """All bank experts in one format as uint8 [n, stride] (zero padded)."""
        from concurrent.futures import ThreadPoolExecutor
        out = np.zeros((self.n, self.stride), dtype=np.uint8)

        def one(b):
            s = self.slot(b, fmt)
            out[b, :s.size] = s

        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(one, range(self.n)))
        return out


def make_bank(cfg: Config) -> ExpertBank:
    fmts = (FMT_FP8_E4M3_ROW, FMT_INT4_G128) if cfg.int4_frac > 0 else (FMT_FP8_E4M3_ROW,)
    return ExpertBank(cfg, fmts)


# ---------------------------------------------------------------- one layer
@dataclass
class LayerInputs:
    cfg: Config
    T: int
    layer: int
    x_bits: np.ndarray          # uint16 [T, H], bf16 bit patterns
    logits: np.ndarray          # float32 [T, E]
    mask: Optional[np.ndarray]  # uint8 [E] (1 = may be routed) or None
    slot_of_expert: np.ndarray  # int32 [E], -1 = not resident
    slot_src: np.ndarray        # int32 [S], bank expert copied into each slot
    slot_fmt: np.ndarray        # uint8 [S]
    expert_fmt: np.ndarray      # uint8 [E]

    @property
    def n_slots(self) -> int:
        return int(self.slot_src.size)


def zipf_prior(cfg: Config, T: int, layer: int) -> np.ndarray:
    perm = _rng(cfg.cfg_id, T, layer, "zipf_perm").permutation(cfg.E)
    p = (perm + 1.0) ** -1.1
    return p / p.sum()


def router_inputs(cfg: Config, T: int, layer: int):
    """The router gate of one layer as fp32 arrays: W_g [E, H] (the layer's
    N(0, wg_std) draw rounded to fp32) and bias [E] (the log-Zipf prior, or
    zeros), for the token rows of make_layer(cfg, T, layer)."""
    c = cfg
    Wg = _rng(c.cfg_id, T, layer, "Wg").standard_normal((c.E, c.H)) * c.wg_std
    bias = np.log(zipf_prior(c, T, layer)) if c.zipf else np.zeros(c.E)
    return Wg.astype(np.float32), bias.astype(np.float32)


def step_tokens(cfg: Config, T: int, layer: int, step: int):
    """Token rows and router logits of decode step `step` of one layer: new
    N(0, 1) rows each step (rounded to bf16), the layer's gate and log-Zipf
    prior fixed across steps (router_inputs), logits = fp32(x W_g^T + bias)
    computed in fp64. Reuse across steps comes from the prior alone."""
    c = cfg
    x = np.random.default_rng(np.random.SeedSequence([c.cfg_id, T, layer, 100, step])).standard_normal(
        (T, c.H), dtype=np.float32)
    x_bits = bf16_round(x)
    Wg, bias = router_inputs(c, T, layer)
    logits = (bf16_bits_to_f64(x_bits) @ Wg.astype(np.float64).T + bias.astype(np.float64)[None, :]).astype(np.float32)
    return x_bits, logits


def make_layer(cfg: Config, T: int, layer: int) -> LayerInputs:
    c = cfg
    E, H, k = c.E, c.H, c.k
    x = _rng(c.cfg_id, T, layer, "x").standard_normal((T, H), dtype=np.float32)
    x_bits = bf16_round(x)
    x64 = bf16_bits_to_f64(x_bits)
    Wg = _rng(c.cfg_id, T, layer, "Wg").standard_normal((E, H)) * c.wg_std
    bias = np.zeros(E)
    p = zipf_prior(c, T, layer) if c.zipf else np.full(E, 1.0 / E)
    if c.zipf:
        bias = np.log(p)
    logits = (x64 @ Wg.T + bias[None, :]).astype(np.float32)

    # which bank expert backs expert e of this layer
    if c.layers == 1:
        bankmap = np.arange(E)
    else:
        bankmap = _rng(c.cfg_id, T, layer, "bankmap").permutation(E)

    expert_fmt = np.zeros(E, dtype=np.uint8)
    if c.int4_frac > 0:
        n4 = int(round(c.int4_frac * E))
        q = (1.0 / p) / (1.0 / p).sum()
        pick = _rng(c.cfg_id, T, layer, "int4_pick").choice(E, n4, replace=False, p=q)
        expert_fmt[pick] = FMT_INT4_G128

    mask = None
    all_resident = c.slots == 0 or T >= c.resident_all_at
    if all_resident:
        resident = np.arange(E)
        if c.name == "C2":
            slot_pos = np.arange(E)  # identity map (prefill working buffer)
        else:
            slot_pos = _rng(c.cfg_id, T, layer, "slot_perm").permutation(E)
    elif c.masked_resident:
        resident = np.sort(_rng(c.cfg_id, T, layer, "resident").choice(E, c.slots, replace=False))
        mask = np.zeros(E, dtype=np.uint8)
        mask[resident] = 1
        slot_pos = _rng(c.cfg_id, T, layer, "slot_perm").permutation(resident.size)
    else:
        top = np.argsort(-logits, axis=1, kind="stable")[:, :k]
        routed = np.unique(top)
        rest = np.setdiff1d(np.arange(E), routed)
        S = max(c.slots, routed.size)
        fill = _rng(c.cfg_id, T, layer, "fill").permutation(rest)[:S - routed.size]
        resident = np.sort(np.concatenate([routed, fill]))
        slot_pos = _rng(c.cfg_id, T, layer, "slot_perm").permutation(resident.size)

    S = resident.size
    slot_of_expert = np.full(E, -1, dtype=np.int32)
    slot_of_expert[resident] = slot_pos.astype(np.int32)
    slot_src = np.full(S, -1, dtype=np.int32)
    slot_fmt = np.zeros(S, dtype=np.uint8)
    slot_src[slot_pos] = bankmap[resident]
    slot_fmt[slot_pos] = expert_fmt[resident]
    return LayerInputs(c, T, layer, x_bits, logits, mask, slot_of_expert, slot_src, slot_fmt, expert_fmt)


def layer_pool_bytes(li: LayerInputs, bank: ExpertBank) -> np.ndarray:
    """Host copy of one layer's slot pool, uint8 [S, stride] (small configs)."""
    out = np.zeros((li.n_slots, bank.stride), dtype=np.uint8)
    for s in range(li.n_slots):
        b = bank.slot(li.slot_src[s], li.slot_fmt[s])
        out[s, :b.size] = b
    return out
