"""Number formats and element-wise steps, written out from their definitions.

The vllm-expert-pager article (rand.pepabo.com, introduction and section
"positioning") serves the model's official FP8 weights unchanged; the page does
not name the FP8 variant. Reading taken: OCP E4M3FN, the variant gfx950
matrix cores consume, decoded from its bit-field definition below.
"""
import numpy as np

ACT_GROUP = 128  # activation-scale group along the contraction axis


def _e4m3_value(code: int) -> float:
    """OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities;
    exponent 15 with mantissa 7 is NaN; exponent 0 is subnormal."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (2.0 ** -6) * (m / 8.0)
    return s * (2.0 ** (e - 7)) * (1.0 + m / 8.0)


E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)

# finite non-negative codes 0x00..0x7E in increasing value order
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALS = E4M3_TABLE[:0x7F]


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode_rne(v: np.ndarray) -> np.ndarray:
    """Nearest E4M3FN code to each value, ties to the even code.

    Inputs must lie in [-448, 448] (the callers scale them there first).
    The sign bit copies the sign of the input, -0.0 included.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if np.any(~np.isfinite(a)) or np.any(a > 448.0):
        raise ValueError("e4m3_encode_rne: input outside [-448, 448]")
    hi = np.clip(np.searchsorted(_POS_VALS, a, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_hi = np.abs(_POS_VALS[hi] - a)
    d_lo = np.abs(a - _POS_VALS[lo])
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (_POS_CODES[lo] % 2 == 0))
    code = np.where(pick_lo, _POS_CODES[lo], _POS_CODES[hi]).astype(np.uint8)
    return np.where(np.signbit(v), code | np.uint8(0x80), code).astype(np.uint8)


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact fp64 values (bf16 is the top half of fp32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f16_decode(raw: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns (as uint16 or a float16 view) -> fp64."""
    return np.asarray(raw).view(np.float16).astype(np.float64)


def pow2_scale_exponent(amax: np.ndarray) -> np.ndarray:
    """Smallest integer s with amax <= 448 * 2**s (s = 0 when amax == 0).

    This is the power-of-two activation scale of the FP8 activation mode: the
    pages fix no activation precision; the reading taken is a per-group
    power-of-two scale so that v / 2**s is exact and the scale is an E8M0
    exponent the gfx950 scaled matrix instructions consume directly.
    """
    amax = np.asarray(amax, dtype=np.float64)
    s = np.zeros(amax.shape, dtype=np.int64)
    nz = amax > 0
    s[nz] = np.ceil(np.log2(amax[nz] / 448.0)).astype(np.int64)
    # make the definition exact whatever log2 rounded to
    for _ in range(2):
        too_small = nz & (amax > np.ldexp(448.0, s))
        s[too_small] += 1
        too_big = nz & (amax <= np.ldexp(448.0, s - 1))
        s[too_big] -= 1
    return s


def act_quant_pow2(v: np.ndarray, group: int = ACT_GROUP):
    """Quantize rows of v to E4M3 with one power-of-two scale per
    (row, group of `group` consecutive columns); the last group of a row
    may be shorter.

    Returns (codes uint8 [R, C], exponents int64 [R, G], dequantized fp64).
    """
    v = np.asarray(v, dtype=np.float64)
    R, C = v.shape
    G = (C + group - 1) // group
    codes = np.zeros((R, C), dtype=np.uint8)
    exps = np.zeros((R, G), dtype=np.int64)
    deq = np.zeros((R, C), dtype=np.float64)
    for g in range(G):
        sl = slice(g * group, min(C, (g + 1) * group))
        blk = v[:, sl]
        s = pow2_scale_exponent(np.abs(blk).max(axis=1))
        exps[:, g] = s
        c = e4m3_encode_rne(np.ldexp(blk, -s[:, None]))
        codes[:, sl] = c
        deq[:, sl] = np.ldexp(E4M3_TABLE[c], s[:, None])
    return codes, exps, deq


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z / (1 + exp(-z)) (the gate nonlinearity of SwiGLU)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))
