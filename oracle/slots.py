"""Decode one VRAM slot (one expert's weights) into fp64 matrices.

vllm-expert-pager article (rand.pepabo.com), section "hierarchical paging of
expert weights": every MoE layer owns a pool of VRAM slots and one slot holds
one expert's weights. The Table 1 set-up names the two tensors each expert
has, w13_weight (gate and up projections fused) and w2_weight (down).
The PagedWeight commentary (spectral-agent.com, section "technically
interesting points") holds each expert at its own bit width; the two storage
formats read here are FP8-E4M3 with one fp32 scale per output row, and
unsigned int4 with an fp16 (scale, zero) pair per 128 consecutive K elements.

Byte layout of a slot (each array starts on a 256-byte boundary, in order):
  FP8 : w13 codes u8[2I][H], w13 scale f32[2I], w2 codes u8[H][I], w2 scale f32[H]
  INT4: w13 u8[2I][H/2], w13 (scale, zero) f16[2I][H/128][2],
        w2 u8[H][I/2],   w2 (scale, zero) f16[H][I/128][2]
  int4 element c of a row sits in the low nibble of byte c/2 when c is even,
  in the high nibble when c is odd.
Rows [0, I) of w13 are the gate projection, rows [I, 2I) the up projection.
"""
import numpy as np

from .numerics import E4M3_TABLE, f16_decode

FMT_FP8_E4M3_ROW = 0
FMT_INT4_G128 = 1
_GROUP = 128


def _up256(n: int) -> int:
    return -(-n // 256) * 256


def slot_offsets(H: int, I: int, fmt: int):
    if fmt == FMT_FP8_E4M3_ROW:
        sizes = [2 * I * H, 2 * I * 4, H * I, H * 4]
    elif fmt == FMT_INT4_G128:
        sizes = [I * H, 2 * I * (H // _GROUP) * 4, H * I // 2, H * (I // _GROUP) * 4]
    else:
        raise ValueError("unknown slot format")
    offs, o = [], 0
    for n in sizes:
        offs.append(o)
        o = _up256(o + n)
    return offs, sizes, o


def _int4_matrix(packed: np.ndarray, sz: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """W[r, c] = (q[r, c] - zero[r, c // 128]) * scale[r, c // 128]."""
    p = packed.reshape(rows, cols // 2)
    q = np.empty((rows, cols), dtype=np.float64)
    q[:, 0::2] = p & 0x0F
    q[:, 1::2] = p >> 4
    sz = f16_decode(sz.view(np.uint16)).reshape(rows, cols // _GROUP, 2)
    scale = np.repeat(sz[:, :, 0], _GROUP, axis=1)
    zero = np.repeat(sz[:, :, 1], _GROUP, axis=1)
    return (q - zero) * scale


def dequant_slot(buf: np.ndarray, fmt: int, H: int, I: int):
    """Return (W13 fp64 [2I, H], W2 fp64 [H, I]) held by one slot's bytes."""
    buf = np.asarray(buf, dtype=np.uint8).reshape(-1)
    offs, sizes, _ = slot_offsets(H, I, fmt)

    def part(i):
        return buf[offs[i]:offs[i] + sizes[i]]

    if fmt == FMT_FP8_E4M3_ROW:
        # W[r, c] = e4m3(q[r, c]) * scale[r]
        c13 = E4M3_TABLE[part(0)].reshape(2 * I, H)
        s13 = part(1).view(np.float32).astype(np.float64)
        c2 = E4M3_TABLE[part(2)].reshape(H, I)
        s2 = part(3).view(np.float32).astype(np.float64)
        return c13 * s13[:, None], c2 * s2[:, None]
    return (_int4_matrix(part(0), part(1), 2 * I, H),
            _int4_matrix(part(2), part(3), H, I))
