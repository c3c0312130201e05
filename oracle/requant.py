"""Quality-aware bit width: which experts to hold in int4, and the FP8 ->
int4-g128 requantization of one slot.

PagedWeight commentary (spectral-agent.com), "technically interesting points":
each expert's bit width is chosen by how much it matters, and switched while
the model serves; rarely used experts can lose precision at little quality
cost. The pages fix no rule or quantizer. Readings taken:

* plan: the n experts routed least often in a batch (per-expert pair counts,
  ties to the lower expert id) are held in int4, the rest in FP8;
* requantization: one expert's FP8 slot (codes with an fp32 row scale)
  becomes the int4-g128 format of its slot table (unsigned 4-bit, one fp16
  (scale, zero) per 128 consecutive K elements of a row), with the same
  quantizer as the int4 experts of the synthetic workloads: for each group
  of 128 decoded values w,
      s = fp16((max w - min w) / 15)   (1 when that is 0)
      z = clip(rint(-min w / s), 0, 15)
      q = clip(rint(w / s) + z, 0, 15),
  where every step that decides an integer (the decode w = e4m3(code) *
  row_scale, the difference, the two divisions, the fp16 rounding, rint with
  ties to even) is carried out in fp32, the precision of the GPU kernel, so
  both sides take the same decisions.
"""
import numpy as np

from .numerics import E4M3_TABLE
from .slots import slot_offsets, FMT_FP8_E4M3_ROW, FMT_INT4_G128

_G = 128


def bitwidth_plan(counts, n_int4: int) -> np.ndarray:
    """uint8 [E]: FMT_INT4_G128 for the n_int4 least-routed experts (ties to
    the lower id), FMT_FP8_E4M3_ROW for the rest."""
    counts = np.asarray(counts, dtype=np.int64)
    E = counts.size
    order = sorted(range(E), key=lambda e: (int(counts[e]), e))
    fmt = np.full(E, FMT_FP8_E4M3_ROW, dtype=np.uint8)
    for e in order[:max(0, min(n_int4, E))]:
        fmt[e] = FMT_INT4_G128
    return fmt


def _int4_rows_fp32(w: np.ndarray):
    """w float32 [R, C] -> (packed uint8 [R, C/2], (scale, zero) fp16 [R, C/128, 2])."""
    R, C = w.shape
    wg = w.reshape(R, C // _G, _G)
    mn, mx = wg.min(axis=2), wg.max(axis=2)
    s = ((mx - mn) / np.float32(15.0)).astype(np.float32).astype(np.float16)
    s[s == 0] = np.float16(1.0)
    s32 = s.astype(np.float32)
    z = np.clip(np.rint((-mn) / s32), 0, 15).astype(np.float32)
    q = np.clip(np.rint(wg / s32[:, :, None]) + z[:, :, None], 0, 15).astype(np.uint8).reshape(R, C)
    packed = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    sz = np.stack([s, z.astype(np.float16)], axis=2)
    return packed, sz


def requant_slot(fp8_slot: np.ndarray, H: int, I: int) -> np.ndarray:
    """The bytes of an int4-g128 slot holding the FP8 slot's expert."""
    src = np.asarray(fp8_slot, dtype=np.uint8).reshape(-1)
    fo, fs, _ = slot_offsets(H, I, FMT_FP8_E4M3_ROW)
    io, isz, itotal = slot_offsets(H, I, FMT_INT4_G128)

    def dec(codes, scale, rows, cols):
        c = E4M3_TABLE[codes].astype(np.float32).reshape(rows, cols)
        return c * scale.view(np.float32)[:, None]        # fp32 products, rounded once each

    w13 = dec(src[fo[0]:fo[0] + fs[0]], src[fo[1]:fo[1] + fs[1]], 2 * I, H)
    w2 = dec(src[fo[2]:fo[2] + fs[2]], src[fo[3]:fo[3] + fs[3]], H, I)
    out = np.zeros(itotal, dtype=np.uint8)
    for (p, sz), (o_p, o_sz) in ((_int4_rows_fp32(w13), (io[0], io[1])), (_int4_rows_fp32(w2), (io[2], io[3]))):
        out[o_p:o_p + p.size] = p.reshape(-1)
        raw = sz.view(np.uint8).reshape(-1)
        out[o_sz:o_sz + raw.size] = raw
    return out
