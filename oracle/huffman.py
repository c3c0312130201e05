"""Lossless compression of FP8 expert slots: per-row Huffman codes of the
exponent fields.

vllm-expert-pager article (rand.pepabo.com), section on weight compression:
FP8 values have a skewed exponent distribution, so the exponent bits of each
row of an expert's weight matrices are Huffman-coded for the RAM (and SSD)
tier and decoded on the GPU right after the copy into VRAM; about a tenth of
the memory is saved. The page fixes no format. Readings taken:

* an e4m3 byte is sign (1 bit) | exponent (4) | mantissa (3); the exponent
  field is the symbol (16 values), the sign and mantissa travel as a raw
  nibble (sign << 3 | mantissa);
* every row has its own code: Huffman code lengths from the row's exponent
  counts, building the tree by repeatedly merging the two lightest nodes,
  a node's weight being its count and ties going to the node holding the
  lower symbol; when the longest code would exceed 8 bits (a decoder then
  needs one 256-entry table per row), every present symbol's count is raised
  by floor(total * 2^k / 256) + 1 for k = 0, 1, 2, ... until it does not;
  a row with a single exponent value gives it length 1;
* codes are canonical (symbols ordered by (length, symbol) take consecutive
  codes), written bit by bit from the code's first bit into a stream filled
  from the least significant bit of each byte;
* each row's stream is cut into chunks of 256 values, whose starting bit
  offsets are stored, so a decoder can start at any chunk.

Packed matrix (R rows x C columns, C a multiple of 256), in order, each part
starting on a 16-byte boundary:
    lens   u8  [R][8]        code length of symbol 2i in the low nibble of byte i
    starts u32 [R][C/256]    bit offset of each chunk in the matrix stream
    nib    u8  [R][C/2]      sign|mantissa nibble of value c in the low nibble of byte c/2 (c even)
    stream u8  [..]          the exponent codes, rows and chunks in order, then 8 zero bytes
Packed slot: a header of eight u32 (magic 0x38504D46, hidden, inter, offset
and size of the w13 part, offset and size of the w2 part, total size), the
w13 matrix, its fp32 row scales [2I], the w2 matrix, its fp32 row scales [H],
each part on a 16-byte boundary; offsets count from the slot's first byte.
"""
import numpy as np

from .slots import slot_offsets, FMT_FP8_E4M3_ROW

CHUNK = 256
MAX_LEN = 8
MAGIC = 0x38504D46


def _al16(n: int) -> int:
    return -(-n // 16) * 16


def _huffman_lengths(counts) -> list:
    present = [s for s in range(16) if counts[s] > 0]
    lens = [0] * 16
    if len(present) == 1:
        lens[present[0]] = 1
        return lens
    # a node: (weight, lowest symbol, symbols below it)
    nodes = [(counts[s], s, [s]) for s in present]
    while len(nodes) > 1:
        nodes.sort(key=lambda n: (n[0], n[1]))
        a, b = nodes[0], nodes[1]
        for s in a[2] + b[2]:
            lens[s] += 1
        nodes = [(a[0] + b[0], min(a[1], b[1]), a[2] + b[2])] + nodes[2:]
    return lens


def code_lengths(counts) -> list:
    """Code length of each of the 16 symbols (0 = absent) for one row."""
    counts = [int(c) for c in counts]
    lens = _huffman_lengths(counts)
    total, k = sum(counts), 0
    while max(lens) > MAX_LEN:
        floor = (total << k) // 256 + 1
        lens = _huffman_lengths([c + floor if c > 0 else 0 for c in counts])
        k += 1
    return lens


def canonical_codes(lens) -> dict:
    """symbol -> (code, length) of the canonical code with these lengths."""
    order = sorted((l, s) for s, l in enumerate(lens) if l > 0)
    codes, code, prev = {}, 0, 0
    for l, s in order:
        code <<= (l - prev)
        codes[s] = (code, l)
        code += 1
        prev = l
    return codes


def _pack_matrix(codes_u8: np.ndarray) -> bytes:
    R, C = codes_u8.shape
    assert C % CHUNK == 0
    nc = C // CHUNK
    expo = (codes_u8 >> 3) & 0xF
    nib = ((codes_u8 >> 4) & 0x8) | (codes_u8 & 0x7)
    lens_b = np.zeros((R, 8), np.uint8)
    starts = np.zeros((R, nc), np.uint32)
    bits = []                                        # the stream, one bit per entry
    for r in range(R):
        lens = code_lengths(np.bincount(expo[r], minlength=16))
        for i in range(8):
            lens_b[r, i] = lens[2 * i] | (lens[2 * i + 1] << 4)
        table = canonical_codes(lens)
        for c in range(C):
            if c % CHUNK == 0:
                starts[r, c // CHUNK] = len(bits)
            code, l = table[int(expo[r, c])]
            for b in range(l - 1, -1, -1):           # first bit of the code first
                bits.append((code >> b) & 1)
    nbytes = -(-len(bits) // 8)
    stream = np.zeros(nbytes + 8, np.uint8)
    for i, b in enumerate(bits):
        if b:
            stream[i >> 3] |= 1 << (i & 7)
    nibp = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    out = bytearray()
    for part in (lens_b.tobytes(), starts.astype("<u4").tobytes(), nibp.tobytes()):
        out += part
        out += bytes(_al16(len(out)) - len(out))
    return bytes(out + stream.tobytes())         # the size counts the stream's 8 zero bytes, no more


def pack_slot(fp8_slot: np.ndarray, H: int, I: int) -> np.ndarray:
    """The packed bytes of an FP8 slot (uint8)."""
    src = np.asarray(fp8_slot, dtype=np.uint8).reshape(-1)
    offs, sizes, _ = slot_offsets(H, I, FMT_FP8_E4M3_ROW)
    w13 = _pack_matrix(src[offs[0]:offs[0] + sizes[0]].reshape(2 * I, H))
    w2 = _pack_matrix(src[offs[2]:offs[2] + sizes[2]].reshape(H, I))
    s13 = src[offs[1]:offs[1] + sizes[1]].tobytes()
    s2 = src[offs[3]:offs[3] + sizes[3]].tobytes()
    out = bytearray(32)
    parts = {}
    for name, data in (("w13", w13), ("s13", s13), ("w2", w2), ("s2", s2)):
        parts[name] = (len(out), len(data))
        out += data
        out += bytes(_al16(len(out)) - len(out))
    hdr = np.array([MAGIC, H, I, parts["w13"][0], parts["w13"][1], parts["w2"][0], parts["w2"][1], len(out)],
                   dtype="<u4")
    out[0:32] = hdr.tobytes()
    return np.frombuffer(bytes(out), dtype=np.uint8).copy()


def _unpack_matrix(buf: np.ndarray, R: int, C: int) -> np.ndarray:
    nc = C // CHUNK
    o = 0
    lens_b = buf[o:o + R * 8].reshape(R, 8); o = _al16(o + R * 8)
    starts = buf[o:o + R * nc * 4].view("<u4").reshape(R, nc); o = _al16(o + R * nc * 4)
    nibp = buf[o:o + R * C // 2].reshape(R, C // 2); o = _al16(o + R * C // 2)
    stream = buf[o:]
    out = np.zeros((R, C), np.uint8)
    for r in range(R):
        lens = [int((lens_b[r, i // 2] >> (4 * (i % 2))) & 0xF) for i in range(16)]
        decode = {(code, l): s for s, (code, l) in canonical_codes(lens).items()}
        for ch in range(nc):
            pos = int(starts[r, ch])
            for c in range(ch * CHUNK, (ch + 1) * CHUNK):
                code, l = 0, 0
                while (code, l) not in decode:
                    code = (code << 1) | ((int(stream[pos >> 3]) >> (pos & 7)) & 1)
                    pos += 1
                    l += 1
                    if l > 15:
                        raise ValueError("bad code")
                e = decode[(code, l)]
                n = (int(nibp[r, c // 2]) >> (4 * (c % 2))) & 0xF
                out[r, c] = ((n & 8) << 4) | (e << 3) | (n & 7)
    return out


def unpack_slot(packed: np.ndarray, H: int, I: int) -> np.ndarray:
    """The FP8 slot bytes a packed slot holds (uint8, the FP8 slot layout)."""
    p = np.asarray(packed, dtype=np.uint8).reshape(-1)
    hdr = p[:32].view("<u4")
    assert int(hdr[0]) == MAGIC and int(hdr[1]) == H and int(hdr[2]) == I
    offs, sizes, total = slot_offsets(H, I, FMT_FP8_E4M3_ROW)
    out = np.zeros(total, np.uint8)
    w13_o, w13_n, w2_o, w2_n = (int(v) for v in hdr[3:7])
    out[offs[0]:offs[0] + sizes[0]] = _unpack_matrix(p[w13_o:w13_o + w13_n], 2 * I, H).reshape(-1)
    s13_o = _al16(w13_o + w13_n)
    out[offs[1]:offs[1] + sizes[1]] = p[s13_o:s13_o + sizes[1]]
    out[offs[2]:offs[2] + sizes[2]] = _unpack_matrix(p[w2_o:w2_o + w2_n], H, I).reshape(-1)
    s2_o = _al16(w2_o + w2_n)
    out[offs[3]:offs[3] + sizes[3]] = p[s2_o:s2_o + sizes[3]]
    return out
