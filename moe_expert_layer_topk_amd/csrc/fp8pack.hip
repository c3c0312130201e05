// Lossless compression of FP8 slots for the host tier: per-row Huffman codes
// of the exponent fields, decoded on the GPU right after the copy to VRAM.
//
// vllm-expert-pager article (rand.pepabo.com), section on weight compression:
// FP8 exponents are skewed, so each row's exponent bits are Huffman-coded in
// RAM and on SSD and expanded on the GPU once copied into VRAM (about a tenth
// of the memory saved).
//
// Format (the packed slot; every part on a 16-byte boundary): a header of
// eight u32 (magic, hidden, inter, offset and size of the packed w13, offset
// and size of the packed w2, total size), packed w13, w13 row scales (fp32),
// packed w2, w2 row scales. A packed matrix of R rows x C values (C a
// multiple of 256): code lengths u8[R][8] (symbol 2i in the low nibble of
// byte i), chunk start bits u32[R][C/256] (bit offsets into the matrix's
// stream), sign|mantissa nibbles u8[R][C/2] (value c in the low nibble of
// byte c/2 when c is even), the exponent stream (least significant bit of
// each byte first) and 8 zero bytes. An e4m3 byte is sign | exponent (4 bits)
// | mantissa (3 bits); the exponent is the coded symbol. Each row has its own
// canonical code: lengths from a Huffman tree over the row's exponent counts
// (merge the two lightest nodes, ties to the node holding the lower symbol;
// one symbol present: length 1); while a length exceeds 8 the counts of the
// present symbols are raised by floor(total 2^k / 256) + 1, k = 0, 1, ...;
// symbols ordered by (length, symbol) take consecutive codes, written first
// bit first.
//
// Decode: one lane per (row, 256-value chunk). The lanes of a wavefront
// first build, in LDS, a 256-entry table per row they cover (entry = symbol
// << 4 | length, indexed by the next 8 stream bits), then each lane walks its
// chunk with a 64-bit bit buffer, 16 values per 16-byte store.
#include "../../include/moe.h"
#include "moe_common.h"
#include "moe_kernels.h"

#include <algorithm>
#include <cstring>
#include <vector>

namespace {

constexpr uint32_t PACK_MAGIC = 0x38504D46u;
constexpr int PACK_CHUNK = 256;
constexpr int PACK_MAX_LEN = 8;

size_t al16(size_t n) { return (n + 15) / 16 * 16; }

// Huffman code lengths of the 16 exponent symbols for these weights
void huffman_lengths(const uint64_t counts[16], int lens[16]) {
    struct Node {
        uint64_t w;
        int low;
        std::vector<int> syms;
    };
    std::vector<Node> nodes;
    for (int s = 0; s < 16; ++s) {
        lens[s] = 0;
        if (counts[s]) nodes.push_back({counts[s], s, {s}});
    }
    if (nodes.size() == 1) {
        lens[nodes[0].low] = 1;
        return;
    }
    while (nodes.size() > 1) {
        std::sort(nodes.begin(), nodes.end(),
                  [](const Node& a, const Node& b) { return a.w != b.w ? a.w < b.w : a.low < b.low; });
        Node m{nodes[0].w + nodes[1].w, std::min(nodes[0].low, nodes[1].low), nodes[0].syms};
        m.syms.insert(m.syms.end(), nodes[1].syms.begin(), nodes[1].syms.end());
        for (int s : m.syms) ++lens[s];
        nodes.erase(nodes.begin(), nodes.begin() + 2);
        nodes.insert(nodes.begin(), m);
    }
}

int max_len(const int lens[16]) {
    int mx = 0;
    for (int s = 0; s < 16; ++s) mx = std::max(mx, lens[s]);
    return mx;
}

// code lengths of one row: the Huffman lengths of its exponent counts, the
// counts of present symbols raised by floor(total 2^k / 256) + 1 (k = 0, 1,
// ...) while a length exceeds 8
void code_lengths(const uint32_t counts[16], int lens[16]) {
    uint64_t c[16], total = 0;
    for (int s = 0; s < 16; ++s) {
        c[s] = counts[s];
        total += counts[s];
    }
    huffman_lengths(c, lens);
    for (int k = 0; max_len(lens) > PACK_MAX_LEN; ++k) {
        const uint64_t floor = (total << k) / 256 + 1;
        uint64_t r[16];
        for (int s = 0; s < 16; ++s) r[s] = c[s] ? c[s] + floor : 0;
        huffman_lengths(r, lens);
    }
}

// canonical codes from the lengths
void canonical(const int lens[16], uint32_t code[16]) {
    int order[16], n = 0;
    for (int l = 1; l <= 15; ++l)
        for (int s = 0; s < 16; ++s)
            if (lens[s] == l) order[n++] = s;
    uint32_t c = 0;
    int prev = 0;
    for (int i = 0; i < n; ++i) {
        const int s = order[i];
        c <<= (lens[s] - prev);
        code[s] = c++;
        prev = lens[s];
    }
}

size_t matrix_bound(int R, int C) {
    return al16((size_t)R * 8) + al16((size_t)R * (C / PACK_CHUNK) * 4) + al16((size_t)R * C / 2) +
           al16((size_t)R * C + 8);
}

// packs one matrix at out (16-byte aligned); returns its size
size_t pack_matrix(const uint8_t* codes, int R, int C, uint8_t* out) {
    const int nc = C / PACK_CHUNK;
    uint8_t* lens_b = out;
    uint32_t* starts = (uint32_t*)(out + al16((size_t)R * 8));
    uint8_t* nib = out + al16((size_t)R * 8) + al16((size_t)R * nc * 4);
    uint8_t* stream = nib + al16((size_t)R * C / 2);
    size_t bit = 0;
    const size_t stream_cap = (size_t)R * C + 8;
    std::memset(stream, 0, stream_cap);
    for (int r = 0; r < R; ++r) {
        const uint8_t* row = codes + (size_t)r * C;
        uint32_t counts[16] = {0};
        for (int c = 0; c < C; ++c) ++counts[(row[c] >> 3) & 0xF];
        int lens[16];
        uint32_t code[16];
        code_lengths(counts, lens);
        canonical(lens, code);
        for (int i = 0; i < 8; ++i) lens_b[(size_t)r * 8 + i] = (uint8_t)(lens[2 * i] | (lens[2 * i + 1] << 4));
        for (int c = 0; c < C; ++c) {
            if (c % PACK_CHUNK == 0) starts[(size_t)r * nc + c / PACK_CHUNK] = (uint32_t)bit;
            const int e = (row[c] >> 3) & 0xF;
            for (int b = lens[e] - 1; b >= 0; --b, ++bit)
                if ((code[e] >> b) & 1) stream[bit >> 3] |= (uint8_t)(1u << (bit & 7));
            const uint8_t n = (uint8_t)(((row[c] >> 4) & 0x8) | (row[c] & 0x7));
            uint8_t& nb = nib[(size_t)r * (C / 2) + c / 2];
            nb = (c & 1) ? (uint8_t)(nb | (n << 4)) : n;
        }
    }
    const size_t used = (bit + 7) / 8 + 8;                 // the stream and its 8 zero bytes
    return (size_t)(stream - out) + used;
}

}  // namespace

namespace moe {

// one 256-thread workgroup covers 256 (row, chunk) lanes
__device__ __forceinline__ void unpack_rows(const uint8_t* __restrict__ pm, uint8_t* __restrict__ out, int R, int C,
                                            int item0, uint8_t* s_tab) {
    const int nc = C / PACK_CHUNK;
    const size_t o_starts = ((size_t)R * 8 + 15) / 16 * 16;
    const size_t o_nib = o_starts + ((size_t)R * nc * 4 + 15) / 16 * 16;
    const size_t o_stream = o_nib + ((size_t)R * C / 2 + 15) / 16 * 16;
    // rows of this workgroup: items item0 .. item0 + 255 (item = row * nc + chunk)
    const int row0 = item0 / nc;
    const int row1 = min(R, (item0 + 255) / nc + 1);
    const int nrows = row1 - row0;                       // at most 256
    // tables: entry t of row r = symbol << 4 | length of the code the stream
    // bits t (first bit lowest) start with; each (row, symbol) writes the
    // 2^(8 - length) entries its bit-reversed canonical code owns
    for (int i = threadIdx.x; i < nrows * 256; i += blockDim.x) s_tab[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < nrows * 16; i += blockDim.x) {
        const int rr = i >> 4, sym = i & 15;
        const uint8_t* lb = pm + (size_t)(row0 + rr) * 8;
        int lens[16];
#pragma unroll
        for (int s = 0; s < 16; ++s) lens[s] = (lb[s >> 1] >> (4 * (s & 1))) & 0xF;
        const int l = lens[sym];
        if (l == 0 || l > PACK_MAX_LEN) continue;
        // canonical code: first code of length l, plus the symbols of that length before sym
        uint32_t code = 0;
        for (int len = 1; len < l; ++len) {
            int cnt = 0;
#pragma unroll
            for (int s = 0; s < 16; ++s) cnt += lens[s] == len;
            code = (code + cnt) << 1;
        }
#pragma unroll
        for (int s = 0; s < 16; ++s) code += (s < sym && lens[s] == l) ? 1u : 0u;
        const uint32_t rev = __builtin_bitreverse32(code) >> (32 - l);
        for (int j = 0; j < (1 << (PACK_MAX_LEN - l)); ++j) s_tab[rr * 256 + (rev | (j << l))] = (uint8_t)((sym << 4) | l);
    }
    __syncthreads();
    const int item = item0 + threadIdx.x;
    if (item >= R * nc) return;
    const int r = item / nc, ch = item % nc;
    const uint8_t* tab = s_tab + (r - row0) * 256;
    const uint32_t* st32 = (const uint32_t*)(pm + o_stream);
    const uint32_t bit0 = ((const uint32_t*)(pm + o_starts))[(size_t)r * nc + ch];
    uint32_t w = bit0 >> 5;
    uint64_t buf = ((uint64_t)st32[w] | ((uint64_t)st32[w + 1] << 32)) >> (bit0 & 31);
    int nbits = 64 - (int)(bit0 & 31);
    w += 2;
    const uint8_t* nib = pm + o_nib + (size_t)r * (C / 2) + ch * (PACK_CHUNK / 2);
    uint8_t* dst = out + (size_t)r * C + ch * PACK_CHUNK;
    for (int g = 0; g < PACK_CHUNK / 16; ++g) {
        const uint2 nb = *(const uint2*)(nib + 8 * g);
        const uint32_t nw[2] = {nb.x, nb.y};
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (nbits < 32) {
                buf |= (uint64_t)st32[w++] << nbits;
                nbits += 32;
            }
            const uint32_t e = tab[buf & 0xFF];
            const int len = e & 0xF;
            buf >>= len;
            nbits -= len;
            const uint32_t n = (nw[i >> 3] >> (4 * (i & 7))) & 0xF;
            const uint32_t byte = ((n & 8) << 4) | ((e >> 4) << 3) | (n & 7);
            if ((i & 3) == 0) o[i >> 2] = byte;
            else o[i >> 2] |= byte << (8 * (i & 3));
        }
        *(uint4*)(dst + 16 * g) = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

// up to 64 packed slots expanded by one launch: job z reads staging +
// src_off[z] and writes slot dst_slot[z]
constexpr int UNPACK_JOBS = 64;
struct UnpackJobs {
    uint64_t src_off[UNPACK_JOBS];
    int32_t dst_slot[UNPACK_JOBS];
};

// grid.y = 0: w13 rows, 1: w2 rows, 2: row scales and the format tag; grid.z: the job
__global__ void __launch_bounds__(256) unpack_kernel(const uint8_t* __restrict__ staging, UnpackJobs jobs,
                                                    uint8_t* __restrict__ base, size_t stride, size_t o_w13,
                                                    size_t o_s13, size_t o_w2, size_t o_s2, int H, int I,
                                                    uint8_t* __restrict__ tags, int32_t* __restrict__ err) {
    __shared__ uint8_t s_tab[256 * 256];                 // the rows of one 256-item group (at most 256)
    const uint8_t* packed = staging + jobs.src_off[blockIdx.z];
    uint8_t* slot = base + (size_t)jobs.dst_slot[blockIdx.z] * stride;
    uint8_t* tag = tags + jobs.dst_slot[blockIdx.z];
    const uint32_t* hdr = (const uint32_t*)packed;
    const bool ok = hdr[0] == PACK_MAGIC && (int)hdr[1] == H && (int)hdr[2] == I;
    if (!ok) {                                           // uniform: nothing written
        if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0 && err) atomicAdd(err, 1);
        return;
    }
    const int part = blockIdx.y;
    if (part == 2) {
        const uint32_t s13_src = (hdr[3] + hdr[4] + 15) / 16 * 16, s2_src = (hdr[5] + hdr[6] + 15) / 16 * 16;
        for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < 2 * I + H; i += gridDim.x * blockDim.x) {
            if (i < 2 * I) ((float*)(slot + o_s13))[i] = ((const float*)(packed + s13_src))[i];
            else ((float*)(slot + o_s2))[i - 2 * I] = ((const float*)(packed + s2_src))[i - 2 * I];
        }
        if (blockIdx.x == 0 && threadIdx.x == 0) *tag = (uint8_t)MOE_FMT_FP8_E4M3_ROW;
        return;
    }
    const int R = part == 0 ? 2 * I : H, C = part == 0 ? H : I;
    const int items = R * (C / PACK_CHUNK);
    const int item0 = blockIdx.x * 256;
    if (item0 >= items) return;
    unpack_rows(packed + (part == 0 ? hdr[3] : hdr[5]), slot + (part == 0 ? o_w13 : o_w2), R, C, item0, s_tab);
}

hipError_t launch_unpack(const PoolArgs& pa, const uint8_t* staging, const UnpackJobs& jobs, int n_jobs, int32_t* err,
                         hipStream_t stream) {
    const int H = pa.hidden, I = pa.inter;
    const int items = std::max(2 * I * (H / PACK_CHUNK), H * (I / PACK_CHUNK));
    MOE_LAUNCH(K_UNPACK, stream, unpack_kernel, dim3((items + 255) / 256, 3, n_jobs), dim3(256), 0, stream, staging,
               jobs, (uint8_t*)pa.base, pa.stride, pa.off[0][0], pa.off[0][1], pa.off[0][2], pa.off[0][3], H, I,
               (uint8_t*)pa.fmt, err);
    return hipGetLastError();
}

// pool view for the unpack kernel (FP8 layout offsets); false on bad arguments
bool unpack_pool(const moe_slot_pool* pool, PoolArgs* pa) {
    if (!pool || !pool->d_base || !pool->d_slot_fmt || pool->n_slots < 1) return false;
    if (pool->hidden < 256 || pool->hidden % 256 || pool->inter < 256 || pool->inter % 256) return false;
    if (pool->slot_bytes < moe_slot_bytes(pool->hidden, pool->inter, MOE_FMT_FP8_E4M3_ROW)) return false;
    pa->base = pool->d_base;
    pa->stride = pool->slot_bytes;
    pa->fmt = pool->d_slot_fmt;
    pa->n_slots = pool->n_slots;
    pa->hidden = pool->hidden;
    pa->inter = pool->inter;
    for (int i = 0; i < 4; ++i) pa->off[0][i] = moe_slot_part_offset(pool->hidden, pool->inter, MOE_FMT_FP8_E4M3_ROW, i);
    return true;
}

}  // namespace moe

extern "C" {

size_t moe_fp8_pack_bound(int hidden, int inter) {
    if (hidden < 256 || hidden % 256 || inter < 256 || inter % 256) return 0;
    return al16(32) + al16(matrix_bound(2 * inter, hidden)) + al16((size_t)2 * inter * 4) +
           al16(matrix_bound(hidden, inter)) + al16((size_t)hidden * 4);
}

size_t moe_fp8_pack(const uint8_t* h_fp8_slot, int hidden, int inter, uint8_t* h_out, size_t cap) {
    const int H = hidden, I = inter;
    if (!h_fp8_slot || !h_out || moe_fp8_pack_bound(H, I) == 0 || cap < moe_fp8_pack_bound(H, I)) return 0;
    const size_t off_w2 = moe_slot_part_offset(H, I, MOE_FMT_FP8_E4M3_ROW, 2);
    const size_t off_s13 = moe_slot_part_offset(H, I, MOE_FMT_FP8_E4M3_ROW, 1);
    const size_t off_s2 = moe_slot_part_offset(H, I, MOE_FMT_FP8_E4M3_ROW, 3);
    std::memset(h_out, 0, moe_fp8_pack_bound(H, I));
    size_t o = 32;
    const size_t w13_o = o, w13_n = pack_matrix(h_fp8_slot, 2 * I, H, h_out + o);
    o = al16(o + w13_n);
    std::memcpy(h_out + o, h_fp8_slot + off_s13, (size_t)2 * I * 4);
    o = al16(o + (size_t)2 * I * 4);
    const size_t w2_o = o, w2_n = pack_matrix(h_fp8_slot + off_w2, H, I, h_out + o);
    o = al16(o + w2_n);
    std::memcpy(h_out + o, h_fp8_slot + off_s2, (size_t)H * 4);
    o = al16(o + (size_t)H * 4);
    const uint32_t hdr[8] = {PACK_MAGIC, (uint32_t)H, (uint32_t)I, (uint32_t)w13_o, (uint32_t)w13_n,
                             (uint32_t)w2_o, (uint32_t)w2_n, (uint32_t)o};
    std::memcpy(h_out, hdr, sizeof(hdr));
    return o;
}

int moe_pager_fill_packed(const moe_slot_pool* pool, const uint8_t* h_packed, const uint64_t* h_offsets,
                          const uint64_t* h_sizes, const int32_t* fill_src, const int32_t* fill_slot, int n_fill,
                          uint8_t* d_staging, size_t staging_bytes, int32_t* d_err, void* copy_stream) {
    moe::PoolArgs pa;
    if (!moe::unpack_pool(pool, &pa) || n_fill < 0 ||
        (n_fill && (!h_packed || !h_offsets || !h_sizes || !fill_src || !fill_slot || !d_staging)))
        return MOE_EINVAL;
    size_t need = 0;
    for (int i = 0; i < n_fill; ++i) {
        if (fill_src[i] < 0 || fill_slot[i] < 0 || fill_slot[i] >= pool->n_slots) return MOE_EINVAL;
        need += al16((size_t)h_sizes[fill_src[i]]);
    }
    if (need > staging_bytes) return MOE_EINVAL;
    hipStream_t s = (hipStream_t)copy_stream;
    (void)hipGetLastError();
    // every copy first (the copy engine streams them back to back), then the
    // expansions, up to 64 slots per launch
    std::vector<uint64_t> off(n_fill);
    size_t o = 0;
    for (int i = 0; i < n_fill; ++i) {
        const size_t n = (size_t)h_sizes[fill_src[i]];
        off[i] = o;
        hipError_t e = hipMemcpyAsync(d_staging + o, h_packed + h_offsets[fill_src[i]], n, hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return moe::record_hip_error((int)e);
        o += al16(n);
    }
    for (int i0 = 0; i0 < n_fill; i0 += moe::UNPACK_JOBS) {
        moe::UnpackJobs jobs;
        const int nj = std::min(moe::UNPACK_JOBS, n_fill - i0);
        for (int j = 0; j < nj; ++j) {
            jobs.src_off[j] = off[i0 + j];
            jobs.dst_slot[j] = fill_slot[i0 + j];
        }
        const hipError_t e = moe::launch_unpack(pa, d_staging, jobs, nj, d_err, s);
        if (e != hipSuccess) return moe::record_hip_error((int)e);
    }
    return MOE_OK;
}

int moe_fp8_unpack(const moe_slot_pool* pool, const uint8_t* d_packed, int dst_slot, int32_t* d_err, void* stream) {
    moe::PoolArgs pa;
    if (!moe::unpack_pool(pool, &pa) || !d_packed || dst_slot < 0 || dst_slot >= pool->n_slots) return MOE_EINVAL;
    moe::UnpackJobs jobs;
    jobs.src_off[0] = 0;
    jobs.dst_slot[0] = dst_slot;
    (void)hipGetLastError();
    const hipError_t e = moe::launch_unpack(pa, d_packed, jobs, 1, d_err, (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : moe::record_hip_error((int)e);
}

}  // extern "C"
