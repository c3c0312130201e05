// Expert FFN, grouped FP8 matrix-core kernels for large batches (block_m 128).
//
// MOE-GEN explainer (aibr.jp), sections 1 and 3: once tokens are gathered per
// expert module each expert runs one dense contraction over many rows, the
// case FP8 matrix cores are built for. Weights come from the expert's VRAM
// slot (vllm-expert-pager article, rand.pepabo.com, "hierarchical paging";
// Table 1 set-up: w13 = gate+up, w2 = down).
//
// gemm1 multiplies the gathered token rows of a 128-row block by 128 gate and
// the matching 128 up rows of W13; its epilogue applies the row scales,
// silu(gate) * up and quantizes h per (row, 128 columns). gemm2 multiplies
// 128 rows of h by 256 rows of W2 and writes w[t][j] * y, in bf16, to the
// pair's row of the combine buffer. Both are built the same way:
// * persistent: one workgroup per CU walks a list of (block, column tile)
//   tiles; the workgroups of one XCD (blocks are dealt round-robin over the 8
//   XCDs) take consecutive tiles, so the same token rows and the same
//   expert's weights are shared in that XCD's L2;
// * the K steps of all tiles of a workgroup form one stream through two LDS
//   buffers filled by direct-to-LDS 16-byte loads: while a step is
//   multiplied from registers, its buffer is refilled two steps ahead by
//   loads issued between the first half of its matrix instructions, and the
//   next step is read into registers between the second half, each fragment
//   as soon as its last instruction of the step has issued (so the load
//   path, the LDS reads and the matrix pipe work at the same time), also
//   across tile boundaries, so the next tile's loads hide behind the current
//   tile's last steps and epilogue;
// * a stage holds 128 A rows and 256 B rows of 128 bytes; one 16-byte load
//   instruction fills 8 whole rows (full 128-byte lines from memory), each
//   row's 16-byte chunks XOR-swizzled through the source address of each
//   lane: chunk c of stage row r sits at c ^ f(r % 16), f(m) = (m / 2) & 5,
//   a placement measured free of LDS bank conflicts for 16-byte fragment
//   reads (rows m of a fragment at lanes m + 16 q, chunk 2q or 2q+1), where
//   the row-index XOR by r % 8 loses half the LDS bandwidth;
// * 8 waves in a 4 x 2 grid over a 256 x 256 tile, 64 x 128 outputs each:
//   32 v_mfma_scale_f32_16x16x128_f8f6f4 per wave and K step, with the
//   power-of-two activation exponents (E8M0) as the instruction's A scales;
// * a lone block (an expert's odd last block) makes a one-block tile; when
//   experts average fewer than three blocks such tiles are a large share, and
//   they run after the two-block tiles on a layout of their own (128 x 256,
//   8 waves in a 2 x 4 grid, 64 x 64 outputs and 16 matrix instructions per
//   wave and step) instead of idling half of the two-block layout's waves;
// * B rows are ordered so that the accumulators a lane holds for one row
//   across fragments are adjacent output columns: epilogue stores are 4-byte
//   fp8 runs (gate/up: four h columns from four gate and four up fragments)
//   or 16-byte bf16 runs (down: eight columns from eight fragments) straight
//   from registers;
// * per-tile metadata (row scales of the expert, pair ids, route weights)
//   reaches LDS by direct-to-LDS loads issued with the tile's first stage;
//   the gate/up kernel's token ids of a tile arrive the same way with the
//   previous tile's first stage, and its workgroup's tile descriptors are
//   read into LDS once at the start, so setting up a tile and its epilogue
//   wait for no memory round trip (the down kernel reads descriptors with
//   scalar loads).
// A prep kernel lists the FP8 blocks and lays out the per-position token
// ids, route weights and activation scales the two kernels read. Blocks whose
// slot is int4-g128 or not usable are handled by the int4 ring kernels of
// ffn_int4.hip.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

constexpr int MM_BM = 128;                              // rows of an align block
constexpr int MM_TM = 256;                              // rows of a tile: two blocks of one expert
constexpr int MM_THREADS = 512;                         // 8 waves: 4 (rows) x 2 (columns)
constexpr int MM_RING = 2;                              // LDS stages
constexpr int MM_OPS = (MM_TM + 256) * 128;             // 256 A rows, 256 B rows of 128 bytes
constexpr int MM_SCL = MM_OPS;                          // 256 row-scale bytes
constexpr int MM_STAGE = MM_OPS + 256;
constexpr int MM_META = 4096;                           // per-tile metadata slot
constexpr int MM_NMETA = 4;                             // tiles that can be in flight at once
constexpr int MM_AMAX = MM_RING * MM_STAGE + MM_NMETA * MM_META;
constexpr int MM_DESC = MM_AMAX + 2 * MM_TM * 4;     // this workgroup's tile descriptors
constexpr int MM_MAXDESC = 512;                         // held in LDS (later tiles: scalar loads)
constexpr int MM_SMEM = MM_DESC + 16 * MM_MAXDESC;
constexpr int MM_TOK = 1024;                            // KIND 0: token ids of the tile, in its metadata slot

// LDS layout and wave shape per tile kind: a two-block tile is 256 A rows x
// 256 B rows, 8 waves as 4 (rows) x 2 (columns), 8 B fragments per wave; a
// one-block tile is 128 A rows x 256 B rows, 8 waves as 2 x 4, 4 B fragments
template <bool ONE>
struct MLay {
    static constexpr int TM = ONE ? MM_BM : MM_TM;          // A rows of a tile
    static constexpr int OPS = (TM + 256) * 128;            // A rows, 256 B rows of 128 bytes
    static constexpr int SCL = OPS;                         // 256 row-scale bytes
    static constexpr int STAGE = OPS + 256;
    static constexpr int AMAX = MM_RING * STAGE + MM_NMETA * MM_META;
    static constexpr int DESC = AMAX + 2048;                // row maxima [column waves][A rows] first
    static constexpr int SMEM = DESC + 16 * MM_MAXDESC;
    static constexpr int NF = ONE ? 4 : 8;                  // B fragments per wave
    static constexpr int NA = ONE ? 2 : 4;                  // A row loads (8 rows each) per wave and step
};
static_assert(MLay<false>::SMEM == MM_SMEM && MLay<true>::SMEM <= MM_SMEM, "LDS layout");
static_assert(MM_RING == 2 && (MM_NMETA & (MM_NMETA - 1)) == 0, "ring and metadata slots index with masks");

template <int V>
struct IC {
    static constexpr int value = V;
};

struct MPool {
    const uint8_t* base;
    size_t stride;
    size_t off[4];            // FP8 slot: w13, s13, w2, s2
};

struct MTiles {
    const int4* tiles;        // (first block, slot, blocks (1 or 2), 0) of each FP8 tile, in order
    const int* n_tiles;
    const int32_t* tokrow;    // token of each sorted position (0 for padding)
    const float* wsort;       // route weight of each sorted position (0 for padding)
    const int32_t* sorted_pair;
    const uint8_t* scl;       // A scale bytes, [block][K step][128 rows]
};

// s_waitcnt with only vmcnt limited (expcnt and lgkmcnt left open)
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Leave at most n of this wave's vector memory operations outstanding
// (waits for all of them when n is outside the table: never too few).
#define MM_W(n) \
    case n: wait_vm<n>(); break;
__device__ __forceinline__ void wait_vm_n(int n) {
    switch (n) {
        MM_W(0) MM_W(6) MM_W(7) MM_W(8) MM_W(9) MM_W(10)
        default: wait_vm<0>(); break;
    }
}
#undef MM_W

// Workgroup barrier without the release fence that __syncthreads() adds: that
// fence waits for every outstanding global load, direct-to-LDS ones included,
// which would drain the stages in flight. The wave's own LDS traffic is
// waited for first; direct-to-LDS data is waited for with wait_vm before it.
// Built from the wait and barrier builtins (the compiler then knows the LDS
// reads before it have completed and adds no waits of its own for them
// later) between two compiler-only fences that keep memory accesses on their
// side.
static __device__ __forceinline__ void barrier_lds() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);                // lgkmcnt(0); vmcnt, expcnt left open
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// lane i writes 16 (4) bytes at lds + 16 i (4 i); lds is wave-uniform
__device__ __forceinline__ void dma16(const void* src, uint8_t* lds) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, uint8_t* lds) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
}

// Scalar loads for per-tile metadata. A vector load here would be waited for
// with the direct-to-LDS loads in flight (vector memory completes in order),
// draining the pipeline; scalar loads count on a separate counter.
__device__ __forceinline__ int4 sload4(const int4* p) {
    i32x4 r;
    asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(r) : "s"(p) : "memory");
    return make_int4(r[0], r[1], r[2], r[3]);
}

// max over each row of 16 lanes (quad swaps, then row rotations by 4 and 8)
// of non-negative values, as integers: the bit patterns of non-negative
// floats order like the floats, and an integer max takes its DPP operand
// directly (a float max would first canonicalise the moved value)
__device__ __forceinline__ float row16_max_nonneg(float v) {
    int x = __float_as_int(v);
    x = max(x, __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true));
    x = max(x, __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true));
    x = max(x, __builtin_amdgcn_mov_dpp(x, 0x124, 0xF, 0xF, true));
    x = max(x, __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, true));
    return __int_as_float(x);
}

typedef short s16x2 __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16, round to nearest even (one hardware conversion of
// the pair)
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, b2));
}


// ------------------------------------------------------------------ prep
// Block 0 lists, in order, the FP8 tiles (pairs of consecutive blocks of one
// resident FP8 expert, counted from the start of the expert's segment; an odd
// last block makes a one-block tile; all tiles in one list for the down
// kernel, the two kinds in lists of their own for the gate/up kernel) and the
// other blocks (int4 or not resident); the other workgroups write, per sorted position, the token, the
// route weight and the token's activation scale bytes transposed to
// [block][K step][row].
__global__ void __launch_bounds__(256) mfma_prep_kernel(const int32_t* __restrict__ sorted_pair,
                                                       const int32_t* __restrict__ block_slot,
                                                       const uint8_t* __restrict__ fmt, int n_slots, int fmt_ok,
                                                       const int32_t* __restrict__ n_padded, int NP, int k,
                                                       const float* __restrict__ topk_w,
                                                       const uint8_t* __restrict__ xs, int groups,
                                                       int4* __restrict__ tiles, int* __restrict__ n_tiles,
                                                       int4* __restrict__ tiles1, int* __restrict__ n_tiles1,
                                                       int4* __restrict__ tiles2, int* __restrict__ n_tiles2,
                                                       int* __restrict__ others, int* __restrict__ n_others,
                                                       int32_t* __restrict__ tokrow, float* __restrict__ wsort,
                                                       uint8_t* __restrict__ scl) {
    const int np = *n_padded;
    if (blockIdx.x == 0) {
        __shared__ int s_cnt[4][4];
        __shared__ int s_last[4];
        __shared__ uint8_t s_fm[MOE_MAX_SLOTS];
        const int lane = lane_id(), wv = threadIdx.x / MOE_WAVE;
        const int nb = np / MM_BM;
        // format tags into LDS, and each round's block slots (blocks b - 1,
        // b, b + 1; clamped indices, no branches) loaded one round ahead, so
        // the rounds wait for no memory round trip of their own
        for (int i = threadIdx.x; i < n_slots; i += 256) s_fm[i] = fmt[i];
        const int last = max(nb - 1, 0);
        int sp = -1, sc = -1, sn = -1;
        auto load3 = [&](int b0) __attribute__((always_inline)) {
            const int b = b0 + (int)threadIdx.x;
            sp = block_slot[min(max(b - 1, 0), last)];
            sc = block_slot[min(b, last)];
            sn = block_slot[min(b + 1, last)];
        };
        if (nb > 0) load3(0);
        __syncthreads();
        // (the round barriers wait for LDS only: the next round's loads stay in flight)
        int base = 0, base1 = 0, base2 = 0, obase = 0, carry = 0;   // carry: last segment start before this chunk
        for (int b0 = 0; b0 < nb; b0 += 256) {
            const int b = b0 + threadIdx.x;
            const bool valid = b < nb;
            const int slot = valid ? sc : -1, prev = sp, next = sn;
            if (b0 + 256 < nb) load3(b0 + 256);
            const bool start = valid && (b == 0 || prev != slot);
            const uint64_t smask = __ballot(start);
            const uint64_t upto = lane == 63 ? ~0ull : ((2ull << lane) - 1);
            if (lane == 0) s_last[wv] = smask ? b0 + 64 * wv + 63 - __clzll(smask) : -1;
            barrier_lds();
            int seg = carry;
            for (int w = 0; w < wv; ++w) seg = s_last[w] > seg ? s_last[w] : seg;
            if (smask & upto) seg = b0 + 64 * wv + 63 - __clzll(smask & upto);
            const bool f = valid && usable_slot(slot, n_slots, fmt_ok, s_fm) >= 0 && s_fm[slot] == 0;
            const bool t = f && ((b - seg) & 1) == 0;
            const bool o = valid && !f;
            const bool t2 = t && b + 1 < nb && next == slot, t1 = t && !t2;   // two-block and one-block tiles
            const uint64_t tbal = __ballot(t), t1bal = __ballot(t1), t2bal = __ballot(t2), obal = __ballot(o);
            if (lane == 0) {
                s_cnt[0][wv] = __popcll(tbal);
                s_cnt[1][wv] = __popcll(obal);
                s_cnt[2][wv] = __popcll(t1bal);
                s_cnt[3][wv] = __popcll(t2bal);
            }
            barrier_lds();
            int off = base, ooff = obase, off1 = base1, off2 = base2;
            for (int w = 0; w < wv; ++w) {
                off += s_cnt[0][w];
                ooff += s_cnt[1][w];
                off1 += s_cnt[2][w];
                off2 += s_cnt[3][w];
            }
            if (t) tiles[off + __popcll(tbal & lanemask_lt())] = make_int4(b, slot, t2 ? 2 : 1, 0);
            if (t1) tiles1[off1 + __popcll(t1bal & lanemask_lt())] = make_int4(b, slot, 1, 0);
            if (t2) tiles2[off2 + __popcll(t2bal & lanemask_lt())] = make_int4(b, slot, 2, 0);
            if (o) others[ooff + __popcll(obal & lanemask_lt())] = b;
            base += s_cnt[0][0] + s_cnt[0][1] + s_cnt[0][2] + s_cnt[0][3];
            obase += s_cnt[1][0] + s_cnt[1][1] + s_cnt[1][2] + s_cnt[1][3];
            base1 += s_cnt[2][0] + s_cnt[2][1] + s_cnt[2][2] + s_cnt[2][3];
            base2 += s_cnt[3][0] + s_cnt[3][1] + s_cnt[3][2] + s_cnt[3][3];
            for (int w = 0; w < 4; ++w) carry = s_last[w] > carry ? s_last[w] : carry;
            barrier_lds();
        }
        if (threadIdx.x == 0) {
            *n_tiles = base;
            *n_others = obase;
            *n_tiles1 = base1;
            *n_tiles2 = base2;
        }
        return;
    }
    const int pos = (blockIdx.x - 1) * 256 + threadIdx.x;
    if (pos >= np) return;
    const int p = sorted_pair[pos];
    const bool v = p < NP;
    const int t = v ? p / k : 0;
    tokrow[pos] = t;
    wsort[pos] = v ? topk_w[p] : 0.f;
    const int mt = pos / MM_BM, r = pos % MM_BM;
    for (int g = 0; g < groups; ++g)
        scl[((size_t)mt * groups + g) * MM_BM + r] = v ? xs[(size_t)t * groups + g] : (uint8_t)127;
}

// ------------------------------------------------------------------ gemm kernels
// KIND 0: gate/up (gemm1), KIND 1: down (gemm2). A tile is 256 rows (two
// blocks; in a one-block tile the second half repeats the first block's rows
// and its results are dropped) by 256 B rows (KIND 0: 128 gate + the matching
// 128 up rows of W13 = 128 columns of h; KIND 1: 256 rows of W2).
template <int KIND, bool ONE>
__device__ __forceinline__ void mfma_tiles(const MPool& pool, const MTiles& tl, const uint8_t* __restrict__ xq,
                                           int NP, int H, int I_arg, uint8_t* __restrict__ hq,
                                           uint8_t* __restrict__ hs, uint16_t* __restrict__ ybuf, uint8_t* smem) {
    using Lay = MLay<ONE>;
    const int I = I_arg;
    const int lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / MOE_WAVE);
    const int m = lane & 15, q = lane >> 4;
    // 64-row group and column group. Two-block tiles: 4 x 2; waves w and
    // w + 4 share a SIMD, so every SIMD holds one wave of each 128-row half
    // of the tile (the waves of an empty half skip their matrix work). One-
    // block tiles: 2 x 4, 64 B rows per wave.
    const int mw = ONE ? (wv >> 2) : 2 * (wv >> 2) + ((wv >> 1) & 1), nw = ONE ? (wv & 3) : (wv & 1);
    constexpr int NF = Lay::NF, NA = Lay::NA;
    const int S = KIND == 0 ? H / 128 : I / 128;          // K steps per tile
    const int NT = KIND == 0 ? I / 128 : H / 256;         // column tiles per block pair
    const int hgroups = I / 128;

    // this workgroup's tiles: start + idx + per_x * j, j < nj
    const int G = *tl.n_tiles * NT;
    const int x = blockIdx.x & 7, idx = blockIdx.x >> 3, per_x = gridDim.x >> 3;
    const int gper = G >> 3, grem = G & 7;
    const int start = x * gper + (x < grem ? x : grem);
    const int cnt = gper + (x < grem ? 1 : 0);
    const int nj = cnt > idx ? (cnt - idx + per_x - 1) / per_x : 0;
    if (nj == 0) return;
    const int N = nj * S;

    // gate/up kernel: this workgroup's tile descriptors into LDS (one round
    // trip for all) and the token ids of tile 0 into its metadata slot; later
    // tiles' token ids arrive with the previous tile's first stage
    // (the down kernel keeps scalar loads: the table measured slower there)
    int4* s_desc = (int4*)(smem + Lay::DESC);
    if (KIND == 0) {
        for (int i = threadIdx.x; i < min(nj, MM_MAXDESC); i += MM_THREADS)
            s_desc[i] = tl.tiles[(start + idx + per_x * i) / NT];
        __syncthreads();
    }
    auto desc_of = [&](int j) __attribute__((always_inline)) {
        if (KIND == 0 && j < MM_MAXDESC) {
            const int4 v = s_desc[j];
            return make_int4(__builtin_amdgcn_readfirstlane(v.x), __builtin_amdgcn_readfirstlane(v.y),
                             __builtin_amdgcn_readfirstlane(v.z), __builtin_amdgcn_readfirstlane(v.w));
        }
        return sload4(tl.tiles + __builtin_amdgcn_readfirstlane((start + idx + per_x * j) / NT));
    };
    if (KIND == 0) {
        const int4 d0 = desc_of(0);
        int32_t* s_tok = (int32_t*)(smem + MM_RING * Lay::STAGE + MM_TOK);
        if (threadIdx.x < Lay::TM) {
            const int r = threadIdx.x;
            s_tok[r] = tl.tokrow[(d0.x + (r >= MM_BM && d0.z == 2 ? 1 : 0)) * MM_BM + r % MM_BM];
        }
        __syncthreads();
    }

    // metadata dword loads (256 B each) of this wave per tile, into the tile's
    // metadata slot at byte meta_off. KIND 0: wave 1 gate, wave 2 up row scales
    // of the 128 columns; KIND 1: waves 1, 2 pair ids of the two blocks, waves
    // 3, 4 their route weights, waves 5, 6 the W2 row scales of the 256 columns.
    const int meta_n = KIND == 0 ? (wv == 1 || wv == 2 ? 2 : 0) : (wv >= 1 && wv <= 6 ? 2 : 0);
    const int meta_off = KIND == 0 ? (wv == 2 ? 512 : 0) : (wv - 1) * 512;

    // ---- issue side: sources of the tile being loaded. Wave w loads A and B
    // rows r = 32 w + 8 j + i / 8 (j < 4); lane i puts the source chunk
    // (i % 8) ^ f(r % 16) of its row at chunk i % 8, f(r % 16) = ((i / 16) & 1)
    // | 4 (j & 1).
    // wave-uniform bases plus 32-bit per-lane offsets (fewer live registers)
    const uint8_t* bA = KIND == 0 ? xq : hq;
    const uint8_t* bB = nullptr;          // B rows of this tile
    const uint8_t* bS = nullptr;          // row-scale bytes of this tile (wave 0)
    const uint8_t* bM = nullptr;          // metadata source (meta_n > 0)
    const int32_t* bT = tl.tokrow;        // KIND 0, waves 4..7: next tile's token ids
    int two_next = 1;                     // the last tile set up has two blocks
    uint32_t oA[4], oB0 = 0, oB1 = 0, oS = 0, oM = 0;   // B row of j: oB(j & 1) + (32 (j & 1) + (j >> 1)) rows
    // B stage row 32 w + 8 j + i / 8 = fragment 2 w + j / 2, fragment row 8 (j & 1) + i / 8;
    // fragment f = 8 nw + n, row m holds output column
    //   KIND 0: nw * 64 + (n / 4) * I + 4 m + n % 4 (n / 4 picks gate or up rows)
    //   KIND 1: nw * 128 + 8 m + n
    auto setup = [&](int j) __attribute__((always_inline)) {
        // per-lane constants formed here from an opaque copy of the lane id,
        // not held in registers across the step loop
        int lane = lane_id();
        asm volatile("" : "+v"(lane));
        const int csw0 = 16 * ((lane & 7) ^ ((lane >> 4) & 1));        // loads j even
        const int csw1 = 16 * ((lane & 7) ^ (4 | ((lane >> 4) & 1)));  // loads j odd
        // one-block tiles: fragment f = 4 nw + n, row m holds output column
        //   KIND 0: nw * 32 + (n / 2) * I + 2 m + n % 2;  KIND 1: nw * 64 + 4 m + n
        const int brow0 = ONE ? (KIND == 0 ? (wv & 1) * I + (wv >> 1) * 32 + 2 * (lane >> 3)
                                           : (wv >> 1) * 64 + 2 * (wv & 1) + 4 * (lane >> 3))
                              : (KIND == 0 ? ((wv & 3) >> 1) * I + (wv >> 2) * 64 + 2 * (wv & 1) + 4 * (lane >> 3)
                                           : (wv >> 2) * 128 + 2 * (wv & 3) + 8 * (lane >> 3));
        const int L = start + idx + per_x * j;
        const int4 d = desc_of(j);
        const int b = d.x, nt = L % NT, two = d.z == 2;
        two_next = two;
        const uint8_t* sb = pool.base + (size_t)d.y * pool.stride;
        const int blk_w = ONE ? b : b + ((wv >> 2) & two);  // block of this wave's A rows
        const int r_w = ONE ? 16 * wv : 32 * (wv & 3);      // first of them inside the block
        bS = tl.scl + (size_t)b * S * MM_BM;
        oS = ((lane >> 5) & two) * S * MM_BM + 4 * (lane & 31);
        if (KIND == 0) {
            // token ids of this wave's 32 rows, from the tile's metadata slot
            const int32_t* s_tok = (const int32_t*)(smem + MM_RING * Lay::STAGE + (j % MM_NMETA) * MM_META + MM_TOK) +
                                   (ONE ? 0 : ((wv >> 2) & 1) * MM_BM) + r_w + (lane >> 3);
#pragma unroll
            for (int j2 = 0; j2 < NA; ++j2) oA[j2] = (uint32_t)s_tok[8 * j2] * H + ((j2 & 1) ? csw1 : csw0);
            // waves 4..7: source of 64 token ids of the next tile (loaded with this tile's first stage)
            const int4 dn = desc_of(min(j + 1, nj - 1));
            const int i4 = (wv - 4) & 3;
            bT = tl.tokrow + (dn.x + (i4 >= 2 && dn.z == 2 ? 1 : 0)) * MM_BM + 64 * (i4 & 1);
            const int c0 = nt * 128;
            bB = sb + pool.off[0] + (size_t)c0 * H;
            oB0 = (uint32_t)brow0 * H + csw0;
            oB1 = (uint32_t)brow0 * H + csw1;
            bM = sb + pool.off[1] + 4 * ((wv == 2 ? I : 0) + c0);
            oM = 4 * lane;
        } else {
            bA = hq + (size_t)(blk_w * MM_BM + r_w) * I;
            oA[0] = (uint32_t)(lane >> 3) * I + csw0;       // row 8 j is + 8 j I (added at issue)
            oA[1] = (uint32_t)(lane >> 3) * I + csw1;
            const int n0 = nt * 256;
            bB = sb + pool.off[2] + (size_t)n0 * I;
            oB0 = (uint32_t)brow0 * I + csw0;
            oB1 = (uint32_t)brow0 * I + csw1;
            const int half = (wv - 1) & 1;                  // waves 1..6: first or second half
            if (wv == 1 || wv == 2) bM = (const uint8_t*)(tl.sorted_pair + (b + (half & two)) * MM_BM);
            else if (wv == 3 || wv == 4) bM = (const uint8_t*)(tl.wsort + (b + (half & two)) * MM_BM);
            else bM = sb + pool.off[3] + 4 * (n0 + 128 * half);
            oM = 4 * lane;
        }
    };
    // A step s of the stream is K step g = s % S of tile jt = s / S; the
    // helpers below take (g, jt), which the loop carries as counters (no
    // division per step).
    // vector memory operations stage g puts in flight for this wave
    auto stage_ops = [&](int g) __attribute__((always_inline)) {
        return NA + 4 + (wv == 0 ? 1 : 0) + (g == 0 ? meta_n + (KIND == 0 && wv >= 4 ? 1 : 0) : 0);
    };
    // the loads of a step into LDS buffer u (u = s % 2, except past the end of
    // the stream, where the last step is loaded again into the buffer the
    // current step left, so the loop needs no branch around them)
    auto dma_a = [&](int g, int u, int j2) __attribute__((always_inline)) {
        uint8_t* st = smem + u * Lay::STAGE;
        const int k0 = g * 128;
        dma16(bA + (KIND == 0 ? oA[j2] : oA[j2 & 1] + (size_t)8 * j2 * I) + k0, st + (8 * NA * wv + 8 * j2) * 128);
    };
    auto dma_b = [&](int g, int u, int j2) __attribute__((always_inline)) {
        uint8_t* st = smem + u * Lay::STAGE;
        const int k0 = g * 128;
        const size_t KB = KIND == 0 ? (size_t)H : (size_t)I;     // B row length
        constexpr int RJ = ONE ? (KIND == 0 ? 16 : 32) : (KIND == 0 ? 32 : 64);   // B rows between loads j and j + 1
        dma16(bB + (RJ * (j2 & 1) + (j2 >> 1)) * KB + k0 + ((j2 & 1) ? oB1 : oB0),
              st + Lay::TM * 128 + (32 * wv + 8 * j2) * 128);
    };
    auto dma_tail = [&](int g, int jt, int u) __attribute__((always_inline)) {
        uint8_t* st = smem + u * Lay::STAGE;
        // opaque copies: the 64-bit addresses are formed here, not kept live
        uint32_t os = oS, om = oM;
        asm volatile("" : "+v"(os));
        asm volatile("" : "+v"(om));
        if (wv == 0) dma4(bS + g * MM_BM + os, st + Lay::SCL);
        if (g == 0) {
            uint8_t* md = smem + MM_RING * Lay::STAGE + (jt & (MM_NMETA - 1)) * MM_META + meta_off;
            for (int h = 0; h < meta_n; ++h) dma4(bM + 256 * h + om, md + 256 * h);
            if (KIND == 0 && wv >= 4)
                dma4((const uint8_t*)bT + om, smem + MM_RING * Lay::STAGE + ((jt + 1) & (MM_NMETA - 1)) * MM_META + MM_TOK +
                                                  256 * (wv - 4));
        }
    };
    auto issue = [&](int s, int u) __attribute__((always_inline)) {
        const int g = s % S, jt = s / S;
        if (g == 0) setup(jt);
#pragma unroll
        for (int j2 = 0; j2 < NA; ++j2) dma_a(g, u, j2);
#pragma unroll
        for (int j2 = 0; j2 < 4; ++j2) dma_b(g, u, j2);
        dma_tail(g, jt, u);
    };

    // ---- compute side
    f32x4 acc[4][NF];
    auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int n = 0; n < NF; ++n) acc[a][n] = f32x4{0, 0, 0, 0};
    };
    // a fragment gives lane m + 16 q the 32 codes of its row m at K bytes
    // [32 q, 32 q + 32): chunks 2q and 2q+1, at swizzled offsets o0, o1 (every
    // row a lane reads shares r % 16 = m)
    const int fm = (m >> 1) & 5;
    const int o0 = ((2 * q) ^ fm) << 4, o1 = ((2 * q + 1) ^ fm) << 4;
    // fragments of a K step in registers: the step being multiplied, and
    // during the second half of its matrix instructions the next step, each
    // fragment read again once its last instruction of the step has issued
    i32x8 FA[4], FB[NF];
    int SA[4];
    // reads at LDS offset so of a stage; each forms its address from an
    // opaque copy of the (wave-uniform) row offset, so no address register
    // stays live across the matrix instructions between the reads
    const int lo0 = m * 128 + o0, lo1 = m * 128 + o1;   // this lane's two chunks of fragment row m
    auto lds_frag = [&](int off) __attribute__((always_inline)) {
        asm volatile("" : "+s"(off));
        const i32x4 lo = *(const i32x4*)(smem + off + lo0);
        const i32x4 hi = *(const i32x4*)(smem + off + lo1);
        return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    auto read_fb = [&](int so, int n) __attribute__((always_inline)) {
        FB[n] = lds_frag(so + (Lay::TM + 16 * (NF * nw + n)) * 128);
    };
    auto read_fa = [&](int so, int a) __attribute__((always_inline)) {
        FA[a] = lds_frag(so + (64 * mw + 16 * a) * 128);
        int off = so + Lay::SCL + 64 * mw + 16 * a;
        asm volatile("" : "+s"(off));
        SA[a] = smem[off + m];
    };
    auto read_step = [&](int so) __attribute__((always_inline)) {
#pragma unroll
        for (int n = 0; n < NF; ++n) read_fb(so, n);
#pragma unroll
        for (int a = 0; a < 4; ++a) read_fa(so, a);
    };
    // the matrix instructions of one K step. First half (A row groups 0, 1):
    // the 16-byte loads of the step two ahead (K step g of tile jt) into
    // buffer u between them (a load instruction waits while the CU's load
    // path is busy, and the matrix pipe keeps working on the instructions
    // issued before it). Then every wave waits for the step after this one to
    // land, and (rd) the second half (row groups 2, 3, alternating) reads it
    // from buffer nx as fragments come free: A groups 0, 1 first, B fragment
    // n after (3, n), A groups 2, 3 at the end.
    auto multiply_issue = [&](bool rd, int g, int jt, int u, int nx, bool live) __attribute__((always_inline)) {
        dma_tail(g, jt, u);                             // branches: kept out of the sequence below
        __builtin_amdgcn_sched_barrier(0);
        constexpr int NK = 4 * NF, HALF = NK / 2;
        constexpr int GRP = KIND == 0 ? 2 : 4;          // matrix instructions per test (measured)
        static_assert(HALF % GRP == 0, "groups stay inside a half");
#pragma unroll
        for (int k = 0; k < NK; ++k) {
            const int a = k < HALF ? k / NF : 2 + ((k - HALF) & 1);
            const int n = k < HALF ? k % NF : (k - HALF) >> 1;
            if (k == HALF) {
                wait_vm_n(stage_ops(g));                // the next step landed
                barrier_lds();                          // ... for every wave
                if (rd) {
                    read_fa(nx, 0);
                    read_fa(nx, 1);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            // (a wave of an empty tile half issues the loads and reads only;
            // one sequence with the test at each group of GRP instructions
            // keeps the register allocation of a single path; the loads and
            // reads placed at an instruction follow its group)
            if (k % GRP == 0 && (ONE || live)) {
#pragma unroll
                for (int d = 0; d < GRP; ++d) {
                    const int kd = k + d;
                    const int ad = kd < HALF ? kd / NF : 2 + ((kd - HALF) & 1);
                    const int nd = kd < HALF ? kd % NF : (kd - HALF) >> 1;
                    acc[ad][nd] = mfma_fp8_16x16x128(FA[ad], FB[nd], acc[ad][nd], SA[ad], 127);
                }
            }
            if (ONE) {
                if (k == 1 || k == 3) dma_a(g, u, k >> 1);
                if (k >= 4 && k < 8) dma_b(g, u, k - 4);
            } else {
                if (k < 16 && (k & 3) == 1) dma_a(g, u, k >> 2);
                if (k < 16 && (k & 3) == 3) dma_b(g, u, k >> 2);
            }
            if (rd) {
                if (k >= HALF && a == 3) read_fb(nx, n);
                if (k == NK - 1) {
                    read_fa(nx, 2);
                    read_fa(nx, 3);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto epilogue = [&](int j) __attribute__((always_inline)) {
        const int L = start + idx + per_x * j;
        const int4 d = desc_of(j);
        const int b = d.x, nt = L % NT, rows = d.z * MM_BM;
        // opaque copies: row addresses are formed here, not hoisted out of the
        // step loop into registers the loop would then have to spill
        int I = I_arg, ln = lane;
        asm volatile("" : "+s"(I));
        asm volatile("" : "+v"(ln));
        const int m = ln & 15, q = ln >> 4;
        const uint8_t* md = smem + MM_RING * Lay::STAGE + (j % MM_NMETA) * MM_META;
        if (KIND == 0) {
            // HN adjacent h columns per lane: fragments n < HN are gate rows,
            // n + HN the matching up rows; NW column waves share a row
            constexpr int HN = NF / 2, NW = ONE ? 4 : 2;
            const int cb = nw * (16 * HN) + HN * m;          // this lane's first h column in the tile
            float* s_amax = (float*)(smem + Lay::AMAX);
            float sg[HN], su[HN];
#pragma unroll
            for (int n = 0; n < HN; ++n) {
                sg[n] = *(const float*)(md + 4 * (cb + n));
                su[n] = *(const float*)(md + 512 + 4 * (cb + n));
            }
            // with z = g sg (g, u: gate and up accumulators, sg, su: row
            // scales), h = silu(z) (u su) = (g u) (sg su) / (1 + 2^(g (-sg log2 e)))
            //   = (g u) / (x c + c),  x = 2^(g ce),  ce = -sg log2 e,  c = 1 / (sg su):
            // two column constants, so an element costs three multiplies, a
            // fused multiply-add, one exp2 and one reciprocal (c is held finite:
            // a zero row scale gives h = 0 as the direct form does)
            float ce[HN], ic[HN];
#pragma unroll
            for (int n = 0; n < HN; ++n) {
                ce[n] = sg[n] * -1.44269504088896341f;
                ic[n] = fminf(__builtin_amdgcn_rcpf(sg[n] * su[n]), 3.0e38f);
            }
            // h replaces the gate accumulators; the 16 row maxima of a lane
            // are reduced and stored after all of them are formed (one
            // straight-line block: independent chains interleave)
            float mx[4][4];
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    mx[a][i] = 0.f;
#pragma unroll
                    for (int n = 0; n < HN; ++n) {
                        const float g = acc[a][n][i];
                        const float x = __builtin_amdgcn_exp2f(g * ce[n]);
                        const float h = (g * acc[a][n + HN][i]) * __builtin_amdgcn_rcpf(fmaf(x, ic[n], ic[n]));
                        acc[a][n][i] = h;
                        mx[a][i] = fmaxf(mx[a][i], fabsf(h));
                    }
                }
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int i = 0; i < 4; ++i) mx[a][i] = row16_max_nonneg(mx[a][i]);
            if (m == 0) {
#pragma unroll
                for (int a = 0; a < 4; ++a)
#pragma unroll
                    for (int i = 0; i < 4; ++i) s_amax[nw * Lay::TM + 64 * mw + 16 * a + 4 * q + i] = mx[a][i];
            }
            barrier_lds();
            // this wave's 64 rows all hold results or all fall in the empty
            // half of a one-block tile (a wave-uniform test). Stores: a
            // wave-uniform row base plus a 32-bit lane offset; the four scale
            // bytes of rows 4q .. 4q+3 (adjacent in hs) in one dword
            if (64 * mw < rows) {
                uint8_t* hrow = hq + ((size_t)b * MM_BM + 64 * mw) * I + nt * 128;
                uint8_t* hsrow = hs + ((size_t)(b + (mw >> 1)) * hgroups + nt) * MM_BM + 64 * (mw & 1);
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    uint32_t eb = 0;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = 64 * mw + 16 * a + 4 * q + i;
                        float amax = s_amax[row];
#pragma unroll
                        for (int w2 = 1; w2 < NW; ++w2) amax = fmaxf(amax, s_amax[w2 * Lay::TM + row]);
                        int e = pow2_exponent_448(amax);
                        e = e < -127 ? -127 : (e > 127 ? 127 : e);
                        eb |= (uint32_t)(e + 127) << (8 * i);
                        // e4m3 codes of h / 2^e: the scaled conversion divides by
                        // its scale operand (the same codes as converting
                        // ldexp(h, -e), measured bit-exact over e in [-127, 20])
                        const float sc = ldexpf(1.0f, e);
                        const s16x2 z = {0, 0};
                        const s16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, acc[a][0][i], acc[a][1][i], sc, false);
                        uint8_t* dst = hrow + (uint32_t)((16 * a + 4 * q + i) * I + cb);
                        if constexpr (HN == 4)
                            *(uint32_t*)dst = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(
                                                                               lo, acc[a][2][i], acc[a][3][i], sc, true));
                        else *(uint16_t*)dst = (uint16_t)(__builtin_bit_cast(uint32_t, lo) & 0xFFFFu);
                    }
                    if (nw == 0 && m == 0) *(uint32_t*)(hsrow + 16 * a + 4 * q) = eb;
                }
            }
        } else {
            const int32_t* s_pr = (const int32_t*)md;
            const float* s_w = (const float*)(md + 1024);
            // NF adjacent columns per lane: one 16-byte (8 columns) or 8-byte store
            const int cb = nw * (16 * NF) + NF * m;
            f32x4 sc[NF / 4];
#pragma unroll
            for (int h = 0; h < NF / 4; ++h) sc[h] = *(const f32x4*)(md + 2048 + 4 * (cb + 4 * h));
            // (a wave-uniform test for the empty half of a one-block tile, as
            // in the gate/up kernel; padding rows per lane)
            if (64 * mw < rows) {
                uint16_t* ycol = ybuf + nt * 256 + cb;
#pragma unroll
                for (int a = 0; a < 4; ++a)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = 64 * mw + 16 * a + 4 * q + i;
                        const int p = s_pr[row];
                        const float w = s_w[row];
                        uint32_t v[NF / 2];
#pragma unroll
                        for (int h = 0; h < NF / 4; ++h) {
                            const float y0 = acc[a][4 * h][i] * sc[h][0] * w, y1 = acc[a][4 * h + 1][i] * sc[h][1] * w;
                            const float y2 = acc[a][4 * h + 2][i] * sc[h][2] * w, y3 = acc[a][4 * h + 3][i] * sc[h][3] * w;
                            v[2 * h] = bf16x2_rne(y0, y1);
                            v[2 * h + 1] = bf16x2_rne(y2, y3);
                        }
                        if (p < NP) {
                            uint16_t* dst = ycol + (size_t)p * H;
                            if constexpr (NF == 8) *(uint4*)dst = make_uint4(v[0], v[1], v[2], v[3]);
                            else *(uint2*)dst = make_uint2(v[0], v[1]);
                        }
                    }
            }
        }
    };

    // ---- the stream of K steps. Step s sits in LDS buffer s % 2. Step cs
    // is in registers when its iteration begins; once every wave has read it
    // its buffer is refilled with step cs+2 during the first half of step
    // cs's matrix instructions, and step cs+1 is read during the second half
    // (at a tile's last step: after the epilogue, whose registers it would
    // otherwise need), so LDS reads, loads and matrix work overlap.
    zero_acc();
    issue(0, 0);
    issue(min(1, N - 1), 1);
    wait_vm_n(stage_ops(min(1, N - 1) % S));            // step 0 landed
    barrier_lds();                                      // ... for every wave
    read_step(0);
    bool live = true;
    // counters: gc = cs % S, jc = cs / S; s2 = min(cs + 2, N - 1) is K step
    // g2 of tile j2
    int gc = 0, jc = 0, s2 = min(2, N - 1);
    int g2 = s2 % S, j2 = s2 / S;
    for (int cs = 0; cs < N; ++cs) {
        // with two or more steps per tile, tile jc was the last one set up
        // when its first step begins
        if (gc == 0 && S >= 2) live = mw < 2 || two_next;
        barrier_lds();                                  // every wave has read step cs
        __builtin_amdgcn_sched_barrier(0);
        if (cs + 2 < N && g2 == 0) setup(j2);
        const int u = cs & 1, nx = ((cs + 1) & 1) * Lay::STAGE;
        const bool end = gc == S - 1;
        multiply_issue(!end, g2, j2, u, nx, live);
        if (end) {
            epilogue(jc);
            zero_acc();
            read_step(nx);                              // (past the last step: unused, no branch)
        }
        if (++gc == S) {
            gc = 0;
            ++jc;
        }
        if (s2 < N - 1) {
            ++s2;
            if (++g2 == S) {
                g2 = 0;
                ++j2;
            }
        }
    }
    wait_vm<0>();      // no load into LDS outlives the workgroup
}

// The FP8 tiles of one GEMM. SPLIT: every workgroup runs its share of the
// two-block tiles (tl2), then its share of the one-block tiles on their own
// layout (tl1), each list split over the XCDs and workgroups on its own.
// Otherwise all tiles (tl) run on the two-block layout, a one-block tile's
// empty half idle.
template <int KIND, bool SPLIT>
__global__ void __launch_bounds__(MM_THREADS, 1)
    mfma_ffn_kernel(MPool pool, MTiles tl, MTiles tl2, MTiles tl1, const uint8_t* __restrict__ xq, int NP, int H,
                    int I, uint8_t* __restrict__ hq, uint8_t* __restrict__ hs, uint16_t* __restrict__ ybuf) {
    extern __shared__ __align__(16) uint8_t smem[];
    if constexpr (SPLIT) {
        mfma_tiles<KIND, false>(pool, tl2, xq, NP, H, I, hq, hs, ybuf, smem);
        __syncthreads();                              // LDS is reused by the one-block tiles
        mfma_tiles<KIND, true>(pool, tl1, xq, NP, H, I, hq, hs, ybuf, smem);
    } else {
        mfma_tiles<KIND, false>(pool, tl, xq, NP, H, I, hq, hs, ybuf, smem);
    }
}

// ------------------------------------------------------------------ host side
bool mfma_path_ok(int H, int I) { return H % 256 == 0 && I % 128 == 0 && H <= 2048 && I <= 2048 && H >= 256; }

// workspace: tiles int4[cap/128], counts (256 B), others int[cap/128], tokrow, wsort, scales, one-block
// and two-block tiles int4[cap/128] each
size_t mfma_ws_bytes(int H, int cap) {
    auto up = [](size_t n) { return (n + 255) / 256 * 256; };
    return up((size_t)(cap / MM_BM) * 16) + 256 + up((size_t)(cap / MM_BM) * 4) + up((size_t)cap * 4) * 2 +
           up((size_t)cap * (H / 128)) + 2 * up((size_t)(cap / MM_BM) * 16);
}

void mfma_other_list(void* ws, int H, int cap, const int** list, const int** n_list) {
    (void)H;
    auto up = [](size_t n) { return (n + 255) / 256 * 256; };
    uint8_t* p = (uint8_t*)ws + up((size_t)(cap / MM_BM) * 16);
    *n_list = (const int*)p + 1;
    *list = (const int*)(p + 256);
}

void mfma_prep_arrays(void* ws, int cap, const int32_t** tokrow, const float** wsort, const uint8_t** scl) {
    auto up = [](size_t n) { return (n + 255) / 256 * 256; };
    const uint8_t* p = (const uint8_t*)ws + up((size_t)(cap / MM_BM) * 16) + 256 + up((size_t)(cap / MM_BM) * 4);
    *tokrow = (const int32_t*)p;
    *wsort = (const float*)(p + up((size_t)cap * 4));
    *scl = p + 2 * up((size_t)cap * 4);
}

hipError_t launch_mfma_ffn(const PoolArgs& pa, const uint8_t* xq, const uint8_t* xs, int NP, int k,
                           const float* topk_w, const int32_t* sorted_pair, const int32_t* block_slot,
                           const int32_t* n_padded, int cap, uint8_t* hq, uint8_t* hs, uint16_t* ybuf, void* ws,
                           int phase, hipStream_t stream) {
    const int H = pa.hidden, I = pa.inter;
    auto up = [](size_t n) { return (n + 255) / 256 * 256; };
    uint8_t* p = (uint8_t*)ws;
    int4* tiles = (int4*)p;
    p += up((size_t)(cap / MM_BM) * 16);
    int* n_tiles = (int*)p;
    int* n_others = n_tiles + 1;
    int* n_tiles1 = n_tiles + 2;
    int* n_tiles2 = n_tiles + 3;
    p += 256;
    int* others = (int*)p;
    p += up((size_t)(cap / MM_BM) * 4);
    int32_t* tokrow = (int32_t*)p;
    p += up((size_t)cap * 4);
    float* wsort = (float*)p;
    p += up((size_t)cap * 4);
    uint8_t* scl = p;
    int4* tiles1 = (int4*)(p + up((size_t)cap * (H / 128)));
    int4* tiles2 = tiles1 + up((size_t)(cap / MM_BM) * 16) / 16;

    MPool mp;
    mp.base = (const uint8_t*)pa.base;
    mp.stride = pa.stride;
    for (int i = 0; i < 4; ++i) mp.off[i] = pa.off[0][i];
    int nwg = device_cus() / 8 * 8;
    if (nwg < 8) nwg = 8;
    // one-block tiles on their own layout when experts average fewer than
    // three blocks of pairs (one-block tiles are then a large share: C3
    // T=4096 80% of the tiles, C4 T=8192 35%); at more (C2: 512 pairs per
    // expert, 29% of the tiles, a fifth of the rows) the second list's
    // pipeline start costs what the layout saves
    const bool split = (long)NP < 384L * pa.n_slots;
    if (phase == 0) {
        MOE_LAUNCH(K_MFMA_PREP, stream, mfma_prep_kernel, dim3(1 + (cap + 255) / 256), dim3(256), 0, stream,
                   sorted_pair, block_slot, pa.fmt, pa.n_slots, pa.fmt_ok, n_padded, NP, k, topk_w, xs, H / 128, tiles,
                   n_tiles, tiles1, n_tiles1, tiles2, n_tiles2, others, n_others, tokrow, wsort, scl);
        MTiles tl{tiles, n_tiles, tokrow, wsort, sorted_pair, scl};
        MTiles tl2{tiles2, n_tiles2, tokrow, wsort, sorted_pair, scl};
        MTiles tl1{tiles1, n_tiles1, tokrow, wsort, sorted_pair, scl};
        if (split) {
            hipError_t e = hipFuncSetAttribute((const void*)mfma_ffn_kernel<0, true>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, MM_SMEM);
            if (e != hipSuccess) return e;
            MOE_LAUNCH(K_GEMM1_FP8, stream, (mfma_ffn_kernel<0, true>), dim3(nwg), dim3(MM_THREADS), MM_SMEM, stream,
                       mp, tl, tl2, tl1, xq, NP, H, I, hq, hs, ybuf);
        } else {
            hipError_t e = hipFuncSetAttribute((const void*)mfma_ffn_kernel<0, false>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, MM_SMEM);
            if (e != hipSuccess) return e;
            MOE_LAUNCH(K_GEMM1_FP8, stream, (mfma_ffn_kernel<0, false>), dim3(nwg), dim3(MM_THREADS), MM_SMEM, stream,
                       mp, tl, tl2, tl1, xq, NP, H, I, hq, hs, ybuf);
        }
    } else {
        MTiles tl{tiles, n_tiles, tokrow, wsort, sorted_pair, hs};
        MTiles tl2{tiles2, n_tiles2, tokrow, wsort, sorted_pair, hs};
        MTiles tl1{tiles1, n_tiles1, tokrow, wsort, sorted_pair, hs};
        if (split) {
            hipError_t e = hipFuncSetAttribute((const void*)mfma_ffn_kernel<1, true>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, MM_SMEM);
            if (e != hipSuccess) return e;
            MOE_LAUNCH(K_GEMM2_FP8, stream, (mfma_ffn_kernel<1, true>), dim3(nwg), dim3(MM_THREADS), MM_SMEM, stream,
                       mp, tl, tl2, tl1, xq, NP, H, I, hq, hs, ybuf);
        } else {
            hipError_t e = hipFuncSetAttribute((const void*)mfma_ffn_kernel<1, false>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, MM_SMEM);
            if (e != hipSuccess) return e;
            MOE_LAUNCH(K_GEMM2_FP8, stream, (mfma_ffn_kernel<1, false>), dim3(nwg), dim3(MM_THREADS), MM_SMEM, stream,
                       mp, tl, tl2, tl1, xq, NP, H, I, hq, hs, ybuf);
        }
    }
    return hipGetLastError();
}

}  // namespace moe
