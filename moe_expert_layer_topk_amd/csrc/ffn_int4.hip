// Expert FFN at batched sizes, gate/up GEMM of the blocks whose expert slot is
// int4-g128.
//
// PagedWeight commentary (spectral-agent.com), "technically interesting
// points" and "hardware requirements": experts are held at their own bit
// width and the GPU kernels switch format per expert. MOE-GEN explainer
// (aibr.jp), sections 1 and 3: tokens gathered per expert make each expert one
// dense contraction. An int4-g128 weight is scale * (q - zero) with one fp16
// (scale, zero) pair per row and 128 columns of K.
//
// The FP8 blocks run on the pipelined matrix-core kernels; the int4 blocks
// (listed by their prep kernel) run here, one tile = half of a 128-row block
// x 128 inter columns (128 gate and the matching 128 up rows of W13), K in
// steps of 128 = one int4 group. Converting the weights costs the same per
// step whatever the rows, so the work is cut by rows: 64-row tiles keep the
// accumulators in registers, give twice the tiles to spread over the CUs and
// fit two workgroups per CU:
// * a ring of three LDS stages filled by direct-to-LDS loads, so two steps
//   are in flight while one is multiplied and no register holds a load: a
//   stage holds the tile's 64 gathered activation rows (e4m3 codes,
//   16-byte chunks XOR-placed for conflict-free fragment reads; each wave
//   loads a quarter and reads all) and, per wave, the int4 codes of the 64
//   weight rows that wave multiplies (its 32 gate and 32 up columns) with
//   their (scale, zero) pairs for the group, so a wave's weight data needs no
//   barrier;
// * each wave turns the next step's int4 codes into e4m3 codes of q - zero
//   in registers (q - zero is an integer in [-15, 15], exact in e4m3) while
//   the current step's matrix instructions run, and issues the loads of the
//   step three ahead between them;
// * one v_mfma_scale_f32_16x16x128_f8f6f4 per (16 rows, 16 columns) with the
//   activation exponents as A scales, from zero, then scaled by the group's
//   fp16 scale of the column and added to the accumulator;
// * the epilogue is the tile kernels' one: silu(gate) * up, e4m3 codes of h
//   with a power-of-two exponent per (row, 128 columns).
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

namespace {

constexpr int Q_THREADS = 256;                    // 4 waves; wave w owns inter columns [32w, 32w + 32)
constexpr int Q_BM = 128;                         // rows of an align block
constexpr int Q_TM = 64;                          // rows of a tile
constexpr int Q_RING = 3;                         // LDS stages
constexpr int Q_A = Q_TM * 128;                   // activation codes: 64 rows x 128 K
constexpr int Q_BQ = 256 * 64;                    // int4 codes: 4 waves x 64 weight rows x 128 K
constexpr int Q_SZ = 256 * 4;                     // (scale, zero) of those rows for the step's group
constexpr int Q_STAGE = Q_A + Q_BQ + Q_SZ;
constexpr int Q_XS = Q_RING * Q_STAGE;            // activation exponent bytes [64 rows][16 groups]
constexpr int Q_SMEM = Q_XS + Q_TM * 16;
constexpr int Q_OPS = 2 + 4 + 1;                  // vector memory operations per wave and stage
constexpr int Q_HROW = 144;                       // epilogue: h code rows staged with 16 bytes of padding
constexpr int Q_AMAX = Q_TM * Q_HROW;             // epilogue: row maxima [4 waves][64 rows] after the staged rows

// position of 16-byte chunk c of stage row r: c ^ qsw(r). Fragment reads take
// rows m of a fragment at lanes m + 16 q, chunks 2q and 2q + 1; this placement
// keeps them free of bank conflicts (the batched FP8 kernels' one).
__device__ __forceinline__ int qsw(int r) { return ((r & 15) >> 1) & 5; }

__device__ __forceinline__ void q_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ i32x8 q_frag(const uint8_t* tile, int r, int o0, int o1) {
    const i32x4 lo = *(const i32x4*)(tile + r * 128 + o0);
    const i32x4 hi = *(const i32x4*)(tile + r * 128 + o1);
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu)); }
__device__ __forceinline__ float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

}  // namespace

struct Q4Pool {
    const uint8_t* base;
    size_t stride;
    const uint8_t* fmt;
    size_t off_sz13;          // int4 slot: (scale, zero) pairs of W13
    int n_slots;
    int fmt_ok;
};

// One-dimensional grid, a multiple of 8 workgroups (about two per CU).
// Workgroups are dealt to the 8 XCDs in turn (workgroup g on XCD g % 8), and
// every tile of a listed block (I / 128 column tiles x 2 row halves) goes to
// the same XCD, so the halves' shared weight rows and the column tiles'
// shared activation rows meet in that XCD's L2: XCD x takes listed blocks
// x, x + 8, ... (count *n_list, known only on the device), its workgroups
// their tiles in turn. FP8 blocks in the list are skipped
// (the list also holds blocks whose slot is not usable: their pairs get zero
// rows from the down kernel).
__global__ void __launch_bounds__(Q_THREADS, 2)
    gemm1_int4_ring_kernel(Q4Pool pool, const uint8_t* __restrict__ xq, const int32_t* __restrict__ tokrow,
                           const uint8_t* __restrict__ scl, const int32_t* __restrict__ block_slot, int H, int I,
                           uint8_t* __restrict__ hq, uint8_t* __restrict__ hs, const int* __restrict__ list,
                           const int* __restrict__ n_list) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / MOE_WAVE);
    const int m = lane & 15, q = lane >> 4;
    const int S = H / 128;                        // K steps = groups of the activation and of W13
    const int hgroups = I / 128;
    const int NT = I / 128;                       // column tiles of a block
    const int xcd = blockIdx.x & 7, P = gridDim.x >> 3;
    uint8_t* s_xs = smem + Q_XS;
    const int fm = qsw(m);
    const int o0 = ((2 * q) ^ fm) << 4, o1 = ((2 * q + 1) ^ fm) << 4;

    const int n = *n_list;
    for (int j = blockIdx.x >> 3;; j += P) {
        const int bi = xcd + 8 * (j / (2 * NT));      // listed block, column tile, row half of tile j
        if (bi >= n) break;
        const int ct = (j % (2 * NT)) >> 1, half = j & 1;
        const int c0 = ct * 128;
        const int b = list[bi];
        const int r0 = b * Q_BM + half * Q_TM;        // first sorted position of the tile
        const int slot = usable_slot(block_slot[b], pool.n_slots, pool.fmt_ok, pool.fmt);
        if (slot < 0 || pool.fmt[slot] != MOE_FMT_INT4_G128) continue;   // (uniform over the workgroup)
        const uint8_t* w13 = pool.base + (size_t)slot * pool.stride;   // int4 codes [2I][H/2]
        const uint8_t* sz13 = w13 + pool.off_sz13;                     // (scale, zero) [2I][H/128]

        // the tile's activation exponents [row][step] (the prep kernel's
        // [block][step][row] bytes), fetched with the token ids
        uint32_t xsw[Q_TM * 16 / 4 / Q_THREADS];
#pragma unroll
        for (int v = 0; v < Q_TM * 16 / 4 / Q_THREADS; ++v) {
            const int i = threadIdx.x + Q_THREADS * v, g = i >> 4, r4 = (i & 15) * 4;   // 4 rows of step g
            xsw[v] = g < S ? *(const uint32_t*)(scl + ((size_t)b * S + g) * Q_BM + half * Q_TM + r4) : 0u;
        }
        // the loads of step g into stage u: wave w fills activation rows
        // 16w .. 16w + 15 and its own weight rows (local row lr < 32: gate
        // column 32w + lr, else up column 32w + lr - 32) with their pairs;
        // this lane's activation sources (row 8 (2w + j) + lane / 8, its chunk
        // placed at lane % 8) are fixed for the tile (padding rows read
        // token 0; their h rows are never used)
        uint32_t aoff[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int r = 8 * (2 * wv + j) + (lane >> 3);
            aoff[j] = (uint32_t)tokrow[r0 + r] * (uint32_t)H + 16u * (uint32_t)((lane & 7) ^ qsw(r));
        }
        auto wrow_of = [&](int lr) __attribute__((always_inline)) { return (lr >> 5) * I + c0 + 32 * wv + (lr & 31); };
        auto issue_a = [&](int g, int u, int j) __attribute__((always_inline)) {
            lds_dma16(xq + aoff[j] + g * 128, smem + u * Q_STAGE + (2 * wv + j) * 1024);
        };
        auto issue_b = [&](int g, int u, int j) __attribute__((always_inline)) {
            const int lr = 16 * j + (lane >> 2);
            lds_dma16(w13 + (size_t)wrow_of(lr) * (H / 2) + g * 64 + 16 * (lane & 3),
                      smem + u * Q_STAGE + Q_A + wv * 4096 + j * 1024);
        };
        auto issue_sz = [&](int g, int u) __attribute__((always_inline)) {
            lds_dma4(sz13 + ((size_t)wrow_of(lane) * S + g) * 4, smem + u * Q_STAGE + Q_A + Q_BQ + wv * 256);
        };
        auto issue = [&](int g, int u) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < 2; ++j) issue_a(g, u, j);
#pragma unroll
            for (int j = 0; j < 4; ++j) issue_b(g, u, j);
            issue_sz(g, u);
        };
        // this lane's weight data of a stage: fragment (gu, c) is local row
        // gu * 32 + c * 16 + m, K bytes [32 q, 32 q + 32) = 16 bytes of codes
        auto read_b = [&](int u, i32x4 raw[2][2], uint32_t zs[2][2]) __attribute__((always_inline)) {
            const uint8_t* st = smem + u * Q_STAGE;
#pragma unroll
            for (int gu = 0; gu < 2; ++gu)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const int lr = gu * 32 + c * 16 + m;
                    raw[gu][c] = *(const i32x4*)(st + Q_A + wv * 4096 + lr * 64 + 16 * q);
                    zs[gu][c] = *(const uint32_t*)(st + Q_A + Q_BQ + wv * 256 + 4 * lr);
                }
        };
        auto convert = [&](const i32x4& raw, uint32_t zs, i32x8& out) __attribute__((always_inline)) {
            uint32_t o[8];
            const float z = f16_hi(zs);
            int4_to_e4m3_16(make_uint2((uint32_t)raw[0], (uint32_t)raw[1]), z, o);
            int4_to_e4m3_16(make_uint2((uint32_t)raw[2], (uint32_t)raw[3]), z, o + 4);
            out = i32x8{(int)o[0], (int)o[1], (int)o[2], (int)o[3], (int)o[4], (int)o[5], (int)o[6], (int)o[7]};
        };

        f32x4 acc[4][2][2];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int gu = 0; gu < 2; ++gu)
#pragma unroll
                for (int c = 0; c < 2; ++c) acc[a][gu][c] = f32x4{0, 0, 0, 0};

        issue(0, 0);
        issue(min(1, S - 1), 1);
        issue(min(2, S - 1), 2);
#pragma unroll
        for (int v = 0; v < Q_TM * 16 / 4 / Q_THREADS; ++v) {
            const int i = threadIdx.x + Q_THREADS * v, g = i >> 4, r4 = (i & 15) * 4;
#pragma unroll
            for (int d = 0; d < 4; ++d) s_xs[(r4 + d) * 16 + g] = (uint8_t)(xsw[v] >> (8 * d));
        }
        // e4m3 codes of q - zero and group scales (this lane's output
        // columns) of a step: two sets, current and next, in turn
        i32x8 bfA[2][2], bfB[2][2];
        float scA[2][2], scB[2][2];
        {
            wait_vmcnt<2 * Q_OPS>();                  // this wave's stage 0
            i32x4 raw[2][2];
            uint32_t zs[2][2];
            read_b(0, raw, zs);
#pragma unroll
            for (int gu = 0; gu < 2; ++gu)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    convert(raw[gu][c], zs[gu][c], bfA[gu][c]);
                    scA[gu][c] = f16_lo(zs[gu][c]);
                }
        }
        auto step = [&](int g, const i32x8 (&bf)[2][2], const float (&sc)[2][2], i32x8 (&bn)[2][2],
                        float (&scn)[2][2]) __attribute__((always_inline)) {
            const int u = g % Q_RING, un = (g + 1) % Q_RING;
            const uint8_t* st = smem + u * Q_STAGE;
            wait_vmcnt<Q_OPS>();                      // this wave's stages g and g + 1 (step g + 2 may fly)
            q_barrier();                              // ... and every wave's activation rows of step g
            i32x8 af8[4];
            int sa8[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                af8[a] = q_frag(st, a * 16 + m, o0, o1);
                sa8[a] = s_xs[(a * 16 + m) * 16 + g];
            }
            i32x4 raw[2][2];                          // next step's codes (past the end: a repeated step)
            uint32_t zs[2][2];
            read_b(un, raw, zs);
            q_barrier();                              // every wave has read stage u's activation rows
            __builtin_amdgcn_sched_barrier(0);
            // 16 matrix instructions; between them the conversion of the next
            // step's codes, the scaling of the previous group's results and
            // the loads of step g + 3 into stage u (past the end: the last
            // step again, so every step leaves the same number of loads behind)
            const int gl = min(g + Q_RING, S - 1);
            f32x4 t4[2][2][2];
#pragma unroll
            for (int a = 0; a < 5; ++a) {
                if (a < 4) {
#pragma unroll
                    for (int gu = 0; gu < 2; ++gu)
#pragma unroll
                        for (int c = 0; c < 2; ++c)
                            t4[a & 1][gu][c] = mfma_fp8_16x16x128(af8[a], bf[gu][c], f32x4{0, 0, 0, 0}, sa8[a], 127);
                }
                if (a > 0) {
#pragma unroll
                    for (int gu = 0; gu < 2; ++gu)
#pragma unroll
                        for (int c = 0; c < 2; ++c) acc[a - 1][gu][c] += sc[gu][c] * t4[(a - 1) & 1][gu][c];
                }
                if (a < 4) convert(raw[a >> 1][a & 1], zs[a >> 1][a & 1], bn[a >> 1][a & 1]);
                if (a < 2) issue_a(gl, u, a);
                if (a < 4) issue_b(gl, u, a);
                if (a == 4) issue_sz(gl, u);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int gu = 0; gu < 2; ++gu)
#pragma unroll
                for (int c = 0; c < 2; ++c) scn[gu][c] = f16_lo(zs[gu][c]);
        };
        // steps in pairs (the sets swap roles), then an odd last one
        int g = 0;
        for (; g + 1 < S; g += 2) {
            step(g, bfA, scA, bfB, scB);
            step(g + 1, bfB, scB, bfA, scA);
        }
        if (g < S) step(g, bfA, scA, bfB, scB);
        wait_vmcnt<0>();
        __syncthreads();

        // epilogue: silu(gate) * up, then e4m3 codes of h with one exponent
        // per (row, 128 columns) (this tile's columns)
        float* s_amax = (float*)(smem + Q_AMAX);      // [4 waves][64 rows]
        float hv[4][2][4];
        float rmax[4][4];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
#pragma unroll
            for (int i = 0; i < 4; ++i) rmax[a][i] = 0.f;
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float h = silu(acc[a][0][c][i]) * acc[a][1][c][i];
                    hv[a][c][i] = h;
                    rmax[a][i] = fmaxf(rmax[a][i], fabsf(h));
                }
        }
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v = rmax[a][i];
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
                if (m == 0) s_amax[wv * Q_TM + a * 16 + 4 * q + i] = v;
            }
        __syncthreads();
        uint8_t* sH = smem;                           // [64][Q_HROW] codes
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = a * 16 + 4 * q + i;
                const float amax = fmaxf(fmaxf(s_amax[row], s_amax[Q_TM + row]),
                                         fmaxf(s_amax[2 * Q_TM + row], s_amax[3 * Q_TM + row]));
                int e = pow2_exponent_448(amax);
                e = e < -127 ? -127 : (e > 127 ? 127 : e);
#pragma unroll
                for (int c = 0; c < 2; ++c)
                    sH[row * Q_HROW + wv * 32 + c * 16 + m] = (uint8_t)(f32x2_to_e4m3(ldexpf(hv[a][c][i], -e), 0.f) & 0xFF);
                if (wv == 0 && m == 0) hs[(size_t)(r0 + row) * hgroups + ct] = (uint8_t)(e + 127);
            }
        __syncthreads();
        for (int i = threadIdx.x; i < Q_TM * 8; i += Q_THREADS) {
            const int r = i >> 3, ch = i & 7;
            *(i32x4*)(hq + (size_t)(r0 + r) * I + c0 + ch * 16) = *(const i32x4*)(sH + r * Q_HROW + ch * 16);
        }
        q_barrier();                                  // LDS is reused by the next listed block (the stores fly on)
    }
}

// ------------------------------------------------------------ down GEMM
// One tile = one 128-row block x 128 hidden columns (128 rows of W2), K = I
// in steps of 128 = one int4 group, built like the gate/up kernel: a ring of
// three direct-to-LDS stages (the block's h codes, rows in sorted order, XOR
// placed; per wave the int4 codes and (scale, zero) pairs of the 32 W2 rows
// it multiplies), conversion of the next step's codes in registers during
// the current step's matrix instructions. The epilogue multiplies by the
// pair's route weight and writes the pair's bf16 row through LDS (16-byte
// stores). Blocks whose slot is not usable write zero rows (a deferred block
// is left alone); FP8 blocks are skipped.
namespace {
constexpr int D_A = Q_BM * 128;                   // h codes: 128 rows x 128 K
constexpr int D_BQ = 4 * 32 * 64;                 // int4 codes: 4 waves x 32 W2 rows x 128 K
constexpr int D_SZ = 4 * 256;                     // (scale, zero) of those rows (lanes 32..63 repeat 0..31)
constexpr int D_STAGE = D_A + D_BQ + D_SZ;
constexpr int D_HS = Q_RING * D_STAGE;            // h exponent bytes [128 rows][16 groups]
constexpr int D_PR = D_HS + Q_BM * 16;            // pair of each row
constexpr int D_W = D_PR + Q_BM * 4;              // route weight of each row (0: padding)
constexpr int D_SMEM = D_W + Q_BM * 4;
constexpr int D_OPS = 4 + 2 + 1;                  // vector memory operations per wave and stage
constexpr int D_YROW = 136;                       // epilogue: bf16 rows staged with 16 bytes of padding
}  // namespace

struct Q4Pool2 {
    const uint8_t* base;
    size_t stride;
    const uint8_t* fmt;
    size_t off_w2, off_sz2;   // int4 slot: W2 codes [H][I/2], (scale, zero) pairs [H][I/128]
    int n_slots;
    int fmt_ok;
};

__global__ void __launch_bounds__(Q_THREADS, 2)
    gemm2_int4_ring_kernel(Q4Pool2 pool, int NP, const float* __restrict__ wsort,
                           const int32_t* __restrict__ sorted_pair, const int32_t* __restrict__ block_slot, int H,
                           int I, const uint8_t* __restrict__ hq, const uint8_t* __restrict__ hs,
                           uint16_t* __restrict__ ybuf, const int* __restrict__ list,
                           const int* __restrict__ n_list) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / MOE_WAVE);
    const int m = lane & 15, q = lane >> 4;
    const int S = I / 128;                        // K steps = groups of h and of W2
    const int NT = H / 128;                       // column tiles of a block
    const int xcd = blockIdx.x & 7, P = gridDim.x >> 3;
    uint8_t* s_hs = smem + D_HS;
    int* s_pr = (int*)(smem + D_PR);
    float* s_w = (float*)(smem + D_W);
    const int fm = qsw(m);
    const int o0 = ((2 * q) ^ fm) << 4, o1 = ((2 * q + 1) ^ fm) << 4;

    const int n = *n_list;
    // XCD x takes listed blocks x, x + 8, ..., its workgroups their column
    // tiles in turn (a block's h rows meet in that XCD's L2)
    for (int j = blockIdx.x >> 3;; j += P) {
        const int bi = xcd + 8 * (j / NT);
        if (bi >= n) break;
        const int n0 = (j % NT) * 128;
        const int b = list[bi];
        const int bs = block_slot[b];
        const int slot = usable_slot(bs, pool.n_slots, pool.fmt_ok, pool.fmt);
        if (slot < 0) {                           // not usable: the block's pairs add zero
            if (bs == MOE_SLOT_DEFERRED) continue;    // (a deferred block's rows are left as they are)
            for (int i = threadIdx.x; i < Q_BM * 16; i += Q_THREADS) {
                const int r = i >> 4, ch = i & 15;
                const int p = sorted_pair[b * Q_BM + r];
                if (p < NP) *(i32x4*)(ybuf + (size_t)p * H + n0 + ch * 8) = i32x4{0, 0, 0, 0};
            }
            continue;
        }
        if (pool.fmt[slot] != MOE_FMT_INT4_G128) continue;   // (uniform over the workgroup)
        const uint8_t* sb = pool.base + (size_t)slot * pool.stride;
        const uint8_t* w2 = sb + pool.off_w2;
        const uint8_t* sz2 = sb + pool.off_sz2;
        const uint8_t* hrow = hq + (size_t)b * Q_BM * I;

        // loads of step g into stage u: wave w fills h rows 32w .. 32w + 31
        // and its own W2 rows n0 + 32w .. n0 + 32w + 31 with their pairs
        auto issue_a = [&](int g, int u, int j) __attribute__((always_inline)) {
            const int r = 8 * (4 * wv + j) + (lane >> 3);
            lds_dma16(hrow + (size_t)r * I + g * 128 + 16 * ((lane & 7) ^ qsw(r)),
                      smem + u * D_STAGE + (4 * wv + j) * 1024);
        };
        auto issue_b = [&](int g, int u, int j) __attribute__((always_inline)) {
            const int lr = 16 * j + (lane >> 2);
            lds_dma16(w2 + (size_t)(n0 + 32 * wv + lr) * (I / 2) + g * 64 + 16 * (lane & 3),
                      smem + u * D_STAGE + D_A + wv * 2048 + j * 1024);
        };
        auto issue_sz = [&](int g, int u) __attribute__((always_inline)) {
            lds_dma4(sz2 + ((size_t)(n0 + 32 * wv + (lane & 31)) * S + g) * 4, smem + u * D_STAGE + D_A + D_BQ + wv * 256);
        };
        auto issue = [&](int g, int u) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < 4; ++j) issue_a(g, u, j);
#pragma unroll
            for (int j = 0; j < 2; ++j) issue_b(g, u, j);
            issue_sz(g, u);
        };
        // this lane's W2 data of a stage: fragment c is local row c * 16 + m
        auto read_b = [&](int u, i32x4 raw[2], uint32_t zs[2]) __attribute__((always_inline)) {
            const uint8_t* st = smem + u * D_STAGE;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int lr = c * 16 + m;
                raw[c] = *(const i32x4*)(st + D_A + wv * 2048 + lr * 64 + 16 * q);
                zs[c] = *(const uint32_t*)(st + D_A + D_BQ + wv * 256 + 4 * lr);
            }
        };
        auto convert = [&](const i32x4& raw, uint32_t zs, i32x8& out) __attribute__((always_inline)) {
            uint32_t o[8];
            const float z = f16_hi(zs);
            int4_to_e4m3_16(make_uint2((uint32_t)raw[0], (uint32_t)raw[1]), z, o);
            int4_to_e4m3_16(make_uint2((uint32_t)raw[2], (uint32_t)raw[3]), z, o + 4);
            out = i32x8{(int)o[0], (int)o[1], (int)o[2], (int)o[3], (int)o[4], (int)o[5], (int)o[6], (int)o[7]};
        };

        f32x4 acc[8][2];
#pragma unroll
        for (int a = 0; a < 8; ++a) acc[a][0] = acc[a][1] = f32x4{0, 0, 0, 0};

        // the block's pairs, route weights and h exponents into LDS while the
        // first stages load (one round trip; the loads are fetched first)
        int pr_v = 0;
        float w_v = 0.f;
        uint32_t hs_v[Q_BM * 16 / 4 / Q_THREADS];
        if (threadIdx.x < Q_BM) {
            pr_v = sorted_pair[b * Q_BM + threadIdx.x];
            w_v = wsort[b * Q_BM + threadIdx.x];
        }
#pragma unroll
        for (int v = 0; v < Q_BM * 16 / 4 / Q_THREADS; ++v) {
            const int i = threadIdx.x + Q_THREADS * v;    // 4 bytes of the block's [128 rows][S] exponents
            hs_v[v] = 4 * i < Q_BM * S ? *(const uint32_t*)(hs + (size_t)b * Q_BM * S + 4 * i) : 0u;
        }
        issue(0, 0);
        issue(min(1, S - 1), 1);
        issue(min(2, S - 1), 2);
        if (threadIdx.x < Q_BM) {
            s_pr[threadIdx.x] = pr_v;
            s_w[threadIdx.x] = w_v;
        }
#pragma unroll
        for (int v = 0; v < Q_BM * 16 / 4 / Q_THREADS; ++v) {
            const int i = threadIdx.x + Q_THREADS * v;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const int e = 4 * i + d;              // row e / S, group e % S
                if (e < Q_BM * S) s_hs[(e / S) * 16 + e % S] = (uint8_t)(hs_v[v] >> (8 * d));
            }
        }
        i32x8 bf[2];
        float sc[2];
        {
            wait_vmcnt<2 * D_OPS>();                  // this wave's stage 0
            i32x4 raw[2];
            uint32_t zs[2];
            read_b(0, raw, zs);
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                convert(raw[c], zs[c], bf[c]);
                sc[c] = f16_lo(zs[c]);
            }
        }
        for (int g = 0; g < S; ++g) {
            const int u = g % Q_RING, un = (g + 1) % Q_RING;
            const uint8_t* st = smem + u * D_STAGE;
            wait_vmcnt<D_OPS>();                      // this wave's stages g and g + 1 (step g + 2 may fly)
            q_barrier();                              // ... and every wave's h rows of step g
            i32x8 af8[8];
            int sa8[8];
#pragma unroll
            for (int a = 0; a < 8; ++a) {
                af8[a] = q_frag(st, a * 16 + m, o0, o1);
                sa8[a] = s_hs[(a * 16 + m) * 16 + g];
            }
            i32x4 raw[2];                             // next step's codes (past the end: a repeated step)
            uint32_t zs[2];
            read_b(un, raw, zs);
            q_barrier();                              // every wave has read stage u's h rows
            __builtin_amdgcn_sched_barrier(0);
            const int gl = min(g + Q_RING, S - 1);
            i32x8 bn[2];
            f32x4 t4[2][2];
#pragma unroll
            for (int a = 0; a < 9; ++a) {
                if (a < 8) {
#pragma unroll
                    for (int c = 0; c < 2; ++c)
                        t4[a & 1][c] = mfma_fp8_16x16x128(af8[a], bf[c], f32x4{0, 0, 0, 0}, sa8[a], 127);
                }
                if (a > 0) {
#pragma unroll
                    for (int c = 0; c < 2; ++c) acc[a - 1][c] += sc[c] * t4[(a - 1) & 1][c];
                }
                if (a < 2) convert(raw[a], zs[a], bn[a]);
                if (a < 4) issue_a(gl, u, a);
                if (a >= 4 && a < 6) issue_b(gl, u, a - 4);
                if (a == 6) issue_sz(gl, u);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                bf[c] = bn[c];
                sc[c] = f16_lo(zs[c]);
            }
        }
        wait_vmcnt<0>();
        __syncthreads();

        // epilogue: route weight, bf16 rows staged in LDS, 16-byte stores to
        // the pairs' rows
        uint16_t* sY = (uint16_t*)smem;               // [128][D_YROW]
#pragma unroll
        for (int a = 0; a < 8; ++a)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = a * 16 + 4 * q + i;
                const float wt = s_w[row];
#pragma unroll
                for (int c = 0; c < 2; ++c) sY[row * D_YROW + wv * 32 + c * 16 + m] = f32_to_bf16(acc[a][c][i] * wt);
            }
        __syncthreads();
        for (int i = threadIdx.x; i < Q_BM * 16; i += Q_THREADS) {
            const int r = i >> 4, ch = i & 15;
            const int p = s_pr[r];
            if (p < NP) *(i32x4*)(ybuf + (size_t)p * H + n0 + ch * 8) = *(const i32x4*)(sY + r * D_YROW + ch * 8);
        }
        q_barrier();                                  // LDS is reused by the next listed block (the stores fly on)
    }
}

bool int4_ring_ok(int H, int I) { return H % 128 == 0 && H <= 2048 && I % 128 == 0 && I <= 2048; }

hipError_t launch_gemm1_int4_ring(const PoolArgs& pa, const uint8_t* xq, const int32_t* tokrow, const uint8_t* scl,
                                  const int32_t* block_slot, int I, uint8_t* hq, uint8_t* hs, const int* list,
                                  const int* n_list, int grid_y, hipStream_t stream) {
    Q4Pool qp;
    qp.base = (const uint8_t*)pa.base;
    qp.stride = pa.stride;
    qp.fmt = pa.fmt;
    qp.off_sz13 = pa.off[1][1];
    qp.n_slots = pa.n_slots;
    qp.fmt_ok = pa.fmt_ok;
    hipError_t e = hipFuncSetAttribute((const void*)gemm1_int4_ring_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       Q_SMEM);
    if (e != hipSuccess) return e;
    // about two workgroups per CU, a multiple of 8, no more than the tiles can use
    const int g = max(8, min(2 * device_cus(), 2 * (I / 128) * grid_y) / 8 * 8);
    MOE_LAUNCH(K_GEMM1_TILE, stream, gemm1_int4_ring_kernel, dim3(g), dim3(Q_THREADS), Q_SMEM, stream, qp,
               xq, tokrow, scl, block_slot, pa.hidden, I, hq, hs, list, n_list);
    return hipGetLastError();
}

hipError_t launch_gemm2_int4_ring(const PoolArgs& pa, int NP, const float* wsort, const int32_t* sorted_pair,
                                  const int32_t* block_slot, int I, const uint8_t* hq, const uint8_t* hs,
                                  uint16_t* ybuf, const int* list, const int* n_list, int grid_y,
                                  hipStream_t stream) {
    Q4Pool2 qp;
    qp.base = (const uint8_t*)pa.base;
    qp.stride = pa.stride;
    qp.fmt = pa.fmt;
    qp.off_w2 = pa.off[1][2];
    qp.off_sz2 = pa.off[1][3];
    qp.n_slots = pa.n_slots;
    qp.fmt_ok = pa.fmt_ok;
    hipError_t e = hipFuncSetAttribute((const void*)gemm2_int4_ring_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       D_SMEM);
    if (e != hipSuccess) return e;
    const int g = max(8, min(2 * device_cus(), (pa.hidden / 128) * grid_y) / 8 * 8);
    MOE_LAUNCH(K_GEMM2_TILE, stream, gemm2_int4_ring_kernel, dim3(g), dim3(Q_THREADS), D_SMEM,
               stream, qp, NP, wsort, sorted_pair, block_slot, pa.hidden, I, hq, hs, ybuf, list, n_list);
    return hipGetLastError();
}

}  // namespace moe
