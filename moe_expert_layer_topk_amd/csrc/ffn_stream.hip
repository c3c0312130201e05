// Expert FFN, streaming path for small token counts (activations in bf16).
//
// vllm-expert-pager article (rand.pepabo.com), Table 1 set-up: each expert
// has w13 (gate and up fused) and w2 (down); "hierarchical paging" section:
// they are read from the expert's VRAM slot. At decode sizes the layer is
// bound by reading those slots once from HBM, so both kernels cut the routed
// experts' weights into many small units spread over the whole chip, issue
// every 16-byte load of a unit before using any (one memory round trip per
// unit), and feed the rows, converted to bf16 (exact for e4m3 codes and for
// int4 q - zero), to bf16 matrix cores against the few token rows of each
// expert.
//
// gemm1 (gate/up): unit = (block of pairs, 16 rows of inter). The 4 waves of
//   a workgroup split K = hidden by 128-wide groups; partial sums meet in
//   LDS; the epilogue applies row scales, silu(gate) * up and stores h (bf16).
// gemm2 (down): unit = (block of pairs, 64 rows of hidden); each wave owns 16
//   rows, multiplies them by h and writes w[t][j] * y for each pair (fp32).
// combine: out[t] = sum_j ybuf[t*k + j], fixed order, rounded once to bf16.
//
// Operand layout of v_mfma_f32_16x16x32_bf16 (lane l = m + 16 q): A row m and
// B column m hold K positions 8q..8q+7; C lane l holds rows 4q..4q+3 of
// column m. Both operands here use the same K permutation (lane group q reads
// 16 consecutive K of a 64-wide chunk and splits them over two instructions),
// which leaves the contraction unchanged.
#include "moe_common.h"
#include "moe_kernels.h"

#include <atomic>
#include "route_dev.h"

namespace moe {

struct SlotView {
    const uint8_t* base;   // slot 0
    size_t stride;         // bytes per slot
    const uint8_t* fmt;    // device u8[n_slots]
    size_t off[2][4];      // part offsets per format
    int fmt_ok;            // bit f: format f fits the stride (usable_slot)
    int spec_fmt;          // a format that fits: loads issued before a slot's tag is known
};

__device__ __forceinline__ void fp8x16_to_bf16(const i32x4& v, bf16x8& s0, bf16x8& s1) {
    uint32_t a0, a1, a2, a3, b0, b1, b2, b3;
    e4m3x4_to_bf16x4((uint32_t)v[0], a0, a1);
    e4m3x4_to_bf16x4((uint32_t)v[1], a2, a3);
    e4m3x4_to_bf16x4((uint32_t)v[2], b0, b1);
    e4m3x4_to_bf16x4((uint32_t)v[3], b2, b3);
    i32x4 x0 = {(int)a0, (int)a1, (int)a2, (int)a3};
    i32x4 x1 = {(int)b0, (int)b1, (int)b2, (int)b3};
    s0 = __builtin_bit_cast(bf16x8, x0);
    s1 = __builtin_bit_cast(bf16x8, x1);
}

__device__ __forceinline__ uint32_t two_bf16(float a, float b) {
    return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

// 16 int4 values (8 bytes) -> q - zero as two bf16x8 operands. For the
// integer zero points the format stores, q - zero is a small integer, exact
// in fp32 and in bf16: the bf16 is the fp32's upper half, no rounding step
// (TRUNC; the rounding form is kept where the shorter sequence measured
// slower: it pushed the twelve-chunk down kernel into more register spills).
template <bool TRUNC = true>
__device__ __forceinline__ void int4x16_to_bf16(uint2 v, float zero, bf16x8& s0, bf16x8& s1) {
    const uint32_t w[2] = {v.x, v.y};
    uint32_t o[8];
#pragma unroll
    for (int d = 0; d < 2; ++d) {
        const uint32_t ev = w[d] & 0x0F0F0F0Fu;           // low nibbles (even elements) as bytes
        const uint32_t od = (w[d] >> 4) & 0x0F0F0F0Fu;    // high nibbles (odd elements)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float a = (float)((ev >> (8 * j)) & 0xFFu) - zero;
            const float b = (float)((od >> (8 * j)) & 0xFFu) - zero;
            o[d * 4 + j] = TRUNC ? __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u)
                                 : two_bf16(a, b);
        }
    }
    i32x4 x0 = {(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
    i32x4 x1 = {(int)o[4], (int)o[5], (int)o[6], (int)o[7]};
    s0 = __builtin_bit_cast(bf16x8, x0);
    s1 = __builtin_bit_cast(bf16x8, x1);
}

__device__ __forceinline__ void split_bf16(const i32x4& lo, const i32x4& hi, bf16x8& s0, bf16x8& s1) {
    s0 = __builtin_bit_cast(bf16x8, lo);
    s1 = __builtin_bit_cast(bf16x8, hi);
}

__device__ __forceinline__ float2 half2_at(const uint8_t* p) {
    const _Float16* h = (const _Float16*)p;
    return make_float2((float)h[0], (float)h[1]);
}

// Workgroup barrier that waits only for the wave's LDS traffic: the fence of
// __syncthreads() would also wait for every global load in flight.
__device__ __forceinline__ void barrier_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

constexpr int G_THREADS = 256;
constexpr int G_WAVES = 4;
constexpr int ROWS = 16;      // inter rows (gate and up each) per gemm1 unit
constexpr int G1_MAXG = 4;    // K groups per wave issued together
constexpr int G2_COLS = 64;   // hidden rows per gemm2 unit
constexpr int G2_MAXC = 8;    // 64-wide K chunks per wave issued together
constexpr int STREAM_MAX_T = 64;

// Unit ranges of the persistent decode kernels (grid G, even: two workgroups
// per CU). Workgroups b and b + G/2 split one contiguous range of
// ceil(n / (G/2)) units in halves, the first half to b, so every workgroup
// holds within one unit of every other (with ceil(n / G) units each, the
// grid's last workgroups were left with short or empty ranges).
__host__ __device__ inline int pair_units(int n, int G) { return (n + G / 2 - 1) / (G / 2); }
__host__ __device__ inline int max_units(int n, int G) { return (pair_units(n, G) + 1) / 2; }
__host__ __device__ inline void unit_range(int n, int G, int b, int& ub, int& ue) {
    const int h = G / 2, pp = pair_units(n, G);
    const int pb = min(n, (b < h ? b : b - h) * pp), pe = min(n, pb + pp);
    const int split = pb + (pe - pb + 1) / 2;
    ub = b < h ? pb : split;
    ue = b < h ? split : pe;
}


// ------------------------------------------------------------ gemm1
// One unit per workgroup. Round trip 1: n_padded, the block's slot and pair
// list, and the pool's format tags (into LDS). Round trip 2: every weight
// row chunk, token row chunk and row scale of the unit at once.
template <int BM>
__global__ void __launch_bounds__(G_THREADS) gemm1_stream_kernel(
    SlotView pool, int n_slots, const uint16_t* __restrict__ x, int NP, int k, const int32_t* __restrict__ sorted_pair,
    const int32_t* __restrict__ block_slot, const int32_t* __restrict__ n_padded, int H, int I,
    uint16_t* __restrict__ hbuf) {
    constexpr int NT = BM / 16;
    __shared__ f32x4 s_red[G_WAVES][NT][2][MOE_WAVE];
    __shared__ uint8_t s_fmt[MOE_MAX_SLOTS];
    const int lane = lane_id(), wv = threadIdx.x / MOE_WAVE;
    const int m = lane & 15, q = lane >> 4;
    const int ntile = I / ROWS;
    const int u = blockIdx.x;
    const int b = u / ntile, i0 = (u % ntile) * ROWS;
    const int groups = H / 128;
    // ---- round trip 1 (all inside the arrays: b < capacity / BM)
    const int npad = *n_padded;
    const int slot_in = block_slot[b];
    int pr[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) pr[nt] = sorted_pair[b * BM + nt * 16 + m];
    for (int i = threadIdx.x; i < n_slots; i += G_THREADS) s_fmt[i] = pool.fmt[i];
    __syncthreads();
    const int slot = usable_slot(slot_in, n_slots, pool.fmt_ok, s_fmt);
    if (b >= npad / BM || slot < 0) return;           // uniform over the workgroup
    const uint8_t* sb = pool.base + (size_t)slot * pool.stride;
    const int fmt = s_fmt[slot];
    const uint16_t* xr[NT];
    bool pv[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        pv[nt] = pr[nt] < NP;
        xr[nt] = x + (size_t)(pv[nt] ? pr[nt] / k : 0) * H;
    }
    f32x4 acc_g[NT], acc_u[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) { acc_g[nt] = f32x4{0, 0, 0, 0}; acc_u[nt] = f32x4{0, 0, 0, 0}; }
    f32x4 sg4 = {1, 1, 1, 1}, su4 = {1, 1, 1, 1};
    if (fmt == 0) {
        // ---- round trip 2
        const float* s13 = (const float*)(sb + pool.off[0][1]);
        sg4 = *(const f32x4*)(s13 + i0 + 4 * q);
        su4 = *(const f32x4*)(s13 + I + i0 + 4 * q);
        const uint8_t* wg = sb + (size_t)(i0 + m) * H;
        const uint8_t* wu = sb + (size_t)(I + i0 + m) * H;
        for (int g0 = wv; g0 < groups; g0 += G_WAVES * G1_MAXG) {
            i32x4 rg[G1_MAXG][2], ru[G1_MAXG][2], rx[G1_MAXG][2][NT][2];
#pragma unroll
            for (int j = 0; j < G1_MAXG; ++j) {
                const int g = g0 + j * G_WAVES;
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const int k0 = g * 128 + c * 64 + q * 16;
                    if (g < groups) {
                        rg[j][c] = *(const i32x4*)(wg + k0);
                        ru[j][c] = *(const i32x4*)(wu + k0);
                    }
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        if (g < groups && pv[nt]) {
                            rx[j][c][nt][0] = *(const i32x4*)(xr[nt] + k0);
                            rx[j][c][nt][1] = *(const i32x4*)(xr[nt] + k0 + 8);
                        } else {
                            rx[j][c][nt][0] = i32x4{0, 0, 0, 0};
                            rx[j][c][nt][1] = i32x4{0, 0, 0, 0};
                        }
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < G1_MAXG; ++j) {
                if (g0 + j * G_WAVES >= groups) break;   // uniform over the wave
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    bf16x8 ga0, ga1, ua0, ua1;
                    fp8x16_to_bf16(rg[j][c], ga0, ga1);
                    fp8x16_to_bf16(ru[j][c], ua0, ua1);
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        bf16x8 xb0, xb1;
                        split_bf16(rx[j][c][nt][0], rx[j][c][nt][1], xb0, xb1);
                        acc_g[nt] = mfma_bf16_16x16x32(ga0, xb0, acc_g[nt]);
                        acc_g[nt] = mfma_bf16_16x16x32(ga1, xb1, acc_g[nt]);
                        acc_u[nt] = mfma_bf16_16x16x32(ua0, xb0, acc_u[nt]);
                        acc_u[nt] = mfma_bf16_16x16x32(ua1, xb1, acc_u[nt]);
                    }
                }
            }
        }
    } else {
        const uint8_t* wg = sb + (size_t)(i0 + m) * (H / 2);
        const uint8_t* wu = sb + (size_t)(I + i0 + m) * (H / 2);
        const uint8_t* sz = sb + pool.off[1][1];
        for (int g = wv; g < groups; g += G_WAVES) {
            const float zg = half2_at(sz + ((size_t)(i0 + m) * groups + g) * 4).y;
            const float zu = half2_at(sz + ((size_t)(I + i0 + m) * groups + g) * 4).y;
            uint2 rg[2], ru[2];
            i32x4 rx[2][NT][2];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int k0 = g * 128 + c * 64 + q * 16;
                rg[c] = *(const uint2*)(wg + k0 / 2);
                ru[c] = *(const uint2*)(wu + k0 / 2);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    if (pv[nt]) {
                        rx[c][nt][0] = *(const i32x4*)(xr[nt] + k0);
                        rx[c][nt][1] = *(const i32x4*)(xr[nt] + k0 + 8);
                    } else {
                        rx[c][nt][0] = i32x4{0, 0, 0, 0};
                        rx[c][nt][1] = i32x4{0, 0, 0, 0};
                    }
                }
            }
            f32x4 tg[NT], tu[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) { tg[nt] = f32x4{0, 0, 0, 0}; tu[nt] = f32x4{0, 0, 0, 0}; }
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                bf16x8 ga0, ga1, ua0, ua1;
                int4x16_to_bf16(rg[c], zg, ga0, ga1);
                int4x16_to_bf16(ru[c], zu, ua0, ua1);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    bf16x8 xb0, xb1;
                    split_bf16(rx[c][nt][0], rx[c][nt][1], xb0, xb1);
                    tg[nt] = mfma_bf16_16x16x32(ga0, xb0, tg[nt]);
                    tg[nt] = mfma_bf16_16x16x32(ga1, xb1, tg[nt]);
                    tu[nt] = mfma_bf16_16x16x32(ua0, xb0, tu[nt]);
                    tu[nt] = mfma_bf16_16x16x32(ua1, xb1, tu[nt]);
                }
            }
            // group scales of the output rows this lane holds (rows 4q..4q+3)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float sg = half2_at(sz + ((size_t)(i0 + 4 * q + i) * groups + g) * 4).x;
                const float su = half2_at(sz + ((size_t)(I + i0 + 4 * q + i) * groups + g) * 4).x;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    acc_g[nt][i] += sg * tg[nt][i];
                    acc_u[nt][i] += su * tu[nt][i];
                }
            }
        }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) { s_red[wv][nt][0][lane] = acc_g[nt]; s_red[wv][nt][1][lane] = acc_u[nt]; }
    __syncthreads();
    if (wv < NT) {                       // wave wv finishes pair tile nt = wv
        const int nt = wv;
        f32x4 g = s_red[0][nt][0][lane], up = s_red[0][nt][1][lane];
#pragma unroll
        for (int w2 = 1; w2 < G_WAVES; ++w2) {
            g += s_red[w2][nt][0][lane];
            up += s_red[w2][nt][1][lane];
        }
        if (pr[nt] < NP) {
            float hv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) hv[i] = silu(g[i] * sg4[i]) * (up[i] * su4[i]);
            *(uint2*)(hbuf + (size_t)(b * BM + nt * 16 + m) * I + i0 + 4 * q) =
                make_uint2(two_bf16(hv[0], hv[1]), two_bf16(hv[2], hv[3]));
        }
    }
}

// ------------------------------------------------------------ gemm1, pipelined
// Persistent gate/up kernel for 16-pair blocks (decode batches).
// * Unit = (block, 8 inter rows): the 16 rows of the matrix-core A tile are
//   8 gate rows and the 8 matching up rows, so one tile yields both halves of
//   silu(gate) * up (swapped between lanes l and l ^ 32 in the epilogue).
// * Each workgroup walks a contiguous range of units, i.e. consecutive 8-row
//   slices of one expert's w13 at a time; the token rows of a block are
//   loaded once per block and kept in registers.
// * While the matrix cores work on unit i, the weight rows and row scales of
//   unit i+1 are in flight (two register sets alternated by a two-step loop
//   body). Loads complete in issue order: each step issues the block's token
//   rows (when the block changes), then unit i+1's weights, then waits for
//   what it needs, which leaves unit i+1's weights in flight.
// int4 units are computed without prefetch.
constexpr int P1_G = 4;          // 128-wide K groups per wave (hidden <= 2048)
constexpr int P1_ROWS = 8;       // inter rows per unit (gate and up each)
constexpr int P1_MAXB = 16;      // blocks per workgroup range the LDS tables hold

// A unit's weights in registers, in one of two layouts (nine 16-byte loads
// either way, with no branch between them, so the compiler's count of loads
// in flight stays exact):
// * FP8 slot: r[2 j + c] = 16 codes of this lane's row, K group g = wv + 4 j,
//   bytes [g 128 + c 64 + q 16, +16); r[8] = fp32 row scales of the C rows
//   4q..4q+3.
// * int4 slot: r[j] = 32 nibbles of this lane's row, K group g = 4 wv + j,
//   elements [g 128 + q 32, +32); r[4] = (scale, zero) of the row for groups
//   4 wv .. 4 wv + 3; r[5], r[6], r[7], r[8] = the same for the C rows
//   4q .. 4q + 3 this lane accumulates (their scales, with no lane exchange).
// The token rows of a block are loaded in the matching K order (p1_issue_x).
struct P1W { i32x4 r[9]; };
struct P1X { i32x4 v[P1_G][2][2]; };         // [group][chunk][half] of this lane's token row

// An empty use of a register set: the compiler waits for its loads here.
__device__ __forceinline__ void p1_landed(const P1W& W) {
#pragma unroll
    for (int i = 0; i < 9; ++i) asm volatile("" ::"v"(W.r[i]));
}

// A-tile row of lane m: gate row i0 + m (m < 8) or up row I + i0 + m - 8
__device__ __forceinline__ int p1_row(int i0, int m, int I) { return m < 8 ? i0 + m : I + i0 + m - 8; }

__device__ __forceinline__ void p1_issue_w(P1W& W, const SlotView& pool, int slot, int fmt, int i0, int m, int q,
                                           int wv, int H, int I, int groups) {
    const uint8_t* sb = pool.base + (size_t)slot * pool.stride;
    const int row = p1_row(i0, m, I);
    // FP8 sources (groups past the row repeat its last group, unused)
    const uint8_t* wr8 = sb + (size_t)row * H;
    const uint8_t* sc8 = sb + pool.off[0][1] + 4 * (q < 2 ? i0 + 4 * q : I + i0 + 4 * (q - 2));
    // int4 sources
    const uint8_t* wr4 = sb + pool.off[1][0] + (size_t)row * (H / 2) + q * 16;
    const uint8_t* szb = sb + pool.off[1][1] + (size_t)min(4 * wv, groups - 1) * 4;
    const uint8_t* sz4 = szb + (size_t)row * groups * 4;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int j = i >> 1, c = i & 1;
        const uint8_t* p8 = wr8 + min(wv + j * G_WAVES, groups - 1) * 128 + c * 64 + q * 16;
        const uint8_t* p4 = i < 4 ? wr4 + min(4 * wv + i, groups - 1) * 64
                          : (i == 4 ? sz4 : szb + (size_t)p1_row(i0, 4 * q + i - 5, I) * groups * 4);
        W.r[i] = *(const i32x4*)(fmt ? p4 : p8);
    }
    W.r[8] = *(const i32x4*)(fmt ? szb + (size_t)p1_row(i0, 4 * q + 3, I) * groups * 4 : sc8);
}

// Token row of this lane (row 0 for a padding lane: its output column is
// never stored) in the K order of the block's weight layout; no branches.
__device__ __forceinline__ void p1_issue_x(P1X& X, const uint16_t* xr, int fmt, int q, int wv, int groups) {
#pragma unroll
    for (int j = 0; j < P1_G; ++j) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int k8 = min(wv + j * G_WAVES, groups - 1) * 128 + c * 64 + q * 16;
            const int k4 = min(4 * wv + j, groups - 1) * 128 + q * 32 + c * 16;
            const int k0 = fmt ? k4 : k8;
            X.v[j][c][0] = *(const i32x4*)(xr + k0);
            X.v[j][c][1] = *(const i32x4*)(xr + k0 + 8);
        }
    }
}

__device__ __forceinline__ f32x4 p1_mma(const P1W& W, const P1X& X, int wv, int groups) {
    f32x4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < P1_G; ++j) {
        if (wv + j * G_WAVES >= groups) break;        // uniform over the wave
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            bf16x8 a0, a1, xb0, xb1;
            fp8x16_to_bf16(W.r[2 * j + c], a0, a1);
            split_bf16(X.v[j][c][0], X.v[j][c][1], xb0, xb1);
            acc = mfma_bf16_16x16x32(a0, xb0, acc);
            acc = mfma_bf16_16x16x32(a1, xb1, acc);
        }
    }
    return acc * __builtin_bit_cast(f32x4, W.r[8]);
}

// int4 unit: (q - z) exactly in bf16 before the matrix instructions, each
// group's scale after them; the scales of C rows 4q..4q+3 come from the
// lanes that loaded those rows.
__device__ __forceinline__ f32x4 p1_int4_mma(const P1W& W, const P1X& X, int q, int wv, int groups) {
    f32x4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < P1_G; ++j) {
        if (4 * wv + j >= groups) break;              // uniform over the wave
        const uint32_t sz = (uint32_t)W.r[4][j];      // (scale, zero) of this lane's row, group 4 wv + j
        const float z = (float)__builtin_bit_cast(_Float16, (uint16_t)(sz >> 16));
        f32x4 t4 = {0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            bf16x8 a0, a1, xb0, xb1;
            int4x16_to_bf16(make_uint2((uint32_t)W.r[j][2 * c], (uint32_t)W.r[j][2 * c + 1]), z, a0, a1);
            split_bf16(X.v[j][c][0], X.v[j][c][1], xb0, xb1);
            t4 = mfma_bf16_16x16x32(a0, xb0, t4);
            t4 = mfma_bf16_16x16x32(a1, xb1, t4);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t szr = (uint32_t)(i < 3 ? W.r[5 + i][j] : W.r[8][j]);   // C row 4q + i, group 4 wv + j
            acc[i] += (float)__builtin_bit_cast(_Float16, (uint16_t)(szr & 0xFFFFu)) * t4[i];
        }
    }
    return acc;
}

// ------------------------------------------------------------ layer prologue
// Decode-sized layers (T <= 64 tokens, 16-pair blocks) skip the separate
// align launch (and, for the smallest batches, the route launch): every
// workgroup of the gate/up kernel sorts the T*k pairs itself, in LDS, from the
// route results, so its tables are ready one LDS pass after the ids arrive.
// The sort is the align call's: MOE-GEN explainer (aibr.jp), sections 1 and
// 3 (pairs grouped per expert, ascending expert id, ascending pair index
// inside a segment, each segment padded to the block with the sentinel T*k);
// vllm-expert-pager article (rand.pepabo.com), "hierarchical paging of expert
// weights" (block -> slot through the layer's table). A pair's position in its
// segment is the number of earlier tokens that chose the same expert, read off
// a per-expert 64-bit token mask (a token lists an expert at most once: the
// router picks distinct experts). Workgroup 0 writes everything the route and
// align calls would have written, for the down and combine kernels and the
// caller; the other workgroups keep only their own blocks' tables.
constexpr int LAYER_MAX_T = 64;
constexpr int LAYER_MAX_NP = 512;
// Route inside the gate/up kernel up to this many tokens and 512 experts (one
// wavefront per token, every workgroup routes them all); otherwise the route
// kernel runs first and the gate/up kernel only sorts the pairs.
constexpr int LAYER_ROUTE_MAX_T = 16;
constexpr int LAYER_EPT = MOE_MAX_E / G_THREADS;     // experts per thread

struct LayerIO {
    const float* logits;            // route inline when not null
    const uint8_t* mask;
    const int32_t* slot_of_expert;
    int E;
    int32_t* ids;                   // read (route done before) or written by workgroup 0
    float* w;                       // written by workgroup 0 when routing inline
    int32_t* sorted_pair;           // outputs of workgroup 0
    int32_t* block_slot;
    int32_t* counts;
    int32_t* seg_offset;
    int32_t* n_padded;
    int32_t* err;                   // [0] route, [1] align
    int4* gdesc;                    // written by workgroup 0 for the down kernel's grid2 workgroups:
    int grid2;                      //   (first unit, end unit, first slot, its format)
    int H;
};

struct P1Range { int u_begin, u_end, b_first, nblk; };

template <int RVPL, int RT>
__device__ __forceinline__ P1Range layer_prologue(const LayerIO& L, const uint8_t* __restrict__ fmt, int n_slots,
                                                  int fmt_ok, int spec_fmt, int T, int k, int ntile, uint8_t* s_fmt,
                                                  int* s_slot, int (*s_pr)[16]) {
    __shared__ unsigned long long s_tok[MOE_MAX_E];  // bit t: token t chose the expert
    __shared__ int s_cnt[MOE_MAX_E];
    __shared__ int s_off[MOE_MAX_E];
    __shared__ int s_ids[LAYER_MAX_NP];
    __shared__ int s_sl[MOE_MAX_E];                   // slot of each expert
    __shared__ int s_wsum[G_WAVES];
    const int tid = threadIdx.x, lane = lane_id(), wv = tid / MOE_WAVE;
    const int NP = T * k, E = L.E;
    // the tables this call hands on, each written by one workgroup (different
    // XCDs): counts and offsets, block slots, padding sentinels, down-kernel
    // descriptors, sorted pairs, route results
    const int G = gridDim.x;
    const bool w_tab = blockIdx.x == 0, w_blk = blockIdx.x == 1 % G, w_pad = blockIdx.x == 2 % G;
    const bool w_desc = blockIdx.x == 3 % G, w_pair = blockIdx.x == 4 % G, w_ids = blockIdx.x == 5 % G;
    // ---- every global load first (one round trip): slot table, format
    // tags, and the route ids or the logits of this wavefront's RT tokens.
    // Each load instruction holds its wave for a while as it issues, so only
    // the loads the shape needs are issued.
    int slot_e[LAYER_EPT];
#pragma unroll
    for (int i = 0; i < LAYER_EPT; ++i) {
        const int e = tid * LAYER_EPT + i;
        slot_e[i] = e < E ? L.slot_of_expert[e] : -1;
    }
    // (an int, not a byte: bytes packed into one register made the compiler
    // wait for each load before issuing the next)
    const int fv0 = fmt[min(tid, n_slots - 1)];
    int pid[2];
    float lg[RT][RVPL == 0 ? 1 : RVPL];
    int mk[RVPL == 0 ? 1 : RVPL];
    if constexpr (RVPL == 0) {
#pragma unroll
        for (int j = 0; j < 2; ++j) pid[j] = tid + j * G_THREADS < NP ? L.ids[tid + j * G_THREADS] : -1;
    } else {
#pragma unroll
        for (int j = 0; j < RT; ++j) {
            const float* row = L.logits + (size_t)min(wv + j * G_WAVES, T - 1) * E;
#pragma unroll
            for (int i = 0; i < RVPL; ++i) lg[j][i] = row[min(i * MOE_WAVE + lane, E - 1)];
        }
#pragma unroll
        for (int i = 0; i < RVPL; ++i) mk[i] = 1;
        if (L.mask) {
#pragma unroll
            for (int i = 0; i < RVPL; ++i) mk[i] = L.mask[min(i * MOE_WAVE + lane, E - 1)];
        }
    }
    // ---- LDS set-up
#pragma unroll
    for (int i = 0; i < LAYER_EPT; ++i) {
        const int e = tid * LAYER_EPT + i;
        if (e < E) {
            s_tok[e] = 0ull;
            s_cnt[e] = 0;
        }
    }
    if (tid < n_slots) s_fmt[tid] = (uint8_t)fv0;
    for (int i = tid + G_THREADS; i < n_slots; i += G_THREADS) s_fmt[i] = fmt[i];   // pools over 256 slots
    if constexpr (RVPL != 0) {
        // the wavefront's RT tokens (wv + 4 j) selected together; a token
        // past T has no keys and gains no choices
        uint32_t key[RT][RVPL];
#pragma unroll
        for (int j = 0; j < RT; ++j)
#pragma unroll
            for (int i = 0; i < RVPL; ++i)
                key[j][i] = (wv + j * G_WAVES < T && i * MOE_WAVE + lane < E && mk[i] != 0) ? route_ord(lg[j][i]) : 0u;
        int id[RT], found[RT];
        float wt[RT];
        route_select_multi<RVPL, RT>(key, k, id, wt, found);
#pragma unroll
        for (int j = 0; j < RT; ++j) {
            const int t = wv + j * G_WAVES;
            if (t >= T) break;                       // uniform over the wave
            if (lane < k) {
                s_ids[t * k + lane] = id[j];
                if (w_ids) {
                    L.ids[t * k + lane] = id[j];
                    L.w[t * k + lane] = wt[j];
                }
            }
            if (w_ids && lane == 0 && found[j] < k) atomicAdd(&L.err[0], 1);
        }
    }
    // (the prologue's barriers wait for LDS only: nothing here reads back the
    // tables handed on, so their stores stay in flight)
    barrier_lds();
    // the format tags are in LDS: a slot outside the pool or with a format
    // that does not fit the stride counts as not resident
#pragma unroll
    for (int i = 0; i < LAYER_EPT; ++i) {
        const int e = tid * LAYER_EPT + i;
        slot_e[i] = usable_slot(slot_e[i], n_slots, fmt_ok, s_fmt);
        if (e < E) s_sl[e] = slot_e[i];
    }
    if constexpr (RVPL != 0) {
#pragma unroll
        for (int j = 0; j < 2; ++j) pid[j] = tid + j * G_THREADS < NP ? s_ids[tid + j * G_THREADS] : -1;
    }
    int bad = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int p = tid + j * G_THREADS, e = pid[j];
        if (p >= NP) continue;
        if (e >= 0 && e < E) {
            atomicOr(&s_tok[e], 1ull << (p / k));
            atomicAdd(&s_cnt[e], 1);
        } else {
            ++bad;
        }
    }
    barrier_lds();
    // padded counts of this thread's experts, then their exclusive scan
    int c[LAYER_EPT], off[LAYER_EPT], sum = 0;
#pragma unroll
    for (int i = 0; i < LAYER_EPT; ++i) {
        const int e = tid * LAYER_EPT + i;
        c[i] = e < E ? s_cnt[e] : 0;
        off[i] = sum;
        sum += (c[i] + 15) & ~15;
        if (slot_e[i] < 0) bad += c[i];             // pairs routed to a non-resident expert
    }
    int incl = sum;
#pragma unroll
    for (int o = 1; o < MOE_WAVE; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
    }
    if (lane == MOE_WAVE - 1) s_wsum[wv] = incl;
    barrier_lds();
    int base = incl - sum, total = 0;
#pragma unroll
    for (int w2 = 0; w2 < G_WAVES; ++w2) {
        const int ws = s_wsum[w2];
        base += w2 < wv ? ws : 0;
        total += ws;
    }
#pragma unroll
    for (int i = 0; i < LAYER_EPT; ++i) {
        const int e = tid * LAYER_EPT + i;
        off[i] += base;
        if (e < E) s_off[e] = off[i];
    }
    if (w_tab || w_blk) {
#pragma unroll
        for (int i = 0; i < LAYER_EPT; ++i) {
            const int e = tid * LAYER_EPT + i;
            if (e >= E) continue;
            const int pad = (c[i] + 15) & ~15;
            if (w_tab) {
                L.counts[e] = c[i];
                L.seg_offset[e] = off[i];
            }
            if (w_blk)
                for (int b = off[i] / 16; b < (off[i] + pad) / 16; ++b) L.block_slot[b] = slot_e[i];
        }
    }
    if (w_tab) {
        if (tid == 0) {
            L.seg_offset[E] = total;
            *L.n_padded = total;
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) bad += __shfl_xor(bad, o, 64);
        if (lane == 0 && bad) atomicAdd(&L.err[1], bad);
    }
    // this workgroup's unit range and its blocks' tables
    P1Range R;
    const int n_units = (total / 16) * ntile;
    unit_range(n_units, gridDim.x, blockIdx.x, R.u_begin, R.u_end);
    R.b_first = R.u_begin / ntile;
    R.nblk = R.u_begin < R.u_end ? (R.u_end - 1) / ntile - R.b_first + 1 : 0;
    for (int i = tid; i < R.nblk * 16; i += G_THREADS) s_pr[i / 16][i % 16] = NP;
#pragma unroll
    for (int i = 0; i < LAYER_EPT; ++i) {
        const int b0 = max(off[i] / 16, R.b_first);
        const int b1 = min((off[i] + ((c[i] + 15) & ~15)) / 16, R.b_first + R.nblk);
        for (int b = b0; b < b1; ++b) s_slot[b - R.b_first] = slot_e[i];
    }
    barrier_lds();                                   // sentinels before the pairs
    if (w_pad) {
        // padding sentinels: the tail of each expert's last block, 16 lanes
        // per expert (one line per store instead of a lane per expert)
        const int j = tid & 15;
#pragma unroll 4
        for (int e = tid >> 4; e < E; e += G_THREADS / 16) {
            const int ce = s_cnt[e], oe = s_off[e];
            const int q = oe + ((ce + 15) & ~15) - 16 + j;
            if (q >= oe + ce) L.sorted_pair[q] = NP;
        }
    }
    if (w_desc && L.gdesc) {
        // the down kernel's unit ranges (its units: block x 64 hidden rows)
        // with the slot and format of each range's first block, so that it
        // loads its first weights without waiting for these tables
        const int ntile2 = L.H / 64;
        const int n_units2 = (total / 16) * ntile2;
        for (int g = tid; g < L.grid2; g += G_THREADS) {
            int ub, ue;
            unit_range(n_units2, L.grid2, g, ub, ue);
            int slot = -1, f = 0;
            if (ub < ue) {
                const int pos = (ub / ntile2) * 16;
                int lo = 0, hi = E - 1;                // last expert whose segment starts at or before pos
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (s_off[mid] <= pos) lo = mid;
                    else hi = mid - 1;
                }
                slot = s_sl[lo];
            }
            f = slot >= 0 ? (int)s_fmt[slot] : spec_fmt;   // (slot -1: the down kernel loads slot 0 in this format)
            L.gdesc[g] = make_int4(ub, ue, slot, f);
        }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int p = tid + j * G_THREADS, e = pid[j];
        if (p >= NP || e < 0 || e >= E) continue;
        const int t = p / k;
        const int pos = s_off[e] + (int)__popcll(s_tok[e] & ((1ull << t) - 1ull));
        if (w_pair) L.sorted_pair[pos] = p;
        const int bb = pos / 16 - R.b_first;
        if (bb >= 0 && bb < R.nblk) s_pr[bb][pos % 16] = p;
    }
    return R;
}

// FUSE 0: the block tables come from a separate align launch. FUSE 1: the
// pairs are sorted here from the route results (layer_prologue). FUSE 2: the
// tokens are routed here too (route_select<RVPL>).
// FUSE 0 and 1 run one workgroup per CU with the weights of the unit two
// ahead in flight (three register sets): one set-up per CU instead of two,
// and one unit stream per CU, which ends evenly (two workgroups per CU each
// sorted the pairs, the second one's set-up took twice as long, and it ended
// several microseconds after the first). FUSE 2, whose set-up routes the
// tokens, keeps two workgroups per CU and one unit of prefetch.
constexpr int gemm1_pipe_wgs_per_cu(int fuse) { return fuse == 2 ? 2 : 1; }

template <int FUSE, int RVPL, int RT>
__global__ void __launch_bounds__(G_THREADS, gemm1_pipe_wgs_per_cu(FUSE)) gemm1_pipe_kernel(
    SlotView pool, int n_slots, const uint16_t* __restrict__ x, int T, int k,
    const int32_t* __restrict__ sorted_pair, const int32_t* __restrict__ block_slot,
    const int32_t* __restrict__ n_padded, int H, int I, uint16_t* __restrict__ hbuf, LayerIO L) {
    __shared__ f32x4 s_red[2][G_WAVES][MOE_WAVE];     // unit u uses half u % 2
    __shared__ uint8_t s_fmt[MOE_MAX_SLOTS];
    __shared__ int s_slot[P1_MAXB];
    __shared__ int s_pr[P1_MAXB][16];
    const int lane = lane_id(), wv = threadIdx.x / MOE_WAVE;
    const int m = lane & 15, q = lane >> 4;
    const int ntile = I / P1_ROWS;
    const int groups = H / 128;
    const int NP = T * k;
    constexpr int PF = gemm1_pipe_wgs_per_cu(FUSE) == 1 ? 2 : 1;   // units of prefetch
    P1W WA, WB, WC;
    P1X X;
    int xblock = -1;
    int u_begin, u_end, b_first, nblk;
    // a block's slot if usable, else -1 (not resident, outside the pool, or a
    // format that does not fit the stride)
    auto ok = [&](int slot) { return usable_slot(slot, n_slots, pool.fmt_ok, s_fmt); };
    // slot and format to load for a table entry: an unusable entry loads slot
    // 0 in a format that fits the stride (its unit ignores the values)
    auto pf_slot = [&](int slot) { return max(ok(slot), 0); };
    auto pf_fmt = [&](int slot) { const int s = ok(slot); return s >= 0 ? (int)s_fmt[s] : pool.spec_fmt; };
    if constexpr (FUSE == 0) {
        const int n_units = (*n_padded / 16) * ntile;
        unit_range(n_units, gridDim.x, blockIdx.x, u_begin, u_end);
        b_first = u_begin / ntile;
        nblk = u_begin < u_end ? (u_end - 1) / ntile - b_first + 1 : 0;
        if (nblk == 0) return;
        // ---- the descriptors of my blocks and the format tags, and the first
        // unit's weights, in one round trip. Loads complete in issue order, so
        // the descriptor loads go first; the weights are loaded before the
        // slot's format is known, from the table entry clamped into the pool
        // and in a format whose layout fits the stride (so every load stays
        // inside the pool), and loaded again if the slot's format differs.
        const int i0f = threadIdx.x;
        const int bb0 = i0f / 17, r0 = i0f % 17;
        uint8_t f0 = 0;
        int d0 = 0;
        if (i0f < n_slots) f0 = pool.fmt[i0f];
        if (i0f < nblk * 17) d0 = r0 == 16 ? block_slot[b_first + bb0] : sorted_pair[(b_first + bb0) * 16 + r0];
        __builtin_amdgcn_sched_barrier(0);          // keep the descriptor loads ahead of the weights
        p1_issue_w(WA, pool, min(max(block_slot[b_first], 0), n_slots - 1), pool.spec_fmt, (u_begin % ntile) * P1_ROWS,
                   m, q, wv, H, I, groups);
        __builtin_amdgcn_sched_barrier(0);
        if (i0f < n_slots) s_fmt[i0f] = f0;
        if (i0f < nblk * 17) {
            if (r0 == 16) s_slot[bb0] = d0;
            else s_pr[bb0][r0] = d0;
        }
        for (int i = i0f + G_THREADS; i < n_slots; i += G_THREADS) s_fmt[i] = pool.fmt[i];
        for (int i = i0f + G_THREADS; i < nblk * 17; i += G_THREADS) {
            const int bb = i / 17, r = i % 17;
            if (r == 16) s_slot[bb] = block_slot[b_first + bb];
            else s_pr[bb][r] = sorted_pair[(b_first + bb) * 16 + r];
        }
        barrier_lds();                               // tables written; the weight loads stay in flight
        const int s0 = ok(s_slot[0]);
        if (s0 >= 0 && s_fmt[s0] != pool.spec_fmt) {  // the first unit's format differs: load it in its own layout
            p1_landed(WA);
            p1_issue_w(WA, pool, s0, s_fmt[s0], (u_begin % ntile) * P1_ROWS, m, q, wv, H, I, groups);
        }
        if constexpr (PF == 2) {
            const int u1 = min(u_begin + 1, u_end - 1), s1 = s_slot[u1 / ntile - b_first];
            p1_issue_w(WB, pool, pf_slot(s1), pf_fmt(s1), (u1 % ntile) * P1_ROWS, m, q, wv, H, I, groups);
        }
    } else {
        const P1Range R = layer_prologue<RVPL, RT>(L, pool.fmt, n_slots, pool.fmt_ok, pool.spec_fmt, T, k, ntile, s_fmt,
                                                   s_slot, s_pr);
        u_begin = R.u_begin;
        u_end = R.u_end;
        b_first = R.b_first;
        nblk = R.nblk;
        if (nblk == 0) return;                       // uniform over the workgroup
        barrier_lds();
        p1_issue_w(WA, pool, pf_slot(s_slot[0]), pf_fmt(s_slot[0]), (u_begin % ntile) * P1_ROWS, m, q, wv, H, I,
                   groups);
        if constexpr (PF == 2) {
            const int u1 = min(u_begin + 1, u_end - 1), s1 = s_slot[u1 / ntile - b_first];
            p1_issue_w(WB, pool, pf_slot(s1), pf_fmt(s1), (u1 % ntile) * P1_ROWS, m, q, wv, H, I, groups);
        }
    }
    auto step = [&](int u, P1W& Wc, P1W& Wn) {
        const int bb = u / ntile - b_first;
        const int i0 = (u % ntile) * P1_ROWS;
        const int slot = ok(s_slot[bb]);
        const int fmt = slot >= 0 ? (int)s_fmt[slot] : 0;
        const int pr = s_pr[bb][m];
        const bool valid = pr < NP;
        if (slot >= 0 && bb != xblock) {              // new block: its token rows, before the prefetch
            p1_issue_x(X, x + (size_t)(valid ? pr / k : 0) * H, fmt, q, wv, groups);
            xblock = bb;
        }
        {
            // the weights of unit u + PF (slot 0 for an unusable slot, whose
            // unit ignores them; past the range: the last unit again)
            const int un = min(u + PF, u_end - 1);
            const int sn = s_slot[un / ntile - b_first];
            p1_issue_w(Wn, pool, pf_slot(sn), pf_fmt(sn), (un % ntile) * P1_ROWS, m, q, wv, H, I, groups);
        }
        // every path waits here for this unit's weight loads, so no load into
        // a register set is still pending when the set is refilled
        p1_landed(Wc);
        if (slot < 0) return;                          // uniform over the workgroup
        f32x4 acc;
        if (fmt == 0) acc = p1_mma(Wc, X, wv, groups);
        else acc = p1_int4_mma(Wc, X, q, wv, groups);
        s_red[u & 1][wv][lane] = acc;
        barrier_lds();
        if (wv == 0) {
            f32x4 v = s_red[u & 1][0][lane];
#pragma unroll
            for (int w2 = 1; w2 < G_WAVES; ++w2) v += s_red[u & 1][w2][lane];
            // lanes q = 0, 1 hold gate rows, q = 2, 3 the up rows of the same inter index
            f32x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = __shfl_xor(v[i], 32, 64);
            if (valid && q < 2) {
                float hv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) hv[i] = silu(v[i]) * o[i];
                *(uint2*)(hbuf + (size_t)((b_first + bb) * 16 + m) * I + i0 + 4 * q) =
                    make_uint2(two_bf16(hv[0], hv[1]), two_bf16(hv[2], hv[3]));
            }
        }
        // no barrier here: unit u+1 writes the other half of s_red, and unit
        // u+2 writes this half only after the barrier of unit u+1, which wave
        // 0 reaches after its reads above
    };
    // pairs of units, then an odd last one after the loop: a path that ran
    // one step and returned to the loop head would leave the other register
    // set's loads pending there, and the compiler would then wait for every
    // load in flight at the head of each iteration (the prefetch included)
    int u = u_begin;
    if constexpr (PF == 2) {                          // three register sets in turn
        for (; u + 2 < u_end; u += 3) {
            step(u, WA, WC);
            step(u + 1, WB, WA);
            step(u + 2, WC, WB);
        }
        if (u < u_end) step(u, WA, WC);
        if (u + 1 < u_end) step(u + 1, WB, WA);
    } else {
        for (; u + 1 < u_end; u += 2) {
            step(u, WA, WB);
            step(u + 1, WB, WA);
        }
        if (u < u_end) step(u, WA, WB);
    }
}

// ------------------------------------------------------------ gemm2
// One unit per workgroup: (block, 64 hidden rows); wave w owns 16 rows.
// Round trip 1 as in gemm1; round trip 2: W2 row chunks, h rows of the
// block's valid pairs, row scales and route weights.
template <int BM>
__global__ void __launch_bounds__(G_THREADS) gemm2_stream_kernel(
    SlotView pool, int n_slots, int NP, int k, const float* __restrict__ topk_w,
    const int32_t* __restrict__ sorted_pair, const int32_t* __restrict__ block_slot,
    const int32_t* __restrict__ n_padded, int H, int I, const uint16_t* __restrict__ hbuf, float* __restrict__ ybuf) {
    constexpr int NT = BM / 16;
    __shared__ uint8_t s_fmt[MOE_MAX_SLOTS];
    const int lane = lane_id(), wv = threadIdx.x / MOE_WAVE;
    const int m = lane & 15, q = lane >> 4;
    const int ntile = H / G2_COLS;
    const int u = blockIdx.x;
    const int b = u / ntile;
    const int n0 = (u % ntile) * G2_COLS + wv * 16;   // this wave's 16 rows
    const int chunks = I / 64;
    const int groups = I / MOE_INT4_G;
    // ---- round trip 1
    const int npad = *n_padded;
    const int slot_in = block_slot[b];
    int pr[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) pr[nt] = sorted_pair[b * BM + nt * 16 + m];
    for (int i = threadIdx.x; i < n_slots; i += G_THREADS) s_fmt[i] = pool.fmt[i];
    __syncthreads();
    if (b >= npad / BM) return;                       // uniform over the workgroup
    const int slot = usable_slot(slot_in, n_slots, pool.fmt_ok, s_fmt);
    bool pv[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) pv[nt] = pr[nt] < NP;
    if (slot < 0) {                                   // non-resident expert: its pairs add zero
        if (slot_in == MOE_SLOT_DEFERRED) return;     // (a deferred block's rows are left as they are)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            if (pv[nt]) *(f32x4*)(ybuf + (size_t)pr[nt] * H + n0 + 4 * q) = f32x4{0, 0, 0, 0};
        return;
    }
    const uint8_t* sb = pool.base + (size_t)slot * pool.stride;
    const int fmt = s_fmt[slot];
    float wt[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) wt[nt] = pv[nt] ? topk_w[pr[nt]] : 0.f;
    f32x4 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0, 0, 0, 0};
    if (fmt == 0) {
        const f32x4 s2 = *(const f32x4*)((const float*)(sb + pool.off[0][3]) + n0 + 4 * q);
        const uint8_t* wr = sb + pool.off[0][2] + (size_t)(n0 + m) * I;
        for (int c0 = 0; c0 < chunks; c0 += G2_MAXC) {
            i32x4 rw[G2_MAXC], rh[G2_MAXC][NT][2];
#pragma unroll
            for (int j = 0; j < G2_MAXC; ++j) {
                const int c = c0 + j;
                const int k0 = c * 64 + q * 16;
                if (c < chunks) rw[j] = *(const i32x4*)(wr + k0);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const uint16_t* hr = hbuf + (size_t)(b * BM + nt * 16 + m) * I;
                    if (c < chunks && pv[nt]) {
                        rh[j][nt][0] = *(const i32x4*)(hr + k0);
                        rh[j][nt][1] = *(const i32x4*)(hr + k0 + 8);
                    } else {
                        rh[j][nt][0] = i32x4{0, 0, 0, 0};
                        rh[j][nt][1] = i32x4{0, 0, 0, 0};
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < G2_MAXC; ++j) {
                if (c0 + j >= chunks) break;             // uniform over the wave
                bf16x8 a0, a1;
                fp8x16_to_bf16(rw[j], a0, a1);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    bf16x8 h0, h1;
                    split_bf16(rh[j][nt][0], rh[j][nt][1], h0, h1);
                    acc[nt] = mfma_bf16_16x16x32(a0, h0, acc[nt]);
                    acc[nt] = mfma_bf16_16x16x32(a1, h1, acc[nt]);
                }
            }
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt] *= s2;
    } else {
        const uint8_t* wr = sb + pool.off[1][2] + (size_t)(n0 + m) * (I / 2);
        const uint8_t* sz = sb + pool.off[1][3];
        for (int g = 0; g < groups; ++g) {
            const float z = half2_at(sz + ((size_t)(n0 + m) * groups + g) * 4).y;
            uint2 rw[2];
            i32x4 rh[2][NT][2];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int k0 = g * 128 + c * 64 + q * 16;
                rw[c] = *(const uint2*)(wr + k0 / 2);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const uint16_t* hr = hbuf + (size_t)(b * BM + nt * 16 + m) * I;
                    if (pv[nt]) {
                        rh[c][nt][0] = *(const i32x4*)(hr + k0);
                        rh[c][nt][1] = *(const i32x4*)(hr + k0 + 8);
                    } else {
                        rh[c][nt][0] = i32x4{0, 0, 0, 0};
                        rh[c][nt][1] = i32x4{0, 0, 0, 0};
                    }
                }
            }
            f32x4 t4[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) t4[nt] = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                bf16x8 a0, a1;
                int4x16_to_bf16(rw[c], z, a0, a1);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    bf16x8 h0, h1;
                    split_bf16(rh[c][nt][0], rh[c][nt][1], h0, h1);
                    t4[nt] = mfma_bf16_16x16x32(a0, h0, t4[nt]);
                    t4[nt] = mfma_bf16_16x16x32(a1, h1, t4[nt]);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float s = half2_at(sz + ((size_t)(n0 + 4 * q + i) * groups + g) * 4).x;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) acc[nt][i] += s * t4[nt][i];
            }
        }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
        if (pv[nt]) *(f32x4*)(ybuf + (size_t)pr[nt] * H + n0 + 4 * q) = acc[nt] * wt[nt];
}

// ------------------------------------------------------------ gemm2, pipelined
// Persistent down-projection kernel for 16-pair blocks, built like the
// pipelined gemm1: contiguous unit ranges per workgroup (unit = block x 64
// hidden rows, wave w owns 16 of them), the block's h rows loaded once per
// block and kept in registers, the next unit's W2 rows and scales in flight
// while the current one is multiplied. int4 units run without prefetch.
constexpr int P2_MAXB = 16;

// C = 64-wide K chunks per wave: 8 (inter <= 512) or 12 (inter <= 768).
//
// A unit's W2 rows in registers, as in gemm1's P1W (C + 1 16-byte loads in
// either layout, no branch between them):
// * FP8 slot: r[c] = 16 codes of this lane's row, bytes [c 64 + q 16, +16);
//   r[C] = fp32 row scales of the C rows 4q..4q+3.
// * int4 slot: r[g] = 32 nibbles of this lane's row, K group g, elements
//   [g 128 + q 32, +32) (g < C / 2); r[C / 2 + g / 4] holds the row's
//   (scale, zero) of group g at dword g % 4; with C = 8, r[5..8] hold those
//   of the C rows 4q..4q+3 the lane accumulates; otherwise the other
//   registers repeat the row's area (unused).
template <int C>
struct P2W { i32x4 r[C + 1]; };
template <int C>
struct P2H { i32x4 v[C][2]; };

template <int C>
__device__ __forceinline__ void p2_landed(const P2W<C>& W) {
#pragma unroll
    for (int i = 0; i <= C; ++i) asm volatile("" ::"v"(W.r[i]));
}

template <int C>
__device__ __forceinline__ void p2_issue_w(P2W<C>& W, const SlotView& pool, int slot, int fmt, int n0, int m, int q,
                                           int I, int chunks) {
    constexpr int NSZ = (C / 2 + 3) / 4;                 // 16-byte (scale, zero) loads per row
    const uint8_t* sb = pool.base + (size_t)slot * pool.stride;
    const int groups = I / MOE_INT4_G;
    const uint8_t* wr8 = sb + pool.off[0][2] + (size_t)(n0 + m) * I + q * 16;
    const uint8_t* sc8 = sb + pool.off[0][3] + 4 * (n0 + 4 * q);
    const uint8_t* wr4 = sb + pool.off[1][2] + (size_t)(n0 + m) * (I / 2) + q * 16;
    const uint8_t* szb = sb + pool.off[1][3];
    const uint8_t* sz4 = szb + (size_t)(n0 + m) * groups * 4;
#pragma unroll
    for (int i = 0; i < C; ++i) {
        const uint8_t* p8 = wr8 + min(i, chunks - 1) * 64;
        const uint8_t* p4 = i < C / 2 ? wr4 + min(i, max(groups, 1) - 1) * 64 : sz4 + 16 * min(i - C / 2, NSZ - 1);
        // C = 8 (one (scale, zero) load per row): registers 5..7 and 8 hold
        // the (scale, zero) of the C rows 4q..4q+3 this lane accumulates
        if (C == 8 && i >= 5) p4 = szb + (size_t)(n0 + 4 * q + i - 5) * groups * 4;
        W.r[i] = *(const i32x4*)(fmt ? p4 : p8);
    }
    W.r[C] = *(const i32x4*)(fmt ? (C == 8 ? szb + (size_t)(n0 + 4 * q + 3) * groups * 4 : sz4) : sc8);
}

// h row of this lane's position in the K order of the block's W2 layout, with
// no branch around the loads (chunks past the row repeat its last one,
// unused). A padding position reads the block's first row (always a real
// pair; the same lines as lane 0): it only feeds that position's output
// column, which is never stored.
template <int C>
__device__ __forceinline__ void p2_issue_h(P2H<C>& Hh, const uint16_t* hr, int fmt, int q, int chunks) {
#pragma unroll
    for (int i = 0; i < C; ++i) {
        const int c = min(i, chunks - 1);
        const int k0 = fmt ? (c >> 1) * 128 + q * 32 + (c & 1) * 16 : c * 64 + q * 16;
        Hh.v[i][0] = *(const i32x4*)(hr + k0);
        Hh.v[i][1] = *(const i32x4*)(hr + k0 + 8);
    }
}

// GD: the unit range and the first block's slot and format come from the
// descriptor the gate/up kernel wrote (whole-layer call), so the first
// weights are loaded in the same round trip as the tables.
// Twelve K chunks (inter 640 or 768): one workgroup per CU with the weights of
// the unit two ahead in flight; at two workgroups per CU the h rows and two
// weight register sets spilled. Eight chunks: the same from 256 pairs up (its
// longer unit ranges end more evenly: 0.7 us less at 32 tokens x 8), two
// workgroups per CU with one unit of prefetch below (one per CU measured
// 0.4-1.4 us slower at 8 tokens). WPC = workgroups per CU.
constexpr int gemm2_pipe_wgs_per_cu(int chunks) { return chunks == 12 ? 1 : 2; }

template <int P2_C, bool GD, int WPC = gemm2_pipe_wgs_per_cu(P2_C)>
__global__ void __launch_bounds__(G_THREADS, WPC) gemm2_pipe_kernel(
    SlotView pool, int n_slots, int NP, int k, const float* __restrict__ topk_w,
    const int32_t* __restrict__ sorted_pair, const int32_t* __restrict__ block_slot,
    const int32_t* __restrict__ n_padded, int H, int I, const uint16_t* __restrict__ hbuf, float* __restrict__ ybuf,
    const int4* __restrict__ gdesc) {
    __shared__ uint8_t s_fmt[MOE_MAX_SLOTS];
    __shared__ int s_slot[P2_MAXB];
    __shared__ int s_pr[P2_MAXB][16];
    const int lane = lane_id(), wv = threadIdx.x / MOE_WAVE;
    const int m = lane & 15, q = lane >> 4;
    const int ntile = H / G2_COLS;
    const int chunks = I / 64;
    const int groups = I / MOE_INT4_G;
    int u_begin, u_end, g_slot = -1, g_fmt = 0;
    if constexpr (GD) {
        const int4 d = gdesc[blockIdx.x];
        u_begin = __builtin_amdgcn_readfirstlane(d.x);
        u_end = __builtin_amdgcn_readfirstlane(d.y);
        g_slot = __builtin_amdgcn_readfirstlane(d.z);
        g_fmt = __builtin_amdgcn_readfirstlane(d.w);
    } else {
        const int n_units = (*n_padded / 16) * ntile;
        unit_range(n_units, gridDim.x, blockIdx.x, u_begin, u_end);
    }
    const int b_first = u_begin / ntile;
    const int nblk = u_begin < u_end ? (u_end - 1) / ntile - b_first + 1 : 0;
    // usable slot or -1, and what to load for a table entry (an unusable one:
    // slot 0 in a format that fits the stride; its unit ignores the values)
    auto ok = [&](int slot) { return usable_slot(slot, n_slots, pool.fmt_ok, s_fmt); };
    auto pf_slot = [&](int slot) { return max(ok(slot), 0); };
    auto pf_fmt = [&](int slot) { const int s = ok(slot); return s >= 0 ? (int)s_fmt[s] : pool.spec_fmt; };
    constexpr int PF = WPC == 1 ? 2 : 1;            // units of prefetch
    P2W<P2_C> WA, WB, WC;
    P2H<P2_C> Hh;
    int hblock = -1;
    float wt = 0.f;
    if constexpr (GD) {
        if (nblk == 0) return;                       // uniform over the workgroup
        // the tables, then the first unit's weights, in one round trip (loads
        // complete in issue order: the tables can be waited for while the
        // weights stay in flight; a non-resident first block reads slot 0's
        // bytes in a format that fits the stride and ignores them)
        const int i0 = threadIdx.x, i1 = threadIdx.x + G_THREADS;
        int f0 = 0, d0 = 0, d1 = 0;
        if (i0 < n_slots) f0 = pool.fmt[i0];
        if (i0 < nblk * 17) d0 = i0 % 17 == 16 ? block_slot[b_first + i0 / 17] : sorted_pair[(b_first + i0 / 17) * 16 + i0 % 17];
        if (i1 < nblk * 17) d1 = i1 % 17 == 16 ? block_slot[b_first + i1 / 17] : sorted_pair[(b_first + i1 / 17) * 16 + i1 % 17];
        __builtin_amdgcn_sched_barrier(0);
        p2_issue_w(WA, pool, max(g_slot, 0), g_fmt, (u_begin % ntile) * G2_COLS + wv * 16, m, q, I, chunks);
        __builtin_amdgcn_sched_barrier(0);
        if (i0 < n_slots) s_fmt[i0] = (uint8_t)f0;
        if (i0 < nblk * 17) {
            if (i0 % 17 == 16) s_slot[i0 / 17] = d0;
            else s_pr[i0 / 17][i0 % 17] = d0;
        }
        if (i1 < nblk * 17) {
            if (i1 % 17 == 16) s_slot[i1 / 17] = d1;
            else s_pr[i1 / 17][i1 % 17] = d1;
        }
        for (int i = i1; i < n_slots; i += G_THREADS) s_fmt[i] = pool.fmt[i];       // pools over 256 slots
        barrier_lds();                               // tables written; the weight loads stay in flight
        if constexpr (PF == 2) {
            const int u1 = min(u_begin + 1, u_end - 1), s1 = s_slot[u1 / ntile - b_first];
            p2_issue_w(WB, pool, pf_slot(s1), pf_fmt(s1), (u1 % ntile) * G2_COLS + wv * 16, m, q, I, chunks);
        }
    } else {
        for (int i = threadIdx.x; i < n_slots; i += G_THREADS) s_fmt[i] = pool.fmt[i];
        for (int i = threadIdx.x; i < nblk * 17; i += G_THREADS) {
            const int bb = i / 17, r = i % 17;
            if (r == 16) s_slot[bb] = block_slot[b_first + bb];
            else s_pr[bb][r] = sorted_pair[(b_first + bb) * 16 + r];
        }
        __syncthreads();
        if (nblk == 0) return;
        const int s0 = s_slot[0];
        p2_issue_w(WA, pool, pf_slot(s0), pf_fmt(s0), (u_begin % ntile) * G2_COLS + wv * 16, m, q, I, chunks);
        if constexpr (PF == 2) {
            const int u1 = min(u_begin + 1, u_end - 1), s1 = s_slot[u1 / ntile - b_first];
            p2_issue_w(WB, pool, pf_slot(s1), pf_fmt(s1), (u1 % ntile) * G2_COLS + wv * 16, m, q, I, chunks);
        }
    }
    auto step = [&](int u, P2W<P2_C>& Wc, P2W<P2_C>& Wn) {
        const int bb = u / ntile - b_first;
        const int n0 = (u % ntile) * G2_COLS + wv * 16;
        const int slot = ok(s_slot[bb]);
        const int fmt = slot >= 0 ? (int)s_fmt[slot] : 0;
        const int pr = s_pr[bb][m];
        const bool valid = pr < NP;
        if (slot >= 0 && bb != hblock) {              // new block: its h rows and route weights
            p2_issue_h(Hh, hbuf + (size_t)((b_first + bb) * 16 + (valid ? m : 0)) * I, fmt, q, chunks);
            wt = topk_w[valid ? pr : 0];              // (used only where valid)
            hblock = bb;
        }
        {
            // the weights of unit u + PF, with no branch around the loads
            // (slot 0 for an unusable slot, whose unit ignores them; past the
            // range: the last unit again), so the compiler's count of loads
            // in flight stays exact and the wait below leaves them in flight
            const int un = min(u + PF, u_end - 1);
            const int sn = s_slot[un / ntile - b_first];
            p2_issue_w(Wn, pool, pf_slot(sn), pf_fmt(sn), (un % ntile) * G2_COLS + wv * 16, m, q, I, chunks);
        }
        // every path waits here for this unit's weight loads, so no load into
        // a register set is still pending when the set is refilled
        p2_landed(Wc);
        float* yrow = ybuf + (size_t)(valid ? pr : 0) * H + n0 + 4 * q;
        if (slot < 0) {                               // non-resident expert: its pairs add zero
            if (valid && s_slot[bb] != MOE_SLOT_DEFERRED) *(f32x4*)yrow = f32x4{0, 0, 0, 0};
            return;                                   // (a deferred block's rows are left as they are)
        }
        f32x4 acc = {0, 0, 0, 0};
        if (fmt == 0) {
#pragma unroll
            for (int c = 0; c < P2_C; ++c) {
                if (c >= chunks) break;                // uniform
                bf16x8 a0, a1, h0, h1;
                fp8x16_to_bf16(Wc.r[c], a0, a1);
                split_bf16(Hh.v[c][0], Hh.v[c][1], h0, h1);
                acc = mfma_bf16_16x16x32(a0, h0, acc);
                acc = mfma_bf16_16x16x32(a1, h1, acc);
            }
            acc *= __builtin_bit_cast(f32x4, Wc.r[P2_C]);
        } else {
            // (q - z) exactly in bf16, each group's scale after its matrix
            // instructions; the scales of C rows 4q..4q+3 from this lane's
            // registers 5..8 (C = 8) or from the lanes that loaded those rows
#pragma unroll
            for (int g = 0; g < P2_C / 2; ++g) {
                if (g >= groups) break;                // uniform
                const uint32_t sz = (uint32_t)Wc.r[P2_C / 2 + g / 4][g % 4];
                const float z = (float)__builtin_bit_cast(_Float16, (uint16_t)(sz >> 16));
                f32x4 t4 = {0, 0, 0, 0};
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    const int c = g * 2 + c2;
                    bf16x8 a0, a1, h0, h1;
                    int4x16_to_bf16<P2_C == 8>(make_uint2((uint32_t)Wc.r[g][2 * c2], (uint32_t)Wc.r[g][2 * c2 + 1]), z,
                                               a0, a1);
                    split_bf16(Hh.v[c][0], Hh.v[c][1], h0, h1);
                    t4 = mfma_bf16_16x16x32(a0, h0, t4);
                    t4 = mfma_bf16_16x16x32(a1, h1, t4);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // C row 4q + i: its own registers at C = 8, else from the lane that loaded it
                    const uint32_t szr = P2_C == 8 ? (uint32_t)(i < 3 ? Wc.r[5 + i][g % 4] : Wc.r[8][g % 4])
                                                   : (uint32_t)__shfl((int)sz, 4 * q + i, 64);
                    acc[i] += (float)__builtin_bit_cast(_Float16, (uint16_t)(szr & 0xFFFFu)) * t4[i];
                }
            }
        }
        if (valid) *(f32x4*)yrow = acc * wt;
    };
    // pairs of units, then an odd last one after the loop: a path that ran
    // one step and returned to the loop head would leave the other register
    // set's loads pending there, and the compiler would then wait for every
    // load in flight at the head of each iteration (the prefetch included)
    int u = u_begin;
    if constexpr (PF == 2) {                          // three register sets in turn
        for (; u + 2 < u_end; u += 3) {
            step(u, WA, WC);
            step(u + 1, WB, WA);
            step(u + 2, WC, WB);
        }
        if (u < u_end) step(u, WA, WC);
        if (u + 1 < u_end) step(u + 1, WB, WA);
    } else {
        for (; u + 1 < u_end; u += 2) {
            step(u, WA, WB);
            step(u + 1, WB, WA);
        }
        if (u < u_end) step(u, WA, WB);
    }
}

// ------------------------------------------------------------ combine
// out[t] = sum over j of ybuf[t*k + j] in fp32 (fixed order), rounded once to
// bf16. Pairs with weight exactly 0 (route entries that were never filled)
// are skipped: their rows were never written.
template <typename YT, int KMAX>
__global__ void __launch_bounds__(256) combine_rows_kernel(const YT* __restrict__ ybuf, const float* __restrict__ topk_w,
                                                          int T, int k, int H, uint16_t* __restrict__ out,
                                                          int pieces) {
    // workgroups walk (token, column piece) items, H / pieces columns each; a
    // token's weights are wave-uniform (scalar loads), each thread sums 8
    // columns of the token's k rows
    const int cw = H / pieces;
    for (int it = blockIdx.x; it < T * pieces; it += gridDim.x) {
        const int t = it / pieces, c0 = (it % pieces) * cw;
        float wj[KMAX];
#pragma unroll
        for (int j = 0; j < KMAX; ++j) wj[j] = j < k ? topk_w[(size_t)t * k + j] : 0.f;
        for (int c = c0 + threadIdx.x * 8; c < c0 + cw; c += blockDim.x * 8) {
            float s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            // every load first (rows of unfilled route entries are read but not used)
            i32x4 v[KMAX][sizeof(YT) == 4 ? 2 : 1];
#pragma unroll
            for (int j = 0; j < KMAX; ++j) {
                if (j < k) {
                    const YT* row = ybuf + ((size_t)t * k + j) * H + c;
                    if constexpr (sizeof(YT) == 4) {
                        v[j][0] = *(const i32x4*)row;
                        v[j][1] = *(const i32x4*)(row + 4);
                    } else {
                        // batched sizes: the weighted pair rows are read once,
                        // and stream past the caches
                        v[j][0] = __builtin_nontemporal_load((const i32x4*)row);
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < KMAX; ++j) {
                const bool use = j < k && wj[j] != 0.f;
                if constexpr (sizeof(YT) == 4) {
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        s[d] += use ? __int_as_float(v[j][0][d]) : 0.f;
                        s[4 + d] += use ? __int_as_float(v[j][1][d]) : 0.f;
                    }
                } else {
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        s[2 * d] += use ? bf16_to_f32((uint16_t)((uint32_t)v[j][0][d] & 0xFFFF)) : 0.f;
                        s[2 * d + 1] += use ? bf16_to_f32((uint16_t)((uint32_t)v[j][0][d] >> 16)) : 0.f;
                    }
                }
            }
            i32x4 o;
#pragma unroll
            for (int d = 0; d < 4; ++d) o[d] = (int)two_bf16(s[2 * d], s[2 * d + 1]);
            *(i32x4*)(out + (size_t)t * H + c) = o;
        }
    }
}

hipError_t launch_combine_f32(const float* ybuf, const float* topk_w, int T, int k, int H, uint16_t* out,
                              hipStream_t stream) {
    // decode sizes: one wave per (token, 512 columns), so a few tokens still
    // spread over many CUs; otherwise a 256-thread workgroup per token
    const bool narrow = H % 512 == 0 && T * (H / 512) <= 4096;
    const int pieces = narrow ? H / 512 : 1, threads = narrow ? MOE_WAVE : 256;
    const int items = T * pieces, blocks = items < 4096 ? items : 4096;
    if (k <= 8)
        MOE_LAUNCH(K_COMBINE, stream, (combine_rows_kernel<float, 8>), dim3(blocks), dim3(threads), 0, stream, ybuf,
                   topk_w, T, k, H, out, pieces);
    else if (k <= 16)
        MOE_LAUNCH(K_COMBINE, stream, (combine_rows_kernel<float, 16>), dim3(blocks), dim3(threads), 0, stream, ybuf,
                   topk_w, T, k, H, out, pieces);
    else
        MOE_LAUNCH(K_COMBINE, stream, (combine_rows_kernel<float, MOE_MAX_K>), dim3(blocks), dim3(threads), 0, stream,
                   ybuf, topk_w, T, k, H, out, pieces);
    return hipGetLastError();
}

hipError_t launch_combine_bf16(const uint16_t* ybuf, const float* topk_w, int T, int k, int H, uint16_t* out,
                               hipStream_t stream) {
    const int blocks = T < 4096 ? T : 4096;
    if (k <= 8)
        MOE_LAUNCH(K_COMBINE, stream, (combine_rows_kernel<uint16_t, 8>), dim3(blocks), dim3(256), 0, stream, ybuf,
                   topk_w, T, k, H, out, 1);
    else if (k <= 16)
        MOE_LAUNCH(K_COMBINE, stream, (combine_rows_kernel<uint16_t, 16>), dim3(blocks), dim3(256), 0, stream, ybuf,
                   topk_w, T, k, H, out, 1);
    else
        MOE_LAUNCH(K_COMBINE, stream, (combine_rows_kernel<uint16_t, MOE_MAX_K>), dim3(blocks), dim3(256), 0, stream,
                   ybuf, topk_w, T, k, H, out, 1);
    return hipGetLastError();
}

// ------------------------------------------------------------ host side
int stream_max_tokens() { return STREAM_MAX_T; }

// compute units of the current device (cached per device id)
int device_cus() {
    // per device, filled once; racing callers store the same value
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int c = cached[dev].load(std::memory_order_relaxed);
    if (c <= 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
        c = n;
    }
    return c;
}

static size_t up256(size_t n) { return (n + 255) / 256 * 256; }

size_t stream_workspace_bytes(int T, int k, int H, int I, int cap) {
    return up256((size_t)cap * I * sizeof(uint16_t)) + up256((size_t)T * k * H * sizeof(float));
}

// the down kernel's grid (the gate/up kernel of a whole-layer call writes one
// descriptor per workgroup of it)
static int gemm2_pipe_wpc(int I, int NP) { return I > 64 * 8 || NP >= 256 ? 1 : 2; }
static int gemm2_pipe_grid(int I, int NP) { return gemm2_pipe_wpc(I, NP) * device_cus(); }

template <int BM>
static void launch_gemm2_stream(const SlotView& sv, int n_slots, int T, int k, const float* topk_w,
                                const int32_t* sorted_pair, const int32_t* block_slot, const int32_t* n_padded,
                                int cap, int H, int I, const uint16_t* hbuf, float* ybuf, hipStream_t stream,
                                const int4* gdesc = nullptr) {
    const int NP = T * k;
    const int nb = cap / BM;
    const int pipe_grid = gemm2_pipe_grid(I, NP);
    const int units2 = nb * (H / G2_COLS);
    const int per2 = max_units(units2, pipe_grid);
    if (BM == 16 && I <= 64 * 8 && per2 / (H / G2_COLS) + 2 <= P2_MAXB) {
        if (gdesc && pipe_grid == device_cus())
            MOE_LAUNCH(K_GEMM2_STREAM, stream, (gemm2_pipe_kernel<8, true, 1>), dim3(pipe_grid), dim3(G_THREADS), 0, stream,
                       sv, n_slots, NP, k, topk_w, sorted_pair, block_slot, n_padded, H, I, hbuf, ybuf, gdesc);
        else if (gdesc)
            MOE_LAUNCH(K_GEMM2_STREAM, stream, (gemm2_pipe_kernel<8, true>), dim3(pipe_grid), dim3(G_THREADS), 0, stream,
                       sv, n_slots, NP, k, topk_w, sorted_pair, block_slot, n_padded, H, I, hbuf, ybuf, gdesc);
        else if (pipe_grid == device_cus())
            MOE_LAUNCH(K_GEMM2_STREAM, stream, (gemm2_pipe_kernel<8, false, 1>), dim3(pipe_grid), dim3(G_THREADS), 0,
                       stream, sv, n_slots, NP, k, topk_w, sorted_pair, block_slot, n_padded, H, I, hbuf, ybuf, gdesc);
        else
            MOE_LAUNCH(K_GEMM2_STREAM, stream, (gemm2_pipe_kernel<8, false>), dim3(pipe_grid), dim3(G_THREADS), 0,
                       stream, sv, n_slots, NP, k, topk_w, sorted_pair, block_slot, n_padded, H, I, hbuf, ybuf, gdesc);
    } else if (BM == 16 && I <= 64 * 12 && per2 / (H / G2_COLS) + 2 <= P2_MAXB) {
        if (gdesc)
            MOE_LAUNCH(K_GEMM2_STREAM, stream, (gemm2_pipe_kernel<12, true>), dim3(pipe_grid), dim3(G_THREADS), 0,
                       stream, sv, n_slots, NP, k, topk_w, sorted_pair, block_slot, n_padded, H, I, hbuf, ybuf, gdesc);
        else
            MOE_LAUNCH(K_GEMM2_STREAM, stream, (gemm2_pipe_kernel<12, false>), dim3(pipe_grid), dim3(G_THREADS), 0,
                       stream, sv, n_slots, NP, k, topk_w, sorted_pair, block_slot, n_padded, H, I, hbuf, ybuf, gdesc);
    } else {
        MOE_LAUNCH(K_GEMM2_STREAM, stream, gemm2_stream_kernel<BM>, dim3(units2), dim3(G_THREADS), 0, stream, sv,
                   n_slots, NP, k, topk_w, sorted_pair, block_slot, n_padded, H, I, hbuf, ybuf);
    }
}

template <int BM>
static void launch_stream_bm(const SlotView& sv, int n_slots, const uint16_t* x, int T, int k, const float* topk_w,
                             const int32_t* sorted_pair, const int32_t* block_slot, const int32_t* n_padded, int cap,
                             int H, int I, uint16_t* hbuf, float* ybuf, hipStream_t stream) {
    const int NP = T * k;
    const int nb = cap / BM;                        // blocks that can exist; the kernels skip the rest
    const int units = nb * (I / ROWS);
    const int pipe_grid = gemm1_pipe_wgs_per_cu(0) * device_cus();
    // the pipelined kernel: 16-pair blocks, hidden <= 2048, and each workgroup's
    // unit range must span at most P1_MAXB blocks (always true unless the grid is tiny)
    const int pipe_units = nb * (I / P1_ROWS);
    const int per = max_units(pipe_units, pipe_grid);
    if (BM == 16 && H <= 128 * G_WAVES * P1_G && per / (I / P1_ROWS) + 2 <= P1_MAXB) {
        MOE_LAUNCH(K_GEMM1_STREAM, stream, (gemm1_pipe_kernel<0, 0, 1>), dim3(pipe_grid), dim3(G_THREADS), 0, stream,
                   sv, n_slots, x, T, k, sorted_pair, block_slot, n_padded, H, I, hbuf, LayerIO{});
    } else {
        MOE_LAUNCH(K_GEMM1_STREAM, stream, gemm1_stream_kernel<BM>, dim3(units), dim3(G_THREADS), 0, stream, sv,
                   n_slots, x, NP, k, sorted_pair, block_slot, n_padded, H, I, hbuf);
    }
    launch_gemm2_stream<BM>(sv, n_slots, T, k, topk_w, sorted_pair, block_slot, n_padded, cap, H, I, hbuf, ybuf,
                            stream);
}

hipError_t launch_ffn_stream(const PoolArgs& pa, const uint16_t* x, int T, int k, const float* topk_w,
                             const int32_t* sorted_pair, const int32_t* block_slot, const int32_t* n_padded,
                             int cap, int block_m, uint16_t* out, void* ws, hipStream_t stream, FfnPass pass) {
    SlotView sv;
    sv.base = (const uint8_t*)pa.base;
    sv.stride = pa.stride;
    sv.fmt = pa.fmt;
    for (int f = 0; f < 2; ++f)
        for (int p = 0; p < 4; ++p) sv.off[f][p] = pa.off[f][p];
    sv.fmt_ok = pa.fmt_ok;
    sv.spec_fmt = pa.spec_fmt;
    const int H = pa.hidden, I = pa.inter;
    uint16_t* hbuf = (uint16_t*)ws;
    float* ybuf = (float*)((uint8_t*)ws + up256((size_t)cap * I * sizeof(uint16_t)));
    if (pass == FFN_WHOLE && debug_poison_on()) {     // h and y rows: NaN until written
        hipError_t e = launch_poison(ws, stream_workspace_bytes(T, k, H, I, cap), stream);
        if (e != hipSuccess) return e;
    }
    switch (block_m) {
        case 16: launch_stream_bm<16>(sv, pa.n_slots, x, T, k, topk_w, sorted_pair, block_slot, n_padded, cap, H, I, hbuf, ybuf, stream); break;
        case 32: launch_stream_bm<32>(sv, pa.n_slots, x, T, k, topk_w, sorted_pair, block_slot, n_padded, cap, H, I, hbuf, ybuf, stream); break;
        case 64: launch_stream_bm<64>(sv, pa.n_slots, x, T, k, topk_w, sorted_pair, block_slot, n_padded, cap, H, I, hbuf, ybuf, stream); break;
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (pass == FFN_PASS) return hipSuccess;          // rows only: a later pass combines
    return launch_combine_f32(ybuf, topk_w, T, k, H, out, stream);
}

// ------------------------------------------------------------ whole layer
size_t layer_stream_workspace_bytes(int T, int k, int H, int I, int cap) {
    return stream_workspace_bytes(T, k, H, I, cap) + up256((size_t)16 * 2 * device_cus());
}

bool layer_stream_ok(int T, int k, int E, int H, int I, int block_m, int cap) {
    if (block_m != 16 || T > LAYER_MAX_T || T * k > LAYER_MAX_NP || E > MOE_MAX_E) return false;
    if (H > 128 * G_WAVES * P1_G) return false;
    const int pipe_grid = device_cus();              // (the smaller of the gate/up grids: the longer ranges)
    const int per = max_units((cap / 16) * (I / P1_ROWS), pipe_grid);
    return per / (I / P1_ROWS) + 2 <= P1_MAXB;
}

template <int RVPL, int RT>
static void launch_gemm1_layer(const SlotView& sv, int n_slots, const uint16_t* x, int T, int k, int H, int I,
                               uint16_t* hbuf, const LayerIO& L, hipStream_t stream) {
    MOE_LAUNCH(K_GEMM1_STREAM, stream, (gemm1_pipe_kernel<RVPL == 0 ? 1 : 2, RVPL, RT>),
               dim3(gemm1_pipe_wgs_per_cu(RVPL == 0 ? 1 : 2) * device_cus()),
               dim3(G_THREADS), 0, stream, sv, n_slots, x, T, k, (const int32_t*)nullptr, (const int32_t*)nullptr,
               (const int32_t*)nullptr, H, I, hbuf, L);
}

// routing inside the gate/up kernel: RT tokens per wavefront, 64 * VPL experts
template <int VPL>
static void launch_gemm1_route(const SlotView& sv, int n_slots, const uint16_t* x, int T, int k, int H, int I,
                               uint16_t* hbuf, const LayerIO& L, hipStream_t stream) {
    if (T <= G_WAVES) launch_gemm1_layer<VPL, 1>(sv, n_slots, x, T, k, H, I, hbuf, L, stream);
    else if (T <= 2 * G_WAVES) launch_gemm1_layer<VPL, 2>(sv, n_slots, x, T, k, H, I, hbuf, L, stream);
    else launch_gemm1_layer<VPL, 4>(sv, n_slots, x, T, k, H, I, hbuf, L, stream);
}

hipError_t launch_layer_stream(const PoolArgs& pa, const float* logits, const uint8_t* mask,
                               const int32_t* slot_of_expert, int E, const uint16_t* x, int T, int k, int32_t* ids,
                               float* w, int32_t* sorted_pair, int32_t* block_slot, int32_t* counts,
                               int32_t* seg_offset, int32_t* n_padded, int32_t* err, int cap, uint16_t* out,
                               void* ws, hipStream_t stream) {
    SlotView sv;
    sv.base = (const uint8_t*)pa.base;
    sv.stride = pa.stride;
    sv.fmt = pa.fmt;
    for (int f = 0; f < 2; ++f)
        for (int p = 0; p < 4; ++p) sv.off[f][p] = pa.off[f][p];
    sv.fmt_ok = pa.fmt_ok;
    sv.spec_fmt = pa.spec_fmt;
    const int H = pa.hidden, I = pa.inter;
    uint16_t* hbuf = (uint16_t*)ws;
    float* ybuf = (float*)((uint8_t*)ws + up256((size_t)cap * I * sizeof(uint16_t)));
    int4* gdesc = (int4*)((uint8_t*)ws + stream_workspace_bytes(T, k, H, I, cap));
    if (debug_poison_on()) {                          // h and y rows: NaN until written
        hipError_t e = launch_poison(ws, stream_workspace_bytes(T, k, H, I, cap), stream);
        if (e != hipSuccess) return e;
    }
    LayerIO L{logits, mask,     slot_of_expert, E,          ids,         w,          sorted_pair,
              block_slot, counts, seg_offset, n_padded, err, gdesc, gemm2_pipe_grid(I, T * k), H};
    if (T <= LAYER_ROUTE_MAX_T && E <= 512) {
        if (E <= 256) launch_gemm1_route<4>(sv, pa.n_slots, x, T, k, H, I, hbuf, L, stream);
        else launch_gemm1_route<8>(sv, pa.n_slots, x, T, k, H, I, hbuf, L, stream);
    } else {
        hipError_t e = launch_route(logits, mask, T, E, k, ids, w, err, stream);
        if (e != hipSuccess) return e;
        L.logits = nullptr;
        launch_gemm1_layer<0, 1>(sv, pa.n_slots, x, T, k, H, I, hbuf, L, stream);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    launch_gemm2_stream<16>(sv, pa.n_slots, T, k, w, sorted_pair, block_slot, n_padded, cap, H, I, hbuf, ybuf,
                            stream, gdesc);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_combine_f32(ybuf, w, T, k, H, out, stream);
}

}  // namespace moe
