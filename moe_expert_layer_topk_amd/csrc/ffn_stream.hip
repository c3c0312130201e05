// Expert FFN, streaming path for small token counts (activations in bf16).
//
// vllm-expert-pager article (rand.pepabo.com), Table 1 set-up: each expert
// has w13 (gate and up fused) and w2 (down); "hierarchical paging" section:
// they are read from the expert's VRAM slot. At decode sizes the layer is
// bound by reading those slots once from HBM, so both kernels stream weight
// rows with 16-byte loads spread over the whole chip and feed them, converted
// to bf16 (exact for e4m3 codes and for int4 q - zero), to bf16 matrix cores
// against the few token rows of each expert.
//
// Kernel 1 (gate/up): unit = (block of pairs, 16 rows of inter). Each of the
//   4 waves takes a quarter of the K = hidden groups; partial sums meet in
//   LDS; the epilogue applies row scales, silu(gate) * up, and stores h (bf16).
// Kernel 2 (down + combine): each workgroup owns 16 output columns of every
//   token. Its 8 waves walk the blocks, multiply W2 rows by h and add
//   w[t][j] * y into per-wave LDS accumulators, which are summed in a fixed
//   order and rounded once to bf16: no atomics, deterministic.
//
// Operand layout of v_mfma_f32_16x16x32_bf16 (lane l = m + 16 q): A row m and
// B column m hold K positions 8q..8q+7; C lane l holds rows 4q..4q+3 of
// column m. Both operands here use the same K permutation (lane group q reads
// 16 consecutive K of a 64-wide chunk and splits them over two instructions),
// which leaves the contraction unchanged.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

struct SlotView {
    const uint8_t* base;   // slot 0
    size_t stride;         // bytes per slot
    const uint8_t* fmt;    // device u8[n_slots]
    size_t off[2][4];      // part offsets per format
};

// 16 K values of row `row` at K offset k0 (multiple of 16) as two bf16x8
// operands. FP8 rows: codes. INT4 rows: q - zero of the row's K group.
__device__ __forceinline__ void load_w16_fp8(const uint8_t* rowp, int k0, bf16x8& s0, bf16x8& s1) {
    i32x4 v = *(const i32x4*)(rowp + k0);
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

__device__ __forceinline__ void load_w16_int4(const uint8_t* rowp_packed, int k0, float zero, bf16x8& s0,
                                              bf16x8& s1) {
    uint2 v = *(const uint2*)(rowp_packed + k0 / 2);
    uint32_t w[2] = {v.x, v.y};
    uint32_t o[8];
#pragma unroll
    for (int d = 0; d < 2; ++d) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t byte = (w[d] >> (8 * j)) & 0xFFu;
            float lo = (float)(byte & 0xFu) - zero;
            float hi = (float)(byte >> 4) - zero;
            o[d * 4 + j] = two_bf16(lo, hi);
        }
    }
    i32x4 x0 = {(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
    i32x4 x1 = {(int)o[4], (int)o[5], (int)o[6], (int)o[7]};
    s0 = __builtin_bit_cast(bf16x8, x0);
    s1 = __builtin_bit_cast(bf16x8, x1);
}

// 16 bf16 of a token row at K offset k0 as two operands (no conversion)
__device__ __forceinline__ void load_x16(const uint16_t* xrow, int k0, bf16x8& s0, bf16x8& s1) {
    const i32x4* p = (const i32x4*)(xrow + k0);
    s0 = __builtin_bit_cast(bf16x8, p[0]);
    s1 = __builtin_bit_cast(bf16x8, p[1]);
}

__device__ __forceinline__ float2 half2_at(const uint8_t* p) {
    const _Float16* h = (const _Float16*)p;
    return make_float2((float)h[0], (float)h[1]);
}

constexpr int G1_THREADS = 256;
constexpr int G1_WAVES = 4;
constexpr int ROWS = 16;    // inter rows (gate and up each) per unit

template <int BM>
__global__ void __launch_bounds__(G1_THREADS) gemm1_stream_kernel(
    SlotView pool, const uint16_t* __restrict__ x, int NP, int k, const int32_t* __restrict__ sorted_pair,
    const int32_t* __restrict__ block_slot, const int32_t* __restrict__ n_padded, int H, int I,
    uint16_t* __restrict__ hbuf) {
    constexpr int NT = BM / 16;
    __shared__ f32x4 s_red[G1_WAVES][NT][2][MOE_WAVE];
    const int lane = lane_id(), wv = threadIdx.x / MOE_WAVE;
    const int m = lane & 15, q = lane >> 4;
    const int ntile = I / ROWS;
    const int nblocks = *n_padded / BM;
    const int n_units = nblocks * ntile;
    const int groups = H / MOE_INT4_G;
    for (int u = blockIdx.x; u < n_units; u += gridDim.x) {
        const int b = u / ntile, i0 = (u % ntile) * ROWS;
        const int slot = block_slot[b];
        if (slot < 0) continue;                       // uniform over the workgroup
        const uint8_t* sb = pool.base + (size_t)slot * pool.stride;
        const int fmt = (pool.fmt[slot] == 1 && I % MOE_INT4_G == 0) ? 1 : 0;
        const uint16_t* xr[NT];
        int pos[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            pos[nt] = b * BM + nt * 16 + m;
            int p = sorted_pair[pos[nt]];
            xr[nt] = x + (size_t)(p < NP ? p / k : 0) * H;
        }
        f32x4 acc_g[NT], acc_u[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) { acc_g[nt] = f32x4{0, 0, 0, 0}; acc_u[nt] = f32x4{0, 0, 0, 0}; }
        if (fmt == 0) {
            const uint8_t* wg = sb + (size_t)(i0 + m) * H;
            const uint8_t* wu = sb + (size_t)(I + i0 + m) * H;
            for (int g = wv; g < groups; g += G1_WAVES) {
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const int k0 = g * 128 + c * 64 + q * 16;
                    bf16x8 ga0, ga1, ua0, ua1;
                    load_w16_fp8(wg, k0, ga0, ga1);
                    load_w16_fp8(wu, k0, ua0, ua1);
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        bf16x8 xb0, xb1;
                        load_x16(xr[nt], k0, xb0, xb1);
                        acc_g[nt] = mfma_bf16_16x16x32(ga0, xb0, acc_g[nt]);
                        acc_g[nt] = mfma_bf16_16x16x32(ga1, xb1, acc_g[nt]);
                        acc_u[nt] = mfma_bf16_16x16x32(ua0, xb0, acc_u[nt]);
                        acc_u[nt] = mfma_bf16_16x16x32(ua1, xb1, acc_u[nt]);
                    }
                }
            }
        } else {
            const uint8_t* wg = sb + (size_t)(i0 + m) * (H / 2);
            const uint8_t* wu = sb + (size_t)(I + i0 + m) * (H / 2);
            const uint8_t* sz = sb + pool.off[1][1];
            for (int g = wv; g < groups; g += G1_WAVES) {
                const float zg = half2_at(sz + ((size_t)(i0 + m) * groups + g) * 4).y;
                const float zu = half2_at(sz + ((size_t)(I + i0 + m) * groups + g) * 4).y;
                f32x4 tg[NT], tu[NT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) { tg[nt] = f32x4{0, 0, 0, 0}; tu[nt] = f32x4{0, 0, 0, 0}; }
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const int k0 = g * 128 + c * 64 + q * 16;
                    bf16x8 ga0, ga1, ua0, ua1;
                    load_w16_int4(wg, k0, zg, ga0, ga1);
                    load_w16_int4(wu, k0, zu, ua0, ua1);
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        bf16x8 xb0, xb1;
                        load_x16(xr[nt], k0, xb0, xb1);
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
            for (int w2 = 1; w2 < G1_WAVES; ++w2) {
                g += s_red[w2][nt][0][lane];
                up += s_red[w2][nt][1][lane];
            }
            int p = sorted_pair[b * BM + nt * 16 + m];
            if (p < NP) {
                uint32_t packed[2];
#pragma unroll
                for (int i = 0; i < 4; i += 2) {
                    float hv[2];
#pragma unroll
                    for (int d = 0; d < 2; ++d) {
                        const int r = i0 + 4 * q + i + d;
                        float gs = g[i + d], us = up[i + d];
                        if (fmt == 0) {
                            gs *= ((const float*)(sb + pool.off[0][1]))[r];
                            us *= ((const float*)(sb + pool.off[0][1]))[I + r];
                        }
                        hv[d] = silu(gs) * us;
                    }
                    packed[i / 2] = two_bf16(hv[0], hv[1]);
                }
                *(uint2*)(hbuf + (size_t)(b * BM + nt * 16 + m) * I + i0 + 4 * q) = make_uint2(packed[0], packed[1]);
            }
        }
        __syncthreads();
    }
}

constexpr int G2_THREADS = 512;
constexpr int G2_WAVES = 8;
constexpr int STREAM_MAX_T = 64;

template <int BM>
__global__ void __launch_bounds__(G2_THREADS) gemm2_stream_kernel(
    SlotView pool, int T, int NP, int k, const float* __restrict__ topk_w, const int32_t* __restrict__ sorted_pair,
    const int32_t* __restrict__ block_slot, const int32_t* __restrict__ n_padded, int H, int I,
    const uint16_t* __restrict__ hbuf, uint16_t* __restrict__ out) {
    constexpr int NT = BM / 16;
    __shared__ float s_acc[G2_WAVES][STREAM_MAX_T][16];
    const int lane = lane_id(), wv = threadIdx.x / MOE_WAVE;
    const int m = lane & 15, q = lane >> 4;
    const int n0 = blockIdx.x * 16;
    for (int i = threadIdx.x; i < G2_WAVES * STREAM_MAX_T * 16; i += G2_THREADS) (&s_acc[0][0][0])[i] = 0.f;
    __syncthreads();
    const int nblocks = *n_padded / BM;
    const int chunks = I / 64;
    const int groups = (I + MOE_INT4_G - 1) / MOE_INT4_G;
    for (int b = wv; b < nblocks; b += G2_WAVES) {
        const int slot = block_slot[b];
        if (slot < 0) continue;                       // uniform over the wave
        const uint8_t* sb = pool.base + (size_t)slot * pool.stride;
        const int fmt = (pool.fmt[slot] == 1 && I % MOE_INT4_G == 0) ? 1 : 0;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int pos = b * BM + nt * 16 + m;
            const int p = sorted_pair[pos];
            const uint16_t* hr = hbuf + (size_t)pos * I;
            f32x4 acc = {0, 0, 0, 0};
            if (fmt == 0) {
                const uint8_t* wr = sb + pool.off[0][2] + (size_t)(n0 + m) * I;
                for (int c = 0; c < chunks; ++c) {
                    const int k0 = c * 64 + q * 16;
                    bf16x8 a0, a1, h0, h1;
                    load_w16_fp8(wr, k0, a0, a1);
                    load_x16(hr, k0, h0, h1);
                    acc = mfma_bf16_16x16x32(a0, h0, acc);
                    acc = mfma_bf16_16x16x32(a1, h1, acc);
                }
                const float* s2 = (const float*)(sb + pool.off[0][3]);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] *= s2[n0 + 4 * q + i];
            } else {
                const uint8_t* wr = sb + pool.off[1][2] + (size_t)(n0 + m) * (I / 2);
                const uint8_t* sz = sb + pool.off[1][3];
                for (int g = 0; g < groups; ++g) {
                    const float z = half2_at(sz + ((size_t)(n0 + m) * groups + g) * 4).y;
                    f32x4 t4 = {0, 0, 0, 0};
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        const int k0 = g * 128 + c * 64 + q * 16;
                        bf16x8 a0, a1, h0, h1;
                        load_w16_int4(wr, k0, z, a0, a1);
                        load_x16(hr, k0, h0, h1);
                        t4 = mfma_bf16_16x16x32(a0, h0, t4);
                        t4 = mfma_bf16_16x16x32(a1, h1, t4);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[i] += half2_at(sz + ((size_t)(n0 + 4 * q + i) * groups + g) * 4).x * t4[i];
                }
            }
            if (p < NP) {
                const int t = p / k;
                const float wt = topk_w[p];
#pragma unroll
                for (int i = 0; i < 4; ++i) s_acc[wv][t][4 * q + i] += wt * acc[i];
            }
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < T * 16; i += G2_THREADS) {
        const int t = i / 16, c = i % 16;
        float s = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < G2_WAVES; ++w2) s += s_acc[w2][t][c];
        out[(size_t)t * H + n0 + c] = f32_to_bf16(s);
    }
}

int stream_max_tokens() { return STREAM_MAX_T; }

size_t stream_workspace_bytes(int cap, int I) { return (size_t)cap * I * sizeof(uint16_t); }

hipError_t launch_ffn_stream(const PoolArgs& pa, const uint16_t* x, int T, int k, const float* topk_w,
                             const int32_t* sorted_pair, const int32_t* block_slot, const int32_t* n_padded,
                             int cap, int block_m, uint16_t* out, void* ws, hipStream_t stream) {
    SlotView sv;
    sv.base = (const uint8_t*)pa.base;
    sv.stride = pa.stride;
    sv.fmt = pa.fmt;
    for (int f = 0; f < 2; ++f)
        for (int p = 0; p < 4; ++p) sv.off[f][p] = pa.off[f][p];
    const int H = pa.hidden, I = pa.inter, NP = T * k;
    uint16_t* hbuf = (uint16_t*)ws;
    const int units_max = (cap / block_m) * (I / ROWS);
    dim3 g1(units_max < 4096 ? units_max : 4096);
    dim3 g2(H / 16);
    switch (block_m) {
        case 16:
            MOE_LAUNCH(K_GEMM1_STREAM, stream, gemm1_stream_kernel<16>, g1, dim3(G1_THREADS), 0, stream, sv, x, NP, k, sorted_pair,
                               block_slot, n_padded, H, I, hbuf);
            MOE_LAUNCH(K_GEMM2_STREAM, stream, gemm2_stream_kernel<16>, g2, dim3(G2_THREADS), 0, stream, sv, T, NP, k, topk_w,
                               sorted_pair, block_slot, n_padded, H, I, hbuf, out);
            break;
        case 32:
            MOE_LAUNCH(K_GEMM1_STREAM, stream, gemm1_stream_kernel<32>, g1, dim3(G1_THREADS), 0, stream, sv, x, NP, k, sorted_pair,
                               block_slot, n_padded, H, I, hbuf);
            MOE_LAUNCH(K_GEMM2_STREAM, stream, gemm2_stream_kernel<32>, g2, dim3(G2_THREADS), 0, stream, sv, T, NP, k, topk_w,
                               sorted_pair, block_slot, n_padded, H, I, hbuf, out);
            break;
        case 64:
            MOE_LAUNCH(K_GEMM1_STREAM, stream, gemm1_stream_kernel<64>, g1, dim3(G1_THREADS), 0, stream, sv, x, NP, k, sorted_pair,
                               block_slot, n_padded, H, I, hbuf);
            MOE_LAUNCH(K_GEMM2_STREAM, stream, gemm2_stream_kernel<64>, g2, dim3(G2_THREADS), 0, stream, sv, T, NP, k, topk_w,
                               sorted_pair, block_slot, n_padded, H, I, hbuf, out);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace moe
