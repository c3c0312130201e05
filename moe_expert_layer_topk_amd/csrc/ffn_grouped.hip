// Expert FFN, grouped FP8 matrix-core path for large token batches.
//
// MOE-GEN explainer (aibr.jp), sections 1 and 3: with tokens accumulated per
// expert module, each expert's work is a dense contraction over many rows,
// the regime where FP8 matrix cores pay. vllm-expert-pager article
// (rand.pepabo.com), "hierarchical paging": weights come from the expert's
// VRAM slot (Table 1 set-up: w13 = gate+up, w2 = down).
//
// Pipeline (all on the caller's stream):
//   quant_act:  x bf16 -> e4m3 codes + one E8M0 exponent per (row, 128 K)
//   gemm1:      per (block of block_m pairs, 128 inter columns): gathered
//               token rows x W13 gate and up rows -> row scales ->
//               silu(gate) * up -> h quantized like x (one exponent per row
//               and 128 inter columns) -> hq, hs in sorted-pair order
//   gemm2:      per (block, 128 hidden columns): hq x W2 rows -> row scale ->
//               times the pair's route weight -> bf16 row of the pair
//   combine:    out[t] = sum_j ybuf[t*k + j] in fp32, rounded once to bf16
// The E8M0 exponents feed the scaled matrix instruction directly, so the
// power-of-two activation scales cost nothing inside the K loop.
//
// v_mfma_scale_f32_16x16x128_f8f6f4: lane l = m + 16q holds 32 codes of row
// (A) / column (B) m; A and B pair up lane group by lane group, so both are
// loaded with the same K permutation (lane group q reads bytes [32q, 32q+32)
// of the 128-wide K step). Scales are uniform over a K step here, so their
// lane mapping does not matter. C lane l holds rows 4q..4q+3 of column m.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

struct GPool {
    const uint8_t* base;
    size_t stride;
    const uint8_t* fmt;
    size_t off[2][4];
    int n_slots;
    int fmt_ok;           // bit f: format f fits the stride (usable_slot)
};

__device__ __forceinline__ float2 f16x2_at(const uint8_t* p) {
    const _Float16* h = (const _Float16*)p;
    return make_float2((float)h[0], (float)h[1]);
}

// ------------------------------------------------------------ activation quant
// 16 lanes per (row, 128-column group), 8 values (16 bytes) per lane; the
// group's absolute maximum is a max over the lane's row of 16 (DPP).
__global__ void __launch_bounds__(256) quant_act_kernel(const uint16_t* __restrict__ x, int rows, int cols,
                                                       uint8_t* __restrict__ xq, uint8_t* __restrict__ xs) {
    const int lane = lane_id();
    const int groups = cols / MOE_ACT_G;
    const long item = ((long)blockIdx.x * 4 + threadIdx.x / MOE_WAVE) * 4 + lane / 16;
    const bool live = item < (long)rows * groups;
    const long it = live ? item : 0;                    // idle lanes redo item 0 and store nothing
    const int r = (int)(it / groups), g = (int)(it % groups);
    const size_t off = (size_t)r * cols + g * MOE_ACT_G + 8 * (lane & 15);
    const i32x4 raw = __builtin_nontemporal_load((const i32x4*)(x + off));   // read once
    float v[8];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        v[2 * d] = bf16_to_f32((uint16_t)((uint32_t)raw[d] & 0xFFFF));
        v[2 * d + 1] = bf16_to_f32((uint16_t)((uint32_t)raw[d] >> 16));
    }
    float amax = 0.f;
#pragma unroll
    for (int d = 0; d < 8; ++d) amax = fmaxf(amax, fabsf(v[d]));
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    int s = pow2_exponent_448(amax);
    s = s < -127 ? -127 : (s > 127 ? 127 : s);
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
        w[h] = f32x2_to_e4m3(ldexpf(v[4 * h], -s), ldexpf(v[4 * h + 1], -s)) |
               (f32x2_to_e4m3(ldexpf(v[4 * h + 2], -s), ldexpf(v[4 * h + 3], -s)) << 16);
    if (live) {
        *(uint2*)(xq + off) = make_uint2(w[0], w[1]);
        if ((lane & 15) == 0) xs[(size_t)r * groups + g] = (uint8_t)(s + 127);
    }
}

hipError_t launch_quant_act(const uint16_t* x, int rows, int cols, uint8_t* codes, uint8_t* exps, hipStream_t stream) {
    const long items = (long)rows * (cols / MOE_ACT_G);   // 16 per workgroup
    MOE_LAUNCH(K_QUANT_ACT, stream, quant_act_kernel, dim3((unsigned)((items + 15) / 16)), dim3(256), 0, stream, x,
               rows, cols, codes, exps);
    return hipGetLastError();
}

// ------------------------------------------------------------ shared GEMM pieces
constexpr int GT = 256;         // threads per workgroup (4 waves)
constexpr int LDS_ROW = 144;    // 128 bytes of K + 16 bytes of padding

// Workgroup barrier that waits only for the wave's LDS traffic. The fence of
// __syncthreads() also waits for every global load in flight, which would
// drain the next K step's loads at each barrier of the step loop.
__device__ __forceinline__ void barrier_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ------------------------------------------------------------ gemm1
// Tile: BM pair rows x 128 inter columns (128 gate rows + 128 up rows of W13).
// Wave w owns inter columns [32w, 32w+32).
template <int BM>
__device__ __forceinline__ void gemm1_tile(const GPool& pool, const uint8_t* __restrict__ xq,
                                           const uint8_t* __restrict__ xs, int NP, int k,
                                           const int32_t* __restrict__ sorted_pair,
                                           const int32_t* __restrict__ block_slot,
                                           const int32_t* __restrict__ n_padded, int H, int I,
                                           uint8_t* __restrict__ hq, uint8_t* __restrict__ hs,
                                           const int mt_idx, const int nt_idx) {
    constexpr int MT = BM / 16;
    extern __shared__ __align__(16) uint8_t smem[];
    uint8_t* sA = smem;                               // [BM][LDS_ROW]
    uint8_t* sB = sA + BM * LDS_ROW;                  // [256][LDS_ROW]: rows 0..127 gate, 128..255 up
    int* s_tok = (int*)(sB + 256 * LDS_ROW);          // [BM]
    uint8_t* s_xs = (uint8_t*)(s_tok + BM);           // [BM][groups]
    const int groups = H / MOE_ACT_G;
    float* s_amax = (float*)(s_xs + ((BM * groups + 15) / 16) * 16);   // [4][BM]

    if (mt_idx >= *n_padded / BM) return;
    // an unusable slot (not resident, outside the pool, format larger than the stride) adds nothing
    const int slot = usable_slot(block_slot[mt_idx], pool.n_slots, pool.fmt_ok, pool.fmt);
    if (slot < 0) return;
    const uint8_t* sb = pool.base + (size_t)slot * pool.stride;
    const int fmt_slot = pool.fmt[slot];
    const int fmt = fmt_slot;
    const int lane = lane_id(), wv = threadIdx.x / MOE_WAVE, m = lane & 15, q = lane >> 4;
    const int c0 = nt_idx * 128;                      // first inter column of the tile
    const int ncols = min(128, I - c0);               // valid inter columns

    for (int r = threadIdx.x; r < BM; r += GT) {
        int p = sorted_pair[mt_idx * BM + r];
        s_tok[r] = p < NP ? p / k : -1;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < BM * groups; i += GT) {
        int r = i / groups, g = i % groups;
        int t = s_tok[r];
        s_xs[i] = t >= 0 ? xs[(size_t)t * groups + g] : (uint8_t)127;
    }

    f32x4 acc[MT][2][2];                              // [m tile][gate/up][n tile]
#pragma unroll
    for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int c = 0; c < 2; ++c) acc[a][b][c] = f32x4{0, 0, 0, 0};

    const uint8_t* w13 = sb;
    const uint8_t* sz13 = sb + pool.off[1][1];
    // K step g: every load of the step first, then the LDS writes. A: BM
    // gathered rows x 128 bytes; B: 256 weight rows x 128 K (gate rows c0..,
    // up rows I+c0..); int4: the codes, the zeros of the rows staged and the
    // scales of this lane's four output columns. The loads of step g + 1 are
    // issued once step g sits in LDS, so they fly during its matrix work.
    constexpr int NA = (BM * 8 + GT - 1) / GT, NB = 256 * 8 / GT;
    i32x4 va[NA];
    i32x4 vb[NB];
    float zb[NB];
    float sgn[2][2] = {{0.f, 0.f}, {0.f, 0.f}};      // scales of the step being loaded
    auto load_step = [&](int g) __attribute__((always_inline)) {
        const int k0 = g * 128;
#pragma unroll
        for (int u = 0; u < NA; ++u) {
            const int i = threadIdx.x + u * GT;
            const int t = i < BM * 8 ? s_tok[i >> 3] : -1;
            // (loads from clamped addresses, values selected after: no branch
            // around a load, so the loads of the next step stay in flight)
            const i32x4 ld = *(const i32x4*)(xq + (size_t)max(t, 0) * H + k0 + (i & 7) * 16);
            va[u] = t >= 0 ? ld : i32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int i = threadIdx.x + u * GT;
            const int r = i >> 3, ch = i & 7, col = r & 127;
            const int wrow = (r < 128 ? 0 : I) + c0 + (col < ncols ? col : 0);
            if (fmt == 0) {
                const i32x4 ld = *(const i32x4*)(w13 + (size_t)wrow * H + k0 + ch * 16);
                vb[u] = col < ncols ? ld : i32x4{0, 0, 0, 0};
            } else {
                const uint2 ld = *(const uint2*)(w13 + (size_t)wrow * (H / 2) + (k0 + ch * 16) / 2);
                const uint2 pk = col < ncols ? ld : make_uint2(0u, 0u);
                vb[u] = i32x4{(int)pk.x, (int)pk.y, 0, 0};
                zb[u] = f16x2_at(sz13 + ((size_t)wrow * groups + g) * 4).y;
            }
        }
        if (fmt == 1) {
#pragma unroll
            for (int gu = 0; gu < 2; ++gu)
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    const int col = wv * 32 + n * 16 + m;
                    const int wrow = (gu ? I : 0) + c0 + (col < ncols ? col : 0);
                    sgn[gu][n] = f16x2_at(sz13 + ((size_t)wrow * groups + g) * 4).x;
                }
        }
    };
    load_step(0);
    for (int g = 0; g < groups; ++g) {
#pragma unroll
        for (int u = 0; u < NA; ++u) {
            const int i = threadIdx.x + u * GT;
            if (i < BM * 8) *(i32x4*)(sA + (i >> 3) * LDS_ROW + (i & 7) * 16) = va[u];
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int i = threadIdx.x + u * GT;
            const int r = i >> 3, ch = i & 7, col = r & 127;
            i32x4 v = vb[u];
            if (fmt == 1) {
                uint32_t o[4];
                int4_to_e4m3_16(make_uint2((uint32_t)vb[u][0], (uint32_t)vb[u][1]), zb[u], o);
                v = col < ncols ? i32x4{(int)o[0], (int)o[1], (int)o[2], (int)o[3]} : i32x4{0, 0, 0, 0};
            }
            *(i32x4*)(sB + r * LDS_ROW + ch * 16) = v;
        }
        float sgu[2][2];
#pragma unroll
        for (int gu = 0; gu < 2; ++gu)
#pragma unroll
            for (int n = 0; n < 2; ++n) sgu[gu][n] = sgn[gu][n];
        barrier_lds();
        load_step(min(g + 1, groups - 1));           // (no branch around the loads: the last step reloads itself)
        // B fragments of this wave: gate cols 32w + 16n + m, up cols likewise
        i32x8 bf[2][2];
#pragma unroll
        for (int gu = 0; gu < 2; ++gu)
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const uint8_t* p = sB + (gu * 128 + wv * 32 + n * 16 + m) * LDS_ROW + q * 32;
                i32x4 lo = *(const i32x4*)p, hi = *(const i32x4*)(p + 16);
                bf[gu][n] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
#pragma unroll
        for (int a = 0; a < MT; ++a) {
            const uint8_t* p = sA + (a * 16 + m) * LDS_ROW + q * 32;
            i32x4 lo = *(const i32x4*)p, hi = *(const i32x4*)(p + 16);
            i32x8 af = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            const int sa = s_xs[(a * 16 + m) * groups + g];
            if (fmt == 0) {
#pragma unroll
                for (int gu = 0; gu < 2; ++gu)
#pragma unroll
                    for (int n = 0; n < 2; ++n) acc[a][gu][n] = mfma_fp8_16x16x128(af, bf[gu][n], acc[a][gu][n], sa, 127);
            } else {
#pragma unroll
                for (int gu = 0; gu < 2; ++gu)
#pragma unroll
                    for (int n = 0; n < 2; ++n) {
                        f32x4 t4 = mfma_fp8_16x16x128(af, bf[gu][n], f32x4{0, 0, 0, 0}, sa, 127);
                        acc[a][gu][n] += sgu[gu][n] * t4;
                    }
            }
        }
        barrier_lds();
    }

    // epilogue: row scales, silu(gate) * up, per-(row, 128 cols) quantization
    const float* s13 = (const float*)(sb + pool.off[0][1]);
    float hv[MT][2][4];
    float rmax[MT][4];
#pragma unroll
    for (int a = 0; a < MT; ++a) {
#pragma unroll
        for (int i = 0; i < 4; ++i) rmax[a][i] = 0.f;
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int col = wv * 32 + n * 16 + m;
            const bool ok = col < ncols;
            float sg = 1.f, su = 1.f;
            if (fmt == 0 && ok) { sg = s13[c0 + col]; su = s13[I + c0 + col]; }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float h = ok ? silu(acc[a][0][n][i] * sg) * (acc[a][1][n][i] * su) : 0.f;
                hv[a][n][i] = h;
                rmax[a][i] = fmaxf(rmax[a][i], fabsf(h));
            }
        }
    }
    // max over the 16 lanes sharing q (same rows), then over the 4 waves
#pragma unroll
    for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float v = rmax[a][i];
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
            rmax[a][i] = v;
        }
    if (m == 0) {
#pragma unroll
        for (int a = 0; a < MT; ++a)
#pragma unroll
            for (int i = 0; i < 4; ++i) s_amax[wv * BM + a * 16 + 4 * q + i] = rmax[a][i];
    }
    __syncthreads();
    uint8_t* sH = sA;                                 // reuse: [BM][LDS_ROW] codes
    const int hgroups = (I + MOE_ACT_G - 1) / MOE_ACT_G;
#pragma unroll
    for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = a * 16 + 4 * q + i;
            float amax = fmaxf(fmaxf(s_amax[row], s_amax[BM + row]), fmaxf(s_amax[2 * BM + row], s_amax[3 * BM + row]));
            int s = pow2_exponent_448(amax);
            s = s < -127 ? -127 : (s > 127 ? 127 : s);
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const int col = wv * 32 + n * 16 + m;
                sH[row * LDS_ROW + col] = (uint8_t)(f32x2_to_e4m3(ldexpf(hv[a][n][i], -s), 0.f) & 0xFF);
            }
            if (wv == 0 && m == 0) {
                const int p = sorted_pair[mt_idx * BM + row];
                (void)p;
                hs[(size_t)(mt_idx * BM + row) * hgroups + nt_idx] = (uint8_t)(s + 127);
            }
        }
    __syncthreads();
    // coalesced store of the code tile: row r -> hq[(mt*BM + r) * I + c0 .. + ncols]
    for (int i = threadIdx.x; i < BM * 8; i += GT) {
        int r = i >> 3, ch = i & 7;
        if (ch * 16 < ncols)
            *(i32x4*)(hq + (size_t)(mt_idx * BM + r) * I + c0 + ch * 16) = *(const i32x4*)(sH + r * LDS_ROW + ch * 16);
    }
}

// ------------------------------------------------------------ gemm2
// Tile: BM pair rows x 128 hidden columns; wave w owns columns [32w, 32w+32).
template <int BM>
__device__ __forceinline__ void gemm2_tile(const GPool& pool, int NP, int k, const float* __restrict__ topk_w,
                                           const int32_t* __restrict__ sorted_pair,
                                           const int32_t* __restrict__ block_slot,
                                           const int32_t* __restrict__ n_padded, int H, int I,
                                           const uint8_t* __restrict__ hq, const uint8_t* __restrict__ hs,
                                           uint16_t* __restrict__ ybuf, const int mt_idx,
                                           const int nt_idx) {
    constexpr int MT = BM / 16;
    extern __shared__ __align__(16) uint8_t smem[];
    uint8_t* sA = smem;                               // [BM][LDS_ROW]
    uint8_t* sB = sA + BM * LDS_ROW;                  // [128][LDS_ROW]
    if (mt_idx >= *n_padded / BM) return;
    const int slot = usable_slot(block_slot[mt_idx], pool.n_slots, pool.fmt_ok, pool.fmt);
    const int lane = lane_id(), wv = threadIdx.x / MOE_WAVE, m = lane & 15, q = lane >> 4;
    const int n0 = nt_idx * 128;
    if (slot < 0) {                                   // unusable slot (e.g. not resident): its pairs add zero
        if (block_slot[mt_idx] == MOE_SLOT_DEFERRED) return;   // (a deferred block's rows are left as they are)
        for (int i = threadIdx.x; i < BM * 16; i += GT) {
            int r = i >> 4, ch = i & 15;
            int p = sorted_pair[mt_idx * BM + r];
            if (p < NP) *(i32x4*)(ybuf + (size_t)p * H + n0 + ch * 8) = i32x4{0, 0, 0, 0};
        }
        return;
    }
    const uint8_t* sb = pool.base + (size_t)slot * pool.stride;
    // (int4 needs inter % 128 == 0)
    const int fmt = (int)pool.fmt[slot];
    const int hgroups = (I + MOE_ACT_G - 1) / MOE_ACT_G;
    const int wgroups = I / MOE_INT4_G;
    f32x4 acc[MT][2];
#pragma unroll
    for (int a = 0; a < MT; ++a) { acc[a][0] = f32x4{0, 0, 0, 0}; acc[a][1] = f32x4{0, 0, 0, 0}; }
    const uint8_t* w2 = sb + pool.off[fmt][2];
    const uint8_t* sz2 = sb + pool.off[1][3];
    // K step g: every load of the step first (A: the block's h codes; B: 128
    // W2 rows x 128 K, int4 with the zeros of the rows staged and the scales
    // of this lane's two output columns), then the LDS writes; the loads of
    // step g + 1 fly during step g's matrix work
    constexpr int NA = BM * 8 / GT, NB = 128 * 8 / GT;
    i32x4 va[NA];
    i32x4 vb[NB];
    float zb[NB];
    float scn[2] = {0.f, 0.f};
    auto load_step = [&](int g) __attribute__((always_inline)) {
        const int k0 = g * 128;
        const int kv = min(128, I - k0);              // valid K bytes in this step
#pragma unroll
        for (int u = 0; u < NA; ++u) {
            const int i = threadIdx.x + u * GT, r = i >> 3, ch = i & 7;
            const uint8_t* src = hq + (size_t)(mt_idx * BM + r) * I + k0 + ch * 16;
            va[u] = ch * 16 < kv ? *(const i32x4*)src : i32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int i = threadIdx.x + u * GT, r = i >> 3, ch = i & 7;
            if (fmt == 0) {
                vb[u] = ch * 16 < kv ? *(const i32x4*)(w2 + (size_t)(n0 + r) * I + k0 + ch * 16) : i32x4{0, 0, 0, 0};
            } else {
                const uint2 pk = *(const uint2*)(w2 + (size_t)(n0 + r) * (I / 2) + (k0 + ch * 16) / 2);
                vb[u] = i32x4{(int)pk.x, (int)pk.y, 0, 0};
                zb[u] = f16x2_at(sz2 + ((size_t)(n0 + r) * wgroups + g) * 4).y;
            }
        }
        if (fmt == 1) {
#pragma unroll
            for (int n = 0; n < 2; ++n)
                scn[n] = f16x2_at(sz2 + ((size_t)(n0 + wv * 32 + n * 16 + m) * wgroups + g) * 4).x;
        }
    };
    load_step(0);
    for (int g = 0; g < hgroups; ++g) {
#pragma unroll
        for (int u = 0; u < NA; ++u) {
            const int i = threadIdx.x + u * GT;
            *(i32x4*)(sA + (i >> 3) * LDS_ROW + (i & 7) * 16) = va[u];
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int i = threadIdx.x + u * GT;
            i32x4 v = vb[u];
            if (fmt == 1) {
                uint32_t o[4];
                int4_to_e4m3_16(make_uint2((uint32_t)vb[u][0], (uint32_t)vb[u][1]), zb[u], o);
                v = i32x4{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
            }
            *(i32x4*)(sB + (i >> 3) * LDS_ROW + (i & 7) * 16) = v;
        }
        const float sc[2] = {scn[0], scn[1]};
        barrier_lds();
        load_step(min(g + 1, hgroups - 1));          // (no branch around the loads: the last step reloads itself)
        i32x8 bf[2];
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const uint8_t* p = sB + (wv * 32 + n * 16 + m) * LDS_ROW + q * 32;
            i32x4 lo = *(const i32x4*)p, hi = *(const i32x4*)(p + 16);
            bf[n] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int a = 0; a < MT; ++a) {
            const uint8_t* p = sA + (a * 16 + m) * LDS_ROW + q * 32;
            i32x4 lo = *(const i32x4*)p, hi = *(const i32x4*)(p + 16);
            i32x8 af = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            const int sa = hs[(size_t)(mt_idx * BM + a * 16 + m) * hgroups + g];
            if (fmt == 0) {
#pragma unroll
                for (int n = 0; n < 2; ++n) acc[a][n] = mfma_fp8_16x16x128(af, bf[n], acc[a][n], sa, 127);
            } else {
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    f32x4 t4 = mfma_fp8_16x16x128(af, bf[n], f32x4{0, 0, 0, 0}, sa, 127);
                    acc[a][n] += sc[n] * t4;
                }
            }
        }
        barrier_lds();
    }
    // epilogue: row scale, route weight, bf16 rows staged in LDS for wide stores
    const float* s2 = (const float*)(sb + pool.off[0][3]);
    uint16_t* sY = (uint16_t*)smem;                   // [BM][128 + 8] bf16
    constexpr int YROW = 136;
#pragma unroll
    for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = a * 16 + 4 * q + i;
            const int p = sorted_pair[mt_idx * BM + row];
            const float wt = p < NP ? topk_w[p] : 0.f;
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const int col = wv * 32 + n * 16 + m;
                float y = acc[a][n][i] * wt;
                if (fmt == 0) y *= s2[n0 + col];
                sY[row * YROW + col] = f32_to_bf16(y);
            }
        }
    __syncthreads();
    for (int i = threadIdx.x; i < BM * 16; i += GT) {
        int r = i >> 4, ch = i & 15;
        int p = sorted_pair[mt_idx * BM + r];
        if (p < NP) *(i32x4*)(ybuf + (size_t)p * H + n0 + ch * 8) = *(const i32x4*)(sY + r * YROW + ch * 8);
    }
}

// ------------------------------------------------------------ kernels
// Grid (column tiles, blocks).
template <int BM>
__global__ void __launch_bounds__(GT) gemm1_fp8_kernel(GPool pool, const uint8_t* __restrict__ xq,
                                                      const uint8_t* __restrict__ xs, int NP, int k,
                                                      const int32_t* __restrict__ sorted_pair,
                                                      const int32_t* __restrict__ block_slot,
                                                      const int32_t* __restrict__ n_padded, int H, int I,
                                                      uint8_t* __restrict__ hq, uint8_t* __restrict__ hs) {
    gemm1_tile<BM>(pool, xq, xs, NP, k, sorted_pair, block_slot, n_padded, H, I, hq, hs, blockIdx.y, blockIdx.x);
}

template <int BM>
__global__ void __launch_bounds__(GT, 2) gemm2_fp8_kernel(GPool pool, int NP, int k, const float* __restrict__ topk_w,
                                                      const int32_t* __restrict__ sorted_pair,
                                                      const int32_t* __restrict__ block_slot,
                                                      const int32_t* __restrict__ n_padded, int H, int I,
                                                      const uint8_t* __restrict__ hq, const uint8_t* __restrict__ hs,
                                                      uint16_t* __restrict__ ybuf) {
    gemm2_tile<BM>(pool, NP, k, topk_w, sorted_pair, block_slot, n_padded, H, I, hq, hs, ybuf, blockIdx.y,
                   blockIdx.x);
}

// ------------------------------------------------------------ host side
static size_t up256(size_t n) { return (n + 255) / 256 * 256; }

struct GroupedWs {
    uint8_t *xq, *xs, *hq, *hs;
    uint16_t* ybuf;
    void* mm;             // workspace of the pipelined kernels
    size_t total;
};

static GroupedWs grouped_ws_layout(void* base, int T, int k, int H, int I, int cap) {
    GroupedWs w;
    uint8_t* p = (uint8_t*)base;
    size_t o = 0;
    w.xq = p + o; o += up256((size_t)T * H);
    w.xs = p + o; o += up256((size_t)T * (H / MOE_ACT_G));
    w.hq = p + o; o += up256((size_t)cap * I);
    w.hs = p + o; o += up256((size_t)cap * ((I + MOE_ACT_G - 1) / MOE_ACT_G));
    w.ybuf = (uint16_t*)(p + o); o += up256((size_t)T * k * H * 2);
    w.mm = p + o; o += up256(mfma_ws_bytes(H, cap));
    w.total = o;
    return w;
}

size_t grouped_workspace_bytes(int T, int k, int H, int I, int cap) {
    return grouped_ws_layout(nullptr, T, k, H, I, cap).total;
}

template <int BM>
static size_t gemm1_smem(int H) {
    return (size_t)BM * LDS_ROW + 256 * LDS_ROW + BM * 4 + ((BM * (H / MOE_ACT_G) + 15) / 16) * 16 + 4 * BM * 4;
}
template <int BM>
static size_t gemm2_smem() {
    size_t a = (size_t)BM * LDS_ROW + 128 * LDS_ROW;
    size_t b = (size_t)BM * 136 * 2;
    return a > b ? a : b;
}

template <int BM>
static hipError_t launch_grouped_bm(const PoolArgs& pa, const GPool& gp, const GroupedWs& w, const uint16_t* x, int T, int k,
                                    const float* topk_w, const int32_t* sorted_pair, const int32_t* block_slot,
                                    const int32_t* n_padded, int cap, int H, int I, uint16_t* out,
                                    hipStream_t stream, FfnPass pass) {
    const int NP = T * k;
    const long qitems = (long)T * (H / MOE_ACT_G);      // 16 per block
    MOE_LAUNCH(K_QUANT_ACT, stream, quant_act_kernel, dim3((unsigned)((qitems + 15) / 16)), dim3(256), 0, stream, x, T, H,
               w.xq, w.xs);
    dim3 g1((I + 127) / 128, cap / BM);
    size_t sm1 = gemm1_smem<BM>(H);
    dim3 g2(H / 128, cap / BM);
    hipError_t e;
    if (BM == 128 && mfma_path_ok(H, I)) {          // (int4_ring_ok(H, I) then holds too)
        // FP8 blocks on the pipelined matrix-core kernels; the prep kernel
        // (first of them) lists the other blocks (int4 or not usable), which
        // run on the int4 ring kernels (those write zero rows for unusable ones)
        const int* olist = nullptr;
        const int* n_olist = nullptr;
        mfma_other_list(w.mm, H, cap, &olist, &n_olist);
        const int oy = cap / BM < 512 ? cap / BM : 512;     // bound on the listed blocks
        e = launch_mfma_ffn(pa, w.xq, w.xs, NP, k, topk_w, sorted_pair, block_slot, n_padded, cap, w.hq, w.hs,
                            w.ybuf, w.mm, 0, stream);
        if (e != hipSuccess) return e;
        const int32_t* tokrow = nullptr;
        const float* wsort = nullptr;
        const uint8_t* scl = nullptr;
        mfma_prep_arrays(w.mm, cap, &tokrow, &wsort, &scl);
        e = launch_gemm1_int4_ring(pa, w.xq, tokrow, scl, block_slot, I, w.hq, w.hs, olist, n_olist, oy, stream);
        if (e != hipSuccess) return e;
        e = launch_mfma_ffn(pa, w.xq, w.xs, NP, k, topk_w, sorted_pair, block_slot, n_padded, cap, w.hq, w.hs,
                            w.ybuf, w.mm, 1, stream);
        if (e != hipSuccess) return e;
        e = launch_gemm2_int4_ring(pa, NP, wsort, sorted_pair, block_slot, I, w.hq, w.hs, w.ybuf, olist, n_olist, oy,
                                   stream);
        if (e != hipSuccess) return e;
    } else {
        MOE_LAUNCH(K_GEMM1_TILE, stream, gemm1_fp8_kernel<BM>, g1, dim3(GT), sm1, stream, gp, w.xq, w.xs, NP, k,
                   sorted_pair, block_slot, n_padded, H, I, w.hq, w.hs);
        MOE_LAUNCH(K_GEMM2_TILE, stream, gemm2_fp8_kernel<BM>, g2, dim3(GT), gemm2_smem<BM>(), stream, gp, NP, k,
                   topk_w, sorted_pair, block_slot, n_padded, H, I, w.hq, w.hs, w.ybuf);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (pass == FFN_PASS) return hipSuccess;          // rows only: a later pass combines
    return launch_combine_bf16(w.ybuf, topk_w, T, k, H, out, stream);
}

hipError_t launch_ffn_grouped(const PoolArgs& pa, const uint16_t* x, int T, int k, const float* topk_w,
                              const int32_t* sorted_pair, const int32_t* block_slot, const int32_t* n_padded,
                              int cap, int block_m, uint16_t* out, void* ws, hipStream_t stream, FfnPass pass) {
    GPool gp;
    gp.base = (const uint8_t*)pa.base;
    gp.stride = pa.stride;
    gp.fmt = pa.fmt;
    for (int f = 0; f < 2; ++f)
        for (int p = 0; p < 4; ++p) gp.off[f][p] = pa.off[f][p];
    gp.n_slots = pa.n_slots;
    gp.fmt_ok = pa.fmt_ok;
    GroupedWs w = grouped_ws_layout(ws, T, k, pa.hidden, pa.inter, cap);
    if (pass == FFN_WHOLE && debug_poison_on()) {     // activation codes, h and y rows: NaN until written
        hipError_t e = launch_poison(ws, (size_t)((uint8_t*)w.mm - (uint8_t*)ws), stream);
        if (e != hipSuccess) return e;
    }
    if (block_m == 64)
        return launch_grouped_bm<64>(pa, gp, w, x, T, k, topk_w, sorted_pair, block_slot, n_padded, cap, pa.hidden,
                                     pa.inter, out, stream, pass);
    if (block_m == 128)
        return launch_grouped_bm<128>(pa, gp, w, x, T, k, topk_w, sorted_pair, block_slot, n_padded, cap, pa.hidden,
                                      pa.inter, out, stream, pass);
    return hipErrorInvalidValue;
}

}  // namespace moe
