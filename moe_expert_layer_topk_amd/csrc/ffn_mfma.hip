// Expert FFN, grouped FP8 matrix-core kernels for large batches (block_m 128).
//
// MOE-GEN explainer (aibr.jp), sections 1 and 3: once tokens are gathered per
// expert module each expert runs one dense contraction over many rows, the
// case FP8 matrix cores are built for. Weights come from the expert's VRAM
// slot (vllm-expert-pager article, rand.pepabo.com, "hierarchical paging";
// Table 1 set-up: w13 = gate+up, w2 = down).
//
// Both kernels compute a 128 x 256 output tile with 4 waves (2 x 2, 64 x 128
// per wave, 32 v_mfma_scale_f32_16x16x128_f8f6f4 per 128-wide K step):
// * operands reach LDS through direct-to-LDS 16-byte loads (no register
//   staging), 3 stages deep: while step g is multiplied, steps g+1 and g+2
//   are in flight;
// * each 128-byte LDS row stores its 16-byte chunks XOR-swizzled by the row
//   index, chosen through the source address of each lane, so the 16 lanes
//   reading one fragment column hit different banks;
// * the tile order is remapped so that the workgroups of one XCD (blocks are
//   dealt round-robin over the 8 XCDs) work on consecutive tiles: the same
//   token rows and the same expert's weights stay in that XCD's L2;
// * the power-of-two activation scales are E8M0 bytes fed to the scaled
//   matrix instruction, so scaling is free inside the K loop.
// gemm1 gathers the token rows of a block of pairs and multiplies them by
// 128 gate and the matching 128 up rows of W13; the epilogue applies the
// row scales, silu(gate) * up and quantizes h per (row, 128 columns).
// gemm2 multiplies 128 rows of h by 256 rows of W2 and writes
// w[t][j] * y, in bf16, to the pair's row of the combine buffer.
// Tiles whose slot is stored int4-g128 are skipped here; the simpler kernels
// of ffn_grouped.hip, launched in their int4-only mode, multiply those.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

constexpr int MM_BM = 128;
constexpr int MM_BN = 256;
constexpr int MM_BK = 128;
constexpr int MM_ST = 3;
constexpr int MM_THREADS = 256;
constexpr int MM_STAGE = (MM_BM + MM_BN) * MM_BK;   // 48 KiB: A rows, then B rows
constexpr int MM_DMA = (MM_BM + MM_BN) / 4 / 8;       // direct-to-LDS loads per wave per stage

struct MPool {
    const uint8_t* base;
    size_t stride;
    const uint8_t* fmt;
    size_t off[2][4];
};

// s_waitcnt with only vmcnt limited (expcnt and lgkmcnt left open)
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without the release fence that __syncthreads() adds: that
// fence waits for every outstanding global load, direct-to-LDS ones included,
// which would drain the stages still in flight. Callers order their own LDS
// traffic with wait_vm / lgkmcnt before it.
__device__ __forceinline__ void barrier_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until the oldest stage in flight has landed, leaving the `ahead` stages
// issued after it outstanding (loads of one wave complete in issue order).
__device__ __forceinline__ void wait_stage(int ahead) {
    if (ahead >= 2) wait_vm<2 * MM_DMA>();
    else if (ahead == 1) wait_vm<MM_DMA>();
    else wait_vm<0>();
}

__device__ __forceinline__ void lds_dma16(const void* src, uint8_t* lds_dst) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_dst, 16, 0, 0);
}

// tile id such that the workgroups of one XCD take consecutive tiles
__device__ __forceinline__ int xcd_tile(int bid, int G) {
    const int x = bid & 7, idx = bid >> 3, per = G >> 3, rem = G & 7;
    return x * per + (x < rem ? x : rem) + idx;
}

// 32 codes of LDS row r (128-byte rows, swizzled chunks), K bytes [32q, 32q+32)
__device__ __forceinline__ i32x8 lds_frag(const uint8_t* st, int r, int q) {
    const int sw = r & 7;
    const i32x4 lo = *(const i32x4*)(st + r * 128 + (((2 * q) ^ sw) << 4));
    const i32x4 hi = *(const i32x4*)(st + r * 128 + (((2 * q + 1) ^ sw) << 4));
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// One wave's share of a stage: rows [row0, row0 + 8N) of an operand, 8 rows
// per instruction; lane i fills LDS chunk i % 8 of row row0 + 8j + i / 8 with
// the global chunk that the swizzle puts there.
template <int N>
__device__ __forceinline__ void dma_rows(uint8_t* st, int row0, int lane, const uint8_t* const (&src_row)[N],
                                         int k0) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
        const int r = row0 + j * 8 + (lane >> 3);
        const int c = (lane & 7) ^ (r & 7);
        lds_dma16(src_row[j] + k0 + c * 16, st + (row0 + j * 8) * 128);
    }
}

// ---------------------------------------------------------------- gemm1

__global__ void __launch_bounds__(MM_THREADS, 1) gemm1_mfma_kernel(MPool pool, const uint8_t* __restrict__ xq,
                                                                  const uint8_t* __restrict__ xs, int NP, int k,
                                                                  const int32_t* __restrict__ sorted_pair,
                                                                  const int32_t* __restrict__ block_slot,
                                                                  const int32_t* __restrict__ n_padded, int H,
                                                                  int I, uint8_t* __restrict__ hq,
                                                                  uint8_t* __restrict__ hs) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int NT = (I + 127) / 128;
    const int tile = xcd_tile(blockIdx.x, gridDim.x);
    const int mt = tile / NT, nt = tile % NT;
    if (mt >= *n_padded / MM_BM) return;
    const int slot = block_slot[mt];
    if (slot < 0) return;
    const int groups = H / 128;
    uint8_t* st0 = smem;
    int* s_tok = (int*)(smem + MM_ST * MM_STAGE);               // [128]
    float* s_amax = (float*)(s_tok + MM_BM);                    // [2][128]
    uint8_t* s_xs = (uint8_t*)(s_amax + 2 * MM_BM);             // [128][groups]
    const int lane = lane_id(), wv = threadIdx.x / MOE_WAVE, m = lane & 15, q = lane >> 4;
    const int mw = wv & 1, nw = wv >> 1;
    const int c0 = nt * 128;
    const int ncols = min(128, I - c0);
    if (threadIdx.x < MM_BM) {
        const int p = sorted_pair[mt * MM_BM + threadIdx.x];
        s_tok[threadIdx.x] = p < NP ? p / k : -1;
    }
    if (pool.fmt[slot] == 1) return;                  // int4 slot
    __syncthreads();
    const uint8_t* sb = pool.base + (size_t)slot * pool.stride;
    for (int i = threadIdx.x; i < MM_BM * groups; i += MM_THREADS) {
        const int r = i / groups, g = i % groups;
        const int t = s_tok[r];
        s_xs[i] = t >= 0 ? xs[(size_t)t * groups + g] : (uint8_t)127;
    }
    // source rows of this wave's DMA share: A rows [32 wv, 32 wv + 32), B rows [64 wv, 64 wv + 64)
    const uint8_t* srcA[4];
    const uint8_t* srcB[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int t = s_tok[wv * 32 + j * 8 + (lane >> 3)];
        srcA[j] = xq + (size_t)(t < 0 ? 0 : t) * H;            // padding rows read token 0; outputs unused
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int rb = wv * 64 + j * 8 + (lane >> 3);
        const int col = rb & 127;
        const int wrow = (rb < 128 ? 0 : I) + c0 + (col < ncols ? col : 0);
        srcB[j] = sb + (size_t)wrow * H;
    }
    auto issue = [&](int g) {
        uint8_t* st = st0 + (g % MM_ST) * MM_STAGE;
        dma_rows<4>(st, wv * 32, lane, srcA, g * 128);
        dma_rows<8>(st + MM_BM * 128, wv * 64, lane, srcB, g * 128);
    };
    f32x4 acc[4][8];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int n = 0; n < 8; ++n) acc[a][n] = f32x4{0, 0, 0, 0};
    for (int g = 0; g < MM_ST - 1 && g < groups; ++g) issue(g);
    for (int g = 0; g < groups; ++g) {
        wait_stage(min(MM_ST - 2, groups - 1 - g));
        barrier_lds();
        if (g + MM_ST - 1 < groups) issue(g + MM_ST - 1);
        const uint8_t* st = st0 + (g % MM_ST) * MM_STAGE;
        const uint8_t* sB = st + MM_BM * 128;
        i32x8 bf[8];
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            // n < 4: gate rows nw*64 + 16n; n >= 4: up rows 128 + nw*64 + 16(n-4)
            const int rb = (n < 4 ? 0 : 128) + nw * 64 + (n & 3) * 16 + m;
            bf[n] = lds_frag(sB, rb, q);
        }
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int r = mw * 64 + a * 16 + m;
            const i32x8 af = lds_frag(st, r, q);
            const int sa = s_xs[r * groups + g];
#pragma unroll
            for (int n = 0; n < 8; ++n) acc[a][n] = mfma_fp8_16x16x128(af, bf[n], acc[a][n], sa, 127);
        }
    }
    // ---- epilogue: row scales, silu(gate) * up, per-(row, 128 columns) power-of-two quantization
    const float* s13 = (const float*)(sb + pool.off[0][1]);
    float sg[4], su[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
        const int col = nw * 64 + n * 16 + m;
        const bool ok = col < ncols;
        sg[n] = ok ? s13[c0 + col] : 0.f;
        su[n] = ok ? s13[I + c0 + col] : 0.f;
    }
    float hv[4][4][4];
    float rmax[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float mx = 0.f;
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                const float h = silu(acc[a][n][i] * sg[n]) * (acc[a][n + 4][i] * su[n]);
                hv[a][n][i] = h;
                mx = fmaxf(mx, fabsf(h));
            }
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
            rmax[a][i] = mx;
        }
    if (m == 0) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int i = 0; i < 4; ++i) s_amax[nw * MM_BM + mw * 64 + a * 16 + 4 * q + i] = rmax[a][i];
    }
    __syncthreads();                                   // also: every wave is done with the stages
    uint8_t* sH = st0;                                 // [128 rows][128 B] codes
    const int hgroups = (I + MOE_ACT_G - 1) / MOE_ACT_G;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = mw * 64 + a * 16 + 4 * q + i;
            int e = pow2_exponent_448(fmaxf(s_amax[row], s_amax[MM_BM + row]));
            e = e < -127 ? -127 : (e > 127 ? 127 : e);
#pragma unroll
            for (int n = 0; n < 4; ++n)
                sH[row * 128 + nw * 64 + n * 16 + m] = (uint8_t)(f32x2_to_e4m3(ldexpf(hv[a][n][i], -e), 0.f) & 0xFF);
            if (nw == 0 && m == 0) hs[(size_t)(mt * MM_BM + row) * hgroups + nt] = (uint8_t)(e + 127);
        }
    __syncthreads();
    for (int i = threadIdx.x; i < MM_BM * 8; i += MM_THREADS) {
        const int r = i >> 3, ch = i & 7;
        if (ch * 16 < ncols)
            *(i32x4*)(hq + (size_t)(mt * MM_BM + r) * I + c0 + ch * 16) = *(const i32x4*)(sH + r * 128 + ch * 16);
    }
}

// ---------------------------------------------------------------- gemm2

__global__ void __launch_bounds__(MM_THREADS, 1) gemm2_mfma_kernel(MPool pool, int NP, const float* __restrict__ topk_w,
                                                                  const int32_t* __restrict__ sorted_pair,
                                                                  const int32_t* __restrict__ block_slot,
                                                                  const int32_t* __restrict__ n_padded, int H,
                                                                  int I, const uint8_t* __restrict__ hq,
                                                                  const uint8_t* __restrict__ hs,
                                                                  uint16_t* __restrict__ ybuf) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int NT = H / MM_BN;
    const int tile = xcd_tile(blockIdx.x, gridDim.x);
    const int mt = tile / NT, nt = tile % NT;
    if (mt >= *n_padded / MM_BM) return;
    const int slot = block_slot[mt];
    const int lane = lane_id(), wv = threadIdx.x / MOE_WAVE, m = lane & 15, q = lane >> 4;
    const int mw = wv & 1, nw = wv >> 1;
    const int n0 = nt * MM_BN;
    int* s_pr = (int*)(smem + MM_ST * MM_STAGE);              // [128]
    float* s_w = (float*)(s_pr + MM_BM);                       // [128]
    uint8_t* s_hs = (uint8_t*)(s_w + MM_BM);                   // [128][I / 128]
    if (threadIdx.x < MM_BM) {
        const int p = sorted_pair[mt * MM_BM + threadIdx.x];
        s_pr[threadIdx.x] = p;
        s_w[threadIdx.x] = p < NP ? topk_w[p] : 0.f;
    }
    __syncthreads();
    if (slot < 0) {                                   // non-resident expert: its pairs add zero
        for (int i = threadIdx.x; i < MM_BM * (MM_BN / 8); i += MM_THREADS) {
            const int r = i / (MM_BN / 8), ch = i % (MM_BN / 8);
            const int p = s_pr[r];
            if (p < NP) *(i32x4*)(ybuf + (size_t)p * H + n0 + ch * 8) = i32x4{0, 0, 0, 0};
        }
        return;
    }
    if (pool.fmt[slot] == 1) return;                  // int4 slot
    const uint8_t* sb = pool.base + (size_t)slot * pool.stride;
    const int steps = I / 128;
    const int hgroups = I / MOE_ACT_G;
    for (int i = threadIdx.x; i < MM_BM * hgroups; i += MM_THREADS) s_hs[i] = hs[(size_t)mt * MM_BM * hgroups + i];
    const uint8_t* srcA[4];
    const uint8_t* srcB[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) srcA[j] = hq + (size_t)(mt * MM_BM + wv * 32 + j * 8 + (lane >> 3)) * I;
    const uint8_t* w2 = sb + pool.off[0][2];
#pragma unroll
    for (int j = 0; j < 8; ++j) srcB[j] = w2 + (size_t)(n0 + wv * 64 + j * 8 + (lane >> 3)) * I;
    auto issue = [&](int g) {
        uint8_t* st = smem + (g % MM_ST) * MM_STAGE;
        dma_rows<4>(st, wv * 32, lane, srcA, g * 128);
        dma_rows<8>(st + MM_BM * 128, wv * 64, lane, srcB, g * 128);
    };
    f32x4 acc[4][8];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int n = 0; n < 8; ++n) acc[a][n] = f32x4{0, 0, 0, 0};
    for (int g = 0; g < MM_ST - 1 && g < steps; ++g) issue(g);
    for (int g = 0; g < steps; ++g) {
        wait_stage(min(MM_ST - 2, steps - 1 - g));
        barrier_lds();
        if (g + MM_ST - 1 < steps) issue(g + MM_ST - 1);
        const uint8_t* st = smem + (g % MM_ST) * MM_STAGE;
        const uint8_t* sB = st + MM_BM * 128;
        i32x8 bf[8];
#pragma unroll
        for (int n = 0; n < 8; ++n) bf[n] = lds_frag(sB, nw * 128 + n * 16 + m, q);
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int r = mw * 64 + a * 16 + m;
            const i32x8 af = lds_frag(st, r, q);
            const int sa = s_hs[r * hgroups + g];
#pragma unroll
            for (int n = 0; n < 8; ++n) acc[a][n] = mfma_fp8_16x16x128(af, bf[n], acc[a][n], sa, 127);
        }
    }
    // ---- epilogue: row scale x route weight, bf16 rows staged in LDS for 512-byte row stores
    const float* s2 = (const float*)(sb + pool.off[0][3]);
    float sc[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) sc[n] = s2[n0 + nw * 128 + n * 16 + m];
    __syncthreads();                                   // every wave is done with the stages
    uint16_t* sY = (uint16_t*)smem;                    // [128][256 + 8] bf16
    constexpr int YROW = MM_BN + 8;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = mw * 64 + a * 16 + 4 * q + i;
            const float wt = s_w[row];
#pragma unroll
            for (int n = 0; n < 8; ++n) sY[row * YROW + nw * 128 + n * 16 + m] = f32_to_bf16(acc[a][n][i] * sc[n] * wt);
        }
    __syncthreads();
    for (int i = threadIdx.x; i < MM_BM * (MM_BN / 8); i += MM_THREADS) {
        const int r = i / (MM_BN / 8), ch = i % (MM_BN / 8);
        const int p = s_pr[r];
        if (p < NP) *(i32x4*)(ybuf + (size_t)p * H + n0 + ch * 8) = *(const i32x4*)(sY + r * YROW + ch * 8);
    }
}

// ---------------------------------------------------------------- host side
size_t mfma_gemm1_smem(int H) {
    return (size_t)MM_ST * MM_STAGE + MM_BM * 4 + 2 * MM_BM * 4 + (size_t)MM_BM * (H / 128);
}
size_t mfma_gemm2_smem(int I) { return (size_t)MM_ST * MM_STAGE + 2 * MM_BM * 4 + (size_t)MM_BM * (I / 128); }

// shapes the two kernels take (the LDS extras grow with H and I)
bool mfma_path_ok(int H, int I) {
    return H % MM_BN == 0 && I % 128 == 0 && H <= 8192 && I <= 8192;
}

static MPool mpool(const PoolArgs& pa) {
    MPool mp;
    mp.base = (const uint8_t*)pa.base;
    mp.stride = pa.stride;
    mp.fmt = pa.fmt;
    for (int f = 0; f < 2; ++f)
        for (int p = 0; p < 4; ++p) mp.off[f][p] = pa.off[f][p];
    return mp;
}

// The 144 KiB of stages exceed the default dynamic LDS limit. The limit is a
// per-kernel, per-device attribute, so it is set before every launch.
hipError_t launch_mfma_gemm1(const PoolArgs& pa, const uint8_t* xq, const uint8_t* xs, int NP, int k,
                             const int32_t* sorted_pair, const int32_t* block_slot, const int32_t* n_padded, int cap,
                             int H, int I, uint8_t* hq, uint8_t* hs, hipStream_t stream) {
    const size_t sm = mfma_gemm1_smem(H);
    hipError_t e = hipFuncSetAttribute((const void*)gemm1_mfma_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)sm);
    if (e != hipSuccess) return e;
    MOE_LAUNCH(K_GEMM1_FP8, stream, gemm1_mfma_kernel, dim3((cap / MM_BM) * (I / 128)), dim3(MM_THREADS), sm, stream,
               mpool(pa), xq, xs, NP, k, sorted_pair, block_slot, n_padded, H, I, hq, hs);
    return hipGetLastError();
}

hipError_t launch_mfma_gemm2(const PoolArgs& pa, int NP, const float* topk_w, const int32_t* sorted_pair,
                             const int32_t* block_slot, const int32_t* n_padded, int cap, int H, int I,
                             const uint8_t* hq, const uint8_t* hs, uint16_t* ybuf, hipStream_t stream) {
    const size_t sm = mfma_gemm2_smem(I);
    hipError_t e = hipFuncSetAttribute((const void*)gemm2_mfma_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)sm);
    if (e != hipSuccess) return e;
    MOE_LAUNCH(K_GEMM2_FP8, stream, gemm2_mfma_kernel, dim3((cap / MM_BM) * (H / MM_BN)), dim3(MM_THREADS), sm,
               stream, mpool(pa), NP, topk_w, sorted_pair, block_slot, n_padded, H, I, hq, hs, ybuf);
    return hipGetLastError();
}

}  // namespace moe
