// Router gate GEMM: logits[t][e] = sum_h x[t][h] * W_g[e][h] + bias[e], in
// fp32, ahead of the top-k selection (PagedWeight commentary,
// spectral-agent.com, "technically interesting points": a router picks each
// token's experts).
//
// x is bf16; W_g is fp32. Each W_g value is split exactly into three bf16
// parts by truncation (hi = the upper half of w, mid = the upper half of
// w - hi, lo = w - hi - mid, which has at most 8 significant bits), so
// w = hi + mid + lo exactly and every product x * part is exact in fp32: the
// bf16 matrix cores (v_mfma_f32_16x16x32_bf16, fp32 accumulate) then give the
// fp32 sum of the exact products x * w, which differs from the exact logit
// only by the rounding of that sum.
//
// Work split: a workgroup owns 16 * MT tokens x 16 experts; its 4 waves
// split the hidden axis in quarters and meet in LDS, where wave 0 adds the
// partial sums in a fixed order and the bias. Each wave issues the loads of
// SB K steps of 32 before using any (one memory round trip per SB steps).
// The expert tiles of one token tile are placed on one XCD (block ids are
// dealt round-robin over the 8 XCDs), so a token tile is read from HBM once
// and then served by that XCD's L2.
//
// Operand layout of the instruction (lane l = m + 16 q): A row m (token) and
// B column m (expert) hold K positions 8q .. 8q+7 of the 32-wide step; C
// lane l holds rows 4q .. 4q+3 (tokens) of column m (expert).
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

constexpr int RG_THREADS = 256;

// three exact bf16 parts of eight fp32 values (upper halves by truncation)
__device__ __forceinline__ void split3(const i32x4& lo4, const i32x4& hi4, bf16x8& a, bf16x8& b, bf16x8& c) {
    uint32_t w[8] = {(uint32_t)lo4[0], (uint32_t)lo4[1], (uint32_t)lo4[2], (uint32_t)lo4[3],
                     (uint32_t)hi4[0], (uint32_t)hi4[1], (uint32_t)hi4[2], (uint32_t)hi4[3]};
    uint32_t p0[4], p1[4], p2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t h[2], md[2], l[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t v = w[2 * i + j];
            h[j] = v & 0xFFFF0000u;
            const float r1 = __uint_as_float(v) - __uint_as_float(h[j]);          // exact
            md[j] = __float_as_uint(r1) & 0xFFFF0000u;
            const float r2 = r1 - __uint_as_float(md[j]);                        // exact, <= 8 bits
            l[j] = __float_as_uint(r2);
        }
        // two upper halves -> one packed bf16 pair (element 2i in the low half)
        p0[i] = __builtin_amdgcn_perm(h[1], h[0], 0x07060302u);
        p1[i] = __builtin_amdgcn_perm(md[1], md[0], 0x07060302u);
        p2[i] = __builtin_amdgcn_perm(l[1], l[0], 0x07060302u);
    }
    a = __builtin_bit_cast(bf16x8, i32x4{(int)p0[0], (int)p0[1], (int)p0[2], (int)p0[3]});
    b = __builtin_bit_cast(bf16x8, i32x4{(int)p1[0], (int)p1[1], (int)p1[2], (int)p1[3]});
    c = __builtin_bit_cast(bf16x8, i32x4{(int)p2[0], (int)p2[1], (int)p2[2], (int)p2[3]});
}

template <int MT, int SB>
__global__ void __launch_bounds__(RG_THREADS) router_gemm_kernel(const uint16_t* __restrict__ x,
                                                                 const float* __restrict__ wg,
                                                                 const float* __restrict__ bias, int T, int H, int E,
                                                                 float* __restrict__ logits) {
    __shared__ f32x4 s_red[4][MT][64];
    const int n_et = (E + 15) / 16, n_tt = (T + 16 * MT - 1) / (16 * MT);
    const int xcd = blockIdx.x & 7, rest = blockIdx.x >> 3;
    const int et = rest % n_et, tt = (rest / n_et) * 8 + xcd;
    if (tt >= n_tt) return;                              // uniform over the workgroup
    const int lane = lane_id(), wv = threadIdx.x / MOE_WAVE;
    const int m = lane & 15, q = lane >> 4;
    const int e = min(et * 16 + m, E - 1);               // clamped rows: results past E are not stored
    const float* wrow = wg + (size_t)e * H;
    const uint16_t* xrow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) xrow[mt] = x + (size_t)min(tt * 16 * MT + mt * 16 + m, T - 1) * H;
    const int steps = H / 128;                           // 32-wide K steps in this wave's quarter
    const int k_base = wv * (H / 4) + 8 * q;
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0, 0, 0, 0};
    for (int s0 = 0; s0 < steps; s0 += SB) {
        i32x4 ra[SB][MT], rw[SB][2];
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            const int k0 = k_base + min(s0 + j, steps - 1) * 32;   // (steps past the end repeat the last; unused)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) ra[j][mt] = *(const i32x4*)(xrow[mt] + k0);
            rw[j][0] = *(const i32x4*)(wrow + k0);
            rw[j][1] = *(const i32x4*)(wrow + k0 + 4);
        }
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            if (s0 + j >= steps) break;                  // uniform over the wave
            bf16x8 bh, bm, bl;
            split3(rw[j][0], rw[j][1], bh, bm, bl);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const bf16x8 a = __builtin_bit_cast(bf16x8, ra[j][mt]);
                acc[mt] = mfma_bf16_16x16x32(a, bh, acc[mt]);
                acc[mt] = mfma_bf16_16x16x32(a, bm, acc[mt]);
                acc[mt] = mfma_bf16_16x16x32(a, bl, acc[mt]);
            }
        }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) s_red[wv][mt][lane] = acc[mt];
    __syncthreads();
    if (wv != 0) return;
    const int ec = et * 16 + m;
    const float b = (bias && ec < E) ? bias[ec] : 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        f32x4 v = s_red[0][mt][lane];
        v += s_red[1][mt][lane];
        v += s_red[2][mt][lane];
        v += s_red[3][mt][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = tt * 16 * MT + mt * 16 + 4 * q + i;
            if (t < T && ec < E) logits[(size_t)t * E + ec] = v[i] + b;
        }
    }
}

hipError_t launch_router_gemm(const uint16_t* x, const float* wg, const float* bias, int T, int H, int E,
                              float* logits, hipStream_t stream) {
    const int n_et = (E + 15) / 16;
    if (T <= 64) {
        const int n_tt = (T + 15) / 16;
        const int grid = (n_tt + 7) / 8 * 8 * n_et;
        MOE_LAUNCH(K_ROUTER_GEMM, stream, (router_gemm_kernel<1, 8>), dim3(grid), dim3(RG_THREADS), 0, stream, x, wg,
                   bias, T, H, E, logits);
    } else {
        const int n_tt = (T + 63) / 64;
        const int grid = (n_tt + 7) / 8 * 8 * n_et;
        MOE_LAUNCH(K_ROUTER_GEMM, stream, (router_gemm_kernel<4, 4>), dim3(grid), dim3(RG_THREADS), 0, stream, x, wg,
                   bias, T, H, E, logits);
    }
    return hipGetLastError();
}

}  // namespace moe
