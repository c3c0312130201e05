// Device-side helpers shared by the gfx950 kernels of the expert layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

#define MOE_WAVE 64
#define MOE_MAX_E 1024
#define MOE_MAX_K 32
#define MOE_MAX_SLOTS 4096     // slots per pool the kernels accept
#define MOE_ACT_G 128          // activation-scale group along K
#define MOE_INT4_G 128         // int4 weight group along K

namespace moe {

// Slot usability. fmt_ok has bit f set when format f's layout fits the pool
// stride (and, for int4, when inter is a multiple of 128). A slot index is
// usable when it lies inside the pool and its format tag is one of those;
// anything else (a table entry past the pool, a tag other than FP8 or int4, a
// format larger than the stride) is treated like a non-resident expert, so no
// kernel reads outside the pool whatever the slot table or the tags hold.
__device__ __forceinline__ bool fmt_usable(int tag, int fmt_ok) { return tag >= 0 && tag < 2 && ((fmt_ok >> tag) & 1); }
template <typename TagPtr>
__device__ __forceinline__ int usable_slot(int slot, int n_slots, int fmt_ok, TagPtr tags) {
    if ((unsigned)slot >= (unsigned)n_slots) return -1;
    return fmt_usable((int)tags[slot], fmt_ok) ? slot : -1;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// round-to-nearest-even fp32 -> bf16 (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Smallest s with amax <= 448 * 2^s (s = 0 for amax == 0), exact: with
// amax = m * 2^e, m in [0.5, 1) and 448 = 0.875 * 2^9.
__device__ __forceinline__ int pow2_exponent_448(float amax) {
    if (!(amax > 0.f)) return 0;
    int e;
    float m = frexpf(amax, &e);
    return (m <= 0.875f) ? e - 9 : e - 8;
}

// two fp32 -> two OCP e4m3 codes packed in the low 16 bits (round to nearest even)
__device__ __forceinline__ uint32_t f32x2_to_e4m3(float a, float b) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// four e4m3 codes (one dword) -> four bf16 (two dwords); exact
__device__ __forceinline__ void e4m3x4_to_bf16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false));
    hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true));
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
    return __builtin_amdgcn_cvt_pk_f32_fp8((int)code, false)[0];
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// wave-wide reductions (64 lanes)
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        uint64_t w = __shfl_xor(v, o, 64);
        v = w > v ? w : v;
    }
    return v;
}
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// Wave-wide max of 64-bit keys through DPP row shifts and row broadcasts
// (lane 63 ends with the maximum, which is then read back to every lane).
// Lanes whose DPP source lies outside the row contribute the identity 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t v) {
    int lo = (int)(uint32_t)v, hi = (int)(uint32_t)(v >> 32);
    uint32_t slo = (uint32_t)__builtin_amdgcn_update_dpp(0, lo, CTRL, ROW_MASK, 0xF, false);
    uint32_t shi = (uint32_t)__builtin_amdgcn_update_dpp(0, hi, CTRL, ROW_MASK, 0xF, false);
    uint64_t o = ((uint64_t)shi << 32) | slo;
    return o > v ? o : v;
}
__device__ __forceinline__ uint64_t wave_max_u64_dpp(uint64_t v) {
    v = dpp_max_step<0x111, 0xF>(v);   // row_shr:1
    v = dpp_max_step<0x112, 0xF>(v);   // row_shr:2
    v = dpp_max_step<0x114, 0xF>(v);   // row_shr:4
    v = dpp_max_step<0x118, 0xF>(v);   // row_shr:8  -> lane 15 of each row holds the row max
    v = dpp_max_step<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
    v = dpp_max_step<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3 -> lane 63 holds the max
    uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
    uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
    return ((uint64_t)hi << 32) | lo;
}

// Max of 64-bit keys over each row of 16 lanes, left in every lane of the row
// (butterfly: swap neighbours, swap pairs, rotate by 4, rotate by 8).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_row_max_step(uint64_t v) {
    uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xF, 0xF, true);
    uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, true);
    uint64_t o = ((uint64_t)hi << 32) | lo;
    return o > v ? o : v;
}
__device__ __forceinline__ uint64_t row16_max_u64(uint64_t v) {
    v = dpp_row_max_step<0xB1>(v);    // quad_perm [1,0,3,2]
    v = dpp_row_max_step<0x4E>(v);    // quad_perm [2,3,0,1]
    v = dpp_row_max_step<0x124>(v);   // row_ror:4
    v = dpp_row_max_step<0x128>(v);   // row_ror:8
    return v;
}
template <int CTRL>
__device__ __forceinline__ float dpp_row_sum_step(float v) {
    return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
// Sum over each row of 16 lanes, left in every lane of the row.
__device__ __forceinline__ float row16_sum(float v) {
    v = dpp_row_sum_step<0xB1>(v);
    v = dpp_row_sum_step<0x4E>(v);
    v = dpp_row_sum_step<0x124>(v);
    v = dpp_row_sum_step<0x128>(v);
    return v;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
    int l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Matrix-core wrappers. Callers keep the whole wave active around them.
__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(const bf16x8& a, const bf16x8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// A, B: 32 e4m3 codes per lane; sa, sb: E8M0 scale bytes (127 = 1.0)
__device__ __forceinline__ f32x4 mfma_fp8_16x16x128(const i32x8& a, const i32x8& b, f32x4 c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// 16 packed int4 codes (8 bytes, low nibble first) -> 16 e4m3 codes of
// q - zero, in K order (exact for integer zero points: q - zero is an integer
// in [-15, 15]). Each pair of nibbles becomes two fp16 values 1024 + q (the
// exponent of 1024 with q in the low mantissa bits), minus 1024 + zero, then
// two e4m3 codes; four vector instructions per pair.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void int4_to_e4m3_16(uint2 packed, float zero, uint32_t out[4]) {
    const _Float16 zz = (_Float16)(-1024.0f - zero);
    const f16x2_t off = {zz, zz};
    const uint32_t w[2] = {packed.x, packed.y};
#pragma unroll
    for (int d = 0; d < 2; ++d) {
        const uint32_t ev = w[d] & 0x0F0F0F0Fu;              // nibbles 0, 2, 4, 6 as bytes
        const uint32_t od = (w[d] >> 4) & 0x0F0F0F0Fu;       // nibbles 1, 3, 5, 7
#pragma unroll
        for (int h = 0; h < 2; ++h) {                         // output dword: nibble pairs 2h, 2h + 1
            f16x2_t v[2];
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                const int p = 2 * h + pp;
                // bytes: ev.p, 0, od.p, 0 (perm selector 12 gives a zero byte)
                const uint32_t sel = (uint32_t)p | (12u << 8) | ((uint32_t)(4 + p) << 16) | (12u << 24);
                const uint32_t bits = __builtin_amdgcn_perm(od, ev, sel) | 0x64006400u;
                v[pp] = __builtin_bit_cast(f16x2_t, bits) + off;
            }
            s16x2_t acc = {0, 0};
            acc = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(acc, v[0], 1.0f, false);   // low word
            acc = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(acc, v[1], 1.0f, true);    // high word
            out[2 * d + h] = __builtin_bit_cast(uint32_t, acc);
        }
    }
}

// Direct-to-LDS loads: lane i writes 16 (4) bytes at lds + 16 i (4 i); lds is
// wave-uniform. They count on the vector memory counter like other loads.
__device__ __forceinline__ void lds_dma16(const void* src, uint8_t* lds) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}
__device__ __forceinline__ void lds_dma4(const void* src, uint8_t* lds) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
}

// s_waitcnt with only vmcnt limited (expcnt and lgkmcnt left open): at most N
// of this wave's vector memory operations stay outstanding
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace moe
