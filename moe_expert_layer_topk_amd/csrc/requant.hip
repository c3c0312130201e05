// Quality-aware bit width (PagedWeight commentary, spectral-agent.com,
// "technically interesting points": experts are held at a bit width chosen
// by how much they matter, and switched while the model serves).
//
// moe_requant_slot turns one expert's FP8 slot into an int4-g128 slot of the
// same pool: for each row and group of 128 consecutive K values w (decoded
// as e4m3(code) * row scale, in fp32):
//   s = fp16((max w - min w) / 15) (1 when that is 0),
//   z = clip(rint(-min w / s), 0, 15),  q = clip(rint(w / s) + z, 0, 15).
// Every step that decides an integer is an fp32 operation with IEEE
// rounding (product, difference, correctly rounded divisions, fp16 round to
// nearest even, rint with ties to even), so results repeat exactly.
// One 16-lane group per (row, group): 8 values per lane, the group's min and
// max through lane exchanges, 8 nibbles (4 bytes) stored per lane.
//
// moe_bitwidth_plan (host) picks the least-routed experts from the
// per-expert pair counts moe_align writes.
#include "../../include/moe.h"
#include "moe_common.h"
#include "moe_kernels.h"

#include <algorithm>
#include <numeric>
#include <vector>

namespace moe {

struct RqOffsets {
    size_t fp8[4], i4[4];
};

// four e4m3 codes (one dword) -> four fp32 (exact)
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float* o) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    o[0] = lo[0];
    o[1] = lo[1];
    o[2] = hi[0];
    o[3] = hi[1];
}

__global__ void __launch_bounds__(256) requant_kernel(const uint8_t* __restrict__ base, size_t stride,
                                                     const uint8_t* __restrict__ fmt, int fmt_ok, int src, int dst,
                                                     RqOffsets off, int H, int I, uint8_t* __restrict__ tags,
                                                     int32_t* __restrict__ err) {
    const int tag = fmt[src];
    if (tag != MOE_FMT_FP8_E4M3_ROW || !fmt_usable(tag, fmt_ok)) {   // uniform: nothing to convert
        if (blockIdx.x == 0 && threadIdx.x == 0 && err) atomicAdd(err, 1);
        return;
    }
    const uint8_t* sb = base + (size_t)src * stride;
    uint8_t* db = (uint8_t*)base + (size_t)dst * stride;
    const long n13 = (long)2 * I * (H / 128), n2 = (long)H * (I / 128);
    const int lane = lane_id(), l16 = lane & 15;
    const long item = ((long)blockIdx.x * 4 + threadIdx.x / MOE_WAVE) * 4 + lane / 16;
    const bool live = item < n13 + n2;
    const long it = live ? item : 0;                    // idle lanes redo item 0 and store nothing
    const bool up = it < n13;                           // w13 (rows x H) or w2 (rows x I)
    const long j = up ? it : it - n13;
    const int cols = up ? H : I, groups = cols / 128;
    const int row = (int)(j / groups), g = (int)(j % groups);
    const uint8_t* codes = sb + (up ? off.fp8[0] : off.fp8[2]) + (size_t)row * cols + g * 128 + 8 * l16;
    const float scale = *(const float*)(sb + (up ? off.fp8[1] : off.fp8[3]) + 4 * (size_t)row);
    const uint2 c = *(const uint2*)codes;
    float w[8];
    e4m3x4_to_f32(c.x, w);
    e4m3x4_to_f32(c.y, w + 4);
    float mn = INFINITY, mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        w[i] = w[i] * scale;
        mn = fminf(mn, w[i]);
        mx = fmaxf(mx, w[i]);
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
        mn = fminf(mn, __shfl_xor(mn, o, 64));
        mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    }
    _Float16 s16 = (_Float16)((mx - mn) / 15.0f);
    if (s16 == (_Float16)0.0f) s16 = (_Float16)1.0f;
    const float s = (float)s16;
    const float z = fminf(fmaxf(rintf(-mn / s), 0.0f), 15.0f);
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float qv = fminf(fmaxf(rintf(w[i] / s) + z, 0.0f), 15.0f);
        packed |= (uint32_t)qv << (4 * i);              // element 2m in the low nibble of byte m
    }
    if (live) {
        *(uint32_t*)(db + (up ? off.i4[0] : off.i4[2]) + (size_t)row * (cols / 2) + g * 64 + 4 * l16) = packed;
        if (l16 == 0) {
            const uint32_t sz = (uint32_t)__builtin_bit_cast(uint16_t, s16) |
                                ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)z) << 16);
            *(uint32_t*)(db + (up ? off.i4[1] : off.i4[3]) + ((size_t)row * groups + g) * 4) = sz;
        }
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) tags[dst] = (uint8_t)MOE_FMT_INT4_G128;
}

hipError_t launch_requant(const PoolArgs& pa, int src, int dst, uint8_t* tags, int32_t* err, hipStream_t stream) {
    RqOffsets off;
    for (int i = 0; i < 4; ++i) {
        off.fp8[i] = pa.off[0][i];
        off.i4[i] = pa.off[1][i];
    }
    const int H = pa.hidden, I = pa.inter;
    const long items = (long)2 * I * (H / 128) + (long)H * (I / 128);
    MOE_LAUNCH(K_REQUANT, stream, requant_kernel, dim3((unsigned)((items + 15) / 16)), dim3(256), 0, stream,
               (const uint8_t*)pa.base, pa.stride, pa.fmt, pa.fmt_ok, src, dst, off, H, I, tags, err);
    return hipGetLastError();
}

}  // namespace moe

extern "C" int moe_bitwidth_plan(const int32_t* counts, int E, int n_int4, uint8_t* fmt_out) {
    if (!counts || !fmt_out || E < 1 || E > MOE_MAX_E || n_int4 < 0) return MOE_EINVAL;
    std::vector<int> order(E);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return counts[a] < counts[b]; });
    for (int e = 0; e < E; ++e) fmt_out[e] = MOE_FMT_FP8_E4M3_ROW;
    for (int i = 0; i < std::min(n_int4, E); ++i) fmt_out[order[i]] = MOE_FMT_INT4_G128;
    return MOE_OK;
}
