// Top-k selection of one token by one wavefront (shared by the route kernel
// and the gate/up kernel that routes small batches itself).
//
// PagedWeight commentary (spectral-agent.com), "what was released" and
// "technically interesting points": the router sends each token to a few
// experts. Order: logit descending, expert id ascending (-0.0 == +0.0);
// weights: softmax over the k chosen logits, in fp32.
#pragma once
#include "moe_common.h"

namespace moe {

// Orderable 32-bit image of a logit (monotone, signed zeros merged); 0 marks
// an absent entry and is below the image of every non-NaN float.
__device__ __forceinline__ uint32_t route_ord(float v) {
    if (v == 0.0f) v = 0.0f;
    const uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float route_ord_value(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t v) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
    return o > v ? o : v;
}
// wave-wide max: row shifts, then row broadcasts; lane 63 ends with the max
__device__ __forceinline__ uint32_t wave_max_u32_dpp(uint32_t v) {
    v = dpp_max_u32<0x111, 0xF>(v);
    v = dpp_max_u32<0x112, 0xF>(v);
    v = dpp_max_u32<0x114, 0xF>(v);
    v = dpp_max_u32<0x118, 0xF>(v);
    v = dpp_max_u32<0x142, 0xA>(v);
    v = dpp_max_u32<0x143, 0xC>(v);
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Keys of one token's logits, entry i of lane l = expert 64 i + l (E <= 64 *
// VPL); 0 for experts past E or masked out. Every load is issued before any
// is used (clamped indices, no branches), so they share one round trip.
template <int VPL>
__device__ __forceinline__ void route_keys(const float* __restrict__ row, const uint8_t* __restrict__ mask, int E,
                                           uint32_t (&key)[VPL]) {
    const int lane = lane_id();
    float v[VPL];
    int mk[VPL];
    const uint8_t* mp = mask ? mask : (const uint8_t*)row;   // no mask: read a byte that exists, ignore it
    const int mlim = mask ? E - 1 : 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        v[i] = row[min(i * MOE_WAVE + lane, E - 1)];
        mk[i] = mp[min(i * MOE_WAVE + lane, mlim)];
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i)
        key[i] = (i * MOE_WAVE + lane < E && (mask == nullptr || mk[i] != 0)) ? route_ord(v[i]) : 0u;
}

// Lane r < found returns choice r in (id, weight); lanes >= found return
// (-1, 0). Each round takes the largest logit image; among equal images the
// lowest expert id (lowest i, then lowest lane) wins. Each lane keeps its own
// largest key and index, so a round is one wave-wide max plus, when a single
// lane holds it, one lane read. Whole wave must call; key is consumed.
template <int VPL>
__device__ __forceinline__ int route_select(uint32_t (&key)[VPL], int k, int& my_id, float& my_w) {
    const int lane = lane_id();
    // this lane's largest key and the lowest index holding it
    uint32_t lb = 0;
    int li = 0;
    auto local_max = [&]() __attribute__((always_inline)) {
        lb = key[0];
        li = 0;
#pragma unroll
        for (int i = 1; i < VPL; ++i) {
            const bool gt = key[i] > lb;
            lb = gt ? key[i] : lb;
            li = gt ? i : li;
        }
    };
    local_max();
    uint32_t my_ord = 0;
    my_id = -1;
    int found = 0;
    for (int r = 0; r < k; ++r) {
        const uint32_t best = wave_max_u32_dpp(lb);
        if (best == 0) break;                            // uniform across the wave
        const uint64_t at = __ballot(lb == best);
        int sel;
        if (__popcll(at) == 1) {                         // one lane holds the maximum: its lowest index
            const int wl = (int)__builtin_ctzll(at);
            sel = __builtin_amdgcn_readlane(li, wl) * MOE_WAVE + wl;
        } else {                                         // equal keys in several lanes: lowest expert id
            sel = -1;
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const uint64_t bi = __ballot(key[i] == best);
                if (sel < 0 && bi != 0) sel = i * MOE_WAVE + (int)__builtin_ctzll(bi);
            }
        }
#pragma unroll
        for (int i = 0; i < VPL; ++i) key[i] = (i * MOE_WAVE + lane == sel) ? 0u : key[i];
        local_max();                                     // changes only the winner lane's (lb, li)
        if (lane == r) {
            my_ord = best;
            my_id = sel;
        }
        ++found;
    }
    const float my_logit = route_ord_value(my_ord);
    const float top = __shfl(my_logit, 0, 64);
    const float z = (lane < found) ? expf(my_logit - top) : 0.f;
    float s = 0.f;
    for (int r = 0; r < found; ++r) s += __shfl(z, r, 64);   // fixed order
    my_w = (lane < found) ? z / s : 0.f;
    if (lane >= found) my_id = -1;
    return found;
}

// One token: route_keys then route_select.
template <int VPL>
__device__ __forceinline__ int route_token(const float* __restrict__ row, const uint8_t* __restrict__ mask, int E,
                                           int k, int& my_id, float& my_w) {
    uint32_t key[VPL];
    route_keys<VPL>(row, mask, E, key);
    return route_select<VPL>(key, k, my_id, my_w);
}

}  // namespace moe
