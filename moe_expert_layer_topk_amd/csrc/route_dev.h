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

// NT tokens at once (one loop of selection rounds for all of them; measured
// on MI355X, a round of two tokens still costs close to two single-token
// rounds, about 700 clocks each). For token n, lane r < found[n] returns
// choice r in (my_id[n], my_w[n]); lanes >= found[n] return (-1, 0). Each
// round takes the largest logit image; among equal images the lowest expert
// id (lowest i, then lowest lane) wins. Each lane keeps its own largest key
// and index, so a round is one wave-wide max plus, when a single lane holds
// it, one lane read. A token whose keys run out (all 0) stops gaining
// choices. Whole wave must call; key is consumed.
template <int VPL, int NT>
__device__ __forceinline__ void route_select_multi(uint32_t (&key)[NT][VPL], int k, int (&my_id)[NT],
                                                   float (&my_w)[NT], int (&found)[NT]) {
    const int lane = lane_id();
    uint32_t lb[NT], my_ord[NT];
    int li[NT];
    // this lane's largest key of token n and the lowest index holding it
    auto local_max = [&](int n) __attribute__((always_inline)) {
        lb[n] = key[n][0];
        li[n] = 0;
#pragma unroll
        for (int i = 1; i < VPL; ++i) {
            const bool gt = key[n][i] > lb[n];
            lb[n] = gt ? key[n][i] : lb[n];
            li[n] = gt ? i : li[n];
        }
    };
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        local_max(n);
        my_ord[n] = 0;
        my_id[n] = -1;
        found[n] = 0;
    }
    for (int r = 0; r < k; ++r) {
        uint32_t best[NT];
        int sel[NT];
        bool tie = false;
#pragma unroll
        for (int n = 0; n < NT; ++n) best[n] = wave_max_u32_dpp(lb[n]);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const uint64_t at = __ballot(lb[n] == best[n]);      // not empty: some lane holds best
            const int wl = (int)__builtin_ctzll(at);
            sel[n] = best[n] == 0 ? -1 : __builtin_amdgcn_readlane(li[n], wl) * MOE_WAVE + wl;
            tie = tie || (best[n] != 0 && __popcll(at) > 1);
        }
        if (tie) {                                              // uniform; rare
#pragma unroll
            for (int n = 0; n < NT; ++n) {                      // equal keys in several lanes: lowest expert id
                if (best[n] == 0) continue;
                int s2 = -1;
#pragma unroll
                for (int i = 0; i < VPL; ++i) {
                    const uint64_t bi = __ballot(key[n][i] == best[n]);
                    if (s2 < 0 && bi != 0) s2 = i * MOE_WAVE + (int)__builtin_ctzll(bi);
                }
                sel[n] = s2;
            }
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) {
#pragma unroll
            for (int i = 0; i < VPL; ++i) key[n][i] = (i * MOE_WAVE + lane == sel[n]) ? 0u : key[n][i];
            local_max(n);                                       // changes only the winner lane's (lb, li)
            if (lane == r && best[n] != 0) {
                my_ord[n] = best[n];
                my_id[n] = sel[n];
            }
            found[n] += best[n] != 0 ? 1 : 0;
        }
    }
    // softmax over the chosen logits, summed in fixed order (choices past
    // found[n] add exact zeros)
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const float my_logit = route_ord_value(my_ord[n]);
        const float top = __shfl(my_logit, 0, 64);
        const float z = (lane < found[n]) ? expf(my_logit - top) : 0.f;
        float s = 0.f;
        for (int r = 0; r < found[n]; ++r) s += __shfl(z, r, 64);
        my_w[n] = (lane < found[n]) ? z / s : 0.f;
        if (lane >= found[n]) my_id[n] = -1;
    }
}

// One token (see route_select_multi).
template <int VPL>
__device__ __forceinline__ int route_select(uint32_t (&key)[VPL], int k, int& my_id, float& my_w) {
    uint32_t kk[1][VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) kk[0][i] = key[i];
    int id[1], found[1];
    float w[1];
    route_select_multi<VPL, 1>(kk, k, id, w, found);
    my_id = id[0];
    my_w = w[0];
    return found[0];
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
