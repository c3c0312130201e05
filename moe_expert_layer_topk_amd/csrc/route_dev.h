// Top-k selection of one token by one wavefront (shared by the route kernel
// and the fused small-batch route + align kernel).
//
// PagedWeight commentary (spectral-agent.com), "what was released" and
// "technically interesting points": the router sends each token to a few
// experts. Order: logit descending, expert id ascending (-0.0 == +0.0);
// weights: softmax over the k chosen logits, in fp32.
#pragma once
#include "moe_common.h"

namespace moe {

// Orderable 64-bit key: high word = monotone image of the float (signed zeros
// merged), low word = 1023 - expert so that a lower id wins ties. 0 = absent.
__device__ __forceinline__ uint64_t route_key(float v, int e) {
    if (v == 0.0f) v = 0.0f;
    uint32_t u = __float_as_uint(v);
    uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)o << 32) | (uint32_t)(MOE_MAX_E - 1 - e);
}
__device__ __forceinline__ float route_key_value(uint64_t key) {
    uint32_t o = (uint32_t)(key >> 32);
    uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
    return __uint_as_float(u);
}

// Lane r < found returns choice r in (id, weight); lanes >= found return
// (-1, 0). VPL = logits held per lane (E <= 64 * VPL). Whole wave must call.
template <int VPL>
__device__ __forceinline__ int route_token(const float* __restrict__ row, const uint8_t* __restrict__ mask, int E,
                                           int k, int& my_id, float& my_w) {
    const int lane = lane_id();
    uint64_t key[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int e = i * MOE_WAVE + lane;
        const bool ok = e < E && (mask == nullptr || mask[e] != 0);
        key[i] = ok ? route_key(row[e], e) : 0ull;
    }
    float my_logit = 0.f;
    my_id = -1;
    int found = 0;
    for (int r = 0; r < k; ++r) {
        uint64_t best = key[0];
#pragma unroll
        for (int i = 1; i < VPL; ++i) best = key[i] > best ? key[i] : best;
        best = wave_max_u64_dpp(best);
        if (best == 0) break;                            // uniform across the wave
#pragma unroll
        for (int i = 0; i < VPL; ++i) key[i] = (key[i] == best) ? 0ull : key[i];
        if (lane == r) {
            my_logit = route_key_value(best);
            my_id = MOE_MAX_E - 1 - (int)(uint32_t)(best & 0xFFFFFFFFu);
        }
        ++found;
    }
    const float top = __shfl(my_logit, 0, 64);
    const float z = (lane < found) ? expf(my_logit - top) : 0.f;
    float s = 0.f;
    for (int r = 0; r < found; ++r) s += __shfl(z, r, 64);   // fixed order
    my_w = (lane < found) ? z / s : 0.f;
    if (lane >= found) my_id = -1;
    return found;
}

}  // namespace moe
