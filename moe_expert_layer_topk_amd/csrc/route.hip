// Top-k routing from fp32 router logits (one wavefront per token).
//
// PagedWeight commentary (spectral-agent.com), "what was released" and
// "technically interesting points": the router sends each token to a few
// experts. Order: logit descending, expert id ascending (-0.0 == +0.0);
// weights: softmax over the k chosen logits.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

// Orderable 64-bit key: high word = monotone image of the float (signed zeros
// merged), low word = 1023 - expert so that a lower id wins ties. 0 = absent.
__device__ __forceinline__ uint64_t route_key(float v, int e) {
    if (v == 0.0f) v = 0.0f;
    uint32_t u = __float_as_uint(v);
    uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)o << 32) | (uint32_t)(MOE_MAX_E - 1 - e);
}
__device__ __forceinline__ float key_value(uint64_t key) {
    uint32_t o = (uint32_t)(key >> 32);
    uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
    return __uint_as_float(u);
}

constexpr int ROUTE_VPL = MOE_MAX_E / MOE_WAVE;   // logits held per lane

__global__ void __launch_bounds__(256) route_kernel(const float* __restrict__ logits,
                                                    const uint8_t* __restrict__ mask, int T, int E, int k,
                                                    int32_t* __restrict__ ids, float* __restrict__ w,
                                                    int32_t* __restrict__ err) {
    const int lane = lane_id();
    const int t = blockIdx.x * (blockDim.x / MOE_WAVE) + (threadIdx.x / MOE_WAVE);
    if (t >= T) return;                                  // whole wave leaves together
    const float* row = logits + (size_t)t * E;
    uint64_t key[ROUTE_VPL];
#pragma unroll
    for (int i = 0; i < ROUTE_VPL; ++i) {
        int e = i * MOE_WAVE + lane;
        bool ok = e < E && (mask == nullptr || mask[e] != 0);
        key[i] = ok ? route_key(row[e], e) : 0ull;
    }
    float my_logit = 0.f;
    int my_id = -1;
    int found = 0;
    for (int r = 0; r < k; ++r) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < ROUTE_VPL; ++i) best = key[i] > best ? key[i] : best;
        best = wave_max_u64(best);
        if (best == 0) break;                            // uniform across the wave
#pragma unroll
        for (int i = 0; i < ROUTE_VPL; ++i) key[i] = (key[i] == best) ? 0ull : key[i];
        if (lane == r) {
            my_logit = key_value(best);
            my_id = MOE_MAX_E - 1 - (int)(uint32_t)(best & 0xFFFFFFFFu);
        }
        ++found;
    }
    // softmax over the chosen logits; lane r < found holds choice r
    float top = __shfl(my_logit, 0, 64);
    float z = (lane < found) ? expf(my_logit - top) : 0.f;
    float s = 0.f;
    for (int r = 0; r < found; ++r) s += __shfl(z, r, 64);   // fixed order
    if (lane < k) {
        ids[(size_t)t * k + lane] = (lane < found) ? my_id : -1;
        w[(size_t)t * k + lane] = (lane < found) ? z / s : 0.f;
    }
    if (lane == 0 && found < k) atomicAdd(err, 1);
}

hipError_t launch_route(const float* logits, const uint8_t* mask, int T, int E, int k, int32_t* ids,
                        float* w, int32_t* err, hipStream_t stream) {
    const int waves_per_block = 4;
    dim3 grid((T + waves_per_block - 1) / waves_per_block);
    MOE_LAUNCH(K_ROUTE, stream, route_kernel, grid, dim3(waves_per_block * MOE_WAVE), 0, stream, logits, mask, T, E,
                       k, ids, w, err);
    return hipGetLastError();
}

}  // namespace moe
