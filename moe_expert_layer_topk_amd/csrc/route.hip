// Top-k routing from fp32 router logits: one wavefront per token
// (selection and weights in route_dev.h).
#include "moe_common.h"
#include "moe_kernels.h"
#include "route_dev.h"

namespace moe {

template <int VPL>
__global__ void __launch_bounds__(256) route_kernel(const float* __restrict__ logits,
                                                    const uint8_t* __restrict__ mask, int T, int E, int k,
                                                    int32_t* __restrict__ ids, float* __restrict__ w,
                                                    int32_t* __restrict__ err) {
    const int lane = lane_id();
    const int t = blockIdx.x * (blockDim.x / MOE_WAVE) + (threadIdx.x / MOE_WAVE);
    if (t >= T) return;                                  // whole wave leaves together
    int id;
    float wt;
    const int found = route_token<VPL>(logits + (size_t)t * E, mask, E, k, id, wt);
    if (lane < k) {
        ids[(size_t)t * k + lane] = id;
        w[(size_t)t * k + lane] = wt;
    }
    if (lane == 0 && found < k) atomicAdd(err, 1);
}

hipError_t launch_route(const float* logits, const uint8_t* mask, int T, int E, int k, int32_t* ids,
                        float* w, int32_t* err, hipStream_t stream) {
    const int waves_per_block = 4;
    dim3 grid((T + waves_per_block - 1) / waves_per_block), block(waves_per_block * MOE_WAVE);
    if (E <= 64)
        MOE_LAUNCH(K_ROUTE, stream, route_kernel<1>, grid, block, 0, stream, logits, mask, T, E, k, ids, w, err);
    else if (E <= 128)
        MOE_LAUNCH(K_ROUTE, stream, route_kernel<2>, grid, block, 0, stream, logits, mask, T, E, k, ids, w, err);
    else if (E <= 256)
        MOE_LAUNCH(K_ROUTE, stream, route_kernel<4>, grid, block, 0, stream, logits, mask, T, E, k, ids, w, err);
    else if (E <= 512)
        MOE_LAUNCH(K_ROUTE, stream, route_kernel<8>, grid, block, 0, stream, logits, mask, T, E, k, ids, w, err);
    else
        MOE_LAUNCH(K_ROUTE, stream, route_kernel<16>, grid, block, 0, stream, logits, mask, T, E, k, ids, w, err);
    return hipGetLastError();
}

}  // namespace moe
