// moe_layer_noalloc: the whole-layer call for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, hosts
// that forbid allocation). It runs moe_layer's kernels with their workspace
// in a fixed array of this library's code object instead of a caller
// workspace, and calls no allocating routine.
//
// The array is a device global: each GPU the library runs on holds its own
// copy at its own address, for the life of the process. Its host-side name
// only stands for the symbol, so the device address is looked up once per
// device (hipGetSymbolAddress, with that device current) and that address is
// what the kernels receive. Nothing in the workspace needs to start at zero:
// every kernel of moe_layer writes each workspace byte before any kernel
// reads it (the poisoned-workspace tests check this), so the array's contents
// left by an earlier call do not matter. Calls on one GPU share the array:
// two calls that overlap in time on one GPU (different streams, or threads)
// race on it.
#include "../../include/moe.h"
#include "moe_common.h"
#include "moe_kernels.h"

#include <hip/hip_runtime.h>

#include <mutex>

static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {nullptr};

// Device address of this device's copy of `scratch` (looked up on first use).
int scratch_for_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return (int)e;
        if (!p) return (int)hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return 0;
}

}  // namespace

extern "C" int moe_layer_noalloc(const moe_slot_pool* pool, const float* d_logits, const uint8_t* d_mask,
                                 const uint16_t* d_x, int T, int E, int k, int block_m, int act_mode,
                                 const int32_t* d_slot_of_expert, int32_t* d_topk_ids, float* d_topk_w,
                                 int32_t* d_sorted_pair, int32_t* d_block_slot, int32_t* d_counts,
                                 int32_t* d_seg_offset, int32_t* d_n_padded, int32_t* d_err, uint16_t* d_out,
                                 void* stream) {
    if (!pool) return MOE_EINVAL;
    const size_t need = moe_layer_workspace_bytes(T, k, E, pool->hidden, pool->inter, block_m, act_mode);
    if (need == 0) return MOE_EINVAL;
    if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ESCRATCH;
    void* ws = nullptr;
    const int e = scratch_for_current_device(&ws);
    if (e != 0) return moe::record_hip_error(e);
    return moe_layer(pool, d_logits, d_mask, d_x, T, E, k, block_m, act_mode, d_slot_of_expert, d_topk_ids, d_topk_w,
                     d_sorted_pair, d_block_slot, d_counts, d_seg_offset, d_n_padded, d_err, d_out, ws,
                     (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}
