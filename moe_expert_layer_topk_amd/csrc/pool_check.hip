// Slot pool validation and the workspace-poisoning debug mode.
//
// vllm-expert-pager article (rand.pepabo.com), "hierarchical paging of expert
// weights": a layer's experts live in VRAM slots that are refilled while the
// model runs, so a slot can hold bytes the kernels were never meant to read.
// The kernels themselves never read outside the pool (unusable slots count as
// not resident); moe_pool_check tells the caller which slots are unusable and
// why, including int4 zero points the kernels' exact q - zero forms assume to
// be integers in [0, 15] (PagedWeight commentary, spectral-agent.com,
// "technically interesting points": experts held at their own bit width).
#include "../../include/moe.h"
#include "moe_common.h"
#include "moe_kernels.h"

#include <atomic>

namespace moe {

// One workgroup per slot. Status: 0 usable, 1 tag is not a format, 2 the
// format does not fit the stride (or int4 with inter % 128 != 0), 3 an int4
// (scale, zero) pair with a zero that is not an integer in [0, 15] or a scale
// that is not finite, 4 an FP8 row scale that is not finite.
__global__ void __launch_bounds__(256) pool_check_kernel(const uint8_t* __restrict__ base, size_t stride,
                                                        const uint8_t* __restrict__ fmt, int fmt_ok, size_t off_s13_8,
                                                        size_t off_s2_8, size_t off_sz13_4, size_t off_sz2_4, int H,
                                                        int I, int32_t* __restrict__ err,
                                                        uint8_t* __restrict__ status) {
    __shared__ int s_bad;
    const int slot = blockIdx.x;
    const int tag = fmt[slot];
    int st = 0;
    if (tag != MOE_FMT_FP8_E4M3_ROW && tag != MOE_FMT_INT4_G128) st = 1;
    else if (!fmt_usable(tag, fmt_ok)) st = 2;
    if (threadIdx.x == 0) s_bad = 0;
    __syncthreads();
    if (st == 0) {
        const uint8_t* sb = base + (size_t)slot * stride;
        int bad = 0;
        if (tag == MOE_FMT_INT4_G128) {
            // (scale, zero) fp16 pairs: 2I rows x H/128 groups, then H rows x I/128 groups
            const size_t n13 = (size_t)2 * I * (H / MOE_INT4_G), n2 = (size_t)H * (I / MOE_INT4_G);
            for (size_t i = threadIdx.x; i < n13 + n2; i += blockDim.x) {
                const uint32_t w = i < n13 ? ((const uint32_t*)(sb + off_sz13_4))[i]
                                           : ((const uint32_t*)(sb + off_sz2_4))[i - n13];
                const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
                const float z = (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
                const bool ok = __builtin_isfinite(s) && z >= 0.f && z <= 15.f && z == rintf(z);
                bad |= ok ? 0 : 1;
            }
        } else {
            for (int i = threadIdx.x; i < 2 * I + H; i += blockDim.x) {
                const float s = i < 2 * I ? ((const float*)(sb + off_s13_8))[i]
                                          : ((const float*)(sb + off_s2_8))[i - 2 * I];
                bad |= __builtin_isfinite(s) ? 0 : 1;
            }
        }
        if (bad) atomicOr(&s_bad, 1);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        if (st == 0 && s_bad) st = tag == MOE_FMT_INT4_G128 ? 3 : 4;
        if (status) status[slot] = (uint8_t)st;
        if (st) atomicAdd(err, 1);
    }
}

hipError_t launch_pool_check(const PoolArgs& pa, int32_t* err, uint8_t* status, hipStream_t stream) {
    MOE_LAUNCH(K_POOL_CHECK, stream, pool_check_kernel, dim3(pa.n_slots), dim3(256), 0, stream,
               (const uint8_t*)pa.base, pa.stride, pa.fmt, pa.fmt_ok, pa.off[0][1], pa.off[0][3], pa.off[1][1],
               pa.off[1][3], pa.hidden, pa.inter, err, status);
    return hipGetLastError();
}

// ------------------------------------------------------------ poison
namespace {
std::atomic<int> g_poison{0};
}

void set_debug_poison(int on) { g_poison.store(on ? 1 : 0); }
bool debug_poison_on() { return g_poison.load() != 0; }

// all-ones bytes: NaN as bf16, fp32 and e4m3, so a read of never-written
// workspace data reaches the output as NaN
__global__ void __launch_bounds__(256) poison_kernel(uint32_t* __restrict__ p, size_t words) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0xFFFFFFFFu;
}

hipError_t launch_poison(void* p, size_t bytes, hipStream_t stream) {
    const size_t words = bytes / 4;
    if (words == 0) return hipSuccess;
    size_t blocks = (words + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    MOE_LAUNCH(K_POISON, stream, poison_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (uint32_t*)p, words);
    return hipGetLastError();
}

}  // namespace moe
