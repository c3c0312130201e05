// Dequantize one slot to fp32 matrices (per-slot bit width: PagedWeight
// commentary, spectral-agent.com, "technically interesting points").
//   FP8 : W[r][c] = e4m3(q[r][c]) * scale[r]
//   INT4: W[r][c] = (q[r][c] - zero[r][c/128]) * scale[r][c/128]
// The slot's format is read on the device, so the launch carries the array
// offsets of both formats. A tag that is neither format, or names a format
// whose layout does not fit the pool stride, yields NaN matrices (nothing is
// read from the slot).
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

struct DqOffsets {
    size_t codes[2], scale[2];
};

__global__ void __launch_bounds__(256) dequant_kernel(const uint8_t* __restrict__ slot_base, const uint8_t* __restrict__ fmtp,
                                                     int slot, int fmt_ok, DqOffsets off, int rows, int cols,
                                                     float* __restrict__ out) {
    const int tag = fmtp[slot];
    const bool usable = fmt_usable(tag, fmt_ok);
    const int fmt = usable ? tag : 0;
    const uint8_t* codes = slot_base + off.codes[fmt];
    const uint8_t* scale = slot_base + off.scale[fmt];
    const size_t n = (size_t)rows * cols;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
        const int r = (int)(i / cols), c = (int)(i % cols);
        float v;
        if (!usable) {
            v = __builtin_nanf("");
        } else if (fmt == 0) {
            v = e4m3_to_f32(codes[i]) * ((const float*)scale)[r];
        } else {
            const uint8_t b = codes[(size_t)r * (cols / 2) + c / 2];
            const int qv = (c & 1) ? (b >> 4) : (b & 0xF);
            const _Float16* sz = (const _Float16*)scale + ((size_t)r * (cols / MOE_INT4_G) + c / MOE_INT4_G) * 2;
            v = ((float)qv - (float)sz[1]) * (float)sz[0];
        }
        out[i] = v;
    }
}

hipError_t launch_dequant(const PoolArgs& pa, int slot, float* w13, float* w2, hipStream_t stream) {
    const uint8_t* base = (const uint8_t*)pa.base + (size_t)slot * pa.stride;
    const int H = pa.hidden, I = pa.inter;
    if (w13) {
        DqOffsets o = {{pa.off[0][0], pa.off[1][0]}, {pa.off[0][1], pa.off[1][1]}};
        MOE_LAUNCH(K_DEQUANT, stream, dequant_kernel, dim3(512), dim3(256), 0, stream, base, pa.fmt, slot, pa.fmt_ok, o, 2 * I,
                   H, w13);
    }
    if (w2) {
        DqOffsets o = {{pa.off[0][2], pa.off[1][2]}, {pa.off[0][3], pa.off[1][3]}};
        MOE_LAUNCH(K_DEQUANT, stream, dequant_kernel, dim3(512), dim3(256), 0, stream, base, pa.fmt, slot, pa.fmt_ok, o, H, I,
                   w2);
    }
    return hipGetLastError();
}

}  // namespace moe
