// Launch tracing: when enabled, every kernel the library launches carries a
// start and a stop HIP event that the dispatch itself stamps (AMD's extended
// launch), so an event pair spans exactly that kernel's execution;
// moe_profile_read() sums the elapsed times per kernel. Off by default;
// skipped while a stream is being captured into a graph. Single-threaded use.
#include "../../include/moe.h"
#include "moe_kernels.h"

#include <vector>

namespace moe {
namespace {

struct Mark {
    int kid;
    hipEvent_t start, stop;
};

bool g_on = false;
std::vector<Mark> g_marks;
std::vector<hipEvent_t> g_free;

const char* kNames[K_COUNT] = {"route", "route_align", "align_single", "align_hist", "align_scan", "align_scatter",
                               "gemm1_stream", "gemm2_stream", "quant_act", "gemm1_fp8", "gemm2_fp8", "gemm1_tile", "gemm2_tile", "mfma_prep",
                               "combine", "dequant", "pool_check", "poison", "router_gemm",
                               "requant", "fp8_unpack"};

hipEvent_t take_event() {
    if (!g_free.empty()) {
        hipEvent_t e = g_free.back();
        g_free.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

void recycle() {
    for (auto& m : g_marks) {
        g_free.push_back(m.start);
        g_free.push_back(m.stop);
    }
    g_marks.clear();
}

}  // namespace

bool prof_events(int kid, hipStream_t s, hipEvent_t* start, hipEvent_t* stop) {
    *start = *stop = nullptr;
    if (!g_on) return false;
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &st) != hipSuccess || st != hipStreamCaptureStatusNone) return false;
    hipEvent_t a = take_event(), b = take_event();
    if (!a || !b) {
        if (a) g_free.push_back(a);
        if (b) g_free.push_back(b);
        return false;
    }
    *start = a;
    *stop = b;
    g_marks.push_back({kid, a, b});
    return true;
}

}  // namespace moe

extern "C" {

int moe_profile_enable(int on) {
    moe::recycle();
    moe::g_on = on != 0;
    if (!on) {
        for (hipEvent_t e : moe::g_free) (void)hipEventDestroy(e);
        moe::g_free.clear();
    }
    return MOE_OK;
}

int moe_profile_kernels(void) { return moe::K_COUNT; }

const char* moe_profile_kernel_name(int kernel) {
    return (kernel >= 0 && kernel < moe::K_COUNT) ? moe::kNames[kernel] : "";
}

int moe_profile_read(int kernel, int* launches, double* total_ms) {
    if (kernel < 0 || kernel >= moe::K_COUNT || !launches || !total_ms) return MOE_EINVAL;
    *launches = 0;
    *total_ms = 0.0;
    for (const auto& m : moe::g_marks) {
        if (m.kid != kernel) continue;
        if (hipEventSynchronize(m.stop) != hipSuccess) return MOE_EHIP;
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, m.start, m.stop) != hipSuccess) return MOE_EHIP;
        *launches += 1;
        *total_ms += ms;
    }
    return MOE_OK;
}

}  // extern "C"
