// Launch tracing: when enabled, every kernel the library launches is
// bracketed by two HIP events on its stream; moe_profile_read() sums the
// elapsed times per kernel. Off by default; skipped while a stream is being
// captured into a graph. Single-threaded use.
#include "../../include/moe.h"
#include "moe_kernels.h"

#include <vector>

namespace moe {
namespace {

struct Mark {
    int kid;
    bool start;
    hipEvent_t ev;
};

bool g_on = false;
std::vector<Mark> g_marks;
std::vector<hipEvent_t> g_free;

const char* kNames[K_COUNT] = {"route", "route_align", "align_single", "align_hist", "align_scan", "align_scatter",
                               "gemm1_stream", "gemm2_stream", "quant_act", "gemm1_fp8", "gemm2_fp8", "gemm1_tile", "gemm2_tile", "mfma_prep",
                               "combine", "dequant"};

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
    for (auto& m : g_marks) g_free.push_back(m.ev);
    g_marks.clear();
}

}  // namespace

void prof_mark(int kid, hipStream_t s, bool start) {
    if (!g_on) return;
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &st) == hipSuccess && st != hipStreamCaptureStatusNone) return;
    hipEvent_t e = take_event();
    if (!e) return;
    if (hipEventRecord(e, s) != hipSuccess) {
        g_free.push_back(e);
        return;
    }
    g_marks.push_back({kid, start, e});
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
    const auto& m = moe::g_marks;
    for (size_t i = 0; i + 1 < m.size(); ++i) {
        if (m[i].kid != kernel || !m[i].start) continue;
        size_t j = i + 1;
        while (j < m.size() && !(m[j].kid == kernel && !m[j].start)) ++j;
        if (j == m.size()) break;
        if (hipEventSynchronize(m[j].ev) != hipSuccess) return MOE_EHIP;
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, m[i].ev, m[j].ev) != hipSuccess) return MOE_EHIP;
        *launches += 1;
        *total_ms += ms;
    }
    return MOE_OK;
}

}  // extern "C"
