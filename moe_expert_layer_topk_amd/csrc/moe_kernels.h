// Host-side launch entry points of the gfx950 kernels (internal to libmoe).
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// remember a failed HIP call for moe_last_hip_error(); returns MOE_EHIP
int record_hip_error(int hip_error);

// kernel ids for launch tracing (names in profile.hip)
enum KernelId { K_ROUTE, K_ROUTE_ALIGN, K_ALIGN_SINGLE, K_ALIGN_HIST, K_ALIGN_SCAN, K_ALIGN_SCATTER, K_GEMM1_STREAM,
                K_GEMM2_STREAM, K_QUANT_ACT, K_GEMM1_FP8, K_GEMM2_FP8, K_GEMM1_TILE, K_GEMM2_TILE, K_MFMA_PREP, K_COMBINE, K_DEQUANT, K_POOL_CHECK, K_POISON, K_ROUTER_GEMM, K_REQUANT, K_UNPACK, K_COUNT };
// events the next launch of kernel `kid` on `s` should stamp (false: not tracing)
bool prof_events(int kid, hipStream_t s, hipEvent_t* start, hipEvent_t* stop);

// launch a kernel; while tracing, its dispatch stamps a start and a stop event
#define MOE_LAUNCH(kid, stream, kernel, grid, block, shmem, strm, ...)                                   \
    do {                                                                                                \
        hipEvent_t moe_ev0_, moe_ev1_;                                                                  \
        if (::moe::prof_events((kid), (stream), &moe_ev0_, &moe_ev1_))                                  \
            hipExtLaunchKernelGGL(kernel, grid, block, shmem, strm, moe_ev0_, moe_ev1_, 0, __VA_ARGS__);  \
        else                                                                                            \
            hipLaunchKernelGGL(kernel, grid, block, shmem, strm, __VA_ARGS__);                          \
    } while (0)

struct PoolArgs {
    const void* base;
    size_t stride;
    const uint8_t* fmt;
    int n_slots;
    int hidden, inter;
    size_t off[2][4];   // byte offsets of the four arrays, per slot format
    int fmt_ok;         // bit f: format f's layout fits the stride (int4 also needs inter % 128 == 0)
    int spec_fmt;       // a format that fits: speculative loads before a slot's tag is known use it
};

// Optional check of slot-table entries against a pool (moe_layer passes one):
// an entry outside the pool or whose format tag is unusable becomes -1.
struct SlotCheck {
    const uint8_t* fmt = nullptr;   // null: entries are copied as given
    int n_slots = 0;
    int fmt_ok = 0;
};

// router gate GEMM (router.hip): logits = x W_g^T + bias in fp32
hipError_t launch_router_gemm(const uint16_t* x, const float* wg, const float* bias, int T, int H, int E,
                              float* logits, hipStream_t stream);

hipError_t launch_route(const float* logits, const uint8_t* mask, int T, int E, int k, int32_t* ids, float* w,
                        int32_t* err, hipStream_t stream);

int align_single_max_pairs();
int route_align_fused_max_pairs();
hipError_t launch_route_align(const float* logits, const uint8_t* mask, int T, int E, int k, int block_m,
                              const int32_t* slot_of_expert, int32_t* ids, float* w, int32_t* sorted_pair,
                              int32_t* block_slot, int32_t* counts, int32_t* seg_offset, int32_t* n_padded,
                              int32_t* err, void* ws, hipStream_t stream, SlotCheck chk = SlotCheck());
size_t align_workspace_bytes(int NP, int E);
hipError_t launch_align(const int32_t* ids, int T, int k, int E, int block_m, const int32_t* slot_of_expert,
                        int32_t* sorted_pair, int32_t* block_slot, int32_t* counts, int32_t* seg_offset,
                        int32_t* n_padded, int32_t* err, void* ws, hipStream_t stream, SlotCheck chk = SlotCheck());

int stream_max_tokens();
int device_cus();
size_t stream_workspace_bytes(int T, int k, int H, int I, int cap);
hipError_t launch_combine_f32(const float* ybuf, const float* topk_w, int T, int k, int H, uint16_t* out,
                              hipStream_t stream);
hipError_t launch_combine_bf16(const uint16_t* ybuf, const float* topk_w, int T, int k, int H, uint16_t* out,
                               hipStream_t stream);
// FFN call kinds: a whole call (workspace poisoning allowed, combine), or one
// pass of a deferred-block sequence (no poisoning; combine on the last pass)
enum FfnPass { FFN_WHOLE = 0, FFN_PASS = 1, FFN_PASS_LAST = 2 };
hipError_t launch_ffn_stream(const PoolArgs& pa, const uint16_t* x, int T, int k, const float* topk_w,
                             const int32_t* sorted_pair, const int32_t* block_slot, const int32_t* n_padded,
                             int cap, int block_m, uint16_t* out, void* ws, hipStream_t stream,
                             FfnPass pass = FFN_WHOLE);
// whole decode layer (route and align inside the gate/up kernel); layer_stream_ok says where it applies
bool layer_stream_ok(int T, int k, int E, int H, int I, int block_m, int cap);
size_t layer_stream_workspace_bytes(int T, int k, int H, int I, int cap);
hipError_t launch_layer_stream(const PoolArgs& pa, const float* logits, const uint8_t* mask,
                               const int32_t* slot_of_expert, int E, const uint16_t* x, int T, int k, int32_t* ids,
                               float* w, int32_t* sorted_pair, int32_t* block_slot, int32_t* counts,
                               int32_t* seg_offset, int32_t* n_padded, int32_t* err, int cap, uint16_t* out,
                               void* ws, hipStream_t stream);

size_t grouped_workspace_bytes(int T, int k, int H, int I, int cap);
hipError_t launch_ffn_grouped(const PoolArgs& pa, const uint16_t* x, int T, int k, const float* topk_w,
                              const int32_t* sorted_pair, const int32_t* block_slot, const int32_t* n_padded,
                              int cap, int block_m, uint16_t* out, void* ws, hipStream_t stream,
                              FfnPass pass = FFN_WHOLE);

bool mfma_path_ok(int H, int I);
size_t mfma_ws_bytes(int H, int cap);
// blocks the prep kernel found int4 or not resident (device list and count)
void mfma_other_list(void* ws, int H, int cap, const int** list, const int** n_list);
// per sorted position, written by the prep kernel: token (0 for padding),
// route weight (0 for padding), activation exponent bytes [block][K step][128 rows]
void mfma_prep_arrays(void* ws, int cap, const int32_t** tokrow, const float** wsort, const uint8_t** scl);
// phase 0: prep + gate/up kernel, phase 1: down kernel
hipError_t launch_mfma_ffn(const PoolArgs& pa, const uint8_t* xq, const uint8_t* xs, int NP, int k,
                           const float* topk_w, const int32_t* sorted_pair, const int32_t* block_slot,
                           const int32_t* n_padded, int cap, uint8_t* hq, uint8_t* hs, uint16_t* ybuf, void* ws,
                           int phase, hipStream_t stream);

hipError_t launch_dequant(const PoolArgs& pa, int slot, float* w13, float* w2, hipStream_t stream);

// activation quantization alone: e4m3 codes [rows][cols], E8M0 bytes [rows][cols / 128]
hipError_t launch_quant_act(const uint16_t* x, int rows, int cols, uint8_t* codes, uint8_t* exps, hipStream_t stream);

// pool validation (pool_check.hip): d_err += unusable slots; status[slot] optional
hipError_t launch_pool_check(const PoolArgs& pa, int32_t* err, uint8_t* status, hipStream_t stream);

// FP8 slot src -> int4-g128 slot dst of the same pool (requant.hip); tags[dst] set to int4
hipError_t launch_requant(const PoolArgs& pa, int src, int dst, uint8_t* tags, int32_t* err, hipStream_t stream);

// debug mode: fill workspace data regions with all-ones bytes (NaN in every
// float format used) before the FFN kernels run
void set_debug_poison(int on);
bool debug_poison_on();
hipError_t launch_poison(void* p, size_t bytes, hipStream_t stream);

// int4 blocks listed beside the FP8 matrix-core kernels (grid_y: a bound on
// the listed blocks), gate/up GEMM on an
// LDS ring (H and I multiples of 128 up to 2048)
bool int4_ring_ok(int H, int I);
hipError_t launch_gemm1_int4_ring(const PoolArgs& pa, const uint8_t* xq, const int32_t* tokrow, const uint8_t* scl,
                                  const int32_t* block_slot, int I, uint8_t* hq, uint8_t* hs, const int* list,
                                  const int* n_list, int grid_y, hipStream_t stream);
// ... and the down GEMM (with zero rows for listed blocks whose slot is not usable)
hipError_t launch_gemm2_int4_ring(const PoolArgs& pa, int NP, const float* wsort, const int32_t* sorted_pair,
                                  const int32_t* block_slot, int I, const uint8_t* hq, const uint8_t* hs,
                                  uint16_t* ybuf, const int* list, const int* n_list, int grid_y,
                                  hipStream_t stream);

}  // namespace moe
