// extern "C" boundary of libmoe: argument checks, workspace carving and
// dispatch to the gfx950 kernels. Declarations and contracts: include/moe.h.
#include "../../include/moe.h"
#include "moe_common.h"
#include "moe_kernels.h"

#include <hip/hip_runtime.h>

namespace {

thread_local int g_last_hip = 0;

// hipGetLastError() reports the last error of any runtime call on the thread,
// including the caller's own earlier calls; clear it before launching so a
// stale value is not taken for a failure of ours.
void clear_stale_error() { (void)hipGetLastError(); }

int hip_status(hipError_t e) {
    if (e == hipSuccess) return MOE_OK;
    g_last_hip = (int)e;
    return MOE_EHIP;
}

size_t up256(size_t n) { return (n + 255) / 256 * 256; }

}  // namespace

int moe::record_hip_error(int hip_error) {
    g_last_hip = hip_error;
    return MOE_EHIP;
}

namespace {

bool valid_block_m(int bm) { return bm == 16 || bm == 32 || bm == 64 || bm == 128 || bm == 256; }

// Byte offsets of the four arrays of a slot (each 256-byte aligned).
void slot_parts(int H, int I, int fmt, size_t off[4], size_t* total) {
    size_t sz[4];
    if (fmt == MOE_FMT_FP8_E4M3_ROW) {
        sz[0] = (size_t)2 * I * H;
        sz[1] = (size_t)2 * I * 4;
        sz[2] = (size_t)H * I;
        sz[3] = (size_t)H * 4;
    } else {
        sz[0] = (size_t)I * H;
        sz[1] = (size_t)2 * I * (H / 128) * 4;
        sz[2] = (size_t)H * I / 2;
        sz[3] = (size_t)H * (I / 128) * 4;
    }
    // An int4 slot keeps 16 bytes after its last array: the kernels read a
    // row's (scale, zero) pairs 16 bytes at a time, which for rows of fewer
    // than four groups runs up to 12 bytes past the row.
    const size_t tail = fmt == MOE_FMT_INT4_G128 ? 16 : 0;
    size_t o = 0;
    for (int i = 0; i < 4; ++i) {
        off[i] = o;
        o = up256(o + sz[i] + (i == 3 ? tail : 0));
    }
    if (total) *total = o;
}

bool pool_args(const moe_slot_pool* pool, moe::PoolArgs* pa) {
    if (!pool || !pool->d_base || !pool->d_slot_fmt || pool->n_slots < 1 || pool->n_slots > MOE_MAX_SLOTS) return false;
    const int H = pool->hidden, I = pool->inter;
    if (H < 128 || H % 128 || I < 64 || I % 64) return false;
    if (pool->slot_bytes % 256) return false;
    size_t fp8_bytes, int4_bytes = 0;
    slot_parts(H, I, MOE_FMT_FP8_E4M3_ROW, pa->off[0], &fp8_bytes);
    if (I % 128 == 0) {
        slot_parts(H, I, MOE_FMT_INT4_G128, pa->off[1], &int4_bytes);
    } else {
        for (int i = 0; i < 4; ++i) pa->off[1][i] = pa->off[0][i];   // int4 slots need inter % 128 == 0
    }
    // The tags live on the device; a format whose layout does not fit the
    // stride makes the slots tagged with it unusable (treated as not
    // resident), and a stride that fits neither format is refused.
    pa->fmt_ok = (pool->slot_bytes >= fp8_bytes ? 1 : 0) | (int4_bytes && pool->slot_bytes >= int4_bytes ? 2 : 0);
    if (!pa->fmt_ok) return false;
    pa->spec_fmt = (pa->fmt_ok & 1) ? MOE_FMT_FP8_E4M3_ROW : MOE_FMT_INT4_G128;
    pa->base = pool->d_base;
    pa->stride = pool->slot_bytes;
    pa->fmt = pool->d_slot_fmt;
    pa->n_slots = pool->n_slots;
    pa->hidden = H;
    pa->inter = I;
    return true;
}

int capacity(int T, int k, int E, int bm) {
    long long np = (long long)T * k;
    long long n = np + (np < E ? np : E) * (long long)(bm - 1);
    return (int)((n + bm - 1) / bm * bm);
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_strerror(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_EINVAL: return "invalid argument";
        case MOE_EHIP: return "HIP launch error";
        case MOE_ESCRATCH: return "workspace needed exceeds moe_layer_noalloc's built-in scratch";
        default: return "unknown status";
    }
}

int moe_last_hip_error(void) { return g_last_hip; }

int moe_route(const float* d_logits, const uint8_t* d_mask, int T, int E, int k, int32_t* d_topk_ids,
              float* d_topk_w, int32_t* d_err, void* stream) {
    if (!d_logits || !d_topk_ids || !d_topk_w || !d_err) return MOE_EINVAL;
    if (T < 1 || E < 1 || E > MOE_MAX_E || k < 1 || k > E || k > MOE_MAX_K) return MOE_EINVAL;
    clear_stale_error();
    return hip_status(moe::launch_route(d_logits, d_mask, T, E, k, d_topk_ids, d_topk_w, d_err, (hipStream_t)stream));
}

int moe_route_gemm(const uint16_t* d_x, const float* d_wg, const float* d_bias, const uint8_t* d_mask, int T, int H,
                   int E, int k, float* d_logits, int32_t* d_topk_ids, float* d_topk_w, int32_t* d_err, void* stream) {
    if (!d_x || !d_wg || !d_logits || !d_topk_ids || !d_topk_w || !d_err) return MOE_EINVAL;
    if (T < 1 || H < 128 || H % 128 || E < 1 || E > MOE_MAX_E || k < 1 || k > E || k > MOE_MAX_K) return MOE_EINVAL;
    clear_stale_error();
    hipError_t e = moe::launch_router_gemm(d_x, d_wg, d_bias, T, H, E, d_logits, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(moe::launch_route(d_logits, d_mask, T, E, k, d_topk_ids, d_topk_w, d_err, (hipStream_t)stream));
}

int moe_align_capacity(int T, int k, int E, int block_m) {
    if (T < 1 || k < 1 || E < 1 || !valid_block_m(block_m)) return MOE_EINVAL;
    if ((long long)T * k >= (1LL << 30)) return MOE_EINVAL;
    return capacity(T, k, E, block_m);
}

size_t moe_align_workspace_bytes(int T, int k, int E, int block_m) {
    if (T < 1 || k < 1 || E < 1 || E > MOE_MAX_E || !valid_block_m(block_m)) return 0;
    return moe::align_workspace_bytes(T * k, E);
}

int moe_align(const int32_t* d_topk_ids, int T, int k, int E, int block_m, const int32_t* d_slot_of_expert,
              int32_t* d_sorted_pair, int32_t* d_block_slot, int32_t* d_counts, int32_t* d_seg_offset,
              int32_t* d_n_padded, int32_t* d_err, void* d_ws, size_t ws_bytes, void* stream) {
    if (!d_topk_ids || !d_slot_of_expert || !d_sorted_pair || !d_block_slot || !d_counts || !d_seg_offset ||
        !d_n_padded || !d_err)
        return MOE_EINVAL;
    if (T < 1 || k < 1 || E < 1 || E > MOE_MAX_E || !valid_block_m(block_m)) return MOE_EINVAL;
    if ((long long)T * k >= (1LL << 30)) return MOE_EINVAL;
    size_t need = moe::align_workspace_bytes(T * k, E);
    if (need && (!d_ws || ws_bytes < need)) return MOE_EINVAL;
    clear_stale_error();
    return hip_status(moe::launch_align(d_topk_ids, T, k, E, block_m, d_slot_of_expert, d_sorted_pair, d_block_slot,
                                        d_counts, d_seg_offset, d_n_padded, d_err, d_ws, (hipStream_t)stream));
}

int moe_route_align(const float* d_logits, const uint8_t* d_mask, int T, int E, int k, int block_m,
                    const int32_t* d_slot_of_expert, int32_t* d_topk_ids, float* d_topk_w, int32_t* d_sorted_pair,
                    int32_t* d_block_slot, int32_t* d_counts, int32_t* d_seg_offset, int32_t* d_n_padded,
                    int32_t* d_err, void* d_ws, size_t ws_bytes, void* stream) {
    if (!d_logits || !d_slot_of_expert || !d_topk_ids || !d_topk_w || !d_sorted_pair || !d_block_slot || !d_counts ||
        !d_seg_offset || !d_n_padded || !d_err)
        return MOE_EINVAL;
    if (T < 1 || E < 1 || E > MOE_MAX_E || k < 1 || k > E || k > MOE_MAX_K || !valid_block_m(block_m))
        return MOE_EINVAL;
    if ((long long)T * k >= (1LL << 30)) return MOE_EINVAL;
    const size_t need = moe_route_align_workspace_bytes(T, k, E, block_m);
    if (need && (!d_ws || ws_bytes < need)) return MOE_EINVAL;
    clear_stale_error();
    return hip_status(moe::launch_route_align(d_logits, d_mask, T, E, k, block_m, d_slot_of_expert, d_topk_ids,
                                              d_topk_w, d_sorted_pair, d_block_slot, d_counts, d_seg_offset,
                                              d_n_padded, d_err, d_ws, (hipStream_t)stream));
}

size_t moe_route_align_workspace_bytes(int T, int k, int E, int block_m) {
    if (T < 1 || k < 1 || E < 1 || E > MOE_MAX_E || !valid_block_m(block_m)) return 0;
    return moe::align_workspace_bytes(T * k, E);
}

size_t moe_slot_bytes(int hidden, int inter, int fmt) {
    if (hidden < 128 || hidden % 128 || inter < 64 || inter % 64) return 0;
    if (fmt != MOE_FMT_FP8_E4M3_ROW && fmt != MOE_FMT_INT4_G128) return 0;
    if (fmt == MOE_FMT_INT4_G128 && inter % 128) return 0;
    size_t off[4], total;
    slot_parts(hidden, inter, fmt, off, &total);
    return total;
}

size_t moe_slot_part_offset(int hidden, int inter, int fmt, int part) {
    if (part < 0 || part > 3 || moe_slot_bytes(hidden, inter, fmt) == 0) return (size_t)-1;
    size_t off[4], total;
    slot_parts(hidden, inter, fmt, off, &total);
    return off[part];
}

size_t moe_ffn_workspace_bytes(int T, int k, int E, int hidden, int inter, int block_m, int act_mode) {
    if (T < 1 || k < 1 || E < 1 || !valid_block_m(block_m)) return 0;
    const int cap = capacity(T, k, E, block_m);
    if (act_mode == MOE_ACT_BF16) return moe::stream_workspace_bytes(T, k, hidden, inter, cap);
    if (act_mode == MOE_ACT_FP8_G128_POW2) return moe::grouped_workspace_bytes(T, k, hidden, inter, cap);
    return 0;
}

}  // extern "C"

namespace {

int expert_ffn(const moe_slot_pool* pool, const uint16_t* d_x, int T, int k, int E, const float* d_topk_w,
               const int32_t* d_sorted_pair, const int32_t* d_block_slot, const int32_t* d_n_padded, int block_m,
               int act_mode, uint16_t* d_out, void* d_ws, size_t ws_bytes, void* stream, moe::FfnPass pass) {
    moe::PoolArgs pa;
    if (!pool_args(pool, &pa)) return MOE_EINVAL;
    if (!d_x || !d_topk_w || !d_sorted_pair || !d_block_slot || !d_n_padded || !d_out || !d_ws) return MOE_EINVAL;
    if (T < 1 || k < 1 || E < 1 || E > MOE_MAX_E || k > E) return MOE_EINVAL;
    if ((long long)T * k >= (1LL << 30)) return MOE_EINVAL;
    const int cap = capacity(T, k, E, block_m < 1 ? 1 : block_m);
    if (act_mode == MOE_ACT_BF16) {
        if (block_m != 16 && block_m != 32 && block_m != 64) return MOE_EINVAL;
        if (T > moe::stream_max_tokens()) return MOE_EINVAL;
        if (ws_bytes < moe::stream_workspace_bytes(T, k, pa.hidden, pa.inter, cap)) return MOE_EINVAL;
        clear_stale_error();
        return hip_status(moe::launch_ffn_stream(pa, d_x, T, k, d_topk_w, d_sorted_pair, d_block_slot, d_n_padded,
                                                 cap, block_m, d_out, d_ws, (hipStream_t)stream, pass));
    }
    if (act_mode == MOE_ACT_FP8_G128_POW2) {
        if (block_m != 64 && block_m != 128) return MOE_EINVAL;
        if (ws_bytes < moe::grouped_workspace_bytes(T, k, pa.hidden, pa.inter, cap)) return MOE_EINVAL;
        clear_stale_error();
        return hip_status(moe::launch_ffn_grouped(pa, d_x, T, k, d_topk_w, d_sorted_pair, d_block_slot, d_n_padded,
                                                  cap, block_m, d_out, d_ws, (hipStream_t)stream, pass));
    }
    return MOE_EINVAL;
}

}  // namespace

extern "C" {

int moe_expert_ffn(const moe_slot_pool* pool, const uint16_t* d_x, int T, int k, int E, const float* d_topk_w,
                   const int32_t* d_sorted_pair, const int32_t* d_block_slot, const int32_t* d_n_padded,
                   int block_m, int act_mode, uint16_t* d_out, void* d_ws, size_t ws_bytes, void* stream) {
    return expert_ffn(pool, d_x, T, k, E, d_topk_w, d_sorted_pair, d_block_slot, d_n_padded, block_m, act_mode, d_out,
                      d_ws, ws_bytes, stream, moe::FFN_WHOLE);
}

int moe_expert_ffn_pass(const moe_slot_pool* pool, const uint16_t* d_x, int T, int k, int E, const float* d_topk_w,
                        const int32_t* d_sorted_pair, const int32_t* d_block_slot, const int32_t* d_n_padded,
                        int block_m, int act_mode, int last_pass, uint16_t* d_out, void* d_ws, size_t ws_bytes,
                        void* stream) {
    return expert_ffn(pool, d_x, T, k, E, d_topk_w, d_sorted_pair, d_block_slot, d_n_padded, block_m, act_mode, d_out,
                      d_ws, ws_bytes, stream, last_pass ? moe::FFN_PASS_LAST : moe::FFN_PASS);
}

size_t moe_layer_workspace_bytes(int T, int k, int E, int hidden, int inter, int block_m, int act_mode) {
    size_t ffn = moe_ffn_workspace_bytes(T, k, E, hidden, inter, block_m, act_mode);
    if (ffn == 0) return 0;
    if (act_mode == MOE_ACT_BF16 && block_m == 16) {          // the decode layer path's larger need
        const size_t lay = moe::layer_stream_workspace_bytes(T, k, hidden, inter, capacity(T, k, E, block_m));
        ffn = ffn > lay ? ffn : lay;
    }
    return up256(moe_route_align_workspace_bytes(T, k, E, block_m)) + ffn;
}

int moe_layer(const moe_slot_pool* pool, const float* d_logits, const uint8_t* d_mask, const uint16_t* d_x, int T,
              int E, int k, int block_m, int act_mode, const int32_t* d_slot_of_expert, int32_t* d_topk_ids,
              float* d_topk_w, int32_t* d_sorted_pair, int32_t* d_block_slot, int32_t* d_counts,
              int32_t* d_seg_offset, int32_t* d_n_padded, int32_t* d_err, uint16_t* d_out, void* d_ws,
              size_t ws_bytes, void* stream) {
    moe::PoolArgs pa;
    if (!pool_args(pool, &pa)) return MOE_EINVAL;
    if (!d_logits || !d_x || !d_slot_of_expert || !d_topk_ids || !d_topk_w || !d_sorted_pair || !d_block_slot ||
        !d_counts || !d_seg_offset || !d_n_padded || !d_err || !d_out || !d_ws)
        return MOE_EINVAL;
    if (T < 1 || E < 1 || E > MOE_MAX_E || k < 1 || k > E || k > MOE_MAX_K || !valid_block_m(block_m))
        return MOE_EINVAL;
    if ((long long)T * k >= (1LL << 30)) return MOE_EINVAL;
    const size_t need = moe_layer_workspace_bytes(T, k, E, pa.hidden, pa.inter, block_m, act_mode);
    if (need == 0 || ws_bytes < need) return MOE_EINVAL;
    const int cap = capacity(T, k, E, block_m);
    if (act_mode == MOE_ACT_BF16 && moe::layer_stream_ok(T, k, E, pa.hidden, pa.inter, block_m, cap)) {
        const size_t aws = up256(moe_route_align_workspace_bytes(T, k, E, block_m));
        clear_stale_error();
        return hip_status(moe::launch_layer_stream(pa, d_logits, d_mask, d_slot_of_expert, E, d_x, T, k, d_topk_ids,
                                                   d_topk_w, d_sorted_pair, d_block_slot, d_counts, d_seg_offset,
                                                   d_n_padded, d_err, cap, d_out, (uint8_t*)d_ws + aws,
                                                   (hipStream_t)stream));
    }
    // other shapes: the separate calls' kernels, on the same stream; the
    // align step checks the slot table against the pool
    const size_t aws_bytes = moe_route_align_workspace_bytes(T, k, E, block_m);
    const size_t aws = up256(aws_bytes);
    moe::SlotCheck chk;
    chk.fmt = pa.fmt;
    chk.n_slots = pa.n_slots;
    chk.fmt_ok = pa.fmt_ok;
    clear_stale_error();
    int st = hip_status(moe::launch_route_align(d_logits, d_mask, T, E, k, block_m, d_slot_of_expert, d_topk_ids,
                                                d_topk_w, d_sorted_pair, d_block_slot, d_counts, d_seg_offset,
                                                d_n_padded, d_err, aws_bytes ? d_ws : nullptr, (hipStream_t)stream,
                                                chk));
    if (st != MOE_OK) return st;
    return moe_expert_ffn(pool, d_x, T, k, E, d_topk_w, d_sorted_pair, d_block_slot, d_n_padded, block_m, act_mode,
                          d_out, (uint8_t*)d_ws + aws, ws_bytes - aws, stream);
}

int moe_quant_act(const uint16_t* d_x, int rows, int cols, uint8_t* d_codes, uint8_t* d_exps, void* stream) {
    if (!d_x || !d_codes || !d_exps || rows < 1 || cols < MOE_ACT_G || cols % MOE_ACT_G) return MOE_EINVAL;
    if ((long long)rows * (cols / MOE_ACT_G) >= (1LL << 31)) return MOE_EINVAL;
    clear_stale_error();
    return hip_status(moe::launch_quant_act(d_x, rows, cols, d_codes, d_exps, (hipStream_t)stream));
}

int moe_pool_check(const moe_slot_pool* pool, int32_t* d_err, uint8_t* d_status, void* stream) {
    moe::PoolArgs pa;
    if (!pool_args(pool, &pa) || !d_err) return MOE_EINVAL;
    clear_stale_error();
    return hip_status(moe::launch_pool_check(pa, d_err, d_status, (hipStream_t)stream));
}

int moe_requant_slot(const moe_slot_pool* pool, int src_slot, int dst_slot, int32_t* d_err, void* stream) {
    moe::PoolArgs pa;
    if (!pool_args(pool, &pa)) return MOE_EINVAL;
    if ((pa.fmt_ok & 3) != 3) return MOE_EINVAL;                 // both formats must fit the stride
    if (src_slot < 0 || src_slot >= pa.n_slots || dst_slot < 0 || dst_slot >= pa.n_slots || src_slot == dst_slot)
        return MOE_EINVAL;
    clear_stale_error();
    return hip_status(moe::launch_requant(pa, src_slot, dst_slot, (uint8_t*)pool->d_slot_fmt, d_err,
                                          (hipStream_t)stream));
}

int moe_debug_poison(int on) {
    moe::set_debug_poison(on);
    return MOE_OK;
}

int moe_dequant_slot(const moe_slot_pool* pool, int slot, float* d_w13, float* d_w2, void* stream) {
    moe::PoolArgs pa;
    if (!pool_args(pool, &pa)) return MOE_EINVAL;
    if (slot < 0 || slot >= pool->n_slots) return MOE_EINVAL;
    if (!d_w13 && !d_w2) return MOE_EINVAL;
    clear_stale_error();
    return hip_status(moe::launch_dequant(pa, slot, d_w13, d_w2, (hipStream_t)stream));
}

}  // extern "C"
