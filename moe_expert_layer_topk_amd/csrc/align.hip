// Align: stable counting sort of token-expert pairs into per-expert segments
// padded to the GEMM tile, plus the expert -> slot indirection.
//
// MOE-GEN explainer (aibr.jp), sections 1 and 3: tokens are grouped per
// expert so each expert runs one large batch. vllm-expert-pager article
// (rand.pepabo.com), "hierarchical paging of expert weights": a per-layer
// table says which VRAM slot holds which expert.
//
// Positions come from counts and wavefront ranks only (ballot / popcount
// matching), never from the order in which atomics land, so every output is
// identical from run to run.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

constexpr int ALIGN_THREADS = 1024;              // 16 waves
constexpr int ALIGN_WAVES = ALIGN_THREADS / MOE_WAVE;
constexpr int ALIGN_CHUNK = 4096;                // pairs per block in the multi-block path

// Lanes of the wave that hold the same key (keys < 2048; -1 = no key).
__device__ __forceinline__ uint64_t match_peers(int key) {
    uint64_t peers = __ballot(key >= 0);
    peers = key >= 0 ? peers : ~peers;
#pragma unroll
    for (int b = 0; b < 11; ++b) {
        uint64_t m = __ballot((key >> b) & 1);
        peers &= ((key >> b) & 1) ? m : ~m;
    }
    return peers;
}

// Block-wide exclusive scan of one int per thread (blockDim == ALIGN_THREADS).
__device__ int block_exclusive_scan(int v, int* s_tmp, int& total) {
    const int lane = lane_id(), wv = threadIdx.x / MOE_WAVE;
    int x = v;
#pragma unroll
    for (int o = 1; o < MOE_WAVE; o <<= 1) {
        int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == MOE_WAVE - 1) s_tmp[wv] = x;
    __syncthreads();
    if (wv == 0) {
        int s = lane < ALIGN_WAVES ? s_tmp[lane] : 0;
#pragma unroll
        for (int o = 1; o < MOE_WAVE; o <<= 1) {
            int y = __shfl_up(s, o, 64);
            if (lane >= o) s += y;
        }
        if (lane < ALIGN_WAVES) s_tmp[ALIGN_WAVES + lane] = s;   // inclusive wave totals
    }
    __syncthreads();
    int wave_base = wv == 0 ? 0 : s_tmp[ALIGN_WAVES + wv - 1];
    total = s_tmp[2 * ALIGN_WAVES - 1];
    __syncthreads();
    return wave_base + x - v;
}

// From per-expert counts: padded offsets, n_padded, block -> slot map, the
// sentinel padding of every segment tail, and the non-resident pair count.
// One block of ALIGN_THREADS threads; counts in s_cnt[E]. With a slot check,
// an entry outside the pool or with an unusable format counts as -1 (not
// resident).
__device__ void segments_from_counts(const int* s_cnt, int* s_off, int* s_sl, int* s_tmp, int E, int block_m,
                                     int sentinel, const int32_t* slot_of_expert, SlotCheck chk, int32_t* counts,
                                     int32_t* seg_offset, int32_t* n_padded, int32_t* block_slot,
                                     int32_t* sorted_pair, int32_t* err) {
    const int e = threadIdx.x;
    int c = e < E ? s_cnt[e] : 0;
    int sl = e < E ? slot_of_expert[e] : -1;
    if (chk.fmt && sl >= 0) sl = usable_slot(sl, chk.n_slots, chk.fmt_ok, chk.fmt);
    int padded = (c + block_m - 1) / block_m * block_m;
    int total;
    int off = block_exclusive_scan(padded, s_tmp, total);
    if (e < E) {
        s_off[e] = off;
        s_sl[e] = sl;
        counts[e] = c;
        seg_offset[e] = off;
        if (sl < 0 && sl != MOE_SLOT_DEFERRED && c > 0) atomicAdd(err, c);   // (deferred: not an error)
    }
    if (e == 0) {
        seg_offset[E] = total;
        *n_padded = total;
    }
    __syncthreads();
    // block -> slot, spread over the workgroup by block (a hot expert's
    // segment spans many blocks): a block's expert is the last one whose
    // segment starts at or before it (empty segments share their offset with
    // the next expert, so the last one is never empty)
    for (int b = threadIdx.x; b < total / block_m; b += blockDim.x) {
        const int pos = b * block_m;
        int lo = 0, hi = E - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_off[mid] <= pos) lo = mid;
            else hi = mid - 1;
        }
        block_slot[b] = s_sl[lo];
    }
    // the sentinel tails (only a segment's last block holds padding): one
    // wave per expert, the tail's positions across the lanes, so each store
    // covers whole lines instead of one lane's run of single positions
    {
        const int lane = lane_id(), wv = threadIdx.x / MOE_WAVE, nw = blockDim.x / MOE_WAVE;
        for (int x = wv; x < E; x += nw) {
            const int c = s_cnt[x], o = s_off[x];
            const int pad = (c + block_m - 1) / block_m * block_m;
            for (int q = o + c + lane; q < o + pad; q += MOE_WAVE) sorted_pair[q] = sentinel;
        }
    }
    __syncthreads();
}

// Scatter pairs [p0, p1) in ascending order; s_run[e] holds the next free
// position of expert e and is advanced. The pairs are taken in rounds of
// ALIGN_THREADS; inside a round, wave w's pairs of expert e are placed after
// those of waves < w (wave counts in s_wcnt[w][e]).
__device__ void scatter_pairs(const int32_t* ids, int p0, int p1, int E, int* s_run, uint8_t* s_wcnt,
                              int32_t* sorted_pair) {
    const int lane = lane_id(), wv = threadIdx.x / MOE_WAVE;
    for (int base = p0; base < p1; base += ALIGN_THREADS) {
        for (int i = threadIdx.x; i < ALIGN_WAVES * E; i += ALIGN_THREADS) s_wcnt[i] = 0;
        __syncthreads();
        int p = base + threadIdx.x;
        int e = p < p1 ? ids[p] : -1;
        if (e >= E) e = -1;
        uint64_t peers = match_peers(e);
        int rank = __popcll(peers & lanemask_lt());
        bool leader = e >= 0 && (peers & lanemask_lt()) == 0;
        if (leader) s_wcnt[wv * E + e] = (uint8_t)__popcll(peers);
        __syncthreads();
        if (e >= 0) {
            int before = 0;
            for (int w2 = 0; w2 < wv; ++w2) before += s_wcnt[w2 * E + e];
            sorted_pair[s_run[e] + before + rank] = p;
        }
        __syncthreads();
        for (int x = threadIdx.x; x < E; x += ALIGN_THREADS) {
            int add = 0;
            for (int w2 = 0; w2 < ALIGN_WAVES; ++w2) add += s_wcnt[w2 * E + x];
            s_run[x] += add;
        }
        __syncthreads();
    }
}

// Whole align in one block (small T*k).
__global__ void __launch_bounds__(ALIGN_THREADS) align_single_kernel(
    const int32_t* __restrict__ ids, int NP, int E, int block_m, const int32_t* __restrict__ slot_of_expert,
    int32_t* sorted_pair, int32_t* block_slot, int32_t* counts, int32_t* seg_offset, int32_t* n_padded,
    int32_t* err, SlotCheck chk) {
    __shared__ int s_cnt[MOE_MAX_E];
    __shared__ int s_run[MOE_MAX_E];
    __shared__ int s_sl[MOE_MAX_E];
    __shared__ int s_tmp[2 * ALIGN_WAVES];
    __shared__ uint8_t s_wcnt[ALIGN_WAVES * MOE_MAX_E];
    for (int i = threadIdx.x; i < E; i += ALIGN_THREADS) s_cnt[i] = 0;
    __syncthreads();
    int bad = 0;
    for (int p = threadIdx.x; p < NP; p += ALIGN_THREADS) {
        int e = ids[p];
        if (e >= 0 && e < E) atomicAdd(&s_cnt[e], 1);
        else ++bad;
    }
    if (bad) atomicAdd(err, bad);
    __syncthreads();
    segments_from_counts(s_cnt, s_run, s_sl, s_tmp, E, block_m, NP, slot_of_expert, chk, counts, seg_offset,
                         n_padded, block_slot, sorted_pair, err);
    scatter_pairs(ids, 0, NP, E, s_run, s_wcnt, sorted_pair);
}

// Multi-block path: 1) per-chunk histograms, 2) one block turns them into
// segments and per-chunk start positions, 3) each chunk scatters its pairs.
__global__ void __launch_bounds__(256) align_hist_kernel(const int32_t* __restrict__ ids, int NP, int E,
                                                        int32_t* __restrict__ hist, int32_t* err) {
    __shared__ int s_cnt[MOE_MAX_E];
    for (int i = threadIdx.x; i < E; i += blockDim.x) s_cnt[i] = 0;
    __syncthreads();
    int p0 = blockIdx.x * ALIGN_CHUNK, p1 = min(NP, p0 + ALIGN_CHUNK);
    int bad = 0;
    for (int p = p0 + threadIdx.x; p < p1; p += blockDim.x) {
        int e = ids[p];
        if (e >= 0 && e < E) atomicAdd(&s_cnt[e], 1);
        else ++bad;
    }
    if (bad) atomicAdd(err, bad);
    __syncthreads();
    for (int i = threadIdx.x; i < E; i += blockDim.x) hist[(size_t)blockIdx.x * E + i] = s_cnt[i];
}

__global__ void __launch_bounds__(ALIGN_THREADS) align_scan_kernel(
    int32_t* __restrict__ hist, int n_chunks, int NP, int E, int block_m,
    const int32_t* __restrict__ slot_of_expert, int32_t* sorted_pair, int32_t* block_slot, int32_t* counts,
    int32_t* seg_offset, int32_t* n_padded, int32_t* err, SlotCheck chk) {
    __shared__ int s_cnt[MOE_MAX_E];
    __shared__ int s_off[MOE_MAX_E];
    __shared__ int s_sl[MOE_MAX_E];
    __shared__ int s_tmp[2 * ALIGN_WAVES];
    const int e = threadIdx.x;
    constexpr int B = 32;                // chunk counts loaded per round trip (clamped, no branches)
    int v[B];                            // the last group read; with n_chunks <= B, all of them
    auto read_group = [&](int b0) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < B; ++j) v[j] = hist[(size_t)min(b0 + j, n_chunks - 1) * E + e];
#pragma unroll
        for (int j = 0; j < B; ++j) v[j] = b0 + j < n_chunks ? v[j] : 0;
    };
    if (e < E) {
        int c = 0;
        for (int b0 = 0; b0 < n_chunks; b0 += B) {
            read_group(b0);
#pragma unroll
            for (int j = 0; j < B; ++j) c += v[j];
        }
        s_cnt[e] = c;
    }
    __syncthreads();
    segments_from_counts(s_cnt, s_off, s_sl, s_tmp, E, block_m, NP, slot_of_expert, chk, counts, seg_offset,
                         n_padded, block_slot, sorted_pair, err);
    if (e < E) {                         // hist[b][e] <- start of chunk b's pairs of expert e
        int run = s_off[e];
        for (int b0 = 0; b0 < n_chunks; b0 += B) {
            if (n_chunks > B) read_group(b0);
#pragma unroll
            for (int j = 0; j < B; ++j) {
                if (b0 + j < n_chunks) hist[(size_t)(b0 + j) * E + e] = run;
                run += v[j];
            }
        }
    }
}

__global__ void __launch_bounds__(ALIGN_THREADS) align_scatter_kernel(const int32_t* __restrict__ ids, int NP,
                                                                     int E, const int32_t* __restrict__ start,
                                                                     int32_t* sorted_pair) {
    __shared__ int s_run[MOE_MAX_E];
    __shared__ uint8_t s_wcnt[ALIGN_WAVES * MOE_MAX_E];
    for (int i = threadIdx.x; i < E; i += ALIGN_THREADS) s_run[i] = start[(size_t)blockIdx.x * E + i];
    __syncthreads();
    int p0 = blockIdx.x * ALIGN_CHUNK, p1 = min(NP, p0 + ALIGN_CHUNK);
    scatter_pairs(ids, p0, p1, E, s_run, s_wcnt, sorted_pair);
}

// Decode-sized batches (T <= 64): the stable rank of pair (t, j) inside
// expert e's segment is the number of earlier tokens that chose e, read off a
// per-expert 64-bit token mask built with LDS atomics. One workgroup, no
// counting rounds; ids and the slot table are loaded in one round trip.
constexpr int MASK_MAX_T = 64;

__global__ void __launch_bounds__(ALIGN_THREADS) align_mask_kernel(
    const int32_t* __restrict__ ids, int T, int k, int E, int block_m, const int32_t* __restrict__ slot_of_expert,
    int32_t* sorted_pair, int32_t* block_slot, int32_t* counts, int32_t* seg_offset, int32_t* n_padded,
    int32_t* err, SlotCheck chk) {
    __shared__ unsigned long long s_tok[MOE_MAX_E];   // bit t set: token t chose the expert
    __shared__ int s_cnt[MOE_MAX_E];
    __shared__ int s_off[MOE_MAX_E];
    __shared__ int s_sl[MOE_MAX_E];
    __shared__ int s_tmp[2 * ALIGN_WAVES];
    __shared__ uint8_t s_wcnt[ALIGN_WAVES * MOE_MAX_E];
    const int tid = threadIdx.x;
    const int NP = T * k;
    const int my_id = tid < NP ? ids[tid] : -1;           // NP <= ALIGN_THREADS is checked by the host
    for (int i = tid; i < E; i += ALIGN_THREADS) {
        s_tok[i] = 0ull;
        s_cnt[i] = 0;
    }
    __syncthreads();
    const bool valid = my_id >= 0 && my_id < E;
    if (valid) {
        atomicOr(&s_tok[my_id], 1ull << (tid / k));
        atomicAdd(&s_cnt[my_id], 1);
    }
    const uint64_t bad = __ballot(tid < NP && !valid);
    if (lane_id() == 0 && bad) atomicAdd(err, (int)__popcll(bad));
    __syncthreads();
    // a token listing one expert twice breaks the mask ranks: take the counting path then
    const bool dup = __syncthreads_or(tid < E && s_cnt[tid] != (int)__popcll(s_tok[tid]));
    segments_from_counts(s_cnt, s_off, s_sl, s_tmp, E, block_m, NP, slot_of_expert, chk, counts, seg_offset,
                         n_padded, block_slot, sorted_pair, err);
    if (dup) {
        scatter_pairs(ids, 0, NP, E, s_off, s_wcnt, sorted_pair);
        return;
    }
    if (valid) {
        const int tt = tid / k;
        const unsigned long long before = tt == 0 ? 0ull : (s_tok[my_id] & (~0ull >> (64 - tt)));
        sorted_pair[s_off[my_id] + (int)__popcll(before)] = tid;
    }
}

int route_align_fused_max_pairs() { return MASK_MAX_T; }

hipError_t launch_route_align(const float* logits, const uint8_t* mask, int T, int E, int k, int block_m,
                              const int32_t* slot_of_expert, int32_t* ids, float* w, int32_t* sorted_pair,
                              int32_t* block_slot, int32_t* counts, int32_t* seg_offset, int32_t* n_padded,
                              int32_t* err, void* ws, hipStream_t stream, SlotCheck chk) {
    // the route error count lands in err[0]; align counts the -1 entries of short tokens in err[1]
    hipError_t e = launch_route(logits, mask, T, E, k, ids, w, err, stream);
    if (e != hipSuccess) return e;
    return launch_align(ids, T, k, E, block_m, slot_of_expert, sorted_pair, block_slot, counts, seg_offset,
                        n_padded, err + 1, ws, stream, chk);
}

int align_single_max_pairs() { return 8192; }

size_t align_workspace_bytes(int NP, int E) {
    if (NP <= align_single_max_pairs()) return 0;   // (the token-mask path needs none either)
    size_t chunks = (size_t)(NP + ALIGN_CHUNK - 1) / ALIGN_CHUNK;
    return chunks * (size_t)E * sizeof(int32_t);
}

hipError_t launch_align(const int32_t* ids, int T, int k, int E, int block_m, const int32_t* slot_of_expert,
                        int32_t* sorted_pair, int32_t* block_slot, int32_t* counts, int32_t* seg_offset,
                        int32_t* n_padded, int32_t* err, void* ws, hipStream_t stream, SlotCheck chk) {
    const int NP = T * k;
    if (T <= MASK_MAX_T && NP <= ALIGN_THREADS) {
        MOE_LAUNCH(K_ALIGN_SINGLE, stream, align_mask_kernel, dim3(1), dim3(ALIGN_THREADS), 0, stream, ids, T, k, E,
                   block_m, slot_of_expert, sorted_pair, block_slot, counts, seg_offset, n_padded, err, chk);
        return hipGetLastError();
    }
    if (NP <= align_single_max_pairs()) {
        MOE_LAUNCH(K_ALIGN_SINGLE, stream, align_single_kernel, dim3(1), dim3(ALIGN_THREADS), 0, stream, ids, NP, E, block_m,
                           slot_of_expert, sorted_pair, block_slot, counts, seg_offset, n_padded, err, chk);
        return hipGetLastError();
    }
    int chunks = (NP + ALIGN_CHUNK - 1) / ALIGN_CHUNK;
    int32_t* hist = (int32_t*)ws;
    MOE_LAUNCH(K_ALIGN_HIST, stream, align_hist_kernel, dim3(chunks), dim3(256), 0, stream, ids, NP, E, hist, err);
    MOE_LAUNCH(K_ALIGN_SCAN, stream, align_scan_kernel, dim3(1), dim3(ALIGN_THREADS), 0, stream, hist, chunks, NP, E, block_m,
                       slot_of_expert, sorted_pair, block_slot, counts, seg_offset, n_padded, err, chk);
    MOE_LAUNCH(K_ALIGN_SCATTER, stream, align_scatter_kernel, dim3(chunks), dim3(ALIGN_THREADS), 0, stream, ids, NP, E, hist,
                       sorted_pair);
    return hipGetLastError();
}

}  // namespace moe
