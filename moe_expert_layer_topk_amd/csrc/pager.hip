// Slot-miss path: a per-layer LRU over the VRAM slots and the asynchronous
// fill of missing experts from host RAM.
//
// vllm-expert-pager article (rand.pepabo.com), "hierarchical paging of expert
// weights": each MoE layer owns its own VRAM slots (and RAM slots), one expert
// per slot, each tier managed LRU; an expert needed but not in VRAM is copied
// in from its RAM slot. MOE-GEN explainer (aibr.jp), section 3: host-to-GPU
// copies run alongside GPU compute. The plan is host logic (the slot table
// lives on the host and is mirrored to the device); the fill is a set of
// asynchronous host-to-device copies on the caller's copy stream, from
// page-locked host memory.
#include "../../include/moe.h"
#include "moe_common.h"
#include "moe_kernels.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <vector>

struct moe_pager {
    int n_layers, E, n_slots;
    struct Layer {
        std::vector<int32_t> slot_of_expert;   // [E], -1 = not resident
        std::vector<int32_t> expert_in_slot;   // [n_slots], -1 = free
        std::vector<int64_t> last_used;        // [E], step of last use (-1 = never)
        int64_t step = 0;
        long long hits = 0, misses = 0;
    };
    std::vector<Layer> layers;
};

extern "C" {

moe_pager* moe_pager_create(int n_layers, int E, int n_slots) {
    if (n_layers < 1 || E < 1 || E > MOE_MAX_E || n_slots < 1) return nullptr;
    moe_pager* p = new moe_pager;
    p->n_layers = n_layers;
    p->E = E;
    p->n_slots = n_slots;
    p->layers.resize(n_layers);
    for (auto& L : p->layers) {
        L.slot_of_expert.assign(E, -1);
        L.expert_in_slot.assign(n_slots, -1);
        L.last_used.assign(E, -1);
    }
    return p;
}

void moe_pager_destroy(moe_pager* p) { delete p; }

int moe_pager_plan(moe_pager* p, int layer, const int32_t* needed, int n_needed, int32_t* slot_of_expert,
                   int32_t* fill_expert, int32_t* fill_slot, int* n_fill) {
    if (!p || layer < 0 || layer >= p->n_layers || n_needed < 0 || (n_needed && !needed) || !slot_of_expert ||
        !fill_expert || !fill_slot || !n_fill)
        return MOE_EINVAL;
    auto& L = p->layers[layer];
    const int E = p->E;
    std::vector<char> want(E, 0);
    int distinct = 0;
    for (int i = 0; i < n_needed; ++i) {
        const int e = needed[i];
        if (e >= 0 && e < E && !want[e]) {
            want[e] = 1;
            ++distinct;
        }
    }
    if (distinct > p->n_slots) return MOE_EINVAL;      // more experts than slots: the working-buffer case
    int nf = 0;
    for (int e = 0; e < E; ++e) {                       // misses in ascending expert id
        if (!want[e]) continue;
        if (L.slot_of_expert[e] >= 0) {
            ++L.hits;
            continue;
        }
        ++L.misses;
        int slot = -1;
        for (int s = 0; s < p->n_slots; ++s)           // a free slot, lowest index first
            if (L.expert_in_slot[s] < 0) {
                slot = s;
                break;
            }
        if (slot < 0) {                                 // else the least recently used unneeded expert
            int victim = -1;
            for (int v = 0; v < E; ++v) {
                if (L.slot_of_expert[v] < 0 || want[v]) continue;
                if (victim < 0 || L.last_used[v] < L.last_used[victim]) victim = v;   // ties: lower id
            }
            slot = L.slot_of_expert[victim];           // exists: distinct <= n_slots and every slot is taken
            L.slot_of_expert[victim] = -1;
        }
        L.slot_of_expert[e] = slot;
        L.expert_in_slot[slot] = e;
        fill_expert[nf] = e;
        fill_slot[nf] = slot;
        ++nf;
    }
    for (int e = 0; e < E; ++e)
        if (want[e]) L.last_used[e] = L.step;
    ++L.step;
    for (int e = 0; e < E; ++e) slot_of_expert[e] = L.slot_of_expert[e];
    *n_fill = nf;
    return MOE_OK;
}

int moe_pager_stats(const moe_pager* p, int layer, long long* hits, long long* misses) {
    if (!p || !hits || !misses || layer < -1 || layer >= p->n_layers) return MOE_EINVAL;
    long long h = 0, m = 0;
    for (int l = 0; l < p->n_layers; ++l)
        if (layer < 0 || l == layer) {
            h += p->layers[l].hits;
            m += p->layers[l].misses;
        }
    *hits = h;
    *misses = m;
    return MOE_OK;
}

int moe_pager_fill(const moe_slot_pool* pool, const void* h_bank, size_t h_bank_stride, const uint8_t* h_bank_fmt,
                   const int32_t* fill_src, const int32_t* fill_slot, int n_fill, void* copy_stream) {
    if (!pool || !pool->d_base || !pool->d_slot_fmt || n_fill < 0) return MOE_EINVAL;
    if (n_fill && (!h_bank || !h_bank_fmt || !fill_src || !fill_slot)) return MOE_EINVAL;
    if (h_bank_stride > pool->slot_bytes) return MOE_EINVAL;
    hipStream_t s = (hipStream_t)copy_stream;
    (void)hipGetLastError();
    for (int i = 0; i < n_fill; ++i) {
        const int slot = fill_slot[i], src = fill_src[i];
        if (slot < 0 || slot >= pool->n_slots || src < 0) return MOE_EINVAL;
        uint8_t* dst = (uint8_t*)pool->d_base + (size_t)slot * pool->slot_bytes;
        hipError_t e = hipMemcpyAsync(dst, (const uint8_t*)h_bank + (size_t)src * h_bank_stride, h_bank_stride,
                                      hipMemcpyHostToDevice, s);
        if (e == hipSuccess)
            e = hipMemcpyAsync((uint8_t*)pool->d_slot_fmt + slot, h_bank_fmt + src, 1, hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return moe::record_hip_error((int)e);
    }
    return MOE_OK;
}

}  // extern "C"
