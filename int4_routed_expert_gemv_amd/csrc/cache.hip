// cache.hip - Place stage: an HBM cache of expert block slots over a host
// tier, per-layer least-recently-used replacement, block copies on a copy
// stream (host code only).
//
// Colibri pages: "Public Colibri Observation and Revision Ledger", section
// "Exact Architecture and Data-Flow Reconstruction" (stage (3) Place) and
// section "Cache/Prefetch Design Comparison" (per-layer LRU of experts).
#include <vector>

#include "internal.h"
#include "moe_cache.h"

struct moe_cache {
    int E = 0, C = 0;
    size_t bytes = 0, stride = 0;
    const uint8_t *host = nullptr;
    uint8_t *slots = nullptr;
    int32_t *table_dev = nullptr;
    std::vector<int> slot_of;         // expert -> slot, or -1
    std::vector<int> expert_in;       // slot -> expert, or -1
    std::vector<unsigned long long> last_use;  // slot -> tick of its last use (0: never)
    std::vector<int> mark;            // scratch: expert seen in this call
    std::vector<char> used;           // scratch: slot held by this call's union
    unsigned long long tick = 0;
    int32_t *staging = nullptr;       // pinned [2][E]: slot tables on their way to the device
    hipEvent_t copied[2] = {nullptr, nullptr};
    bool pending[2] = {false, false};
    hipEvent_t computed = nullptr;    // work on the compute stream before the copies
    int cur = 0;
    unsigned long long hits = 0, misses = 0;
};

namespace {

void release(moe_cache *c)
{
    if (!c) return;
    for (int i = 0; i < 2; ++i) {
        if (c->copied[i]) {
            if (c->pending[i]) (void)hipEventSynchronize(c->copied[i]);
            (void)hipEventDestroy(c->copied[i]);
        }
    }
    if (c->computed) (void)hipEventDestroy(c->computed);
    if (c->staging) (void)hipHostFree(c->staging);
    delete c;
}

}  // namespace

extern "C" {

moe_status moe_cache_create(int n_experts, int n_slots, size_t block_bytes, size_t block_stride,
                            const void *host_blocks, void *slots, int32_t *slot_table,
                            moe_cache **out)
{
    if (!out) return MOE_EINVAL;
    *out = nullptr;
    if (n_experts < 1 || n_experts > MOE_MAX_EXPERTS || n_slots < 1 || n_slots > n_experts)
        return MOE_EINVAL;
    if (!host_blocks || !slots || !slot_table || block_bytes == 0 || block_bytes > block_stride)
        return MOE_EINVAL;
    if (block_stride % MOE_ALIGN || (uintptr_t)slots % MOE_ALIGN || (uintptr_t)slot_table % 4)
        return MOE_EALIGN;
    moe_cache *c = new moe_cache;
    c->E = n_experts;
    c->C = n_slots;
    c->bytes = block_bytes;
    c->stride = block_stride;
    c->host = static_cast<const uint8_t *>(host_blocks);
    c->slots = static_cast<uint8_t *>(slots);
    c->table_dev = slot_table;
    c->slot_of.assign(n_experts, -1);
    c->expert_in.assign(n_slots, -1);
    c->last_use.assign(n_slots, 0);
    c->mark.assign(n_experts, 0);
    c->used.assign(n_slots, 0);
    if (hipHostMalloc(reinterpret_cast<void **>(&c->staging), 2 * sizeof(int32_t) * n_experts,
                      hipHostMallocDefault) != hipSuccess ||
        hipEventCreateWithFlags(&c->copied[0], hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&c->copied[1], hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&c->computed, hipEventDisableTiming) != hipSuccess) {
        release(c);
        return MOE_EHIP;
    }
    for (int e = 0; e < n_experts; ++e) c->staging[e] = -1;
    if (hipMemcpy(slot_table, c->staging, sizeof(int32_t) * n_experts, hipMemcpyHostToDevice) !=
        hipSuccess) {
        release(c);
        return MOE_EHIP;
    }
    *out = c;
    return MOE_OK;
}

void moe_cache_destroy(moe_cache *cache) { release(cache); }

moe_status moe_cache_place(moe_cache *c, const int32_t *union_ids, int n_union,
                           hipStream_t copy_stream, hipStream_t compute_stream, int32_t *n_missed)
{
    if (!c || n_union < 0 || (n_union > 0 && !union_ids)) return MOE_EINVAL;
    if (n_missed) *n_missed = 0;
    // the distinct valid ids of this call; more than the slots: change nothing
    int distinct = 0;
    for (int i = 0; i < n_union; ++i) {
        const int e = union_ids[i];
        if (e >= 0 && e < c->E && !c->mark[e]) {
            c->mark[e] = 1;
            ++distinct;
        }
    }
    for (int i = 0; i < n_union; ++i) {
        const int e = union_ids[i];
        if (e >= 0 && e < c->E) c->mark[e] = 0;
    }
    if (distinct > c->C) return MOE_ESHAPE;

    ++c->tick;
    std::fill(c->used.begin(), c->used.end(), 0);
    // hits first: they keep their slots, which no miss may then take
    for (int i = 0; i < n_union; ++i) {
        const int e = union_ids[i];
        if (e < 0 || e >= c->E) continue;
        const int s = c->slot_of[e];
        if (s >= 0 && !c->used[s]) {
            c->used[s] = 1;
            c->last_use[s] = c->tick;
            ++c->hits;
        }
    }
    int missed = 0;
    bool waited = false;
    for (int i = 0; i < n_union; ++i) {
        const int e = union_ids[i];
        if (e < 0 || e >= c->E || c->slot_of[e] >= 0) continue;  // out of range, or resident
        // the least recently used slot this union does not hold (free slots first)
        int victim = -1;
        for (int s = 0; s < c->C; ++s)
            if (!c->used[s] && (victim < 0 || c->last_use[s] < c->last_use[victim])) victim = s;
        if (victim < 0) return MOE_EHIP;  // cannot happen: distinct <= C
        if (!waited) {
            // a replaced block may still be read by work already on the
            // compute stream: the copies start after it
            if (hipEventRecord(c->computed, compute_stream) != hipSuccess ||
                hipStreamWaitEvent(copy_stream, c->computed, 0) != hipSuccess)
                return MOE_EHIP;
            waited = true;
        }
        const int old = c->expert_in[victim];
        if (old >= 0) c->slot_of[old] = -1;
        c->expert_in[victim] = e;
        c->slot_of[e] = victim;
        c->used[victim] = 1;
        c->last_use[victim] = c->tick;
        if (hipMemcpyAsync(c->slots + (size_t)victim * c->stride, c->host + (size_t)e * c->stride,
                           c->bytes, hipMemcpyHostToDevice, copy_stream) != hipSuccess)
            return MOE_EHIP;
        ++missed;
        ++c->misses;
    }
    if (n_missed) *n_missed = missed;
    if (!missed) return MOE_OK;
    // the new table, through a staging buffer no copy in flight still reads
    const int b = c->cur;
    if (c->pending[b] && hipEventSynchronize(c->copied[b]) != hipSuccess) return MOE_EHIP;
    int32_t *st = c->staging + (size_t)b * c->E;
    for (int e = 0; e < c->E; ++e) st[e] = c->slot_of[e];
    if (hipMemcpyAsync(c->table_dev, st, sizeof(int32_t) * c->E, hipMemcpyHostToDevice,
                       copy_stream) != hipSuccess ||
        hipEventRecord(c->copied[b], copy_stream) != hipSuccess)
        return MOE_EHIP;
    c->pending[b] = true;
    c->cur = b ^ 1;
    if (hipStreamWaitEvent(compute_stream, c->copied[b], 0) != hipSuccess) return MOE_EHIP;
    return MOE_OK;
}

moe_status moe_cache_stats(const moe_cache *c, uint64_t *hits, uint64_t *misses)
{
    if (!c) return MOE_EINVAL;
    if (hits) *hits = c->hits;
    if (misses) *misses = c->misses;
    return MOE_OK;
}

}  // extern "C"
