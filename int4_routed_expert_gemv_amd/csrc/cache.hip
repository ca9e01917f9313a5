// cache.hip - Place and Overlap stages: an HBM cache of expert block slots
// over a host tier, per-layer least-recently-used replacement, block copies
// on a copy stream while the resident experts compute, pinned experts,
// prefetch hints, and the persisted hit counters (host code only).
//
// Colibri pages: "Public Colibri Observation and Revision Ledger", section
// "Exact Architecture and Data-Flow Reconstruction" (stage (3) Place, stage
// (5) Learn: hit counters that later runs use to pin the hottest experts) and
// section "Cache/Prefetch Design Comparison" (per-layer LRU of experts,
// pinning by measured heat, prefetch of the next layer's experts from a
// lookahead router); README "Never wait for the disk twice" (the usage file
// that a run writes and the next run reads).
#include <stdio.h>
#include <string.h>

#include <algorithm>
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
    std::vector<char> pinned;         // slot -> never replaced
    int n_pinned = 0;
    bool unwaited = false;            // copies (prefetch) the compute stream has not waited for
    std::vector<int> mark;            // scratch: expert seen in this call
    std::vector<char> used;           // scratch: slot held by this call's union
    unsigned long long tick = 0;
    int32_t *staging = nullptr;       // pinned [2][E]: slot tables on their way to the device
    hipEvent_t copied[2] = {nullptr, nullptr};
    bool pending[2] = {false, false};
    hipEvent_t computed = nullptr;    // work on the compute stream before the copies
    int cur = 0;
    unsigned long long hits = 0, misses = 0;
    // Overlap (moe_cache_forward): which experts of a step wait for copies
    uint8_t *phase_dev = nullptr;     // device [E]: 0 resident, 1 being copied in
    uint8_t *phase_staging = nullptr; // pinned [2][E]
    hipEvent_t phase_sent[2] = {nullptr, nullptr};
    bool phase_pending[2] = {false, false};
    int phase_cur = 0;
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
    for (int i = 0; i < 2; ++i) {
        if (c->phase_sent[i]) {
            if (c->phase_pending[i]) (void)hipEventSynchronize(c->phase_sent[i]);
            (void)hipEventDestroy(c->phase_sent[i]);
        }
    }
    if (c->phase_staging) (void)hipHostFree(c->phase_staging);
    if (c->phase_dev) (void)hipFree(c->phase_dev);
    delete c;
}

// Distinct valid ids of a call (ids outside [0, E) ignored); how many of
// them are not resident in a pinned slot.
void count_distinct(moe_cache *c, const int32_t *ids, int n, int *distinct, int *unpinned)
{
    *distinct = *unpinned = 0;
    for (int i = 0; i < n; ++i) {
        const int e = ids[i];
        if (e >= 0 && e < c->E && !c->mark[e]) {
            c->mark[e] = 1;
            ++*distinct;
            const int s = c->slot_of[e];
            if (s < 0 || !c->pinned[s]) ++*unpinned;
        }
    }
    for (int i = 0; i < n; ++i) {
        const int e = ids[i];
        if (e >= 0 && e < c->E) c->mark[e] = 0;
    }
}

// Make ids[0..n) resident (the caller has checked that they fit): hits are
// refreshed first, then each missing expert takes the least recently used
// slot that is neither pinned nor held by this call, its block copied on
// copy_stream after the work already on compute_stream. The new slot table
// follows on copy_stream. wait: compute_stream waits for every copy so far
// (Place); otherwise the copies are left for the next Place to wait for
// (prefetch). count: add the hits and copies to the cache's totals (Place
// only). Returns MOE_OK or MOE_EHIP; *missed = experts copied.
moe_status place_ids(moe_cache *c, const int32_t *ids, int n, hipStream_t copy_stream,
                     hipStream_t compute_stream, bool wait, bool count, int *missed_out)
{
    ++c->tick;
    std::fill(c->used.begin(), c->used.end(), 0);
    // hits first: they keep their slots, which no miss may then take
    for (int i = 0; i < n; ++i) {
        const int e = ids[i];
        if (e < 0 || e >= c->E) continue;
        const int s = c->slot_of[e];
        if (s >= 0 && !c->used[s]) {
            c->used[s] = 1;
            c->last_use[s] = c->tick;
            if (count) ++c->hits;
        }
    }
    int missed = 0;
    bool waited = false;
    for (int i = 0; i < n; ++i) {
        const int e = ids[i];
        if (e < 0 || e >= c->E || c->slot_of[e] >= 0) continue;  // out of range, or resident
        // the least recently used slot this call does not hold and no pin
        // keeps (free slots first, lowest index among equals)
        int victim = -1;
        for (int s = 0; s < c->C; ++s)
            if (!c->used[s] && !c->pinned[s] &&
                (victim < 0 || c->last_use[s] < c->last_use[victim]))
                victim = s;
        if (victim < 0) return MOE_EHIP;  // cannot happen: the caller checked the room
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
        if (count) ++c->misses;
    }
    *missed_out = missed;
    if (!missed && !(wait && c->unwaited)) return MOE_OK;
    // the new table (or, for a Place with no copies of its own, only the wait
    // on earlier prefetch copies), through a staging buffer no copy in flight
    // still reads
    const int b = c->cur;
    if (c->pending[b] && hipEventSynchronize(c->copied[b]) != hipSuccess) return MOE_EHIP;
    if (missed) {
        int32_t *st = c->staging + (size_t)b * c->E;
        for (int e = 0; e < c->E; ++e) st[e] = c->slot_of[e];
        if (hipMemcpyAsync(c->table_dev, st, sizeof(int32_t) * c->E, hipMemcpyHostToDevice,
                           copy_stream) != hipSuccess)
            return MOE_EHIP;
    }
    if (hipEventRecord(c->copied[b], copy_stream) != hipSuccess) return MOE_EHIP;
    c->pending[b] = true;
    c->cur = b ^ 1;
    if (wait) {
        if (hipStreamWaitEvent(compute_stream, c->copied[b], 0) != hipSuccess) return MOE_EHIP;
        c->unwaited = false;
    } else {
        c->unwaited = true;
    }
    return MOE_OK;
}

const char kUsageMagic[8] = {'M', 'O', 'E', 'U', 'S', 'A', 'G', 'E'};
constexpr uint32_t kUsageVersion = 1;

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
    c->pinned.assign(n_slots, 0);
    c->mark.assign(n_experts, 0);
    c->used.assign(n_slots, 0);
    if (hipHostMalloc(reinterpret_cast<void **>(&c->staging), 2 * sizeof(int32_t) * n_experts,
                      hipHostMallocDefault) != hipSuccess ||
        hipHostMalloc(reinterpret_cast<void **>(&c->phase_staging), 2 * (size_t)n_experts,
                      hipHostMallocDefault) != hipSuccess ||
        hipMalloc(reinterpret_cast<void **>(&c->phase_dev), (size_t)n_experts) != hipSuccess ||
        hipEventCreateWithFlags(&c->copied[0], hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&c->copied[1], hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&c->phase_sent[0], hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&c->phase_sent[1], hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&c->computed, hipEventDisableTiming) != hipSuccess) {
        release(c);
        return MOE_EHIP;
    }
    for (int e = 0; e < n_experts; ++e) c->staging[e] = -1;
    memset(c->phase_staging, 0, 2 * (size_t)n_experts);
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
    // more distinct experts than the slots no pin keeps: change nothing
    int distinct, unpinned;
    count_distinct(c, union_ids, n_union, &distinct, &unpinned);
    if (unpinned > c->C - c->n_pinned) return MOE_ESHAPE;
    int missed = 0;
    const moe_status st = place_ids(c, union_ids, n_union, copy_stream, compute_stream, true,
                                    true, &missed);
    if (n_missed) *n_missed = missed;
    return st;
}

moe_status moe_cache_forward(moe_cache *c, const moe_expert_pool *shape, const float *x,
                             int n_tokens, int k, const float *topk_w, const int32_t *union_ids,
                             const int32_t *n_union, const int32_t *expert_offsets,
                             const int32_t *perm, const int32_t *union_host, int n_union_host,
                             float *y, void *workspace, size_t ws_bytes, hipStream_t copy_stream,
                             hipStream_t compute_stream, int32_t *n_missed)
{
    if (!c || !shape || n_union_host < 0 || (n_union_host > 0 && !union_host)) return MOE_EINVAL;
    if (n_missed) *n_missed = 0;
    if (shape->n_experts != c->E) return MOE_ESHAPE;
    if (moe_block_bytes(shape->d_model, shape->d_ff, shape->wbits, shape->group) != c->bytes)
        return MOE_ESHAPE;
    // the layer as the expert kernels see it: the cache's slots and table
    moe_expert_pool p = *shape;
    p.pool = c->slots;
    p.expert_bytes = c->stride;
    p.slot_of = c->table_dev;
    p.n_slots = c->C;
    // every check of moe_expert_forward, and the room for the union, before
    // anything changes or is enqueued
    moe_status st = moe::expert_forward_phase(&p, x, n_tokens, k, topk_w, union_ids, n_union,
                                              expert_offsets, perm, y, workspace, ws_bytes,
                                              compute_stream, c->phase_dev, 0, true);
    if (st != MOE_OK) return st;
    int distinct, unpinned;
    count_distinct(c, union_host, n_union_host, &distinct, &unpinned);
    if (unpinned > c->C - c->n_pinned) return MOE_ESHAPE;
    if (n_tokens == 0) return MOE_OK;
    // copies of an earlier prefetch, not yet waited for: their experts count
    // as resident below, so the compute stream waits for them first
    if (c->unwaited) {
        const int last = c->cur ^ 1;
        if (hipStreamWaitEvent(compute_stream, c->copied[last], 0) != hipSuccess) return MOE_EHIP;
        c->unwaited = false;
    }
    // phase of each union expert before placement: 0 resident, 1 copied in
    const int b = c->phase_cur;
    if (c->phase_pending[b] && hipEventSynchronize(c->phase_sent[b]) != hipSuccess)
        return MOE_EHIP;
    uint8_t *ph = c->phase_staging + (size_t)b * c->E;
    int to_copy = 0;
    for (int i = 0; i < n_union_host; ++i) {
        const int e = union_host[i];
        if (e < 0 || e >= c->E) continue;
        ph[e] = c->slot_of[e] >= 0 ? 0 : 1;
        to_copy += ph[e];
    }
    int missed = 0;
    if (to_copy == 0) {
        // nothing to copy: one plain forward
        st = place_ids(c, union_host, n_union_host, copy_stream, compute_stream, true, true,
                       &missed);
        if (st != MOE_OK) return st;
        return moe::expert_forward_phase(&p, x, n_tokens, k, topk_w, union_ids, n_union,
                                         expert_offsets, perm, y, workspace, ws_bytes,
                                         compute_stream, nullptr, 0, false);
    }
    if (hipMemcpyAsync(c->phase_dev, ph, (size_t)c->E, hipMemcpyHostToDevice, compute_stream) !=
            hipSuccess ||
        hipEventRecord(c->phase_sent[b], compute_stream) != hipSuccess)
        return MOE_EHIP;
    c->phase_pending[b] = true;
    c->phase_cur = b ^ 1;
    // Place: block copies and the new slot table on the copy stream (after
    // the work already on the compute stream); the compute stream does not
    // wait for them yet
    st = place_ids(c, union_host, n_union_host, copy_stream, compute_stream, false, true, &missed);
    if (st != MOE_OK) return st;
    if (n_missed) *n_missed = missed;
    // Overlap: the resident experts and the shared expert while the copies
    // run (their slots and table entries do not change in this call), then
    // the copied experts and the combine
    st = moe::expert_forward_phase(&p, x, n_tokens, k, topk_w, union_ids, n_union,
                                   expert_offsets, perm, y, workspace, ws_bytes, compute_stream,
                                   c->phase_dev, 0, false);
    if (st != MOE_OK) return st;
    const int last = c->cur ^ 1;  // the event place_ids recorded after this call's copies
    if (hipStreamWaitEvent(compute_stream, c->copied[last], 0) != hipSuccess) return MOE_EHIP;
    c->unwaited = false;
    return moe::expert_forward_phase(&p, x, n_tokens, k, topk_w, union_ids, n_union,
                                     expert_offsets, perm, y, workspace, ws_bytes,
                                     compute_stream, c->phase_dev, 1, false);
}

moe_status moe_cache_prefetch(moe_cache *c, const int32_t *ids, int n, hipStream_t copy_stream,
                              hipStream_t compute_stream, int32_t *n_copied)
{
    if (!c || n < 0 || (n > 0 && !ids)) return MOE_EINVAL;
    if (n_copied) *n_copied = 0;
    // a hint: the longest prefix of ids whose distinct experts fit in the
    // slots no pin keeps (one pass, marks cleared after)
    const int room = c->C - c->n_pinned;
    int take = 0, need = 0;
    for (int i = 0; i < n; ++i) {
        const int e = ids[i];
        if (e >= 0 && e < c->E && !c->mark[e]) {
            const int s = c->slot_of[e];
            const bool kept = s >= 0 && c->pinned[s];
            if (!kept && need + 1 > room) break;
            c->mark[e] = 1;
            if (!kept) ++need;
        }
        take = i + 1;
    }
    for (int i = 0; i < take; ++i) {
        const int e = ids[i];
        if (e >= 0 && e < c->E) c->mark[e] = 0;
    }
    int copied = 0;
    const moe_status st = place_ids(c, ids, take, copy_stream, compute_stream, false, false,
                                    &copied);
    if (n_copied) *n_copied = copied;
    return st;
}

moe_status moe_cache_pin(moe_cache *c, const int32_t *ids, int n, hipStream_t copy_stream,
                         hipStream_t compute_stream, int32_t *n_missed)
{
    if (!c || n < 0 || (n > 0 && !ids)) return MOE_EINVAL;
    if (n_missed) *n_missed = 0;
    int distinct, unpinned;
    count_distinct(c, ids, n, &distinct, &unpinned);
    if (distinct > c->C) return MOE_ESHAPE;
    // the new pin set replaces the old one: unpin, place, then pin its slots
    std::fill(c->pinned.begin(), c->pinned.end(), 0);
    c->n_pinned = 0;
    int missed = 0;
    const moe_status st = place_ids(c, ids, n, copy_stream, compute_stream, true, false, &missed);
    if (st != MOE_OK) return st;
    for (int i = 0; i < n; ++i) {
        const int e = ids[i];
        if (e < 0 || e >= c->E) continue;
        const int s = c->slot_of[e];
        if (s >= 0 && !c->pinned[s]) {
            c->pinned[s] = 1;
            ++c->n_pinned;
        }
    }
    if (n_missed) *n_missed = missed;
    return MOE_OK;
}

moe_status moe_cache_stats(const moe_cache *c, uint64_t *hits, uint64_t *misses)
{
    if (!c) return MOE_EINVAL;
    if (hits) *hits = c->hits;
    if (misses) *misses = c->misses;
    return MOE_OK;
}

moe_status moe_cache_resident(const moe_cache *c, int32_t *slot_of, int32_t *pinned)
{
    if (!c) return MOE_EINVAL;
    for (int e = 0; e < c->E; ++e) {
        const int s = c->slot_of[e];
        if (slot_of) slot_of[e] = s;
        if (pinned) pinned[e] = (s >= 0 && c->pinned[s]) ? 1 : 0;
    }
    return MOE_OK;
}

moe_status moe_usage_hottest(const uint64_t *counters, int n_experts, int n, int32_t *ids)
{
    if (!counters || n_experts < 1 || n_experts > MOE_MAX_EXPERTS || n < 0 || n > n_experts ||
        (n > 0 && !ids))
        return MOE_EINVAL;
    std::vector<int32_t> order(n_experts);
    for (int e = 0; e < n_experts; ++e) order[e] = e;
    // most hits first, the lower id among equal counts
    std::stable_sort(order.begin(), order.end(),
                     [&](int32_t a, int32_t b) { return counters[a] > counters[b]; });
    for (int i = 0; i < n; ++i) ids[i] = order[i];
    return MOE_OK;
}

moe_status moe_usage_write(const char *path, const uint64_t *counters, int n_layers,
                           int n_experts)
{
    if (!path || !counters || n_layers < 1 || n_experts < 1 || n_experts > MOE_MAX_EXPERTS)
        return MOE_EINVAL;
    FILE *fp = fopen(path, "wb");
    if (!fp) return MOE_EIO;
    const uint32_t head[3] = {kUsageVersion, (uint32_t)n_layers, (uint32_t)n_experts};
    const size_t n = (size_t)n_layers * n_experts;
    bool ok = fwrite(kUsageMagic, 1, 8, fp) == 8 && fwrite(head, 4, 3, fp) == 3 &&
              fwrite(counters, 8, n, fp) == n;
    ok = (fclose(fp) == 0) && ok;
    return ok ? MOE_OK : MOE_EIO;
}

moe_status moe_usage_read(const char *path, uint64_t *counters, int n_layers, int n_experts)
{
    if (!path || !counters || n_layers < 1 || n_experts < 1 || n_experts > MOE_MAX_EXPERTS)
        return MOE_EINVAL;
    FILE *fp = fopen(path, "rb");
    if (!fp) return MOE_EIO;
    char magic[8];
    uint32_t head[3];
    const size_t n = (size_t)n_layers * n_experts;
    moe_status st = MOE_OK;
    if (fread(magic, 1, 8, fp) != 8 || memcmp(magic, kUsageMagic, 8) != 0 ||
        fread(head, 4, 3, fp) != 3 || head[0] != kUsageVersion)
        st = MOE_EIO;
    else if (head[1] != (uint32_t)n_layers || head[2] != (uint32_t)n_experts)
        st = MOE_ESHAPE;
    else {
        // read into a copy, so that a short or overlong file leaves counters
        // as they were (no exception crosses the C interface)
        std::vector<uint64_t> tmp;
        try {
            tmp.resize(n);
        } catch (...) {
            st = MOE_EIO;
        }
        char extra;
        if (st == MOE_OK) {
            if (fread(tmp.data(), 8, n, fp) != n || fread(&extra, 1, 1, fp) != 0)
                st = MOE_EIO;
            else
                memcpy(counters, tmp.data(), 8 * n);
        }
    }
    fclose(fp);
    return st;
}

}  // extern "C"
