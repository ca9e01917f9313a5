/*
 * moe_cache.h - Place stage: a layer's routed experts held in a host tier
 * (pinned host memory) with an HBM cache of a fixed number of block slots,
 * per-layer least-recently-used replacement, and missing experts copied in
 * on a copy stream (the GPU's DMA engines) before the expert math that
 * needs them.
 *
 * Colibri pages: "Public Colibri Observation and Revision Ledger", section
 * "Exact Architecture and Data-Flow Reconstruction" (stage (3) Place: load
 * the experts a batch is missing, reuse the cached ones) and section
 * "Cache/Prefetch Design Comparison" (a per-layer LRU cache of experts);
 * README "The idea" / "Never wait for the disk twice" (experts placed in a
 * memory hierarchy, each needed expert read once).
 *
 * Use per layer step: moe_route_union (device results), copy n_union and
 * union_ids to the host, moe_cache_place, then moe_expert_forward with a
 * pool descriptor whose pool is `slots`, expert_bytes the block stride,
 * slot_of moe_cache_slot_table(...) and n_slots the cache's slot count.
 * Placement changes where blocks live, never the results: the forward reads
 * the same bytes as with every expert resident.
 *
 * A cache object is host state; calls on one cache must not overlap.
 */
#ifndef MOE_CACHE_H
#define MOE_CACHE_H

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_cache moe_cache;

/*
 * host_blocks: (host, pinned with hipHostMalloc or equivalent) n_experts
 *   device-layout blocks (moe_pack_expert output), block_stride bytes apart.
 * slots: (device) n_slots blocks, block_stride bytes apart, MOE_ALIGN-aligned.
 * slot_table: (device) int32 [n_experts], written by the cache: the slot of
 *   each resident expert, -1 for the others.
 * block_stride: a multiple of MOE_ALIGN; block_bytes <= block_stride bytes
 *   of each block are copied.
 * n_slots: 1 .. n_experts.
 * The table is cleared (all -1) with a synchronous copy before returning.
 * Errors: MOE_EINVAL (null pointer, bad count), MOE_EALIGN, MOE_EHIP.
 */
moe_status moe_cache_create(int n_experts, int n_slots, size_t block_bytes, size_t block_stride,
                            const void *host_blocks, void *slots, int32_t *slot_table,
                            moe_cache **out /* (host) */);

void moe_cache_destroy(moe_cache *cache);

/*
 * Make every expert of the union resident. union_ids (host) holds n_union
 * distinct expert ids (ids outside [0, n_experts) are ignored). Hits move to
 * the most recent end of the LRU order. Each missing expert takes the least
 * recently used slot that no expert of this union holds; its block copy is
 * enqueued on copy_stream, followed by the updated slot table; compute_stream
 * then waits for them (an event), so work enqueued on compute_stream after
 * this call sees the blocks and the table. Copies of one call overlap
 * whatever compute_stream is still running from before.
 * n_missed (host, may be NULL): the number of experts copied.
 * Errors: MOE_EINVAL (null cache, n_union < 0, union_ids NULL with
 * n_union > 0), MOE_ESHAPE (more distinct experts than slots: nothing is
 * changed), MOE_EHIP.
 */
moe_status moe_cache_place(moe_cache *cache, const int32_t *union_ids, int n_union,
                           hipStream_t copy_stream, hipStream_t compute_stream,
                           int32_t *n_missed);

/* Totals since creation: experts found resident, experts copied in. */
moe_status moe_cache_stats(const moe_cache *cache, uint64_t *hits, uint64_t *misses);

#ifdef __cplusplus
}
#endif

#endif /* MOE_CACHE_H */
