/*
 * moe_cache.h - Place and Overlap stages: a layer's routed experts held in a
 * host tier (pinned host memory) with an HBM cache of a fixed number of block
 * slots, per-layer least-recently-used replacement, and missing experts
 * copied in on a copy stream (the GPU's DMA engines), either before the
 * expert math (moe_cache_place) or while the resident experts compute
 * (moe_cache_forward).
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

/*
 * Place and Overlap, then the expert math, of one layer step through the
 * cache (the pages' stages (3) and (4): the experts of a batch that are
 * already in the fast tier are computed while the missing ones are read in).
 * The union (union_host, as for moe_cache_place) is placed: hits and misses
 * as in moe_cache_place, the block copies and the new slot table enqueued on
 * copy_stream after the work already on compute_stream. Then, on
 * compute_stream, without waiting for the copies: the expert kernels of the
 * union's resident experts and of the shared expert. Then compute_stream
 * waits for the copies and runs the kernels of the copied experts and the
 * combine. When nothing is missing, one ordinary forward. y equals
 * moe_expert_forward on a pool with every expert resident, bit for bit (the
 * same kernels on the same work items).
 *   shape: the layer's descriptor (d_model, d_ff, n_experts == the cache's,
 *     wbits, group, shared); its pool, expert_bytes, slot_of and n_slots
 *     are replaced by the cache's slots and table.
 *   x ... perm, y, workspace, ws_bytes: as for moe_expert_forward (the device
 *     union outputs of the same batch); union_host / n_union_host: the same
 *     union on the host.
 *   n_missed (host, may be NULL): experts copied in.
 * Hits and misses count in moe_cache_stats. The cache keeps a small device
 * array of each call's split, so successive calls on one cache must be
 * ordered on compute_stream (the same stream, or streams the caller orders).
 * Errors: those of moe_expert_forward and moe_cache_place (MOE_ESHAPE also
 * when shape does not match the cache's blocks), checked before anything is
 * enqueued or changed.
 */
moe_status moe_cache_forward(moe_cache *cache, const moe_expert_pool *shape /* (host) */,
                             const float *x, int n_tokens, int k, const float *topk_w,
                             const int32_t *union_ids, const int32_t *n_union,
                             const int32_t *expert_offsets, const int32_t *perm,
                             const int32_t *union_host /* (host) */, int n_union_host,
                             float *y, void *workspace, size_t ws_bytes,
                             hipStream_t copy_stream, hipStream_t compute_stream,
                             int32_t *n_missed);

/* Totals of moe_cache_place and moe_cache_forward since creation: experts
 * found resident, experts copied in (pins and prefetches are not counted). */
moe_status moe_cache_stats(const moe_cache *cache, uint64_t *hits, uint64_t *misses);

/*
 * Pin: make the experts of ids (host, n of them, ids outside [0, n_experts)
 * ignored) resident as moe_cache_place does, then keep them: no later Place
 * or prefetch replaces a pinned slot. The call replaces the previous pin set
 * (n = 0 unpins everything). A Place whose union needs more slots than the
 * unpinned ones returns MOE_ESHAPE. The pages pin the experts their hit
 * counters show hottest ("Cache/Prefetch Design Comparison"; Learn stage);
 * moe_usage_hottest picks them.
 * Errors: MOE_EINVAL, MOE_ESHAPE (more distinct ids than slots; nothing is
 * changed), MOE_EHIP (the pin set is then empty). n_missed (host, may be
 * NULL): experts copied in.
 */
moe_status moe_cache_pin(moe_cache *cache, const int32_t *ids, int n,
                         hipStream_t copy_stream, hipStream_t compute_stream,
                         int32_t *n_missed);

/*
 * Prefetch hint: start copying the experts of ids (host) that are not
 * resident, in order, as far as the unpinned slots allow (the rest of the
 * list is ignored), into least-recently-used slots, after the work already
 * on compute_stream; unlike Place, compute_stream does not wait for these
 * copies here: the next moe_cache_place on this cache makes it wait. The
 * experts count as just used. For the next layer's experts predicted by a
 * lookahead router while the current layer computes (the pages' prefetch of
 * layer l+1 from layer l's hidden state). n_copied (host, may be NULL).
 * Errors: MOE_EINVAL, MOE_EHIP.
 */
moe_status moe_cache_prefetch(moe_cache *cache, const int32_t *ids, int n,
                              hipStream_t copy_stream, hipStream_t compute_stream,
                              int32_t *n_copied);

/* Host view of the cache: slot_of[n_experts] (slot or -1) and
 * pinned[n_experts] (1 when the expert sits in a pinned slot); either may be
 * NULL. */
moe_status moe_cache_resident(const moe_cache *cache, int32_t *slot_of, int32_t *pinned);

/*
 * Learn across runs: the per-layer hit counters (moe_hit_count /
 * moe_route_union output, uint64 [n_layers][n_experts], copied to the host)
 * saved to and loaded from a small file, the counterpart of the pages' usage
 * file that a run leaves for the next one ("Never wait for the disk twice").
 * Format: the 8 bytes "MOEUSAGE", uint32 version 1, uint32 n_layers, uint32
 * n_experts, then the counters, all little-endian.
 * moe_usage_read: MOE_ESHAPE when the file holds other dimensions, MOE_EIO
 * when it cannot be read or is not such a file (counters unchanged then).
 * moe_usage_hottest: the n experts with the most hits (ties to the lower id),
 * most hits first, from one layer's counters (n_experts up to
 * MOE_MAX_EXPERTS).
 */
moe_status moe_usage_write(const char *path /* (host) */, const uint64_t *counters /* (host) */,
                           int n_layers, int n_experts);
moe_status moe_usage_read(const char *path /* (host) */, uint64_t *counters /* (host) */,
                          int n_layers, int n_experts);
moe_status moe_usage_hottest(const uint64_t *counters /* (host) */, int n_experts, int n,
                             int32_t *ids /* (host) */);

#ifdef __cplusplus
}
#endif

#endif /* MOE_CACHE_H */
