// noalloc.hip - moe_layer_step for callers that cannot allocate memory.
//
// The layer step needs a workspace (router scores, work lists, hidden and
// output rows of the experts). moe_layer_step takes it from the caller; this
// entry point uses a fixed array in the library's own device memory instead,
// so a caller under HIP graph capture, in a tight serving loop or in a harness
// that forbids hipMalloc passes only its inputs and outputs. The array is part
// of the code object: each GPU the library is loaded on holds one copy of
// MOE_SCRATCH_BYTES until the process ends.
//
// The array's name is only a host-side handle: its device address is looked up
// once per device (hipGetSymbolAddress, with that device current) and that
// address is what the kernels receive. Every call on a device uses the same
// array, so calls that overlap on one device (different streams, or threads)
// race on it; no kernel of the step reads a workspace byte it has not written
// in the same call, so nothing has to be cleared between calls.
#include <mutex>

#include "internal.h"

namespace {

static __device__ __align__(256) uint8_t scratch[MOE_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void *g_scratch[kMaxDevices];  // device address of `scratch` per device, once looked up

// The current device's address of `scratch` (looked up on the first call on
// that device).
moe_status scratch_address(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_EHIP;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_EHIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_layer_step_noalloc(const moe_expert_pool *pool, const float *x,
                                             int n_tokens, int d_model, const float *w_router,
                                             const float *b_router, int k, int32_t *topk_ids,
                                             float *topk_w, int32_t *union_ids, int32_t *n_union,
                                             int32_t *expert_offsets, int32_t *perm,
                                             uint64_t *counters, float *y, hipStream_t stream,
                                             const moe_forward_options *opt)
{
    if (!pool) return MOE_EINVAL;
    // a step whose workspace does not fit the array is rejected before any
    // HIP call (invalid arguments give a size of 0 and are reported by
    // moe_layer_step's own checks)
    if (n_tokens > 0 && moe_layer_step_workspace_size(pool, n_tokens, k) > MOE_SCRATCH_BYTES)
        return MOE_EWORKSPACE;
    void *ws = nullptr;
    const moe_status st = scratch_address(&ws);
    if (st != MOE_OK) return st;
    return moe_layer_step(pool, x, n_tokens, d_model, w_router, b_router, k, topk_ids, topk_w,
                          union_ids, n_union, expert_offsets, perm, counters, y, ws,
                          MOE_SCRATCH_BYTES, stream, opt);
}
