// stack.hip - a stack of MoE layers chained through the residual stream, one
// call: for each layer, the residual RMS norm of the stream, the layer step
// (route, union, counters, experts, combine), and the layer's output added
// back. Where a layer step ends with the combine kernel, that launch also adds
// the output into the stream and takes the next norm. This is how the speculative-decoding flow runs its draft steps (the
// int8 draft-head layer) and its verify batch (the int4 layers) through the
// same kernels (Colibri README, "Speculative decoding, honestly": draft
// tokens are verified as one batch by the main layers).
#include <string.h>

#include "internal.h"

namespace {

constexpr long long kAlign = MOE_ALIGN;
long long align_up(long long v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Workspace of moe_stack_forward, in this order: the normalised layer input
// a and the layer output y ([N][d] float32 each), the routing buffers of one
// layer (ids, w, union, count, offsets, permutation), then the layer step's
// own workspace (the largest over the layers).
struct StackLayout {
    long long a, y, ids, w, uid, nu, off, perm, step, total;
};

bool stack_layout(const moe_layer_desc *layers, int n_layers, int N, int k, StackLayout *L)
{
    if (!layers || n_layers < 1 || N < 0 || k < 1) return false;
    const int d = layers[0].pool.d_model, E = layers[0].pool.n_experts;
    size_t step = 0;
    for (int l = 0; l < n_layers; ++l) {
        if (layers[l].pool.d_model != d || layers[l].pool.n_experts != E) return false;
        const size_t s = moe_layer_step_workspace_size(&layers[l].pool, N, k);
        if (N > 0 && s == 0) return false;
        step = s > step ? s : step;
    }
    long long off = 0;
    L->a = off; off = align_up(off + 4LL * N * d);
    L->y = off; off = align_up(off + 4LL * N * d);
    L->ids = off; off = align_up(off + 4LL * N * k);
    L->w = off; off = align_up(off + 4LL * N * k);
    L->uid = off; off = align_up(off + 4LL * E);
    L->nu = off; off = align_up(off + 4);
    L->off = off; off = align_up(off + 4LL * (E + 1));
    L->perm = off; off = align_up(off + 4LL * N * k);
    L->step = off; off = align_up(off + (long long)step);
    L->total = off;
    return true;
}

}  // namespace

extern "C" {

size_t moe_stack_workspace_size(const moe_layer_desc *layers, int n_layers, int n_tokens, int k)
{
    StackLayout L;
    return stack_layout(layers, n_layers, n_tokens, k, &L) ? (size_t)L.total : 0;
}

moe_status moe_stack_forward(const moe_layer_desc *layers, int n_layers, int n_tokens, int k,
                             float eps, float *h, int32_t *topk_ids_out, void *workspace,
                             size_t ws_bytes, hipStream_t stream)
{
    if (!layers || n_layers < 1 || n_tokens < 0 || !(eps >= 0.0f)) return MOE_EINVAL;
    StackLayout L;
    if (!stack_layout(layers, n_layers, n_tokens, k, &L)) {
        // report the first layer's own error when there is one
        for (int l = 0; l < n_layers; ++l) {
            moe::Geo g;
            const moe_status st = moe::resolve_geo(&layers[l].pool, &g);
            if (st != MOE_OK) return st;
        }
        return k < 1 || k > MOE_MAX_K ? MOE_EINVAL : MOE_ESHAPE;
    }
    if (n_tokens == 0) return MOE_OK;
    if (!h) return MOE_EINVAL;
    if ((uintptr_t)h % 16) return MOE_EALIGN;
    if (!workspace || ws_bytes < (size_t)L.total) return MOE_EWORKSPACE;
    if ((uintptr_t)workspace % MOE_ALIGN) return MOE_EALIGN;
    char *ws = static_cast<char *>(workspace);
    float *a = reinterpret_cast<float *>(ws + L.a);
    float *y = reinterpret_cast<float *>(ws + L.y);
    float *w = reinterpret_cast<float *>(ws + L.w);
    int32_t *uid = reinterpret_cast<int32_t *>(ws + L.uid);
    int32_t *nu = reinterpret_cast<int32_t *>(ws + L.nu);
    int32_t *off = reinterpret_cast<int32_t *>(ws + L.off);
    int32_t *perm = reinterpret_cast<int32_t *>(ws + L.perm);
    void *sws = ws + L.step;
    const size_t sbytes = ws_bytes - (size_t)L.step;
    const int d = layers[0].pool.d_model;
    const size_t nk = (size_t)n_tokens * k;
    // every layer's checks before anything is enqueued
    for (int l = 0; l < n_layers; ++l) {
        int32_t *ids = topk_ids_out ? topk_ids_out + l * nk : reinterpret_cast<int32_t *>(ws + L.ids);
        const moe_layer_desc &ly = layers[l];
        const moe_status st =
            moe::layer_step_check(&ly.pool, a, n_tokens, d, ly.w_router, ly.b_router, k, ids, w,
                                  uid, nu, off, perm, ly.counters, y, sws, sbytes);
        if (st != MOE_OK) return st;
    }
    if (topk_ids_out && ((uintptr_t)topk_ids_out % 4)) return MOE_EALIGN;
    bool normed = false;  // the last layer step ended with h += y, a = rms(h)
    for (int l = 0; l < n_layers; ++l) {
        const moe_layer_desc &ly = layers[l];
        int32_t *ids = topk_ids_out ? topk_ids_out + l * nk : reinterpret_cast<int32_t *>(ws + L.ids);
        // h += y of the layer before (none before the first), a = rms(h),
        // unless that layer's combine did it
        moe_status st = MOE_OK;
        if (!normed) st = moe_residual_rmsnorm(h, l ? y : nullptr, a, n_tokens, d, eps, stream);
        if (st != MOE_OK) return st;
        const moe::StackNorm sn{h, a, eps};
        st = moe::layer_step_norm(&ly.pool, a, n_tokens, d, ly.w_router, ly.b_router, k, ids, w,
                                  uid, nu, off, perm, ly.counters, y, sws, sbytes, stream, &sn,
                                  &normed);
        if (st != MOE_OK) return st;
    }
    // the last layer's output joins the stream (the norm it also computes
    // goes to the scratch a)
    return normed ? MOE_OK : moe_residual_rmsnorm(h, y, a, n_tokens, d, eps, stream);
}

}  // extern "C"
