// abi.hip - the C entry points: argument checks, workspace layout, launches.
//
// Every check runs on the host before any HIP call, so a rejected call
// enqueues nothing. The Colibri pages' engine stops the process on bad input
// ("Failure, Corruption, and Restart Behavior" on the ledger page, which also
// recommends turning such failures into clear errors); here each failure is a
// status code instead.
#include <string.h>

#include <vector>

#include "internal.h"
#include "topk.h"

namespace moe {

namespace {

constexpr long long kAlign = MOE_ALIGN;

long long align_up(long long v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void *p) { return ((uintptr_t)p % kAlign) == 0; }


long long n_scales(long long rows, long long cols, int group)
{
    return group ? rows * (cols / group) : rows;
}

// Batches of at most this many tokens keep every expert on the GEMV by default
// (measured through the stack workload: 2 tokens 1.49 -> 1.03 ms per step on
// the GEMV; 4 tokens 1.70 ms on the 32-token pass against 1.82 on the GEMV)
constexpr int kGemvBatchTokens = 2;

// Defaults: experts with at least this many tokens use the 128-token MFMA
// pass, all others the 32-token MFMA pass (batches of up to kGemvBatchTokens
// tokens aside). Single-token experts of larger batches used to stay on the
// GEMV; on the 32-token pass they measured faster at every batch size tried
// (the stack workload at 3 to 32 tokens per step: +6% to +17% tokens/s;
// decode64 81.7K -> 84.2K), one pass fewer and its launches gone.
constexpr int kDefaultMfmaMinTokens = 32;
constexpr int kDefaultSmallMinTokens = 1;

// Workspace of moe_expert_forward, laid out in this order.
struct FwdLayout {
    int tb, max_items, max_mitems, max_sitems, tstar, tsmall, P;
    long long items, n_items, mitems, n_mitems, sitems, n_sitems, h, o, x16, h16, total;
};

long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

// The passes and work-list bounds of one call. upper = true: a bound of the
// layout over every option value, for sizing the workspace.
FwdLayout fwd_layout(const Geo &g, int N, int k, int has_shared, int mfma_min_tokens,
                     int small_min_tokens, bool upper = false)
{
    FwdLayout L;
    const long long A = (long long)N * k;
    const long long ue = A < g.E ? A : g.E;  // union experts at most
    const bool mf = mfma_supported(g);
    L.tstar = mfma_min_tokens > 0 ? mfma_min_tokens : kDefaultMfmaMinTokens;
    L.tsmall = small_min_tokens > 0 ? small_min_tokens : kDefaultSmallMinTokens;
    // a pass runs when some expert can reach its threshold (an expert has at
    // most N tokens); the small pass only takes what the large one leaves
    bool big = mf && mfma_min_tokens >= 0 && N >= L.tstar;
    if (big && mf && small_min_tokens >= 0 && N >= L.tsmall && L.tsmall < L.tstar) {
        // at most this many 128-token items: each expert reaching tstar adds
        // one partly filled item. Below kMinBigItems the planner moves them
        // all to the 32-token pass, so that pass alone is launched. With the
        // default thresholds, batches of fewer assignments than kMinBigItems
        // full items take the 32-token pass alone as well: there the planner
        // nearly always leaves the 128-token pass empty, and an empty launch
        // pair still costs about 9 us
        const long long most = ceil_div(A, kMfmaBigTokens) + A / L.tstar +
                               (has_shared && N >= L.tstar ? ceil_div(N, kMfmaBigTokens) : 0);
        if (most < kMinBigItems ||
            (mfma_min_tokens == 0 && A < (long long)kMinBigItems * kMfmaBigTokens))
            big = false;
    }
    bool small = mf && small_min_tokens >= 0 && N >= L.tsmall && !(big && L.tsmall >= L.tstar);
    // By default, the smallest batches stay on the GEMV: one item per expert
    // reads its weights once, while the 32-token pass would give a handful of
    // experts a handful of workgroups each, behind extra launches
    if (small && small_min_tokens == 0 && !big && N <= kGemvBatchTokens) small = false;
    // most tokens of an expert on the GEMV pass
    long long cap = N;
    if (small) cap = L.tsmall - 1;
    else if (big) cap = L.tstar - 1;
    L.tb = gemv_tokens_per_item(g, (int)(cap < 1 ? 1 : cap));
    if (upper) {
        // every list at the most items any threshold can give it (1-token
        // GEMV items, and every assignment its own MFMA expert)
        L.tb = gemv_tokens_per_item(g, N);
        L.max_items = (int)(A + ue + N);
        L.max_mitems = mf ? (int)(ceil_div(A, kMfmaBigTokens) + A + ceil_div(N, kMfmaBigTokens)) : 0;
        L.max_sitems = mf ? (int)(ceil_div(A, kMfmaSmallTokens) + A + ceil_div(N, kMfmaSmallTokens)) : 0;
    } else {
        if (cap < 1) {
            L.max_items = 0;
        } else {
            // each expert adds at most one partly filled item; none has more
            // than cap tokens
            const long long per = ceil_div(cap, L.tb);
            long long routed = ceil_div(A, L.tb) + ue;
            if (ue * per < routed) routed = ue * per;
            L.max_items = (int)(routed + (has_shared && N <= cap ? ceil_div(N, L.tb) : 0));
        }
        // each expert on a pass adds at most one partly filled item; at most
        // min(ue, A / threshold) experts reach a threshold
        const long long ue_big = ue < A / L.tstar ? ue : A / L.tstar;
        const long long ue_small = ue < A / L.tsmall ? ue : A / L.tsmall;
        L.max_mitems = big ? (int)(ceil_div(A, kMfmaBigTokens) + ue_big +
                                   (has_shared ? ceil_div(N, kMfmaBigTokens) : 0))
                           : 0;
        // every group on this pass, and (with the 128-token pass) the
        // remainder of each group on that one, adds at most one partly
        // filled item
        long long sm = ceil_div(A, kMfmaSmallTokens) + (big ? ue : ue_small) +
                       (has_shared ? ceil_div(N, kMfmaSmallTokens) : 0);
        if (big) {
            // below tstar an expert is at most ceil((tstar - 1) / 32) items; experts
            // moved over from the 128-token pass had fewer than kMinBigItems of
            // its items between them, so at most (kMinBigItems - 1) * 128 tokens;
            // each group left on the 128-token pass adds at most one remainder
            const long long below = (ue + (has_shared ? 1 : 0)) * ceil_div(L.tstar - 1, kMfmaSmallTokens);
            const long long moved = (long long)(kMinBigItems - 1) * (kMfmaBigTokens / kMfmaSmallTokens + 1);
            const long long rems = ue_big + (has_shared ? 1 : 0);
            if (below + moved + rems < sm) sm = below + moved + rems;
        }
        L.max_sitems = small ? (int)sm : 0;
    }
    L.P = (int)(A + (has_shared ? N : 0));
    long long off = 0;
    L.items = off; off = align_up(off + (long long)L.max_items * (long long)sizeof(Item));
    L.n_items = off; off = align_up(off + 4);
    L.mitems = off; off = align_up(off + (long long)L.max_mitems * (long long)sizeof(Item));
    L.n_mitems = off; off = align_up(off + 4);
    L.sitems = off; off = align_up(off + (long long)L.max_sitems * (long long)sizeof(Item));
    L.n_sitems = off; off = align_up(off + 4);
    L.h = off; off = align_up(off + (long long)L.P * g.f * 4);
    L.o = off; off = align_up(off + (long long)L.P * g.d * 4);
    // float16 operands, when a matrix-core pass can run
    const bool any_mfma = L.max_mitems > 0 || L.max_sitems > 0;
    L.x16 = off; off = align_up(off + (any_mfma ? (long long)N * g.d * 2 : 0));
    L.h16 = off; off = align_up(off + (any_mfma ? (long long)L.P * g.f * 2 : 0));
    L.total = off;
    return L;
}

moe_status check_k(int k, int E)
{
    if (E < 1 || E > MOE_MAX_EXPERTS) return MOE_EINVAL;
    if (k < 1 || k > MOE_MAX_K || k > E) return MOE_EINVAL;
    return MOE_OK;
}

}  // namespace

moe_status resolve_geo(const moe_expert_pool *p, Geo *g)
{
    if (!p) return MOE_EINVAL;
    if (p->wbits != 4 && p->wbits != 8) return MOE_EINVAL;
    if (p->n_experts < 1 || p->n_experts > MOE_MAX_EXPERTS) return MOE_EINVAL;
    if (p->d_model <= 0 || p->d_ff <= 0 || p->group < 0) return MOE_EINVAL;
    Geo r;
    memset(&r, 0, sizeof(r));
    r.d = p->d_model;
    r.f = p->d_ff;
    r.E = p->n_experts;
    r.wbits = p->wbits;
    r.group = p->group;
    r.epc = p->wbits == 4 ? 32 : 16;
    r.ucols = 4 * r.epc;
    // whole units along both matrices' rows and columns; activations of one
    // token row staged in LDS stay within budget
    if (r.d % r.ucols || r.f % r.ucols) return MOE_ESHAPE;
    if (r.d > kMaxModelDim || r.f > kMaxModelDim) return MOE_ESHAPE;
    if (r.group) {
        if (r.group % r.epc || r.d % r.group || r.f % r.group) return MOE_ESHAPE;
    }
    r.kb_gu = r.d / r.ucols;
    r.kb_dn = r.f / r.ucols;
    r.ng_gu = r.group ? r.d / r.group : 1;
    r.ng_dn = r.group ? r.f / r.group : 1;
    const long long q_gu = (long long)r.f * r.d * r.wbits / 8, q_dn = q_gu;
    r.off_up = q_gu;
    r.off_dn = 2 * q_gu;
    r.off_gs = 2 * q_gu + q_dn;
    r.off_us = r.off_gs + 4 * n_scales(r.f, r.d, r.group);
    r.off_ds = r.off_us + 4 * n_scales(r.f, r.d, r.group);
    *g = r;
    return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_block_bytes(int d_model, int d_ff, int wbits, int group)
{
    if (d_model <= 0 || d_ff <= 0 || (wbits != 4 && wbits != 8) || group < 0) return 0;
    if (group && (d_model % group || d_ff % group)) return 0;
    const long long q = (long long)d_model * d_ff * wbits / 8;
    return (size_t)(3 * q + 4 * (2 * n_scales(d_ff, d_model, group) + n_scales(d_model, d_ff, group)));
}

size_t moe_route_workspace_size(int n_tokens, int n_experts)
{
    if (n_tokens < 0 || n_experts < 1) return 0;
    // scores, or the router's partial sums over up to router_slices_bound slices
    const long long slices = n_tokens > 0 ? router_slices_bound(n_tokens, n_experts) : 1;
    return (size_t)align_up(slices * n_tokens * n_experts * 4);
}

size_t moe_forward_workspace_size(const moe_expert_pool *pool, int n_tokens, int k)
{
    Geo g;
    if (resolve_geo(pool, &g) != MOE_OK || n_tokens < 0 || k < 1) return 0;
    return (size_t)fwd_layout(g, n_tokens, k, pool->shared != nullptr, 0, 0, true).total;
}

size_t moe_workspace_size(const moe_expert_pool *pool, int n_tokens, int k)
{
    if (!pool) return 0;
    size_t a = moe_route_workspace_size(n_tokens, pool->n_experts);
    size_t b = moe_forward_workspace_size(pool, n_tokens, k);
    return a > b ? a : b;
}

const char *moe_strerror(moe_status st)
{
    switch (st) {
    case MOE_OK: return "success";
    case MOE_EINVAL: return "invalid argument (null pointer, negative size, bad k or wbits)";
    case MOE_ESHAPE: return "unsupported shape (d_model, d_ff or group)";
    case MOE_EALIGN: return "pointer or stride not aligned to MOE_ALIGN";
    case MOE_EWORKSPACE: return "workspace missing or too small";
    case MOE_EHIP: return "HIP runtime call or kernel launch failed";
    case MOE_EIO: return "file not readable, not writable, or not a usage file";
    }
    return "unknown status";
}

}  // extern "C"

namespace {

// Route options -> (bias for the router, top-k options); false on a bad option
bool route_options(const moe_route_options *opt, const float *b_router, const float **b_in,
                   TopkOpt *to)
{
    *b_in = b_router;
    *to = TopkOpt();
    if (!opt) return true;
    if ((opt->bias_select_only != 0 && opt->bias_select_only != 1) ||
        (opt->normalize != 0 && opt->normalize != 1) || !(opt->scale > 0.0f) ||
        !(opt->scale < 3.0e38f) || !(opt->top_p >= 0.0f) || !(opt->top_p < 3.0e38f))
        return false;
    if (opt->bias_select_only) {
        *b_in = nullptr;       // scores without the bias
        to->sel = b_router;    // the bias only in the selection keys (null: none)
    }
    to->norm = opt->normalize;
    to->scale = opt->scale;
    to->top_p = opt->top_p;
    return true;
}

}  // namespace

extern "C" {

moe_status moe_route_topk(const float *x, int n_tokens, int d_model, const float *w_router,
                          const float *b_router, int n_experts, int k, int32_t *topk_ids,
                          float *topk_w, void *workspace, size_t ws_bytes, hipStream_t stream)
{
    return moe_route_topk_ex(x, n_tokens, d_model, w_router, b_router, n_experts, k, topk_ids,
                             topk_w, workspace, ws_bytes, stream, nullptr);
}

moe_status moe_route_topk_ex(const float *x, int n_tokens, int d_model, const float *w_router,
                             const float *b_router, int n_experts, int k, int32_t *topk_ids,
                             float *topk_w, void *workspace, size_t ws_bytes, hipStream_t stream,
                             const moe_route_options *opt)
{
    if (n_tokens < 0 || d_model <= 0) return MOE_EINVAL;
    moe_status st = check_k(k, n_experts);
    if (st != MOE_OK) return st;
    if (d_model % 32) return MOE_ESHAPE;
    if ((long long)n_tokens * n_experts > 0x7FFFFFFFLL || (long long)n_tokens * d_model > 0x7FFFFFFFLL)
        return MOE_ESHAPE;
    if (n_tokens == 0) return MOE_OK;
    if (!x || !w_router || !topk_ids || !topk_w) return MOE_EINVAL;
    if (((uintptr_t)x % 16) || ((uintptr_t)w_router % 16)) return MOE_EALIGN;
    if (!workspace || ws_bytes < moe_route_workspace_size(n_tokens, n_experts)) return MOE_EWORKSPACE;
    if (!aligned(workspace)) return MOE_EALIGN;
    const float *b_in;
    TopkOpt to;
    if (!route_options(opt, b_router, &b_in, &to)) return MOE_EINVAL;
    if (to.sel && ((uintptr_t)to.sel % 4)) return MOE_EALIGN;
    float *scores = static_cast<float *>(workspace);
    if (launch_router(x, n_tokens, d_model, w_router, b_in, n_experts, scores, stream) !=
        hipSuccess)
        return MOE_EHIP;
    if (launch_topk(scores, router_slices(n_tokens, d_model, n_experts), b_in, n_tokens,
                    n_experts, k, topk_ids, topk_w, stream, to) != hipSuccess)
        return MOE_EHIP;
    return MOE_OK;
}

moe_status moe_union(const int32_t *topk_ids, int n_tokens, int k, int n_experts,
                     int32_t *union_ids, int32_t *n_union, int32_t *expert_offsets, int32_t *perm,
                     hipStream_t stream)
{
    if (n_tokens < 0) return MOE_EINVAL;
    moe_status st = check_k(k, n_experts);
    if (st != MOE_OK) return st;
    if ((long long)n_tokens * k > 0x7FFFFFFFLL) return MOE_ESHAPE;
    if (n_tokens == 0) return MOE_OK;
    if (!topk_ids || !union_ids || !n_union || !expert_offsets || !perm) return MOE_EINVAL;
    if (launch_union(topk_ids, n_tokens * k, n_experts, union_ids, n_union, expert_offsets, perm,
                     nullptr, stream) != hipSuccess)
        return MOE_EHIP;
    return MOE_OK;
}

moe_status moe_hit_count(const int32_t *topk_ids, int n_tokens, int k, int n_experts,
                         uint64_t *counters, hipStream_t stream)
{
    if (n_tokens < 0) return MOE_EINVAL;
    moe_status st = check_k(k, n_experts);
    if (st != MOE_OK) return st;
    if ((long long)n_tokens * k > 0x7FFFFFFFLL) return MOE_ESHAPE;
    if (n_tokens == 0) return MOE_OK;
    if (!topk_ids || !counters) return MOE_EINVAL;
    if ((uintptr_t)counters % 8) return MOE_EALIGN;
    if (launch_hit_count(topk_ids, n_tokens * k, n_experts, counters, stream) != hipSuccess)
        return MOE_EHIP;
    return MOE_OK;
}

// batches of at least this many assignments form the union over several
// workgroups (moe_route_union only: it has the router's workspace as scratch)
constexpr int kChunkedUnionMin = 4096;

moe_status moe_route_union(const float *x, int n_tokens, int d_model, const float *w_router,
                           const float *b_router, int n_experts, int k, int32_t *topk_ids,
                           float *topk_w, int32_t *union_ids, int32_t *n_union,
                           int32_t *expert_offsets, int32_t *perm, uint64_t *counters,
                           void *workspace, size_t ws_bytes, hipStream_t stream)
{
    return moe_route_union_ex(x, n_tokens, d_model, w_router, b_router, n_experts, k, topk_ids,
                              topk_w, union_ids, n_union, expert_offsets, perm, counters,
                              workspace, ws_bytes, stream, nullptr);
}

// What route_union_impl does after its checks (router_plan: nothing, but
// the router's slice count and bias are returned).
enum class RouteMode { all, check_only, router_plan };

static moe_status route_union_impl(const float *x, int n_tokens, int d_model,
                                   const float *w_router, const float *b_router, int n_experts,
                                   int k, int32_t *topk_ids, float *topk_w, int32_t *union_ids,
                                   int32_t *n_union, int32_t *expert_offsets, int32_t *perm,
                                   uint64_t *counters, void *workspace, size_t ws_bytes,
                                   hipStream_t stream, const moe_route_options *opt,
                                   RouteMode mode, int *P_out, const float **b_out)
{
    // every check of moe_route_topk, moe_union and moe_hit_count, before any launch
    if (n_tokens < 0 || d_model <= 0) return MOE_EINVAL;
    moe_status st = check_k(k, n_experts);
    if (st != MOE_OK) return st;
    if (d_model % 32) return MOE_ESHAPE;
    if ((long long)n_tokens * n_experts > 0x7FFFFFFFLL || (long long)n_tokens * d_model > 0x7FFFFFFFLL ||
        (long long)n_tokens * k > 0x7FFFFFFFLL)
        return MOE_ESHAPE;
    if (n_tokens == 0) return MOE_OK;
    if (!x || !w_router || !topk_ids || !topk_w || !union_ids || !n_union || !expert_offsets ||
        !perm)
        return MOE_EINVAL;
    if (((uintptr_t)x % 16) || ((uintptr_t)w_router % 16)) return MOE_EALIGN;
    if (counters && ((uintptr_t)counters % 8)) return MOE_EALIGN;
    if (!workspace || ws_bytes < moe_route_workspace_size(n_tokens, n_experts))
        return MOE_EWORKSPACE;
    if (!aligned(workspace)) return MOE_EALIGN;
    const float *b_in;
    TopkOpt to;
    if (!route_options(opt, b_router, &b_in, &to)) return MOE_EINVAL;
    if (to.sel && ((uintptr_t)to.sel % 4)) return MOE_EALIGN;
    if (mode == RouteMode::check_only) return MOE_OK;
    float *scores = static_cast<float *>(workspace);
    const int P = router_slices(n_tokens, d_model, n_experts);
    if (mode == RouteMode::router_plan) {
        *P_out = P;
        *b_out = b_in;
        return MOE_OK;
    }
    if (launch_router(x, n_tokens, d_model, w_router, b_in, n_experts, scores, stream) !=
        hipSuccess)
        return MOE_EHIP;
    if (n_tokens <= route_tail_max_tokens())
        return launch_route_tail(scores, P, b_in, n_tokens, n_experts, k, topk_ids, topk_w,
                                 union_ids, n_union, expert_offsets, perm, counters, stream,
                                 to) == hipSuccess
                   ? MOE_OK
                   : MOE_EHIP;
    if (launch_topk(scores, P, b_in, n_tokens, n_experts, k, topk_ids, topk_w, stream, to) !=
        hipSuccess)
        return MOE_EHIP;
    const int A = n_tokens * k;
    if (A >= kChunkedUnionMin) {
        // the router's output has been consumed (stream order): the
        // workspace is the chunked union's scratch
        return launch_union_chunked(topk_ids, A, n_experts, union_ids, n_union, expert_offsets,
                                    perm, counters, workspace,
                                    moe_route_workspace_size(n_tokens, n_experts),
                                    stream) == hipSuccess
                   ? MOE_OK
                   : MOE_EHIP;
    }
    // the union kernel adds the hit counts itself
    if (launch_union(topk_ids, A, n_experts, union_ids, n_union, expert_offsets, perm, counters,
                     stream) != hipSuccess)
        return MOE_EHIP;
    return MOE_OK;
}

moe_status moe_route_union_ex(const float *x, int n_tokens, int d_model, const float *w_router,
                              const float *b_router, int n_experts, int k, int32_t *topk_ids,
                              float *topk_w, int32_t *union_ids, int32_t *n_union,
                              int32_t *expert_offsets, int32_t *perm, uint64_t *counters,
                              void *workspace, size_t ws_bytes, hipStream_t stream,
                              const moe_route_options *opt)
{
    return route_union_impl(x, n_tokens, d_model, w_router, b_router, n_experts, k, topk_ids,
                            topk_w, union_ids, n_union, expert_offsets, perm, counters, workspace,
                            ws_bytes, stream, opt, RouteMode::all, nullptr, nullptr);
}

moe_status moe_expert_forward(const moe_expert_pool *pool, const float *x, int n_tokens, int k,
                              const float *topk_w, const int32_t *union_ids,
                              const int32_t *n_union, const int32_t *expert_offsets,
                              const int32_t *perm, float *y, void *workspace, size_t ws_bytes,
                              hipStream_t stream)
{
    return moe_expert_forward_ex(pool, x, n_tokens, k, topk_w, union_ids, n_union, expert_offsets,
                                 perm, y, workspace, ws_bytes, stream, nullptr);
}

// The routing a one- or two-token moe_layer_step hands to the expert
// kernels: the router (launched by forward_impl) writes scores, and the
// gate/up kernel takes the top-k.
struct InRoute {
    float *scores;
    int P;
    const float *b;
    int32_t *ids;
    float *w;
    uint64_t *counters;
    const float *x, *wr;  // router inputs
    int d;
};

// The phase of a two-phase forward (Fwd::phase), or none.
struct Phase {
    const uint8_t *mask;
    int sel;
};

static moe_status forward_impl(const moe_expert_pool *pool, const float *x, int n_tokens, int k,
                               const float *topk_w, const int32_t *union_ids,
                               const int32_t *n_union, const int32_t *expert_offsets,
                               const int32_t *perm, float *y, void *workspace, size_t ws_bytes,
                               hipStream_t stream, const moe_forward_options *ev,
                               bool check_only, const InRoute *ir, const Phase *ph = nullptr,
                               const StackNorm *sn = nullptr, bool *normed = nullptr)
{
    Geo g;
    moe_status st = resolve_geo(pool, &g);
    if (st != MOE_OK) return st;
    if (n_tokens < 0) return MOE_EINVAL;
    st = check_k(k, g.E);
    if (st != MOE_OK) return st;
    if (!pool->pool) return MOE_EINVAL;
    if (pool->slot_of && pool->n_slots < 1) return MOE_EINVAL;
    if (!aligned(pool->pool) || (pool->shared && !aligned(pool->shared)) ||
        pool->expert_bytes % kAlign)
        return MOE_EALIGN;
    if (pool->expert_bytes < moe_block_bytes(g.d, g.f, g.wbits, g.group)) return MOE_ESHAPE;
    const long long A = (long long)n_tokens * k;
    if (A + n_tokens > 0x7FFFFFFFLL || (A + n_tokens) * (long long)(g.d > g.f ? g.d : g.f) > 0x7FFFFFFFFFFFLL)
        return MOE_ESHAPE;
    if (n_tokens == 0) return MOE_OK;
    if (!x || !topk_w || !union_ids || !n_union || !expert_offsets || !perm || !y)
        return MOE_EINVAL;
    if (((uintptr_t)x % 16) || ((uintptr_t)y % 16)) return MOE_EALIGN;
    const int has_shared = pool->shared != nullptr;
    const FwdLayout L = fwd_layout(g, n_tokens, k, has_shared, ev ? ev->mfma_min_tokens : 0,
                                   ev ? ev->mfma_small_min_tokens : 0);
    if (!workspace || ws_bytes < (size_t)L.total) return MOE_EWORKSPACE;
    if (!aligned(workspace)) return MOE_EALIGN;
    if (check_only) return MOE_OK;

    char *ws = static_cast<char *>(workspace);
    Fwd f;
    f.route_in = ir ? ir->scores : nullptr;
    f.route_P = ir ? ir->P : 1;
    f.route_b = ir ? ir->b : nullptr;
    f.route_ids = ir ? ir->ids : nullptr;
    f.route_w = ir ? ir->w : nullptr;
    f.route_counters = ir ? reinterpret_cast<unsigned long long *>(ir->counters) : nullptr;
    f.g = g;
    f.pool = static_cast<const uint8_t *>(pool->pool);
    f.stride = pool->expert_bytes;
    f.slot_of = pool->slot_of;
    f.n_slots = pool->n_slots;
    f.shared = static_cast<const uint8_t *>(pool->shared);
    f.x = x;
    f.w = topk_w;
    f.k = k;
    f.N = n_tokens;
    f.A = (int)A;
    f.has_shared = has_shared;
    f.union_ids = union_ids;
    f.n_union = n_union;
    f.offsets = expert_offsets;
    f.perm = perm;
    f.h = reinterpret_cast<float *>(ws + L.h);
    f.o = reinterpret_cast<float *>(ws + L.o);
    f.x16 = reinterpret_cast<uint16_t *>(ws + L.x16);
    f.h16 = reinterpret_cast<uint16_t *>(ws + L.h16);
    f.y = y;
    f.items = reinterpret_cast<Item *>(ws + L.items);
    f.n_items = reinterpret_cast<int32_t *>(ws + L.n_items);
    f.tb = L.tb;
    f.max_items = L.max_items;
    f.mitems = reinterpret_cast<Item *>(ws + L.mitems);
    f.n_mitems = reinterpret_cast<int32_t *>(ws + L.n_mitems);
    f.max_mitems = L.max_mitems;
    f.tstar = L.tstar;
    f.sitems = reinterpret_cast<Item *>(ws + L.sitems);
    f.n_sitems = reinterpret_cast<int32_t *>(ws + L.n_sitems);
    f.max_sitems = L.max_sitems;
    f.tsmall = L.tsmall;
    // Every expert on the GEMV pass and at most two terms per output element
    // (top-1 with the shared expert, or top-2 without): the down kernel adds
    // its gate-weighted rows into y with float atomics. Two addends onto zero
    // give the same sum in either order, so y is deterministic and equal to
    // the combine kernel's; one launch fewer.
    f.direct = (L.max_mitems == 0 && L.max_sitems == 0 && k + has_shared <= 2) ? 1 : 0;
    // a two-phase forward combines once, after its second phase
    f.phase = ph ? ph->mask : nullptr;
    f.phase_sel = ph ? ph->sel : 0;
    if (ph) f.direct = 0;

    f.ev_gu[0] = ev ? ev->gateup_start : nullptr;
    f.ev_gu[1] = ev ? ev->gateup_end : nullptr;
    f.ev_dn[0] = ev ? ev->down_start : nullptr;
    f.ev_dn[1] = ev ? ev->down_end : nullptr;
    f.ev_mgu[0] = ev ? ev->mfma_gateup_start : nullptr;
    f.ev_mgu[1] = ev ? ev->mfma_gateup_end : nullptr;
    f.ev_mdn[0] = ev ? ev->mfma_down_start : nullptr;
    f.ev_mdn[1] = ev ? ev->mfma_down_end : nullptr;
    f.ev_sgu[0] = ev ? ev->small_gateup_start : nullptr;
    f.ev_sgu[1] = ev ? ev->small_gateup_end : nullptr;
    f.ev_sdn[0] = ev ? ev->small_down_start : nullptr;
    f.ev_sdn[1] = ev ? ev->small_down_end : nullptr;
    if (ir && launch_router(ir->x, n_tokens, ir->d, ir->wr, ir->b, g.E, ir->scores, stream) !=
                  hipSuccess)
        return MOE_EHIP;
    // gate/up of every pass (the first launch also builds the work lists),
    // then down of every pass, then the combine
    bool x16_staged = false;
    if (launch_gateup(f, stream, &x16_staged) != hipSuccess) return MOE_EHIP;
    if ((f.max_mitems > 0 || f.max_sitems > 0) && !x16_staged &&
        launch_stage_x16(f, stream) != hipSuccess)
        return MOE_EHIP;
    if (launch_mfma(f, true, false, stream) != hipSuccess) return MOE_EHIP;
    if (launch_mfma(f, true, true, stream) != hipSuccess) return MOE_EHIP;
    if (launch_down(f, stream) != hipSuccess) return MOE_EHIP;
    if (launch_mfma(f, false, false, stream) != hipSuccess) return MOE_EHIP;
    if (launch_mfma(f, false, true, stream) != hipSuccess) return MOE_EHIP;
    if (!f.direct && (!ph || ph->sel == 1)) {
        if (sn && combine_norm_supported(g.d, sn->h, sn->a)) {
            // a layer stack: the combine goes straight into the residual
            // stream and the next layer's norm
            if (launch_combine_norm(f.o, topk_w, n_tokens, k, g.d, (int)A, has_shared, sn->h,
                                    sn->a, sn->eps, stream) != hipSuccess)
                return MOE_EHIP;
            if (normed) *normed = true;
        } else if (launch_combine(f.o, topk_w, n_tokens, k, g.d, (int)A, has_shared, y, stream) !=
                   hipSuccess) {
            return MOE_EHIP;
        }
    }
    return MOE_OK;
}


moe_status moe_expert_forward_ex(const moe_expert_pool *pool, const float *x, int n_tokens, int k,
                                 const float *topk_w, const int32_t *union_ids,
                                 const int32_t *n_union, const int32_t *expert_offsets,
                                 const int32_t *perm, float *y, void *workspace, size_t ws_bytes,
                                 hipStream_t stream, const moe_forward_options *ev)
{
    return forward_impl(pool, x, n_tokens, k, topk_w, union_ids, n_union, expert_offsets, perm, y,
                        workspace, ws_bytes, stream, ev, false, nullptr);
}

// moe_layer_step takes the routing inside the gate/up launch up to this k:
// every workgroup of a routed expert pays k argmax rounds before its weight
// loads, which outweighs the route-tail launch it saves at larger k.
constexpr int kInsideMaxK = 2;

size_t moe_layer_step_workspace_size(const moe_expert_pool *pool, int n_tokens, int k)
{
    if (!pool) return 0;
    const size_t a = moe_route_workspace_size(n_tokens, pool->n_experts);
    const size_t b = moe_forward_workspace_size(pool, n_tokens, k);
    return a && b ? a + b : 0;
}

static moe_status layer_step_impl(const moe_expert_pool *pool, const float *x, int n_tokens,
                                  int d_model, const float *w_router, const float *b_router, int k,
                                  int32_t *topk_ids, float *topk_w, int32_t *union_ids,
                                  int32_t *n_union, int32_t *expert_offsets, int32_t *perm,
                                  uint64_t *counters, float *y, void *workspace, size_t ws_bytes,
                                  hipStream_t stream, const moe_forward_options *opt,
                                  bool check_only, const StackNorm *sn = nullptr,
                                  bool *normed = nullptr);

moe_status moe_layer_step(const moe_expert_pool *pool, const float *x, int n_tokens, int d_model,
                          const float *w_router, const float *b_router, int k, int32_t *topk_ids,
                          float *topk_w, int32_t *union_ids, int32_t *n_union,
                          int32_t *expert_offsets, int32_t *perm, uint64_t *counters, float *y,
                          void *workspace, size_t ws_bytes, hipStream_t stream,
                          const moe_forward_options *opt)
{
    return layer_step_impl(pool, x, n_tokens, d_model, w_router, b_router, k, topk_ids, topk_w,
                           union_ids, n_union, expert_offsets, perm, counters, y, workspace,
                           ws_bytes, stream, opt, false);
}

static moe_status layer_step_impl(const moe_expert_pool *pool, const float *x, int n_tokens,
                                  int d_model, const float *w_router, const float *b_router, int k,
                                  int32_t *topk_ids, float *topk_w, int32_t *union_ids,
                                  int32_t *n_union, int32_t *expert_offsets, int32_t *perm,
                                  uint64_t *counters, float *y, void *workspace, size_t ws_bytes,
                                  hipStream_t stream, const moe_forward_options *opt,
                                  bool check_only, const StackNorm *sn, bool *normed)
{
    if (!pool) return MOE_EINVAL;
    Geo g;
    moe_status st = resolve_geo(pool, &g);
    if (st != MOE_OK) return st;
    if (d_model != pool->d_model) return MOE_ESHAPE;
    st = check_k(k, pool->n_experts);
    if (st != MOE_OK) return st;
    if (n_tokens < 0) return MOE_EINVAL;
    const size_t need = moe_layer_step_workspace_size(pool, n_tokens, k);
    if (n_tokens > 0 && (!workspace || need == 0 || ws_bytes < need)) return MOE_EWORKSPACE;
    // the router's output first, the expert step's workspace after it
    const size_t rs = moe_route_workspace_size(n_tokens, pool->n_experts);
    char *ws = static_cast<char *>(workspace);
    void *fws = ws ? ws + rs : nullptr;
    const size_t fbytes = ws_bytes > rs ? ws_bytes - rs : 0;
    // every check of both calls before anything is enqueued
    st = route_union_impl(x, n_tokens, d_model, w_router, b_router, pool->n_experts, k,
                                     topk_ids, topk_w, union_ids, n_union, expert_offsets, perm,
                                     counters, workspace, rs, stream, nullptr,
                                     RouteMode::check_only, nullptr, nullptr);
    if (st != MOE_OK) return st;
    st = forward_impl(pool, x, n_tokens, k, topk_w, union_ids, n_union, expert_offsets, perm, y,
                      fws, fbytes, stream, opt, true, nullptr);
    if (st != MOE_OK || n_tokens == 0 || check_only) return st;
    // Up to two tokens whose experts all stay on the GEMV with one item per
    // expert (a positive threshold can move them to the matrix cores) take
    // the routing inside the gate/up launch.
    const FwdLayout L = fwd_layout(g, n_tokens, k, pool->shared != nullptr,
                                   opt ? opt->mfma_min_tokens : 0,
                                   opt ? opt->mfma_small_min_tokens : 0);
    const bool inside = n_tokens <= 2 && k <= kInsideMaxK && L.max_mitems == 0 &&
                        L.max_sitems == 0 && n_tokens <= L.tb;
    if (!inside) {
        st = route_union_impl(x, n_tokens, d_model, w_router, b_router, pool->n_experts, k,
                              topk_ids, topk_w, union_ids, n_union, expert_offsets, perm,
                              counters, workspace, rs, stream, nullptr, RouteMode::all, nullptr,
                              nullptr);
        if (st != MOE_OK) return st;
        return forward_impl(pool, x, n_tokens, k, topk_w, union_ids, n_union, expert_offsets,
                            perm, y, fws, fbytes, stream, opt, false, nullptr, nullptr, sn,
                            normed);
    }
    // the router, then the expert kernels, the top-k, union and counting
    // taken inside the gate/up GEMV launch
    InRoute ir;
    ir.scores = static_cast<float *>(workspace);
    ir.ids = topk_ids;
    ir.w = topk_w;
    ir.counters = counters;
    ir.x = x;
    ir.wr = w_router;
    ir.d = d_model;
    st = route_union_impl(x, n_tokens, d_model, w_router, b_router, pool->n_experts, k, topk_ids,
                          topk_w, union_ids, n_union, expert_offsets, perm, counters, workspace,
                          rs, stream, nullptr, RouteMode::router_plan, &ir.P, &ir.b);
    if (st != MOE_OK) return st;
    return forward_impl(pool, x, n_tokens, k, topk_w, union_ids, n_union, expert_offsets, perm, y,
                        fws, fbytes, stream, opt, false, &ir, nullptr, sn, normed);
}

moe_status moe_residual_rmsnorm(float *h, const float *y, float *a, int n_tokens, int d_model,
                                float eps, hipStream_t stream)
{
    if (n_tokens < 0 || d_model <= 0 || !(eps >= 0.0f)) return MOE_EINVAL;
    if (n_tokens == 0) return MOE_OK;
    if (!h || !a || a == h) return MOE_EINVAL;
    if (launch_residual_rmsnorm(h, y, a, n_tokens, d_model, eps, stream) != hipSuccess)
        return MOE_EHIP;
    return MOE_OK;
}

moe_status moe_pack_expert(const void *canonical_block, const moe_expert_pool *shape,
                           void *block_out)
{
    Geo g;
    moe_status st = resolve_geo(shape, &g);
    if (st != MOE_OK) return st;
    if (!canonical_block || !block_out) return MOE_EINVAL;
    const size_t bytes = moe_block_bytes(g.d, g.f, g.wbits, g.group);
    // build in a host copy, so that the output may be the input
    std::vector<uint8_t> tmp(bytes);
    const uint8_t *src = static_cast<const uint8_t *>(canonical_block);
    uint8_t *dst = tmp.data();
    const uint8_t flip = g.wbits == 4 ? 0x88 : 0x80;  // two's complement -> offset binary
    const uint64_t flip8 = 0x0101010101010101ULL * flip;
    // the three code matrices: canonical row-major [R][K] -> units
    struct Mat { long long off; int R, K; };
    const Mat mats[3] = {{0, g.f, g.d}, {g.off_up, g.f, g.d}, {g.off_dn, g.d, g.f}};
    for (const Mat &m : mats) {
        const long long row_bytes = (long long)m.K * g.wbits / 8;
        const int n_kb = m.K / g.ucols;
        for (int rt = 0; rt < m.R / kUnitRows; ++rt)
            for (int kb = 0; kb < n_kb; ++kb)
                for (int slot = 0; slot < kWave; ++slot) {
                    const int r = slot % kUnitRows, q = slot / kUnitRows;
                    const long long row = (long long)rt * kUnitRows + r;
                    const long long from = m.off + row * row_bytes +
                                           ((long long)kb * g.ucols + (long long)q * g.epc) *
                                               g.wbits / 8;
                    const long long to = m.off + ((long long)rt * n_kb + kb) * kUnitBytes + 16LL * slot;
                    uint64_t v[2];
                    memcpy(v, src + from, 16);
                    v[0] ^= flip8;
                    v[1] ^= flip8;
                    memcpy(dst + to, v, 16);
                }
    }
    // scales: canonical [R][groups] -> [R / 16][groups][16]
    struct Sc { long long off; int R, ng; };
    const Sc scs[3] = {{g.off_gs, g.f, g.ng_gu}, {g.off_us, g.f, g.ng_gu}, {g.off_ds, g.d, g.ng_dn}};
    for (const Sc &sc : scs)
        for (int row = 0; row < sc.R; ++row)
            for (int gi = 0; gi < sc.ng; ++gi) {
                const long long from = sc.off + ((long long)row * sc.ng + gi) * 4;
                const long long to = sc.off + (((long long)(row / kUnitRows) * sc.ng + gi) * kUnitRows +
                                               row % kUnitRows) * 4;
                memcpy(dst + to, src + from, 4);
            }
    memcpy(block_out, dst, bytes);
    return MOE_OK;
}

}  // extern "C"

namespace moe {

moe_status layer_step_check(const moe_expert_pool *pool, const float *x, int n_tokens, int d_model,
                            const float *w_router, const float *b_router, int k,
                            int32_t *topk_ids, float *topk_w, int32_t *union_ids,
                            int32_t *n_union, int32_t *expert_offsets, int32_t *perm,
                            uint64_t *counters, float *y, void *workspace, size_t ws_bytes)
{
    return layer_step_impl(pool, x, n_tokens, d_model, w_router, b_router, k, topk_ids, topk_w,
                           union_ids, n_union, expert_offsets, perm, counters, y, workspace,
                           ws_bytes, nullptr, nullptr, true);
}

moe_status layer_step_norm(const moe_expert_pool *pool, const float *x, int n_tokens, int d_model,
                           const float *w_router, const float *b_router, int k,
                           int32_t *topk_ids, float *topk_w, int32_t *union_ids,
                           int32_t *n_union, int32_t *expert_offsets, int32_t *perm,
                           uint64_t *counters, float *y, void *workspace, size_t ws_bytes,
                           hipStream_t stream, const StackNorm *sn, bool *normed)
{
    *normed = false;
    return layer_step_impl(pool, x, n_tokens, d_model, w_router, b_router, k, topk_ids, topk_w,
                           union_ids, n_union, expert_offsets, perm, counters, y, workspace,
                           ws_bytes, stream, nullptr, false, sn, normed);
}

moe_status expert_forward_phase(const moe_expert_pool *pool, const float *x, int n_tokens, int k,
                                const float *topk_w, const int32_t *union_ids,
                                const int32_t *n_union, const int32_t *expert_offsets,
                                const int32_t *perm, float *y, void *workspace, size_t ws_bytes,
                                hipStream_t stream, const uint8_t *phase, int phase_sel,
                                bool check_only)
{
    Phase ph{phase, phase_sel};
    return forward_impl(pool, x, n_tokens, k, topk_w, union_ids, n_union, expert_offsets, perm,
                        y, workspace, ws_bytes, stream, nullptr, check_only, nullptr,
                        phase ? &ph : nullptr);
}

}  // namespace moe
