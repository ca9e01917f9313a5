/*
 * oracle.c - plain CPU reference of one MoE layer's routed-expert step.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library. It shares no code
 * with the GPU library. It is written for clarity, not speed: every sum runs in
 * index order in double precision, and OpenMP only splits independent rows.
 *
 * What it computes, after the Colibri pages:
 *  - "Public Colibri Observation and Revision Ledger", section "Exact
 *    Architecture and Data-Flow Reconstruction": a sigmoid gate scores every
 *    expert for every token (n_group = 1, gate parameters in float32); the
 *    chosen experts are three-matrix MLPs; a shared expert is always applied;
 *    per layer the work is Route, Union, Place, Overlap, Learn, and the Learn
 *    step bumps per-expert hit counters.
 *  - Same page, "Cache/Prefetch Design Comparison" (figure on async I/O and
 *    prefetch): batch-union, each distinct expert of a batch is used once.
 *  - Colibri README, "Get started" (model container: int4 experts with group
 *    scales) and "Speculative decoding, honestly" (int8 draft head).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - score s = sigmoid(Wr x + b); the top-k is taken on the float32 score,
 *    ties going to the lower expert id; ids are returned in rank order and the
 *    gate weight of a slot is the chosen expert's raw score (no renormalising).
 *  - the three-matrix MLP is SwiGLU: o = Wd (silu(Wg x) * (Wu x)),
 *    silu(z) = z / (1 + exp(-z)), no biases.
 *  - weights: W[r][c] = q[r][c] * scale[r][c / G] (symmetric, no zero point);
 *    G == 0 means one scale per row.
 *  - combine: y[t] = shared(x_t) + sum over slots j in order of w[t][j] * o_j.
 *  - hit counters count (token, slot) assignments per expert; the shared
 *    expert is not counted.
 *
 * Precision: inputs are float32 as the pages fix for the gate and the
 * activations; all arithmetic is in double. The router score is rounded to
 * float32 because the top-k decision is taken on float32 scores.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Number of threads an OpenMP parallel region of this library runs with
 * (reported next to timings of the oracle; no arithmetic). */
int oracle_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
}

/* ---- canonical expert block ------------------------------------------- */

typedef struct {
    const uint8_t *gate_q, *up_q, *down_q;
    const float *gate_s, *up_s, *down_s;
} block_view;

static size_t q_bytes(int rows, int cols, int wbits) { return (size_t)rows * cols * wbits / 8; }
static size_t n_scales(int rows, int cols, int group) { return group ? (size_t)rows * (cols / group) : (size_t)rows; }

size_t oracle_block_bytes(int d, int f, int wbits, int group)
{
    return q_bytes(f, d, wbits) * 2 + q_bytes(d, f, wbits)
         + 4 * (2 * n_scales(f, d, group) + n_scales(d, f, group));
}

static block_view view_block(const uint8_t *blk, int d, int f, int wbits, int group)
{
    block_view v;
    size_t qgu = q_bytes(f, d, wbits), qdn = q_bytes(d, f, wbits);
    v.gate_q = blk;
    v.up_q = blk + qgu;
    v.down_q = blk + 2 * qgu;
    v.gate_s = (const float *)(blk + 2 * qgu + qdn);
    v.up_s = v.gate_s + n_scales(f, d, group);
    v.down_s = v.up_s + n_scales(f, d, group);
    return v;
}

/* signed code of element c of a packed row */
static int code_at(const uint8_t *row, int c, int wbits)
{
    if (wbits == 8)
        return (int)(int8_t)row[c];
    int nib = (row[c >> 1] >> ((c & 1) * 4)) & 0xF; /* element 2i is the low nibble */
    return (nib ^ 8) - 8;                           /* two's complement nibble */
}

/* Dequantise row r of a [rows][cols] matrix: W[r][c] = q[r][c] * scale[r][c/G]. */
void oracle_dequant_row(const uint8_t *q, const float *scales, int r, int cols, int wbits,
                        int group, double *w_out)
{
    const uint8_t *row = q + (size_t)r * cols * wbits / 8;
    int gs = group ? group : cols;
    const float *srow = scales + (size_t)r * (cols / gs);
    for (int c = 0; c < cols; ++c)
        w_out[c] = (double)code_at(row, c, wbits) * (double)srow[c / gs];
}

/* ---- Route ------------------------------------------------------------ */

/* s[t][e] = float32( 1 / (1 + exp(-(b[e] + sum_i Wr[e][i] x[t][i]))) ).
 * b may be NULL (no bias). Optionally also returns the double logits. */
void oracle_router(const float *x, int n_tokens, int d, const float *w_router,
                   const float *b_router, int n_experts, float *scores, double *logits)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int t = 0; t < n_tokens; ++t)
        for (int e = 0; e < n_experts; ++e) {
            double l = b_router ? (double)b_router[e] : 0.0;
            const float *wr = w_router + (size_t)e * d;
            const float *xt = x + (size_t)t * d;
            for (int i = 0; i < d; ++i)
                l += (double)wr[i] * (double)xt[i];
            if (logits) logits[(size_t)t * n_experts + e] = l;
            scores[(size_t)t * n_experts + e] = (float)(1.0 / (1.0 + exp(-l)));
        }
}

/* key order: higher score first; equal scores -> lower id first */
static int ranks_before(float sa, int ia, float sb, int ib)
{
    return sa > sb || (sa == sb && ia < ib);
}

/* Stable top-k per token: sort all expert ids by (score desc, id asc) with a
 * plain insertion sort, keep the first k. */
void oracle_topk(const float *scores, int n_tokens, int n_experts, int k,
                 int32_t *topk_ids, float *topk_w)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < n_tokens; ++t) {
        const float *s = scores + (size_t)t * n_experts;
        int *order = (int *)malloc(sizeof(int) * n_experts);
        for (int e = 0; e < n_experts; ++e) {
            int j = e;
            while (j > 0 && ranks_before(s[e], e, s[order[j - 1]], order[j - 1])) {
                order[j] = order[j - 1];
                --j;
            }
            order[j] = e;
        }
        for (int j = 0; j < k; ++j) {
            topk_ids[(size_t)t * k + j] = order[j];
            topk_w[(size_t)t * k + j] = s[order[j]];
        }
        free(order);
    }
}

/* Router variant (opt-in; the default reading keeps the bias inside the
 * sigmoid and the raw score as the weight): the bias only steers the
 * selection, and the weights may be normalised. scores are the unbiased
 * sigmoid scores (oracle_router with no bias). Per token:
 *   key[e] = s[e] + b_sel[e]        (float32 addition: the selection is
 *                                     decided in float32, like the scores)
 *   ids    = the k best experts by (key desc, id asc), in rank order
 *   w[j]   = s[ids[j]] * scale, or with normalize
 *            s[ids[j]] / sum_j' s[ids[j']] * scale (double, rounded to
 *            float32 once);
 *   top_p in (0, 1): a lossy cutoff on the ranked slots. With S the float32
 *            sum of the k chosen scores in rank order and c_j the float32 sum
 *            of the scores ranked before slot j, slot j is kept when j == 0
 *            or c_j < top_p * S (float32); a dropped slot gets id -1 and
 *            weight 0, and the kept weights are left as above. Off when
 *            top_p <= 0 or >= 1. (The pages mention a top-p option that trades
 *            accuracy for speed without defining it; this is the plainest
 *            reading: the smallest ranked prefix holding a fraction top_p of
 *            the chosen score mass.)
 * b_sel may be NULL (no selection bias).
 * Rows of the pages this follows: the sigmoid gate over all experts with
 * n_group = 1 ("Public Colibri Observation and Revision Ledger", "Exact
 * Architecture and Data-Flow Reconstruction"); where the bias enters and
 * whether weights are renormalised the pages leave open. */
void oracle_topk_select(const float *scores, const float *b_sel, int n_tokens, int n_experts,
                        int k, int normalize, double scale, float top_p, int32_t *topk_ids,
                        float *topk_w)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < n_tokens; ++t) {
        const float *s = scores + (size_t)t * n_experts;
        float *key = (float *)malloc(sizeof(float) * n_experts);
        int *order = (int *)malloc(sizeof(int) * n_experts);
        for (int e = 0; e < n_experts; ++e) {
            volatile float kv = s[e] + (b_sel ? b_sel[e] : 0.0f);  /* one float32 rounding */
            key[e] = kv;
        }
        for (int e = 0; e < n_experts; ++e) {
            int j = e;
            while (j > 0 && ranks_before(key[e], e, key[order[j - 1]], order[j - 1])) {
                order[j] = order[j - 1];
                --j;
            }
            order[j] = e;
        }
        double sum = 0.0;
        for (int j = 0; j < k; ++j) sum += (double)s[order[j]];
        const int cut = top_p > 0.0f && top_p < 1.0f;
        volatile float mass = 0.0f;  /* float32 sums in rank order */
        for (int j = 0; j < k; ++j) mass = mass + s[order[j]];
        volatile float thr = top_p * mass;
        volatile float before = 0.0f;
        for (int j = 0; j < k; ++j) {
            const int keep = !cut || j == 0 || before < thr;
            before = before + s[order[j]];
            topk_ids[(size_t)t * k + j] = keep ? order[j] : -1;
            topk_w[(size_t)t * k + j] =
                !keep ? 0.0f
                      : normalize ? (float)((double)s[order[j]] / sum * scale)
                                  : (float)((double)s[order[j]] * scale);
        }
        free(key);
        free(order);
    }
}

/* ---- Union and the token -> expert permutation ------------------------- */

/* union_ids: the distinct routed ids in ascending order (n_union of them);
 * offsets[e] .. offsets[e+1]: the slice of perm holding expert e's
 * assignments a = t*k + j, in ascending a. Returns n_union. */
int oracle_union(const int32_t *topk_ids, int n_tokens, int k, int n_experts,
                 int32_t *union_ids, int32_t *offsets, int32_t *perm)
{
    int n_assign = n_tokens * k;
    int *cnt = (int *)calloc((size_t)n_experts, sizeof(int));
    int *cur = (int *)calloc((size_t)n_experts, sizeof(int));
    /* ids outside [0, n_experts) (a dropped slot is -1) are left out */
    for (int a = 0; a < n_assign; ++a)
        if (topk_ids[a] >= 0 && topk_ids[a] < n_experts) cnt[topk_ids[a]]++;
    int n_union = 0;
    for (int e = 0; e < n_experts; ++e)
        if (cnt[e]) union_ids[n_union++] = e;
    offsets[0] = 0;
    for (int e = 0; e < n_experts; ++e) offsets[e + 1] = offsets[e] + cnt[e];
    for (int a = 0; a < n_assign; ++a) {
        int e = topk_ids[a];
        if (e >= 0 && e < n_experts) perm[offsets[e] + cur[e]++] = a;
    }
    free(cnt);
    free(cur);
    return n_union;
}

/* ---- Learn ------------------------------------------------------------ */

void oracle_hit_count(const int32_t *topk_ids, int n_tokens, int k, int n_experts,
                      uint64_t *counters)
{
    for (int a = 0; a < n_tokens * k; ++a)
        if (topk_ids[a] >= 0 && topk_ids[a] < n_experts) counters[topk_ids[a]] += 1;
}

/* ---- Expert math ------------------------------------------------------- */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* One expert on T token vectors X[T][d] (double): O[T][d] = Wd (silu(Wg x) * (Wu x)).
 * Each weight row is dequantised once and used for all T tokens; every dot
 * product is a plain sum in index order (the T sums of a row advance together,
 * which leaves each one's order unchanged). */
void oracle_expert_mlp(const uint8_t *block, int d, int f, int wbits, int group,
                       const double *X, int T, double *O)
{
    block_view v = view_block(block, d, f, wbits, group);
    double *XT = (double *)malloc(sizeof(double) * (size_t)T * d); /* [d][T] */
    double *HT = (double *)malloc(sizeof(double) * (size_t)T * f); /* [f][T] */
    for (int t = 0; t < T; ++t)
        for (int i = 0; i < d; ++i) XT[(size_t)i * T + t] = X[(size_t)t * d + i];
#pragma omp parallel
    {
        double *wg = (double *)malloc(sizeof(double) * (size_t)d);
        double *wu = (double *)malloc(sizeof(double) * (size_t)d);
        double *g = (double *)malloc(sizeof(double) * (size_t)T);
        double *u = (double *)malloc(sizeof(double) * (size_t)T);
#pragma omp for schedule(static)
        for (int r = 0; r < f; ++r) {
            oracle_dequant_row(v.gate_q, v.gate_s, r, d, wbits, group, wg);
            oracle_dequant_row(v.up_q, v.up_s, r, d, wbits, group, wu);
            for (int t = 0; t < T; ++t) g[t] = u[t] = 0.0;
            for (int i = 0; i < d; ++i) {
                const double *xi = XT + (size_t)i * T;
                for (int t = 0; t < T; ++t) {
                    g[t] += wg[i] * xi[t];
                    u[t] += wu[i] * xi[t];
                }
            }
            for (int t = 0; t < T; ++t) HT[(size_t)r * T + t] = silu(g[t]) * u[t];
        }
        free(wg);
        free(wu);
        double *wd = (double *)malloc(sizeof(double) * (size_t)f);
#pragma omp for schedule(static)
        for (int r = 0; r < d; ++r) {
            oracle_dequant_row(v.down_q, v.down_s, r, f, wbits, group, wd);
            for (int t = 0; t < T; ++t) g[t] = 0.0;
            for (int i = 0; i < f; ++i) {
                const double *hi = HT + (size_t)i * T;
                for (int t = 0; t < T; ++t) g[t] += wd[i] * hi[t];
            }
            for (int t = 0; t < T; ++t) O[(size_t)t * d + r] = g[t];
        }
        free(wd);
        free(g);
        free(u);
    }
    free(XT);
    free(HT);
}

/* Expert forward of one layer for a batch of N tokens, given the routing.
 *   pool:  n_experts canonical blocks, `stride` bytes apart
 *   shared: the shared expert's block, or NULL
 *   y[N][d] (double) = shared(x_t) + sum_j w[t][j] * expert_{ids[t][j]}(x_t)
 * Each distinct routed expert is visited once (batch union) with all of its
 * assignments; the sum over slots runs in slot order. Returns 0, or -1 on a
 * bad expert id. */
int oracle_expert_forward(const uint8_t *pool, size_t stride, int n_experts,
                          const uint8_t *shared, int d, int f, int wbits, int group,
                          const float *x, int n_tokens, int k,
                          const int32_t *topk_ids, const float *topk_w, double *y)
{
    int n_assign = n_tokens * k;
    /* -1 marks a dropped slot (top-p cutoff): no expert, nothing added */
    for (int a = 0; a < n_assign; ++a)
        if (topk_ids[a] < -1 || topk_ids[a] >= n_experts) return -1;

    double *Xd = (double *)malloc(sizeof(double) * (size_t)n_tokens * d);
    for (size_t i = 0; i < (size_t)n_tokens * d; ++i) Xd[i] = (double)x[i];

    double *o = (double *)malloc(sizeof(double) * ((size_t)n_assign + 1) * d);
    int32_t *union_ids = (int32_t *)malloc(sizeof(int32_t) * n_experts);
    int32_t *offsets = (int32_t *)malloc(sizeof(int32_t) * (n_experts + 1));
    int32_t *perm = (int32_t *)malloc(sizeof(int32_t) * (n_assign + 1));
    int n_union = oracle_union(topk_ids, n_tokens, k, n_experts, union_ids, offsets, perm);

    double *Xg = (double *)malloc(sizeof(double) * ((size_t)n_assign + 1) * d);
    double *Og = (double *)malloc(sizeof(double) * ((size_t)n_assign + 1) * d);
    for (int ui = 0; ui < n_union; ++ui) {
        int e = union_ids[ui];
        int T = offsets[e + 1] - offsets[e];
        for (int i = 0; i < T; ++i) {
            int a = perm[offsets[e] + i];
            memcpy(Xg + (size_t)i * d, Xd + (size_t)(a / k) * d, sizeof(double) * d);
        }
        oracle_expert_mlp(pool + (size_t)e * stride, d, f, wbits, group, Xg, T, Og);
        for (int i = 0; i < T; ++i) {
            int a = perm[offsets[e] + i];
            memcpy(o + (size_t)a * d, Og + (size_t)i * d, sizeof(double) * d);
        }
    }
    free(Xg);
    free(Og);

    if (shared)
        oracle_expert_mlp(shared, d, f, wbits, group, Xd, n_tokens, y);
    else
        memset(y, 0, sizeof(double) * (size_t)n_tokens * d);
    for (int t = 0; t < n_tokens; ++t)
        for (int j = 0; j < k; ++j) {
            if (topk_ids[(size_t)t * k + j] < 0) continue;
            double w = (double)topk_w[(size_t)t * k + j];
            const double *oj = o + ((size_t)t * k + j) * d;
            double *yt = y + (size_t)t * d;
            for (int i = 0; i < d; ++i) yt[i] += w * oj[i];
        }

    free(Xd);
    free(o);
    free(union_ids);
    free(offsets);
    free(perm);
    return 0;
}

/* ---- Layer chaining for a stack of layers ----------------------------- */

/* a[t] = float32( h[t] / sqrt(mean_i h[t][i]^2 + eps) ), parameter-free RMS
 * normalisation used only to feed one layer's output to the next. */
void oracle_rms_normalize(const double *h, int n_tokens, int d, double eps, float *a)
{
    for (int t = 0; t < n_tokens; ++t) {
        const double *ht = h + (size_t)t * d;
        double ss = 0.0;
        for (int i = 0; i < d; ++i) ss += ht[i] * ht[i];
        double inv = 1.0 / sqrt(ss / d + eps);
        for (int i = 0; i < d; ++i) a[(size_t)t * d + i] = (float)(ht[i] * inv);
    }
}

/* ---- Place: a per-layer LRU cache of expert blocks -------------------- */

/* The pages' stage (3) Place loads the experts a batch is missing into a
 * faster tier and reuses the resident ones, with a per-layer LRU cache;
 * hot experts may be pinned from the hit counters, and the next layer's
 * experts may be prefetched ("Public Colibri Observation and Revision
 * Ledger", "Exact Architecture and Data-Flow Reconstruction" stage (3) and
 * "Cache/Prefetch Design Comparison"). The pages give no tie rule; the
 * reading here:
 *   - a call takes a list of expert ids; ids outside [0, n_experts) and
 *     repeats are ignored;
 *   - the call is refused (state unchanged, return -1) when its distinct
 *     experts not held by a pinned slot outnumber the unpinned slots;
 *   - the call's clock advances by one; every resident id is a hit and its
 *     slot's last use becomes the clock;
 *   - then, in list order, every missing id takes the slot with the
 *     smallest last use among the slots that are not pinned and not
 *     already taken by this call (never-used slots have last use 0; the
 *     lowest slot index among equals), evicting its expert.
 * State lives in caller arrays: expert_in[n_slots] (expert or -1),
 * last_use[n_slots], pinned[n_slots] (0/1), *clock. */
int oracle_cache_place(int n_slots, int n_experts, int32_t *expert_in, uint64_t *last_use,
                       const int32_t *pinned, uint64_t *clock, const int32_t *ids, int n,
                       int32_t *hits, int32_t *misses)
{
    int *seen = (int *)calloc((size_t)n_experts, sizeof(int));
    int *taken = (int *)calloc((size_t)n_slots, sizeof(int));
    int n_unpinned_slots = 0, need = 0;
    for (int s = 0; s < n_slots; ++s) n_unpinned_slots += !pinned[s];
    for (int i = 0; i < n; ++i) {
        int e = ids[i];
        if (e < 0 || e >= n_experts || seen[e]) continue;
        seen[e] = 1;
        int in_pinned = 0;
        for (int s = 0; s < n_slots; ++s)
            if (expert_in[s] == e && pinned[s]) in_pinned = 1;
        need += !in_pinned;
    }
    if (need > n_unpinned_slots) {
        free(seen);
        free(taken);
        return -1;
    }
    memset(seen, 0, sizeof(int) * (size_t)n_experts);
    *clock += 1;
    int h = 0, m = 0;
    for (int i = 0; i < n; ++i) {  /* hits */
        int e = ids[i];
        if (e < 0 || e >= n_experts || seen[e]) continue;
        for (int s = 0; s < n_slots; ++s)
            if (expert_in[s] == e) {
                seen[e] = 1;
                taken[s] = 1;
                last_use[s] = *clock;
                ++h;
            }
    }
    for (int i = 0; i < n; ++i) {  /* misses, in list order */
        int e = ids[i];
        if (e < 0 || e >= n_experts || seen[e]) continue;
        seen[e] = 1;
        int victim = -1;
        for (int s = 0; s < n_slots; ++s)
            if (!pinned[s] && !taken[s] && (victim < 0 || last_use[s] < last_use[victim]))
                victim = s;
        expert_in[victim] = e;
        taken[victim] = 1;
        last_use[victim] = *clock;
        ++m;
    }
    free(seen);
    free(taken);
    if (hits) *hits = h;
    if (misses) *misses = m;
    return 0;
}

/* Pin: the new pin set replaces the old one. A set of more distinct experts
 * than slots is refused (-1, nothing changed); otherwise every slot is
 * unpinned, the ids are placed as above and the slots holding them are
 * pinned. *misses = experts copied in. */
int oracle_cache_pin(int n_slots, int n_experts, int32_t *expert_in, uint64_t *last_use,
                     int32_t *pinned, uint64_t *clock, const int32_t *ids, int n,
                     int32_t *misses)
{
    int distinct = 0;
    for (int i = 0; i < n; ++i) {
        int dup = 0;
        if (ids[i] < 0 || ids[i] >= n_experts) continue;
        for (int j = 0; j < i; ++j) dup |= ids[j] == ids[i];
        distinct += !dup;
    }
    if (distinct > n_slots) return -1;
    for (int s = 0; s < n_slots; ++s) pinned[s] = 0;
    int32_t h = 0, m = 0;
    if (oracle_cache_place(n_slots, n_experts, expert_in, last_use, pinned, clock, ids, n, &h, &m))
        return -1;
    for (int i = 0; i < n; ++i)
        for (int s = 0; s < n_slots; ++s)
            if (ids[i] >= 0 && ids[i] < n_experts && expert_in[s] == ids[i]) pinned[s] = 1;
    if (misses) *misses = m;
    return 0;
}

/* Prefetch: place the longest prefix of ids whose distinct experts not held
 * by a pinned slot fit in the unpinned slots. *copied = experts copied in. */
void oracle_cache_prefetch(int n_slots, int n_experts, int32_t *expert_in, uint64_t *last_use,
                           const int32_t *pinned, uint64_t *clock, const int32_t *ids, int n,
                           int32_t *copied)
{
    int take = 0;
    for (int len = 1; len <= n; ++len) {
        /* does the prefix of this length fit? (count as oracle_cache_place) */
        int need = 0, room = 0;
        for (int s = 0; s < n_slots; ++s) room += !pinned[s];
        for (int i = 0; i < len; ++i) {
            int e = ids[i], dup = 0, in_pinned = 0;
            if (e < 0 || e >= n_experts) continue;
            for (int j = 0; j < i; ++j) dup |= ids[j] == e;
            if (dup) continue;
            for (int s = 0; s < n_slots; ++s)
                if (expert_in[s] == e && pinned[s]) in_pinned = 1;
            need += !in_pinned;
        }
        if (need > room) break;
        take = len;
    }
    int32_t h = 0, m = 0;
    oracle_cache_place(n_slots, n_experts, expert_in, last_use, pinned, clock, ids, take, &h, &m);
    if (copied) *copied = m;
}

/* The n experts with the most hits, most first, the lower id among equal
 * counts (the pages pin the experts their hit counters show hottest). */
void oracle_usage_hottest(const uint64_t *counters, int n_experts, int n, int32_t *ids)
{
    int *order = (int *)malloc(sizeof(int) * (size_t)n_experts);
    for (int e = 0; e < n_experts; ++e) {  /* insertion sort by (count desc, id asc) */
        int j = e;
        while (j > 0 && counters[order[j - 1]] < counters[e]) {
            order[j] = order[j - 1];
            --j;
        }
        order[j] = e;
    }
    for (int i = 0; i < n; ++i) ids[i] = order[i];
    free(order);
}
