/*
 * moe.h - C ABI of the routed-expert layer step on AMD Instinct MI355X (gfx950).
 *
 * One MoE layer of a GLM-5.2-shaped model, as the Colibri pages state it
 * ("Public Colibri Observation and Revision Ledger", section "Exact
 * Architecture and Data-Flow Reconstruction"): per layer and batch,
 * (1) Route: a float32 sigmoid gate scores every expert (n_group = 1) and the
 *     top-k experts are selected,
 * (2) Union: requests of the batch are merged so each distinct expert is used
 *     once (same page, "Cache/Prefetch Design Comparison", figure on async
 *     I/O and prefetch: "batch-union"),
 * (5) Learn: per-expert hit counters are bumped,
 * and the expert math: each chosen expert is a three-matrix MLP, plus an
 * always-on shared expert. The experts sit in an HBM-resident pool; the
 * pages' Place and Overlap stages (disk, RAM and VRAM tiers) have no
 * counterpart here because every expert is resident.
 *
 * Readings where the pages are silent:
 *   score      s[t][e] = sigmoid(b[e] + sum_i Wr[e][i] x[t][i]), float32
 *   top-k      k largest s per token, ties to the lower expert id, ids in rank
 *              order; the gate weight of a slot is its raw score
 *   expert     o = Wd (silu(Wg x) * (Wu x)), silu(z) = z / (1 + exp(-z))
 *   weights    W[r][c] = q[r][c] * scale[r][c / G] (symmetric codes)
 *   combine    y[t] = shared(x_t) + sum_j w[t][j] * o_{t,j}
 *   counters   counters[e] += number of (token, slot) assignments to e
 *
 * Conventions for every call:
 *   - Array arguments are DEVICE pointers unless marked (host). The caller
 *     owns every buffer; the library allocates nothing and keeps no state
 *     between calls. Calls on different streams with disjoint outputs may
 *     run concurrently.
 *   - Calls enqueue work on `stream` and return without synchronising.
 *     n_union and the permutation stay on the device; moe_expert_forward
 *     reads them there, so a layer step needs no host round trip.
 *   - Arguments are checked on the host before any HIP call. A failed check
 *     returns a negative moe_status and enqueues nothing. A launch failure
 *     returns MOE_EHIP. Faults during execution surface at the caller's next
 *     synchronisation. After an error the outputs are unspecified.
 *   - n_tokens == 0 is a successful no-op.
 *   - Row-major layouts throughout. x is [n_tokens][d_model] float32.
 *   - Arithmetic of the expert kernels (routing, SiLU and the combine are
 *     float32 throughout):
 *       GEMV pass (experts with one or a few tokens): each run of 32 (int4)
 *       or 16 (int8) consecutive activations is scaled by the power of two
 *       that brings its largest magnitude into [2^13, 2^14) and rounded to a
 *       16-bit integer; the products with the codes are exact integer dot
 *       products (v_dot8c_i32_i4 on four base-16 digit planes, or
 *       v_dot4c_i32_i8 on two base-256 planes), scaled in float32 per run.
 *       Matrix-core passes (groups of tokens): x and the hidden values are
 *       rounded to float16, unscaled, and multiplied with float16 codes on
 *       v_mfma_f32_16x16x32_f16 with float32 accumulation. The group scale is
 *       applied to the float32 products of each 128-column step when the
 *       scale groups cover whole 128-column units (G == 0 or a multiple of
 *       128); otherwise (and on the 128-token pass) code * scale is rounded
 *       to float16 before the product, so such scales must be normal float16
 *       values (2^-14 <= scale <= 65504; the host does not check this).
 *     Inputs must be finite, and |x| and every hidden value |silu(g) * u|
 *     must stay below 65504, which holds with a wide margin for normalised
 *     activations.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,          /* null pointer, negative size, bad k, bad wbits */
    MOE_ESHAPE = -2,          /* shape the kernels do not support (see below) */
    MOE_EALIGN = -3,          /* pointer or stride not aligned as required */
    MOE_EWORKSPACE = -4,      /* workspace missing or smaller than required */
    MOE_EHIP = -5,            /* a HIP runtime call or kernel launch failed */
    MOE_EIO = -6              /* a file could not be read or written, or is not a usage file */
} moe_status;

#define MOE_MAX_K 32          /* largest top-k */
#define MOE_MAX_EXPERTS 1024  /* largest number of routed experts per layer */
#define MOE_ALIGN 256         /* alignment of pools, blocks and workspaces */

/*
 * One layer's expert pool (the struct itself is host memory; the blocks are
 * device memory).
 *
 * Block format. The Colibri pages store an expert's three matrices next to
 * each other and read them as one block ("Storage, Memory, and I/O Formulas";
 * README "Never wait for the disk twice"); their container is int4 with
 * group scales (README "Get started") and the draft head is int8 (README
 * "Speculative decoding, honestly").
 *
 * Canonical block (the input of moe_pack_expert), in order:
 *   gate codes [f][d], up codes [f][d], down codes [d][f]   (row-major)
 *   gate scales [f][d/G], up scales [f][d/G], down scales [d][f/G] (float32)
 * with f = d_ff, d = d_model and G = group (G == 0: one scale per row).
 * Codes are two's-complement wbits-bit integers; int4 packs element 2i in
 * the low nibble of byte i.
 *
 * Device block (what the pool holds): the same sections at the same
 * offsets, rearranged for the kernels. Each code matrix [R][K] is cut into
 * 1024-byte units of 16 rows x U columns (U = 128 for int4, 64 for int8),
 * stored by unit row then unit column: unit (rt, kb) at byte offset
 * (rt * K/U + kb) * 1024 of the matrix. Slot L = r + 16 q (r = 0..15,
 * q = 0..3) of a unit holds bytes 16 L .. 16 L + 15: the 16 canonical bytes
 * of row 16 rt + r covering columns kb U + q U/4 .. + U/4, with the codes
 * made offset-binary (code + 8 per nibble, code + 128 per byte). Each scale
 * matrix [R][groups] becomes [R/16][groups][16]. moe_pack_expert writes this
 * layout; moe_block_bytes is the same for both.
 *
 * Supported shapes: wbits 4 or 8; d and f multiples of 128 (int4) or 64
 * (int8), at most 16384; G == 0 or G a multiple of 32 (int4) or 16 (int8)
 * dividing both d and f; pool, shared and expert_bytes multiples of
 * MOE_ALIGN, expert_bytes >= moe_block_bytes(...).
 */
typedef struct {
    int32_t d_model;
    int32_t d_ff;
    int32_t n_experts;        /* routed experts, 1..MOE_MAX_EXPERTS */
    int32_t wbits;            /* 4 or 8 */
    int32_t group;            /* scale group along the input dimension; 0 = per row */
    const void *pool;         /* n_experts blocks, expert_bytes apart */
    size_t expert_bytes;      /* block stride */
    const void *shared;       /* the shared expert's block, or NULL for none */
    /* NULL: routed expert e's block is at pool + e * expert_bytes. Otherwise
     * (device, [n_experts] int32, a pool held partly in HBM, see moe_cache.h)
     * its block is at pool + slot_of[e] * expert_bytes, pool holding n_slots
     * blocks; every expert a call uses must then have a slot (slot values
     * are clamped into [0, n_slots) before use, so a wrong table gives wrong
     * results, never an access outside the pool). */
    const int32_t *slot_of;
    int32_t n_slots;
} moe_expert_pool;

/*
 * Route. scores = sigmoid(x Wr^T + b) in float32, then per token the k best
 * experts: topk_ids [n_tokens][k] int32 in rank order (ties to the lower id;
 * a NaN score ranks above every number) and topk_w [n_tokens][k] float32,
 * the chosen scores. Batches above 16 tokens sum the router products in up to
 * 16 slices of the contraction (partial sums in the workspace, added in
 * slice order before the sigmoid).
 *   w_router [n_experts][d_model] float32; b_router [n_experts] or NULL.
 *   d_model must be a multiple of 32; x and w_router 16-byte aligned.
 *   workspace: at least moe_route_workspace_size(n_tokens, n_experts) bytes,
 *   MOE_ALIGN-aligned.
 * Colibri pages: "Exact Architecture and Data-Flow Reconstruction" (sigmoid
 * router, n_group = 1, float32 gate parameters).
 */
moe_status moe_route_topk(const float *x, int n_tokens, int d_model,
                          const float *w_router, const float *b_router,
                          int n_experts, int k,
                          int32_t *topk_ids, float *topk_w,
                          void *workspace, size_t ws_bytes, hipStream_t stream);

/*
 * Union and permutation of the batch's n_tokens*k assignments a = t*k + j.
 *   union_ids [n_experts]: the distinct routed ids ascending (first *n_union
 *   entries valid); n_union [1]; expert_offsets [n_experts+1]: exclusive
 *   prefix of the per-expert counts; perm [n_tokens*k]: the assignments
 *   grouped by expert, expert_offsets[e] .. expert_offsets[e+1] holding
 *   expert e's assignments in ascending a (a stable counting sort, so the
 *   result does not depend on thread timing). Ids outside [0, n_experts) are
 *   left out of every output.
 * Colibri pages: "Exact Architecture and Data-Flow Reconstruction", stage (2)
 * Union; "Cache/Prefetch Design Comparison", batch-union.
 */
moe_status moe_union(const int32_t *topk_ids, int n_tokens, int k, int n_experts,
                     int32_t *union_ids, int32_t *n_union,
                     int32_t *expert_offsets, int32_t *perm, hipStream_t stream);

/*
 * Route, Union and (when counters is not NULL) Learn of one layer in one call:
 * the same outputs as moe_route_topk, then moe_union, then moe_hit_count on
 * the same arguments (same checks, nothing enqueued on an error). Batches of
 * up to 16 tokens take the top-k, the union and the counting in a single
 * workgroup after the router kernel (two kernel launches instead of four);
 * from 4096 assignments the union and counting run over several workgroups,
 * with the workspace (whose router output the top-k has consumed by then) as
 * scratch. workspace: at least moe_route_workspace_size(n_tokens, n_experts)
 * bytes; its contents afterwards are unspecified.
 * Colibri pages: "Exact Architecture and Data-Flow Reconstruction", stages
 * (1) Route, (2) Union and (5) Learn.
 */
moe_status moe_route_union(const float *x, int n_tokens, int d_model,
                           const float *w_router, const float *b_router,
                           int n_experts, int k,
                           int32_t *topk_ids, float *topk_w,
                           int32_t *union_ids, int32_t *n_union,
                           int32_t *expert_offsets, int32_t *perm,
                           uint64_t *counters /* may be NULL */,
                           void *workspace, size_t ws_bytes, hipStream_t stream);

/*
 * Router variant (opt-in). The pages give a sigmoid gate over all experts
 * with n_group = 1 and float32 gate parameters ("Exact Architecture and
 * Data-Flow Reconstruction") and leave open where the bias enters and whether
 * the chosen weights are rescaled; the calls above read them as a bias inside
 * the sigmoid and the raw score as the weight. The _ex calls take the other
 * reading on request:
 *   bias_select_only = 1: scores s = sigmoid(x Wr^T) without the bias; the
 *     top-k key of expert e is the float32 sum s[e] + b_router[e] (ties to
 *     the lower id), the weight stays s;
 *   normalize = 1: each chosen weight is divided by the sum of the token's
 *     k chosen scores (added in rank order);
 *   scale: multiplies every chosen weight (after normalising), > 0 and
 *     finite; 1 leaves the weights as they are;
 *   top_p: a lossy cutoff (the pages mention a top-p option that trades
 *     accuracy for speed without defining it), off at 0 or >= 1. With S the
 *     float32 sum of the token's k chosen scores in rank order, slot j is kept
 *     when j == 0 or the float32 sum of the scores ranked before it is below
 *     top_p * S; a dropped slot gets topk_ids -1 and topk_w 0, and the union,
 *     the permutation, the hit counts and moe_expert_forward leave it out.
 * opt == NULL is the default reading (the same results as the calls above).
 * A bad option is MOE_EINVAL before anything is enqueued; b_router must be
 * 4-byte aligned.
 */
typedef struct {
    int32_t bias_select_only; /* 0 or 1 */
    int32_t normalize;        /* 0 or 1 */
    float scale;              /* weight multiplier */
    float top_p;              /* 0: no cutoff */
} moe_route_options;

moe_status moe_route_topk_ex(const float *x, int n_tokens, int d_model,
                             const float *w_router, const float *b_router,
                             int n_experts, int k,
                             int32_t *topk_ids, float *topk_w,
                             void *workspace, size_t ws_bytes, hipStream_t stream,
                             const moe_route_options *opt);

moe_status moe_route_union_ex(const float *x, int n_tokens, int d_model,
                              const float *w_router, const float *b_router,
                              int n_experts, int k,
                              int32_t *topk_ids, float *topk_w,
                              int32_t *union_ids, int32_t *n_union,
                              int32_t *expert_offsets, int32_t *perm,
                              uint64_t *counters /* may be NULL */,
                              void *workspace, size_t ws_bytes, hipStream_t stream,
                              const moe_route_options *opt);

/*
 * Expert math and combine:
 *   y[t] = shared(x_t) + sum_{j<k} topk_w[t][j] * E_{e(t,j)}(x_t),
 *   E(x) = Wd (silu(Wg x) * (Wu x)),
 * over the union produced by moe_union (union_ids, n_union, expert_offsets,
 * perm are its outputs for the same n_tokens and k). topk_w is an input, so a
 * caller may inject gate weights; a slot with weight 0 adds nothing, and a
 * slot left out of the permutation (an id outside [0, n_experts), such as a
 * slot the top-p cutoff dropped) must have weight 0. Each distinct expert's
 * weights are streamed
 * from HBM once per work item: single tokens on GEMV kernels, groups of up to
 * 32 or 128 tokens on the matrix cores (see moe_expert_forward_ex). y
 * [n_tokens][d_model] float32 is overwritten. workspace: at least
 * moe_forward_workspace_size(pool, n_tokens, k) bytes, MOE_ALIGN-aligned.
 * Colibri pages: "Exact Architecture and Data-Flow Reconstruction" (three-
 * matrix expert MLP, always-on shared expert); README "Get started" (int4
 * group-scaled experts).
 */
moe_status moe_expert_forward(const moe_expert_pool *pool /* (host) */,
                              const float *x, int n_tokens, int k,
                              const float *topk_w,
                              const int32_t *union_ids, const int32_t *n_union,
                              const int32_t *expert_offsets, const int32_t *perm,
                              float *y, void *workspace, size_t ws_bytes,
                              hipStream_t stream);

/*
 * moe_expert_forward with options (options may be NULL: same as
 * moe_expert_forward). Each expert of the call is computed by one of three
 * passes, chosen by its number of tokens T in the batch (the shared expert
 * by n_tokens):
 *   T >= mfma_min_tokens: grouped GEMM on the matrix cores, 128-token tiles;
 *     0 selects the default (32), a negative value turns this pass off;
 *   mfma_small_min_tokens <= T < mfma_min_tokens: the same kernels with
 *     32-token tiles; 0 selects the default (1: every expert not on the
 *     128-token pass; off for batches of up to 2 tokens, which the GEMV
 *     takes in one item per expert), negative turns it off;
 *   otherwise: the streaming GEMV kernels.
 * When both matrix-core passes are on, a group on the 128-token pass whose
 * last item would hold at most 32 tokens past a full one gives those tokens
 * to the 32-token pass (a 128-token item computes all of its tile), and
 * when the 128-token pass would get fewer than 32 items, those experts join
 * the 32-token pass (a few large items
 * would otherwise run with a few workgroups each); when n_tokens and k alone
 * bound it below 32 items, or (default thresholds) n_tokens * k is below
 * 32 * 128, the 128-token kernels are not launched at all.
 * The matrix-core passes take int4 and int8 layers alike (every supported
 * shape is a whole number of 1 KB code units per row).
 * events: each non-NULL event is taken by the dispatch of the kernel it
 *   names (hipExtLaunchKernelGGL), at that kernel's start or end. Events are
 *   created and owned by the caller; a kernel that a call does not launch
 *   leaves its events untouched.
 * The results agree with moe_expert_forward to the library's tolerance for
 * every choice of thresholds (bit for bit when the same kernels are chosen).
 */
typedef struct {
    hipEvent_t gateup_start, gateup_end;              /* GEMV gate/up kernel */
    hipEvent_t down_start, down_end;                  /* GEMV down kernel */
    hipEvent_t mfma_gateup_start, mfma_gateup_end;    /* 128-token matrix-core gate/up */
    hipEvent_t mfma_down_start, mfma_down_end;        /* 128-token matrix-core down */
    hipEvent_t small_gateup_start, small_gateup_end;  /* 32-token matrix-core gate/up */
    hipEvent_t small_down_start, small_down_end;      /* 32-token matrix-core down */
    int32_t mfma_min_tokens;
    int32_t mfma_small_min_tokens;
} moe_forward_options;

moe_status moe_expert_forward_ex(const moe_expert_pool *pool /* (host) */,
                                 const float *x, int n_tokens, int k,
                                 const float *topk_w,
                                 const int32_t *union_ids, const int32_t *n_union,
                                 const int32_t *expert_offsets, const int32_t *perm,
                                 float *y, void *workspace, size_t ws_bytes,
                                 hipStream_t stream,
                                 const moe_forward_options *options /* (host) */);

/*
 * Learn: counters[e] += #{(t, j) : topk_ids[t][j] == e}, uint64, accumulated
 * in place (device atomics, so concurrent calls on one counter table add up).
 * The shared expert is not counted. Ids outside [0, n_experts) are ignored.
 * Colibri pages: "Exact Architecture and Data-Flow Reconstruction", stage (5)
 * Learn: per-expert hit counters.
 */
moe_status moe_hit_count(const int32_t *topk_ids, int n_tokens, int k, int n_experts,
                         uint64_t *counters, hipStream_t stream);

/*
 * Residual chaining of stacked layers (not one of the pages' stages; the
 * pages keep layer norms resident in float32 and give no formula):
 *   h[t] += y[t] (skipped when y is NULL), then
 *   a[t] = h[t] / sqrt(mean_i h[t][i]^2 + eps).
 * h, y, a are [n_tokens][d_model] float32; a may not alias h.
 */
moe_status moe_residual_rmsnorm(float *h, const float *y, float *a, int n_tokens,
                                int d_model, float eps, hipStream_t stream);

/*
 * A whole layer step in one call: moe_route_union (router bias inside the
 * sigmoid, no options) followed by moe_expert_forward, with the same
 * arguments, checks (all made before anything is enqueued) and outputs, bit
 * for bit; d_model must equal pool->d_model and the router has
 * pool->n_experts rows. counters may be NULL. For one or two tokens with
 * k <= 2 whose experts all stay on the GEMV pass (the default thresholds),
 * the top-k, union, permutation and counting run inside the gate/up GEMV
 * launch: every workgroup of a routed expert takes the top-k of the router's
 * scores itself and workgroup 0 writes the routing outputs, so a decode step
 * is three launches (router, gate/up, down; a combine after them when an
 * output row has more than two terms) instead of four or five. At larger k
 * the argmax rounds every workgroup would run cost more than the launch they
 * save, and the two calls' kernels run. workspace: at least
 * moe_layer_step_workspace_size(pool, n_tokens, k) bytes, 256-byte aligned
 * (the router's output, then the expert step's workspace); its contents
 * afterwards are unspecified. opt (host, may be NULL): as for
 * moe_expert_forward_ex (events around the expert kernels, pass thresholds);
 * a threshold that moves an expert to the matrix cores makes the step take
 * the two calls' kernels.
 * Colibri pages: "Exact Architecture and Data-Flow Reconstruction", stages
 * (1) Route, (2) Union and (5) Learn, and the three-matrix expert MLP with
 * the always-on shared expert.
 */
moe_status moe_layer_step(const moe_expert_pool *pool /* (host) */, const float *x,
                          int n_tokens, int d_model, const float *w_router,
                          const float *b_router, int k, int32_t *topk_ids, float *topk_w,
                          int32_t *union_ids, int32_t *n_union, int32_t *expert_offsets,
                          int32_t *perm, uint64_t *counters, float *y, void *workspace,
                          size_t ws_bytes, hipStream_t stream,
                          const moe_forward_options *opt /* (host) */);

/*
 * moe_layer_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). The workspace is a fixed array of
 * MOE_SCRATCH_BYTES in the library's own device memory, one per GPU, held
 * until the process ends; the call allocates nothing. Same arguments (minus
 * workspace and ws_bytes), checks, kernels and outputs as moe_layer_step.
 * A step whose moe_layer_step_workspace_size exceeds MOE_SCRATCH_BYTES is
 * rejected with MOE_EWORKSPACE before any HIP call (at the GLM-5.2 shapes,
 * d_model 6144, d_ff 2048, 256 experts: up to 128 tokens at top-8, 256
 * tokens at top-1). Every call on one GPU shares that GPU's array and leaves
 * its contents behind (the step reads nothing it has not written in the same
 * call): calls that overlap on one GPU (other streams or threads) race and
 * must be ordered by the caller. MOE_EHIP if the array's device address
 * cannot be found (first call on a device).
 */
#define MOE_SCRATCH_BYTES ((size_t)64 << 20)

moe_status moe_layer_step_noalloc(const moe_expert_pool *pool /* (host) */, const float *x,
                                  int n_tokens, int d_model, const float *w_router,
                                  const float *b_router, int k, int32_t *topk_ids,
                                  float *topk_w, int32_t *union_ids, int32_t *n_union,
                                  int32_t *expert_offsets, int32_t *perm, uint64_t *counters,
                                  float *y, hipStream_t stream,
                                  const moe_forward_options *opt /* (host) */);

/*
 * A stack of layers chained through a residual stream, in one call. The
 * pages keep the dense layers (attention, norms) out of the expert path and
 * give no formula for joining the MoE layers; the reading here is a pre-norm
 * residual with a parameter-free RMS norm: for l = 0 .. n_layers-1,
 *   a = h / sqrt(mean_i h[i]^2 + eps),  y = layer_l(a),  h += y,
 * each layer_l a moe_layer_step (router bias inside the sigmoid, top-k,
 * union, counters, experts, combine) with its own pool, router and hit
 * counters. This is the path of a stack workload and of the speculative
 * decoding flow: draft steps through the int8 draft-head layer, then the
 * 1 + D token verify batch through the main layers with the same kernels
 * (Colibri README, "Speculative decoding, honestly").
 *   layers (host) [n_layers]: every pool with the same d_model and
 *     n_experts; w_router [n_experts][d_model] (16-byte aligned),
 *     b_router [n_experts] or NULL, counters [n_experts] uint64 (8-byte
 *     aligned) or NULL (device pointers).
 *   h [n_tokens][d_model] float32 (device, 16-byte aligned): the stack's
 *     input, overwritten with its output.
 *   topk_ids_out (device [n_layers][n_tokens][k] int32, or NULL): each
 *     layer's expert ids.
 *   workspace: moe_stack_workspace_size(layers, n_layers, n_tokens, k) bytes,
 *     MOE_ALIGN-aligned; its contents afterwards are unspecified.
 * Every layer's checks are made before anything is enqueued.
 */
typedef struct {
    moe_expert_pool pool;
    const float *w_router;
    const float *b_router;
    uint64_t *counters;
} moe_layer_desc;

moe_status moe_stack_forward(const moe_layer_desc *layers /* (host) */, int n_layers,
                             int n_tokens, int k, float eps, float *h, int32_t *topk_ids_out,
                             void *workspace, size_t ws_bytes, hipStream_t stream);

/* Workspace of moe_stack_forward (0 for invalid arguments). */
size_t moe_stack_workspace_size(const moe_layer_desc *layers /* (host) */, int n_layers,
                                int n_tokens, int k);

/* Workspace sizes in bytes (host-only arithmetic, no HIP calls). */
size_t moe_route_workspace_size(int n_tokens, int n_experts);
size_t moe_forward_workspace_size(const moe_expert_pool *pool, int n_tokens, int k);
/* The larger of the two, for one buffer shared by a layer step's calls. */
size_t moe_workspace_size(const moe_expert_pool *pool, int n_tokens, int k);
/* The sum of the two (0 for invalid arguments): moe_layer_step's workspace. */
size_t moe_layer_step_workspace_size(const moe_expert_pool *pool, int n_tokens, int k);

/* Bytes of one expert block (same for the canonical and device layouts). */
size_t moe_block_bytes(int d_model, int d_ff, int wbits, int group);

/*
 * (host) Converts one canonical block (two's-complement codes, layout as
 * above) into the device layout. Both buffers are host memory of
 * moe_block_bytes(...) bytes; they may be the same buffer.
 */
moe_status moe_pack_expert(const void *canonical_block, const moe_expert_pool *shape,
                           void *block_out);

/* Static text for a status code. */
const char *moe_strerror(moe_status status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
