// internal.h - shared declarations of the routed-expert library (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;

// One unit of expert work: up to TB consecutive positions p0 .. p0+count-1 of
// one expert's slice of the permutation (expert >= 0), or of the shared
// expert (expert == -1), whose positions are A + t for token t.
struct Item {
    int32_t expert;
    int32_t p0;
    int32_t count;
    int32_t pad;
};

// Geometry of one layer's expert blocks, resolved and checked on the host.
//
// Device block layout. Each code matrix [R rows][K columns] is cut into
// 1 KB units of 16 rows x U columns (U = 128 int4 codes or 64 int8 codes
// per row), stored unit-row by unit-row: unit (rt, kb) at byte
// (rt * (K / U) + kb) * 1024. Inside a unit, lane slot L = r + 16 q (r the
// row within the unit, q = 0..3) holds the 16 bytes of row 16 rt + r that
// cover columns kb * U + q * U/4 .. + U/4, in canonical byte order with
// offset-binary codes. One 16-byte load per lane of a wave reads one whole
// unit, which is also the weight operand of four (int4) or two (int8)
// 16x16x32 MFMA steps. Scales of a matrix: [R / 16][groups per row][16]
// float32, so the 16 rows of a unit read one 64-byte run per group.
struct Geo {
    int d, f, E, wbits, group;
    int epc;                 // codes per 16-byte lane chunk (32 int4, 16 int8)
    int ucols;               // columns per unit = 4 * epc
    int kb_gu, kb_dn;        // units along a gate/up row (d / ucols), a down row (f / ucols)
    int ng_gu, ng_dn;        // scale groups per gate/up row (d / G or 1), per down row
    long long off_up, off_dn, off_gs, off_us, off_ds;  // byte offsets in a block
};

constexpr int kUnitRows = 16;
constexpr int kMaxModelDim = 16384;  // largest d_model or d_ff
constexpr int kUnitBytes = 1024;

// Everything the expert kernels of one moe_expert_forward call need.
struct Fwd {
    Geo g;
    const uint8_t *pool;
    size_t stride;
    const int32_t *slot_of;  // null, or the block slot of each routed expert
    int n_slots;             // blocks in the pool when slot_of is not null
    const uint8_t *shared;
    const float *x;          // [N][d] layer input
    const float *w;          // [N][k] gate weights
    int k, N, A, has_shared; // A = N * k assignments
    const int32_t *union_ids, *n_union, *offsets, *perm;  // moe_union outputs
    float *h;                // [A + N][f] hidden of the GEMV pass (workspace)
    float *o;                // [A + N][d] expert outputs (workspace)
    // float16 operands of the matrix-core passes (workspace), each 8-column
    // group in the order the MFMA weight operand takes its codes:
    uint16_t *x16;           // [N][d] layer input
    uint16_t *h16;           // [A + N][f] hidden
    float *y;                // [N][d] layer output
    // Two-phase forward (the cache's Overlap): when phase is not null, the
    // expert kernels compute only the items of routed experts e with
    // phase[e] == phase_sel, and of the shared expert when phase_sel == 0;
    // the other workgroups leave at once.
    const uint8_t *phase;    // [E] 0 or 1, or null: every item
    int phase_sel;
    int direct;              // 1: the GEMV down kernel adds the gate-weighted rows into y
                             // itself (at most two addends per element, y cleared by
                             // the gate/up kernel); 0: the combine kernel writes y
    // One-token layer step (moe_layer_step): when route_in is not null the
    // gate/up GEMV kernel takes the top-k of the router's output itself, and
    // workgroup 0 writes the top-k (route_ids, route_w = w), the union,
    // offsets, permutation (into union_ids, n_union, offsets, perm) and the
    // hit counts; the down kernel reads them after the launch boundary.
    const float *route_in;   // router output: P slices of [E] (P = 1: final scores)
    int route_P;
    const float *route_b;    // router bias (used when P > 1), may be null
    int32_t *route_ids;      // [k]
    float *route_w;          // [k], the same buffer as w
    unsigned long long *route_counters;  // [E] or null
    Item *items;             // [max_items] work list (workspace)
    int32_t *n_items;        // [1]
    int tb;                  // tokens per GEMV work item
    int max_items;           // host bound of the number of GEMV items
    Item *mitems;            // [max_mitems] MFMA work list, 128-token items (workspace)
    int32_t *n_mitems;       // [1]
    int max_mitems;          // host bound of the number of 128-token items (0: no such pass)
    int tstar;               // experts with at least this many tokens use 128-token items
    Item *sitems;            // [max_sitems] MFMA work list, 32-token items (workspace)
    int32_t *n_sitems;       // [1]
    int max_sitems;          // host bound of the number of 32-token items (0: no such pass)
    int tsmall;              // experts with tsmall <= tokens < tstar use 32-token items
    hipEvent_t ev_gu[2];     // optional: taken at the GEMV gate/up kernel's start and end
    hipEvent_t ev_dn[2];     // optional: the same for the GEMV down kernel
    hipEvent_t ev_mgu[2];    // optional: the same for the 128-token MFMA gate/up kernel
    hipEvent_t ev_mdn[2];    // optional: the same for the 128-token MFMA down kernel
    hipEvent_t ev_sgu[2];    // optional: the same for the 32-token MFMA gate/up kernel
    hipEvent_t ev_sdn[2];    // optional: the same for the 32-token MFMA down kernel
};

// Whether the current phase computes the item of this expert (-1: shared).
__device__ __forceinline__ bool in_phase(const Fwd &f, int expert)
{
    if (!f.phase) return true;
    return (expert >= 0 ? (int)f.phase[expert] : 0) == f.phase_sel;
}

// Block of routed expert e (0 <= e < E): its own place in the pool, or the
// slot the expert cache gave it.
__device__ __forceinline__ const uint8_t *expert_block(const Fwd &f, int e)
{
    const int s = f.slot_of ? min(max(f.slot_of[e], 0), f.n_slots - 1) : e;
    return f.pool + (size_t)s * f.stride;
}

// ---- host helpers (abi.hip) --------------------------------------------
moe_status resolve_geo(const moe_expert_pool *p, Geo *g);
// Every check of moe_layer_step on these arguments, nothing enqueued.
moe_status layer_step_check(const moe_expert_pool *pool, const float *x, int n_tokens, int d_model,
                            const float *w_router, const float *b_router, int k,
                            int32_t *topk_ids, float *topk_w, int32_t *union_ids,
                            int32_t *n_union, int32_t *expert_offsets, int32_t *perm,
                            uint64_t *counters, float *y, void *workspace, size_t ws_bytes);
// The residual stream of a layer stack: a layer step given one may end with
// h += y and a = rms_norm(h, eps) in its combine launch (y is then not
// written) and says so in *normed.
struct StackNorm {
    float *h;
    float *a;
    float eps;
};
moe_status layer_step_norm(const moe_expert_pool *pool, const float *x, int n_tokens, int d_model,
                           const float *w_router, const float *b_router, int k,
                           int32_t *topk_ids, float *topk_w, int32_t *union_ids,
                           int32_t *n_union, int32_t *expert_offsets, int32_t *perm,
                           uint64_t *counters, float *y, void *workspace, size_t ws_bytes,
                           hipStream_t stream, const StackNorm *sn, bool *normed);
// moe_expert_forward restricted to one phase of a two-phase forward (see
// Fwd::phase): phase_sel 0 computes the experts with phase[e] == 0 and the
// shared expert, 1 the others and then the combine. check_only: the
// argument checks alone, nothing enqueued.
moe_status expert_forward_phase(const moe_expert_pool *pool, const float *x, int n_tokens, int k,
                                const float *topk_w, const int32_t *union_ids,
                                const int32_t *n_union, const int32_t *expert_offsets,
                                const int32_t *perm, float *y, void *workspace, size_t ws_bytes,
                                hipStream_t stream, const uint8_t *phase, int phase_sel,
                                bool check_only);

// ---- launchers (each in its own translation unit) ----------------------
// Router: final scores [N][E], or raw partial sums [P][N][E] over P slices of
// the contraction (P = router_slices(N, d, E)) that launch_topk adds up.
int router_slices_bound(int N, int E);   // the largest P any d can give
int router_slices(int N, int d, int E);
hipError_t launch_router(const float *x, int N, int d, const float *wr, const float *b,
                         int E, float *out, hipStream_t s);
struct TopkOpt;
hipError_t launch_topk(const float *in, int P, const float *b, int N, int E, int k,
                       int32_t *ids, float *w, hipStream_t s, TopkOpt opt);
// union and permutation in one workgroup; counters (may be null) += the counts
hipError_t launch_union(const int32_t *ids, int A, int E, int32_t *union_ids, int32_t *n_union,
                        int32_t *offsets, int32_t *perm, uint64_t *counters, hipStream_t s);
hipError_t launch_hit_count(const int32_t *ids, int A, int E, uint64_t *counters, hipStream_t s);
// Top-k, union and hit counting of a batch of at most route_tail_max_tokens()
// tokens in one workgroup (counters may be null).
int route_tail_max_tokens();
// Union, permutation and (counters not null) hit counts of a large batch
// over several workgroups, with scratch of at least E * 4 bytes (more allows
// more chunks); the same outputs as launch_union + launch_hit_count.
int union_chunks(int A, int E, size_t scratch_bytes);
hipError_t launch_union_chunked(const int32_t *ids, int A, int E, int32_t *union_ids,
                                int32_t *n_union, int32_t *offsets, int32_t *perm,
                                uint64_t *counters, void *scratch, size_t scratch_bytes,
                                hipStream_t s);
hipError_t launch_route_tail(const float *in, int P, const float *b, int N, int E, int k,
                             int32_t *ids, float *w, int32_t *union_ids, int32_t *n_union,
                             int32_t *offsets, int32_t *perm, uint64_t *counters, hipStream_t s,
                             TopkOpt opt);
int gemv_tokens_per_item(const Geo &g, int n_tokens);
// The GEMV gate/up pass and, when a planning launch is needed, that launch
// first; *x16_staged: whether it also wrote x16 (the matrix-core passes').
hipError_t launch_gateup(const Fwd &f, hipStream_t s, bool *x16_staged);
hipError_t launch_down(const Fwd &f, hipStream_t s);
bool mfma_supported(const Geo &g);
constexpr int kMfmaBigTokens = 128;   // tokens per item of the large-group MFMA pass
constexpr int kMfmaSmallTokens = 32;  // tokens per item of the small-group MFMA pass
// fewer 128-token items than this go to the 32-token pass (when both run)
constexpr int kMinBigItems = 32;
// small = false: the 128-token items (mitems), true: the 32-token items (sitems)
hipError_t launch_mfma(const Fwd &f, bool gateup, bool small, hipStream_t s);
// x -> x16 for the matrix-core passes (launch_gateup does it in the
// planning launch when that runs; launch_stage_x16 on its own otherwise)
hipError_t launch_stage_x16(const Fwd &f, hipStream_t s);
hipError_t launch_combine(const float *o, const float *w, int N, int k, int d, int A,
                          int has_shared, float *y, hipStream_t s);
hipError_t launch_residual_rmsnorm(float *h, const float *y, float *a, int N, int d, float eps,
                                   hipStream_t s);
// The combine followed by the residual norm of a layer stack (h += y, a =
// rms_norm(h), y not written), when the rows take the register-resident norm.
bool combine_norm_supported(int d, const float *h, const float *a);
hipError_t launch_combine_norm(const float *o, const float *w, int N, int k, int d, int A,
                               int has_shared, float *h, float *a, float eps, hipStream_t s);

// ---- device helpers ----------------------------------------------------

// Column j of an 8-column group goes to position perm8<WB>(j) of the matrix
// cores' float16 operand, in the order the weight operand takes its codes
// (int4: columns 0,4,1,5,2,6,3,7, i.e. the low nibbles of bytes 0 and 2,
// their high nibbles, then the same of bytes 1 and 3; int8: 0,2,1,3,4,6,5,7).
template <int WB>
__device__ __forceinline__ int perm8(int j)
{
    if constexpr (WB == 4) return j < 4 ? 2 * j : 2 * (j - 4) + 1;
    else return (j & 4) | ((j & 1) << 1) | ((j >> 1) & 1);
}

// Factor applied to column j of an 8-column group in the matrix cores'
// float16 operand: int4 codes in the high nibble of their byte (odd j) enter
// the products as 16 u (the nibble's own bit position in a float16 mantissa),
// so their activations are stored divided by 16 (exact: a power of two).
template <int WB>
__host__ __device__ constexpr float act16_factor(int j)
{
    return (WB == 4 && (j & 1)) ? 0.0625f : 1.0f;
}

// x [N][d] float32 -> x16 [N][d] float16 for the matrix-core passes: the
// 8-column group i, each column at its perm8 position, times act16_factor.
template <int WB>
__device__ __forceinline__ void stage_x16_group(const float *__restrict__ x, long long i,
                                                uint16_t *__restrict__ x16)
{
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    const float4 a = reinterpret_cast<const float4 *>(x)[2 * i];
    const float4 b = reinterpret_cast<const float4 *>(x)[2 * i + 1];
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    h8 h;
#pragma unroll
    for (int j = 0; j < 8; ++j) h[perm8<WB>(j)] = (_Float16)(v[j] * act16_factor<WB>(j));
    reinterpret_cast<h8 *>(x16)[i] = h;
}

// (a & m) | o in one instruction (v_and_or_b32; the compiler emits an AND
// and an OR for constant masks). m goes in a scalar register, o in a vector
// register: one scalar operand per instruction.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o)
{
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m), "v"(o));
    return r;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// sum over aligned groups of L lanes (L a power of two <= 64)
template <int L>
__device__ __forceinline__ float segment_sum(float v) {
#pragma unroll
    for (int o = L / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

}  // namespace moe
