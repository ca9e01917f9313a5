// expert_gemv.hip - expert math for decode-sized token groups, and the combine.
//
// Colibri pages: "Public Colibri Observation and Revision Ledger", section
// "Exact Architecture and Data-Flow Reconstruction" (each chosen expert is a
// three-matrix MLP; a shared expert is always applied; the experts' weights
// are int4), Colibri README "Get started" (int4 with group scales) and
// "Speculative decoding, honestly" (int8 draft head).
//
//   h = silu(Wg x) * (Wu x),  o = Wd h,  y[t] = o_shared[t] + sum_j w[t][j] o[t*k+j]
//   W[r][c] = q[r][c] * scale[r][c / G]
//
// Streaming design (HBM-bound at a few tokens per expert):
//  * a workgroup owns a block of rows of one expert and up to 4 of its
//    tokens; each row is cut into 16-byte chunks (32 int4 or 16 int8 codes),
//    one chunk per lane, so every 128-bit load instruction of a wave covers
//    1 KB of contiguous row; rows longer than 64 chunks are split across the
//    waves of the workgroup, shorter rows share a wave;
//  * a work item's activations are staged once per workgroup in LDS, each
//    chunk scaled by the power of two that brings its largest magnitude into
//    [2^13, 2^14) (exact, undone on the chunk's partial sum together with
//    the group scale);
//  * int4: each staged chunk is rounded to 16-bit integers and kept as four
//    signed base-16 digit planes; a dword of codes (offset binary, one XOR
//    to two's complement) meets each plane in one v_dot8c_i32_i4, exact in
//    int32 (stage_chunk_int4, dot_int4);
//  * int8: the same with two signed base-256 digit planes and
//    v_dot4c_i32_i8 (stage_chunk_int8, dot_int8);
//  * partial sums of a row are added across its lanes with DPP and lane
//    reads, always in the same order.
#include <hip/hip_ext.h>

#include <type_traits>

#include "internal.h"
#include "topk.h"

namespace moe {
namespace {

// codes per 16-byte lane chunk, staged activation dwords per chunk
template <int WB> struct Fmt;
template <> struct Fmt<4> { static constexpr int epc = 32, xdw = 16; };
template <> struct Fmt<8> { static constexpr int epc = 16, xdw = 8; };

// int8 codes against integer activations: v_dot4c_i32_i8 (four signed
// 8-bit products into an int32). A staged run of 16 activations, scaled into
// [-2^14, 2^14], is rounded to integers X and kept as two signed base-256
// digit planes (the bytes of X + 0x8080, each XOR 0x80: X = d_0 + 256 d_1);
// a dword of codes (offset binary, XOR 0x80808080 gives two's complement)
// meets each plane in one instruction. The run's sum is exact in int32; its
// conversion to float32 rounds once (relative 2^-24) above 2^24.
__device__ __forceinline__ void stage_chunk_int8(const float4 *src, float scale, uint32_t *xs)
{
    int u[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float4 f4 = src[q];
        u[4 * q + 0] = (int)rintf(f4.x * scale) + 0x8080;
        u[4 * q + 1] = (int)rintf(f4.y * scale) + 0x8080;
        u[4 * q + 2] = (int)rintf(f4.z * scale) + 0x8080;
        u[4 * q + 3] = (int)rintf(f4.w * scale) + 0x8080;
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        // elements e and e + 2 of the group in one word: their bytes of plane
        // p land at bytes e and e + 2 once shifted by 8 (e - p)
        const uint32_t p0 = (uint32_t)(u[4 * g] & 0xFFFF) | ((uint32_t)(u[4 * g + 2] & 0xFFFF) << 16);
        const uint32_t p1 = (uint32_t)(u[4 * g + 1] & 0xFFFF) | ((uint32_t)(u[4 * g + 3] & 0xFFFF) << 16);
        xs[2 * g + 0] = ((p0 & 0x00FF00FFu) | ((p1 & 0x00FF00FFu) << 8)) ^ 0x80808080u;
        xs[2 * g + 1] = (((p0 >> 8) & 0x00FF00FFu) | (p1 & 0xFF00FF00u)) ^ 0x80808080u;
    }
}

// sum of the lane's 16 int8 codes (one 16-byte chunk, offset binary) times
// the staged integer activations of the chunk
__device__ __forceinline__ int dot_int8(const uint4 &w, const uint32_t *xs)
{
    const uint32_t cw[4] = {w.x ^ 0x80808080u, w.y ^ 0x80808080u, w.z ^ 0x80808080u,
                            w.w ^ 0x80808080u};
    int a0 = 0, a1 = 0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        a0 = __builtin_amdgcn_sdot4((int)cw[g], (int)xs[2 * g], a0, false);
        a1 = __builtin_amdgcn_sdot4((int)cw[g], (int)xs[2 * g + 1], a1, false);
    }
    return a1 * 256 + a0;
}

// int4 codes against integer activations: v_dot8c_i32_i4 (eight signed
// 4-bit products into an int32). Each staged chunk of 32 activations,
// already scaled into [-2^14, 2^14], is rounded to integers X and written
// as four signed base-16 digit planes (X = sum_p 16^p d_p, d_p in [-8, 7]:
// the nibbles of X + 0x8888, each XOR 8); a dword of codes (offset binary,
// XOR 0x88888888 gives two's complement) meets each plane in one
// instruction. Every product and sum is exact in int32 and the chunk total
// (below 2^23) converts to float32 exactly: the only rounding is x -> X, 16
// bits against float16's 11.
// Stage one chunk (32 scaled values) as digit planes: xs[4 g + p] holds
// plane p of elements 8g .. 8g+7, element 8g+j in nibble j.
__device__ __forceinline__ void stage_chunk_int4(const float4 *src, float scale, uint32_t *xs)
{
    int u[32];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const float4 f4 = src[q];
        u[4 * q + 0] = (int)rintf(f4.x * scale) + 0x8888;
        u[4 * q + 1] = (int)rintf(f4.y * scale) + 0x8888;
        u[4 * q + 2] = (int)rintf(f4.z * scale) + 0x8888;
        u[4 * q + 3] = (int)rintf(f4.w * scale) + 0x8888;
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        // element e and e + 4 of the group in one word: their nibbles of
        // plane p land at bits 4e and 4e + 16 once shifted by 4e - 4p
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            pk[e] = (uint32_t)(u[8 * g + e] & 0xFFFF) | ((uint32_t)(u[8 * g + e + 4] & 0xFFFF) << 16);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            uint32_t word = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t nib = pk[e] & (0x000F000Fu << (4 * p));
                word |= (e >= p) ? (nib << (4 * (e - p))) : (nib >> (4 * (p - e)));
            }
            xs[4 * g + p] = word ^ 0x88888888u;
        }
    }
}

// sum of the lane's 32 codes (one 16-byte chunk, offset binary) times the
// staged integer activations of the chunk
__device__ __forceinline__ int dot_int4(const uint4 &w, const uint32_t *xs)
{
    const uint32_t cw[4] = {w.x ^ 0x88888888u, w.y ^ 0x88888888u, w.z ^ 0x88888888u,
                            w.w ^ 0x88888888u};
    int a[4] = {0, 0, 0, 0};
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int p = 0; p < 4; ++p)
            a[p] = __builtin_amdgcn_sdot8((int)cw[g], (int)xs[4 * g + p], a[p], false);
    return ((a[3] * 16 + a[2]) * 16 + a[1]) * 16 + a[0];
}

// staged activations per token per chunk: XDW dwords, and a float2 whose
// second member is the chunk's inverse scale
__host__ __device__ constexpr int stage_bytes(int wb) { return (wb == 4 ? 16 : 8) * 4 + 8; }

// rounds of (token, chunk) activation pairs loaded before the weight loads
__host__ __device__ constexpr int pre_rounds(int tb) { return tb == 1 ? 1 : 2; }

// units a wave holds in registers at a time: 4 to 16 (a template parameter)
constexpr int kUnitBatch = 12;

// below this many 4-wave workgroups in a pass, single-token rows of 17..48
// units go to 8-wave workgroups instead (more waves per unit row to overlap
// the products with the loads when few items fill the chip)
constexpr long long kFewWorkgroups = 1024;

// LDS a GEMV workgroup may use for staged activations
constexpr int kStageBudget = 150 * 1024;

__device__ __forceinline__ int wave_incl_scan(int v)
{
    const int lane = threadIdx.x % kWave;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int u = __shfl_up(v, o, kWave);
        if (lane >= o) v += u;
    }
    return v;
}

struct GemvArgs {
    Fwd f;
    int n_wg;               // workgroups per item
    int plan_here;          // gate/up pass: 0 read the work list, 1 scan a union of
                            // <= 64 in-kernel, 2 one item per union slot (n_tokens <= TB)
};

// Finds work item `item_idx` of the current call when the union has at most
// 64 experts. Items are the shared expert's tokens in slices of TB first
// (their workgroups need nothing from the union to start loading weights),
// then the union experts in union order, each cut into slices of TB of its
// permutation positions. One wave; writes *out (count == 0: no such item)
// and returns the item total.
template <int TB>
__device__ int find_item(const Fwd &f, int item_idx, Item *out)
{
    const int lane = threadIdx.x % kWave;
    const int nsh = f.has_shared ? (f.N + TB - 1) / TB : 0;
    if (item_idx < nsh) {
        if (lane == 0) {
            Item it;
            it.expert = -1;
            it.p0 = f.A + item_idx * TB;
            it.count = min(TB, f.N - item_idx * TB);
            it.pad = 0;
            *out = it;
        }
        return -1;  // total not needed by shared-expert workgroups
    }
    const int E = f.g.E;
    const int nu = min(max(*f.n_union, 0), min(E, kWave));
    int e = -1, s0 = 0, T = 0;
    if (lane < nu) {
        e = f.union_ids[lane];
        if (e >= 0 && e < E) {
            s0 = min(max(f.offsets[e], 0), f.A);
            T = min(max(f.offsets[e + 1], s0), f.A) - s0;
        } else {
            e = -1;
        }
    }
    if (lane == 0) out->count = 0;
    const int nb = (T + TB - 1) / TB;
    const int incl = wave_incl_scan(nb);
    const int excl = incl - nb;
    const int rel = item_idx - nsh;
    if (nb > 0 && rel >= excl && rel < incl) {
        const int b = rel - excl;
        Item it;
        it.expert = e;
        it.p0 = s0 + b * TB;
        it.count = min(TB, T - b * TB);
        it.pad = 0;
        *out = it;
    }
    return nsh + __builtin_amdgcn_readlane(incl, kWave - 1);
}

// One workgroup (NW waves) computes NW/KS unit rows (16 output rows each) of
// one work item: up to TB tokens of one expert. KS waves share a unit row,
// each taking every KS-th unit along it. The item's activations are staged
// once in LDS as integer digit planes (each chunk scaled by a power of two
// and rounded to 16 bits, in the order the dot product consumes them). Each
// lane reads one 16-byte slot per unit (a wave reads the whole 1 KB unit) and
// takes exact integer dot products of its 32 (int4) or 16 (int8) codes with
// every token's staged chunk (dot_int4 / dot_int8), scaled in float32 per
// chunk. Partial sums are added over the four lanes of a row with lane
// shuffles and over the KS waves of a unit row in LDS, always in the same
// order.
//
// gate/up pass with a union of at most 64 experts: the workgroup finds its
// item from the union itself (no separate planning launch) and records the
// item list for the down pass.
template <bool GATEUP, int WB, int TB, int NW, int KS, int UB>
__device__ __forceinline__ void gemv_body(const GemvArgs &ga, const int bid, const int nblk)
{
    constexpr int kGemvThreads = NW * kWave;
    constexpr int XDW = Fmt<WB>::xdw, EPC = Fmt<WB>::epc;
    constexpr int XQ = XDW / 4;              // uint4 per staged chunk
    constexpr int UC = 4 * EPC;              // columns per unit
    constexpr int NM = GATEUP ? 2 : 1;       // gate and up, or down
    constexpr int TPW = NW / KS;             // unit rows per workgroup
    static_assert(!GATEUP || NW >= 2, "routing inside takes a wave per token, two tokens");

    extern __shared__ uint4 lds_x[];         // [TB][XQ][NCH] staged activations
    __shared__ Item s_item;
    __shared__ int s_expert;
    __shared__ float red[NW][TB][NM][kUnitRows];
    // routing inside (one or two tokens)
    __shared__ int32_t s_rt_lds[2 * MOE_MAX_K], s_rt_ids[2 * MOE_MAX_K];
    __shared__ float s_rt_w[2 * MOE_MAX_K];
    __shared__ int s_rt_tok[2];  // tokens of this item, in assignment order

    const Fwd &f = ga.f;
    const Geo &g = f.g;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    if (GATEUP && f.direct) {
        // the down kernel adds its rows into y: clear y one launch ahead
        // (every workgroup a part, before any of them can leave early)
        const long long n4 = (long long)f.N * g.d / 4;
        for (long long i = (long long)bid * kGemvThreads + tid; i < n4;
             i += (long long)nblk * kGemvThreads)
            reinterpret_cast<float4 *>(f.y)[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
    const int item_idx = bid / ga.n_wg;
    const int wg = bid % ga.n_wg;
    // The expert is needed first (the weight loads only depend on it); the
    // item's tokens are resolved after when possible.
    int expert;
    Item it;
    bool resolved = true;
    if (GATEUP && ga.plan_here == 2 && f.route_in) {
        // one or two tokens, routed here: every workgroup of a routed item
        // takes the top-k of the router's output (a wave per token; the same
        // code and inputs as the route tail, so the same ids). Union slot u
        // holds the u-th smallest distinct id; the permutation is the stable
        // sort of the assignments by id. Workgroup 0 also writes the routing
        // outputs for the down kernel and the caller (an extra workgroup
        // doing only that measured slower).
        const int nsh = f.has_shared ? 1 : 0;
        const bool writer = bid == 0;
        const bool route = writer || item_idx >= nsh;
        const int A = f.A;  // at most 2 * MOE_MAX_K = 64 assignments: one per lane
        if (tid == 0) {
            Item none;
            none.expert = -2;
            none.p0 = 0;
            none.count = 0;
            none.pad = 0;
            s_item = none;
        }
        if (route && wave < f.N)
            topk_wave<false>(f.route_in, f.route_P, f.route_b, f.N, g.E, f.k, wave,
                             writer ? f.route_ids : s_rt_ids, writer ? f.route_w : s_rt_w,
                             s_rt_lds);
        __syncthreads();
        if (wave == 0 && route) {
            const int id = lane < A ? s_rt_lds[lane] : 0x7FFFFFFF;
            int lt = 0, cnt = 0, before = 0;  // ids below, equal ids, equal ids of lower lanes
            for (int b = 0; b < A; ++b) {
                const int o = s_rt_lds[b];
                lt += o < id ? 1 : 0;
                cnt += o == id ? 1 : 0;
                before += (o == id && b < lane) ? 1 : 0;
            }
            const bool first = lane < A && before == 0;
            const unsigned long long fm = __ballot(first);
            int u = 0;  // distinct ids below this one
            for (int b = 0; b < A; ++b)
                u += (((fm >> b) & 1ull) && s_rt_lds[b] < id) ? 1 : 0;
            // the permutation is written in this launch: the item's tokens
            // come from LDS (at most two occurrences of an id, one per token)
            if (lane < A && item_idx - nsh == u) s_rt_tok[before] = lane / f.k;
            if (first && item_idx - nsh == u) {
                Item r;
                r.expert = id;
                r.p0 = lt;
                r.count = cnt;
                r.pad = 0;
                s_item = r;
            }
            if (writer) {
                if (lane < A) const_cast<int32_t *>(f.perm)[lt + before] = lane;
                if (first) {
                    const_cast<int32_t *>(f.union_ids)[u] = id;
                    if (f.route_counters)
                        atomicAdd(&f.route_counters[id], (unsigned long long)cnt);
                }
                for (int e = lane; e <= g.E; e += kWave) {
                    int c = 0;
                    for (int b = 0; b < A; ++b) c += s_rt_lds[b] < e ? 1 : 0;
                    const_cast<int32_t *>(f.offsets)[e] = c;
                }
                if (lane == 0) {
                    *const_cast<int32_t *>(f.n_union) = __popcll(fm);
                    *f.n_items = nsh + __popcll(fm);
                }
            }
        }
        __syncthreads();
        if (item_idx < nsh) {
            it.expert = -1;
            it.p0 = f.A;
            it.count = f.N;
            it.pad = 0;
        } else {
            it = s_item;
            if (it.expert == -2) return;  // beyond the union: uniform exit
        }
        expert = it.expert;
        if (wg == 0 && tid == 0) f.items[item_idx] = it;
    } else if (GATEUP && ga.plan_here == 2) {
        // every expert has at most n_tokens <= TB tokens: one item per union
        // slot, after the shared expert's single item
        const int nsh = f.has_shared ? 1 : 0;
        resolved = false;
        if (item_idx < nsh) {
            expert = -1;
        } else {
            if (tid == 0) {
                const int rel = item_idx - nsh;
                const int lim = min(g.E, f.A);
                const int nu = min(max(*f.n_union, 0), lim);   // both loads in flight together
                const int e = rel < lim ? f.union_ids[rel] : -1;
                s_expert = (rel < nu && e >= 0 && e < g.E) ? e : -2;
                if (wg == 0 && rel == 0) *f.n_items = nsh + nu;
            }
            __syncthreads();
            expert = s_expert;
            if (expert == -2) return;  // beyond the union: uniform exit
        }
    } else if (GATEUP && ga.plan_here == 1) {
        if (wave == 0) {
            const int total = find_item<TB>(f, item_idx, &s_item);
            if (lane == 0) {
                if (wg == 0 && s_item.count > 0) f.items[item_idx] = s_item;
                // the first routed item's first workgroup publishes the total
                const int nsh = f.has_shared ? (f.N + TB - 1) / TB : 0;
                if (wg == 0 && item_idx == nsh) *f.n_items = min(total, f.max_items);
            }
        }
        __syncthreads();
        it = s_item;
        expert = it.expert;
    } else {
        if (item_idx >= *f.n_items) return;  // uniform over the workgroup
        if (tid == 0) s_item = f.items[item_idx];
        __syncthreads();
        it = s_item;
        expert = it.expert;
    }
    if (resolved && it.count <= 0) return;  // no such item: uniform exit
    if (!resolved) {
        if (expert < 0) {
            it.expert = -1;
            it.p0 = f.A;
            it.count = f.N;
            it.pad = 0;
        } else if (f.N == 1) {
            // one token: every union expert holds one assignment, at the
            // permutation position equal to its union slot
            it.expert = expert;
            it.p0 = item_idx - (f.has_shared ? 1 : 0);
            it.count = 1;
            it.pad = 0;
        } else {
            if (tid == 0) {
                const int s0 = min(max(f.offsets[expert], 0), f.A);
                Item r;
                r.expert = expert;
                r.p0 = s0;
                r.count = min(max(f.offsets[expert + 1], s0), f.A) - s0;
                r.pad = 0;
                s_item = r;
            }
            __syncthreads();
            it = s_item;
        }
        if (wg == 0 && tid == 0 && it.count > 0) f.items[item_idx] = it;
        if (it.count <= 0) return;  // uniform: inconsistent offsets give no tokens
    }
    if (!in_phase(f, it.expert)) return;  // uniform: the other phase's item
    const int count = min(it.count, TB);

    const uint8_t *blk = expert >= 0 ? expert_block(f, expert) : f.shared;
    const int K = GATEUP ? g.d : g.f;        // contraction length
    const int rows = GATEUP ? g.f : g.d;     // output rows
    const int NCH = K / EPC;                 // chunks per row
    const int n_kb = K / UC;                 // units per row
    const int ng = GATEUP ? g.ng_gu : g.ng_dn;
    float2 *lds_ci = reinterpret_cast<float2 *>(lds_x + TB * XQ * NCH);  // [TB][NCH]
    const float *in = GATEUP ? f.x : f.h;
    float *out = GATEUP ? f.h : f.o;
    const int r16 = lane % kUnitRows, q = lane / kUnitRows;
    const int tw = wave / KS, slice = wave % KS;   // unit row in the workgroup, K slice
    const int n_rt = rows / kUnitRows;
    const int rt = wg * TPW + tw;
    const bool live = rt < n_rt;                    // uniform per wave
    const size_t unit0 = (size_t)min(rt, n_rt - 1) * n_kb * kUnitBytes + (size_t)lane * 16;
    const uint8_t *q0 = blk + (GATEUP ? 0 : g.off_dn) + unit0;
    const uint8_t *q1 = blk + g.off_up + unit0;
    const size_t sc0 = (size_t)min(rt, n_rt - 1) * ng * kUnitRows + r16;
    const float *s0 = reinterpret_cast<const float *>(blk + (GATEUP ? g.off_gs : g.off_ds)) + sc0;
    const float *s1 = reinterpret_cast<const float *>(blk + g.off_us) + sc0;

    // units kb = slice + KS * j of this wave, UB at a time. Every load of a
    // batch is issued (past the wave's last unit it reads that unit again),
    // so the number of loads in flight is the same on every path and each
    // unit's products wait for that unit only.
    const int n_mine = live ? (n_kb - slice + KS - 1) / KS : 0;
    uint4 w[UB][NM];
    float sc[UB][NM];
    auto load_units = [&](int j0) {
#pragma unroll
        for (int u = 0; u < UB; ++u) {
            const int kb = slice + KS * max(min(j0 + u, n_mine - 1), 0);
            const int grp = g.group ? (kb * UC + q * EPC) / g.group : 0;
            w[u][0] = *reinterpret_cast<const uint4 *>(q0 + (size_t)kb * kUnitBytes);
            sc[u][0] = s0[grp * kUnitRows];
            if (GATEUP) {
                w[u][NM - 1] = *reinterpret_cast<const uint4 *>(q1 + (size_t)kb * kUnitBytes);
                sc[u][NM - 1] = s1[grp * kUnitRows];
            }
        }
    };

    // ---- stage the activations: loads first, then the weights ----------------
    // (token, chunk) pairs are spread over the threads; a round covers one
    // pair per thread. Each pair is staged on its own: scaled by the power of
    // two that brings the chunk's largest magnitude into [2^13, 2^14),
    // rounded to 16-bit integers and split into digit planes (the scale is
    // undone per chunk with the group scale). The first rounds are loaded
    // before the weight loads are issued, so their data do not wait behind
    // the weights.
    const int NPAIR = TB * NCH;
    const int ROUNDS = (NPAIR + kGemvThreads - 1) / kGemvThreads;
    auto pair_src = [&](int pq) -> const float * {
        const int i = pq / NCH, c = pq % NCH;
        if (i >= count) return nullptr;
        const int p = it.p0 + i;
        size_t r;
        if (!GATEUP)
            r = (size_t)p;
        else if (it.expert < 0)
            r = (size_t)(p - f.A);
        else if (f.N == 1)
            r = 0;
        else if (f.route_in)  // routing inside: the permutation is still being written
            r = (size_t)s_rt_tok[i];
        else  // values read from the permutation are clamped into range
            r = (size_t)(min(max(f.perm[p], 0), f.A - 1) / f.k);
        return in + r * K + (size_t)c * EPC;
    };
    constexpr int PRE = pre_rounds(TB);
    float4 xv[PRE][EPC / 4];
#pragma unroll
    for (int r = 0; r < PRE; ++r) {
        const int pq = tid + r * kGemvThreads;
        const float *src = pq < NPAIR ? pair_src(pq) : nullptr;
        if (src) {
#pragma unroll
            for (int v = 0; v < EPC / 4; ++v) xv[r][v] = reinterpret_cast<const float4 *>(src)[v];
        }
    }
    load_units(0);
    auto stage_pair = [&](int pq, const float4 (&v)[EPC / 4]) {
        const int i = pq / NCH, c = pq % NCH;
        float m = 0.0f;
#pragma unroll
        for (int u = 0; u < EPC / 4; ++u)
            m = fmaxf(m, fmaxf(fmaxf(fabsf(v[u].x), fabsf(v[u].y)),
                               fmaxf(fabsf(v[u].z), fabsf(v[u].w))));
        int sh = 0;
        if (m > 0.0f && m <= 3.4e38f) {
            int ex;
            frexpf(m, &ex);
            sh = min(126, max(-126, 14 - ex));
        }
        uint32_t xs[XDW];
        if constexpr (WB == 4)
            stage_chunk_int4(v, ldexpf(1.0f, sh), xs);
        else
            stage_chunk_int8(v, ldexpf(1.0f, sh), xs);
        lds_ci[i * NCH + c] = make_float2(0.0f, ldexpf(1.0f, -sh));
#pragma unroll
        for (int u = 0; u < XQ; ++u)
            lds_x[(i * XQ + u) * NCH + c] = make_uint4(xs[4 * u], xs[4 * u + 1], xs[4 * u + 2],
                                                       xs[4 * u + 3]);
    };
#pragma unroll
    for (int r = 0; r < PRE; ++r) {
        const int pq = tid + r * kGemvThreads;
        if (pq < NPAIR && pq / NCH < count) stage_pair(pq, xv[r]);
    }
#pragma unroll 1
    for (int r = PRE; r < ROUNDS; ++r) {
        const int pq = tid + r * kGemvThreads;
        const float *src = pq < NPAIR ? pair_src(pq) : nullptr;
        if (src) {
            float4 v[EPC / 4];
#pragma unroll
            for (int u = 0; u < EPC / 4; ++u) v[u] = reinterpret_cast<const float4 *>(src)[u];
            stage_pair(pq, v);
        }
    }
    __syncthreads();

    // ---- stream this wave's units ---------------------------------------------
    float acc[TB][NM];
#pragma unroll
    for (int i = 0; i < TB; ++i)
#pragma unroll
        for (int m = 0; m < NM; ++m) acc[i][m] = 0.0f;
#pragma unroll 1
    for (int j0 = 0; j0 < n_mine; j0 += UB) {
        if (j0 > 0) load_units(j0);  // the first batch was issued before staging
#pragma unroll
        for (int u = 0; u < UB; ++u) {
            if (j0 + u >= n_mine) break;
            const int c = (slice + KS * (j0 + u)) * 4 + q;  // this lane's chunk

#pragma unroll
            for (int i = 0; i < TB; ++i) {
                if (i >= count) break;
                uint32_t xs[XDW];
#pragma unroll
                for (int qq = 0; qq < XQ; ++qq) {
                    const uint4 v = lds_x[(i * XQ + qq) * NCH + c];
                    xs[4 * qq] = v.x;
                    xs[4 * qq + 1] = v.y;
                    xs[4 * qq + 2] = v.z;
                    xs[4 * qq + 3] = v.w;
                }
                const float2 ci = lds_ci[i * NCH + c];  // (unused, inverse scale)
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    const int d = WB == 4 ? dot_int4(w[u][m], xs) : dot_int8(w[u][m], xs);
                    acc[i][m] = fmaf(sc[u][m] * ci.y, (float)d, acc[i][m]);
                }
            }
        }
    }

    // ---- row sums: the four lanes of a row, then the waves of a unit row -----
#pragma unroll
    for (int i = 0; i < TB; ++i)
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            float v = acc[i][m];
            v += __shfl_xor(v, 16, kWave);
            v += __shfl_xor(v, 32, kWave);
            if (lane < kUnitRows) red[wave][i][m][lane] = v;
        }
    __syncthreads();
    if (tid < TPW * TB * kUnitRows) {
        const int t = tid / (TB * kUnitRows), i = (tid / kUnitRows) % TB, r = tid % kUnitRows;
        const int row_tile = wg * TPW + t;
        if (i < count && row_tile < n_rt) {
            float v[NM];
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                float sum = 0.0f;
#pragma unroll
                for (int ww = 0; ww < KS; ++ww) sum += red[t * KS + ww][i][m][r];
                v[m] = sum;
            }
            const int p = it.p0 + i;
            const int orow = (!GATEUP && it.expert >= 0) ? min(max(f.perm[p], 0), f.A - 1) : p;
            const int row = row_tile * kUnitRows + r;
            if (GATEUP) {
                const float gv = v[0], uv = v[NM - 1];
                out[(size_t)orow * rows + row] = gv / (1.0f + expf(-gv)) * uv;
            } else if (f.direct) {
                // y[t] gets the shared row and one routed row, or two routed
                // rows: float atomics onto the cleared y, the same sum in
                // either order (the combine kernel's order of rounding)
                const bool routed = it.expert >= 0;
                const int t = routed ? orow / f.k : p - f.A;
                const float wt = routed ? f.w[orow] : 1.0f;
                atomicAdd(&f.y[(size_t)t * rows + row], wt * v[0]);
            } else {
                out[(size_t)orow * rows + row] = v[0];
            }
        }
    }
}

template <bool GATEUP, int WB, int TB, int NW, int KS, int UB>
__global__ __launch_bounds__(NW * kWave) void gemv_kernel(GemvArgs ga)
{
    gemv_body<GATEUP, WB, TB, NW, KS, UB>(ga, blockIdx.x, gridDim.x);
}

// ---- work list for larger unions ---------------------------------------------

constexpr int kPlanThreads = 1024;

__device__ int block_excl_scan(int v, int &total)
{
    __shared__ int wt[kPlanThreads / kWave];
    const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
    const int incl = wave_incl_scan(v);
    if (lane == kWave - 1) wt[wv] = incl;
    __syncthreads();
    if (wv == 0) {
        int x = lane < kPlanThreads / kWave ? wt[lane] : 0;
        x = wave_incl_scan(x);
        if (lane < kPlanThreads / kWave) wt[lane] = x;
    }
    __syncthreads();
    total = wt[kPlanThreads / kWave - 1];
    const int r = incl - v + (wv > 0 ? wt[wv - 1] : 0);
    __syncthreads();
    return r;
}

// Which pass computes an expert with T tokens: 0 the GEMV kernels, 1 the
// 128-token MFMA kernels (T >= tstar), 2 the 32-token MFMA kernels
// (tsmall <= T < tstar). A pass with no list (max_* == 0) takes nothing.
__device__ __forceinline__ int pass_of(const Fwd &f, int T)
{
    if (f.max_mitems > 0 && T >= f.tstar) return 1;
    if (f.max_sitems > 0 && T >= f.tsmall) return 2;
    return 0;
}

// Work lists for unions of any size (<= 1024 experts), one thread per union
// slot. Each expert goes to the list of its pass in slices of that list's
// tokens per item (tb, 128 or 32); in every list the shared expert comes
// first, then the union experts in union order.
__device__ __forceinline__ void plan_body(const Fwd &f)
{
    const int u = threadIdx.x;
    const int E = f.g.E;
    const int nu = min(max(*f.n_union, 0), E);
    int e = -1, s0 = 0, T = 0;
    if (u < nu) {
        e = f.union_ids[u];
        if (e >= 0 && e < E) {
            s0 = min(max(f.offsets[e], 0), f.A);
            T = min(max(f.offsets[e + 1], s0), f.A) - s0;
        } else {
            e = -1;
        }
    }
    int pass = pass_of(f, T);
    int sh_pass = f.has_shared ? pass_of(f, f.N) : -1;
    // A group on the 128-token pass whose last item would hold at most 32
    // tokens past a full one gives that remainder to the 32-token pass: a
    // 128-token item computes all of its token blocks whatever it holds.
    const bool small_on = f.max_sitems > 0;
    auto big_part = [&](int cnt) {
        const int r = cnt % kMfmaBigTokens;
        return (small_on && cnt > kMfmaBigTokens && r > 0 && r <= kMfmaSmallTokens) ? cnt - r
                                                                                      : cnt;
    };
    if (f.max_mitems > 0 && f.max_sitems > 0) {
        // a handful of 128-token items would run nearly alone (a few
        // workgroups each): give them to the 32-token pass instead, where
        // they run among the others
        int n_big;
        block_excl_scan(pass == 1 ? (big_part(T) + kMfmaBigTokens - 1) / kMfmaBigTokens : 0,
                        n_big);
        if (sh_pass == 1) n_big += (big_part(f.N) + kMfmaBigTokens - 1) / kMfmaBigTokens;
        if (n_big < kMinBigItems) {
            if (pass == 1) pass = 2;
            if (sh_pass == 1) sh_pass = 2;
        }
    }
    Item *const lists[3] = {f.items, f.mitems, f.sitems};
    int32_t *const counts[3] = {f.n_items, f.n_mitems, f.n_sitems};
    const int maxes[3] = {f.max_items, f.max_mitems, f.max_sitems};
    const int sizes[3] = {f.tb, kMfmaBigTokens, kMfmaSmallTokens};
#pragma unroll
    for (int l = 0; l < 3; ++l) {
        const int sz = sizes[l], mx = maxes[l];
        // the tokens [beg, end) of a group of cnt tokens on pass p that list l takes
        auto span = [&](int p, int cnt, int &beg, int &end) {
            beg = end = 0;
            if (p == l) {
                end = l == 1 ? big_part(cnt) : cnt;
            } else if (p == 1 && l == 2) {  // the remainder of a 128-token group
                beg = big_part(cnt);
                end = cnt;
            }
        };
        int sb, se, eb, ee;
        span(sh_pass, f.N, sb, se);
        span(pass, T, eb, ee);
        const int nsh = (se - sb + sz - 1) / sz;
        const int nb = (ee - eb + sz - 1) / sz;
        int tot;
        const int base = nsh + block_excl_scan(nb, tot);  // uniform call: every thread
        if (mx <= 0) continue;
        for (int b = u; b < nsh && b < mx; b += kPlanThreads) {
            Item it = {-1, f.A + sb + b * sz, min(sz, se - sb - b * sz), 0};
            lists[l][b] = it;
        }
        for (int b = 0; b < nb && base + b < mx; ++b) {
            Item it = {e, s0 + eb + b * sz, min(sz, ee - eb - b * sz), 0};
            lists[l][base + b] = it;
        }
        if (u == 0) *counts[l] = min(nsh + tot, mx);
    }
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(Fwd f) { plan_body(f); }

// The planning workgroup (block 0) and, in the other blocks, the float16
// copy of x for the matrix-core passes (independent work, one launch).
template <int WB>
__global__ __launch_bounds__(kPlanThreads) void plan_stage_kernel(Fwd f, long long n8)
{
    if (blockIdx.x == 0) {
        plan_body(f);
        return;
    }
    const long long i = (long long)(blockIdx.x - 1) * kPlanThreads + threadIdx.x;
    if (i < n8) stage_x16_group<WB>(f.x, i, f.x16);
}

// ---- combine and chaining ---------------------------------------------------

__global__ __launch_bounds__(256) void combine_kernel(
    const float *__restrict__ o, const float *__restrict__ w, int N, int k, int d, int A,
    int has_shared, float *__restrict__ y)
{
    // acc + (w * o), each rounded (not fused): the order of rounding of the
    // direct combine in the down kernel
#pragma clang fp contract(off)
    const int nq = d / 4;
    const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long long)N * nq) return;
    const int t = (int)(idx / nq), q = (int)(idx % nq);
    float4 acc = has_shared ? reinterpret_cast<const float4 *>(o + (size_t)(A + t) * d)[q]
                            : make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
        const float wj = w[(size_t)t * k + j];
        if (wj == 0.0f) continue;  // adds nothing; a dropped slot's row is never written
        const float4 v = reinterpret_cast<const float4 *>(o + ((size_t)t * k + j) * d)[q];
        acc.x = acc.x + wj * v.x;
        acc.y = acc.y + wj * v.y;
        acc.z = acc.z + wj * v.z;
        acc.w = acc.w + wj * v.w;
    }
    reinterpret_cast<float4 *>(y + (size_t)t * d)[q] = acc;
}

// Residual RMS norm of token rows, one workgroup of kNormThreads per token.
// Rows of d = 4 nq floats (nq <= RV * kNormThreads, 16-byte aligned) keep
// their values in registers: thread j owns the float4 chunks j, j +
// kNormThreads, ...; its sum of squares runs over its chunks in order (x, y,
// z, w), then over the wave, then the four waves' sums pairwise. Other rows
// take residual_rmsnorm_kernel, with one element per thread at a time.
constexpr int kNormThreads = 256;

// The rest of the norm for a row whose values (h + y) are in v: the sum of
// squares, then a = v / sqrt(mean + eps). Shared by the residual norm and the
// combine that ends in it, so both give the same a for the same v.
template <int RV>
__device__ __forceinline__ void norm_finish(const float4 (&v)[RV], int nq, int d, float eps,
                                            float4 *__restrict__ a4)
{
    __shared__ float part[kNormThreads / kWave];
    const int tid = threadIdx.x;
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < RV; ++j) {
        if (tid + j * kNormThreads < nq) {
            ss = fmaf(v[j].x, v[j].x, ss);
            ss = fmaf(v[j].y, v[j].y, ss);
            ss = fmaf(v[j].z, v[j].z, ss);
            ss = fmaf(v[j].w, v[j].w, ss);
        }
    }
    ss = wave_sum(ss);
    if (tid % kWave == 0) part[tid / kWave] = ss;
    __syncthreads();
    const float tot = (part[0] + part[1]) + (part[2] + part[3]);
    const float r = 1.0f / sqrtf(tot / (float)d + eps);
#pragma unroll
    for (int j = 0; j < RV; ++j) {
        const int q = tid + j * kNormThreads;
        if (q < nq) a4[q] = make_float4(v[j].x * r, v[j].y * r, v[j].z * r, v[j].w * r);
    }
}

template <int RV>
__global__ __launch_bounds__(kNormThreads) void residual_rmsnorm_vec_kernel(
    float *__restrict__ h, const float *__restrict__ y, float *__restrict__ a, int d, float eps)
{
    const int t = blockIdx.x, tid = threadIdx.x, nq = d / 4;
    float4 *h4 = reinterpret_cast<float4 *>(h + (size_t)t * d);
    float4 v[RV], u[RV];
#pragma unroll
    for (int j = 0; j < RV; ++j) {  // every load issued before the first add
        const int q = min(tid + j * kNormThreads, nq - 1);
        v[j] = h4[q];
        if (y) u[j] = reinterpret_cast<const float4 *>(y + (size_t)t * d)[q];
    }
    if (y) {
#pragma unroll
        for (int j = 0; j < RV; ++j) {
            v[j] = make_float4(v[j].x + u[j].x, v[j].y + u[j].y, v[j].z + u[j].z, v[j].w + u[j].w);
            const int q = tid + j * kNormThreads;
            if (q < nq) h4[q] = v[j];
        }
    }
    norm_finish<RV>(v, nq, d, eps, reinterpret_cast<float4 *>(a + (size_t)t * d));
}

__global__ __launch_bounds__(kNormThreads) void residual_rmsnorm_kernel(
    float *__restrict__ h, const float *__restrict__ y, float *__restrict__ a, int d, float eps)
{
    __shared__ float part[kNormThreads / kWave];
    const int t = blockIdx.x;
    float *ht = h + (size_t)t * d;
    float ss = 0.0f;
    for (int i = threadIdx.x; i < d; i += kNormThreads) {
        float v = ht[i];
        if (y) {
            v += y[(size_t)t * d + i];
            ht[i] = v;
        }
        ss = fmaf(v, v, ss);
    }
    ss = wave_sum(ss);
    if (threadIdx.x % kWave == 0) part[threadIdx.x / kWave] = ss;
    __syncthreads();
    const float tot = (part[0] + part[1]) + (part[2] + part[3]);
    const float r = 1.0f / sqrtf(tot / (float)d + eps);
    for (int i = threadIdx.x; i < d; i += kNormThreads) a[(size_t)t * d + i] = ht[i] * r;
}

// The combine of a layer step followed by the residual norm that starts the
// next one, for a stack of layers: y[t] (the combine's value, in its order
// of rounding) is added into h[t] and a[t] = rms_norm(h[t]), without writing
// y. Gives exactly the h and a of combine_kernel then
// residual_rmsnorm_vec_kernel.
template <int RV>
__global__ __launch_bounds__(kNormThreads) void combine_norm_kernel(
    const float *__restrict__ o, const float *__restrict__ w, int k, int d, int A, int has_shared,
    float *__restrict__ h, float *__restrict__ a, float eps)
{
#pragma clang fp contract(off)
    const int t = blockIdx.x, tid = threadIdx.x, nq = d / 4;
    float4 *h4 = reinterpret_cast<float4 *>(h + (size_t)t * d);
    float4 v[RV], acc[RV];
#pragma unroll
    for (int j = 0; j < RV; ++j) {
        const int q = min(tid + j * kNormThreads, nq - 1);
        v[j] = h4[q];
        acc[j] = has_shared ? reinterpret_cast<const float4 *>(o + (size_t)(A + t) * d)[q]
                            : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    // the rows of KC slots are loaded together, then added in slot order
    constexpr int KC = RV <= 6 ? 8 : (RV <= 12 ? 4 : 2);
    for (int i0 = 0; i0 < k; i0 += KC) {
        float4 u[KC][RV];
        float wc[KC];
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            const int i = min(i0 + c, k - 1);
            wc[c] = i0 + c < k ? w[(size_t)t * k + i] : 0.0f;
            const float4 *oi = reinterpret_cast<const float4 *>(o + ((size_t)t * k + i) * d);
#pragma unroll
            for (int j = 0; j < RV; ++j) u[c][j] = oi[min(tid + j * kNormThreads, nq - 1)];
        }
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            const float wi = wc[c];
            if (wi == 0.0f) continue;  // adds nothing; a dropped slot's row is never written
#pragma unroll
            for (int j = 0; j < RV; ++j) {
                acc[j].x = acc[j].x + wi * u[c][j].x;
                acc[j].y = acc[j].y + wi * u[c][j].y;
                acc[j].z = acc[j].z + wi * u[c][j].z;
                acc[j].w = acc[j].w + wi * u[c][j].w;
            }
        }
    }
#pragma unroll
    for (int j = 0; j < RV; ++j) {
        v[j] = make_float4(v[j].x + acc[j].x, v[j].y + acc[j].y, v[j].z + acc[j].z,
                           v[j].w + acc[j].w);
        const int q = tid + j * kNormThreads;
        if (q < nq) h4[q] = v[j];
    }
    norm_finish<RV>(v, nq, d, eps, reinterpret_cast<float4 *>(a + (size_t)t * d));
}

// float4 chunks per thread of the register-resident norm for rows of d
// floats, or 0 when such rows take the element-wise kernel
int norm_vec_width(int d)
{
    if (d % 4) return 0;
    const int rv = (d / 4 + kNormThreads - 1) / kNormThreads;
    for (int w : {1, 2, 4, 6, 8, 12, 16})
        if (rv <= w) return w;
    return 0;
}

template <typename F>
hipError_t with_norm_width(int rv, F &&go)
{
    switch (rv) {
    case 1: return go(std::integral_constant<int, 1>());
    case 2: return go(std::integral_constant<int, 2>());
    case 4: return go(std::integral_constant<int, 4>());
    case 6: return go(std::integral_constant<int, 6>());
    case 8: return go(std::integral_constant<int, 8>());
    case 12: return go(std::integral_constant<int, 12>());
    case 16: return go(std::integral_constant<int, 16>());
    default: return hipErrorInvalidValue;
    }
}

// ---- dispatch -------------------------------------------------------------

template <bool GATEUP, int WB, int TB, int NW, int KS, int UB>
hipError_t run_gemv(GemvArgs a, hipStream_t s)
{
    const Geo &g = a.f.g;
    const int K = GATEUP ? g.d : g.f;
    const int rows = GATEUP ? g.f : g.d;
    const size_t lds = (size_t)TB * (K / Fmt<WB>::epc) * stage_bytes(WB);
    constexpr int TPW = NW / KS;
    a.n_wg = (rows / kUnitRows + TPW - 1) / TPW;
    const long long blocks = (long long)a.f.max_items * a.n_wg;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7FFFFFFFLL || lds > (size_t)kStageBudget) return hipErrorInvalidValue;
    const hipEvent_t *ev = GATEUP ? a.f.ev_gu : a.f.ev_dn;
    if (ev[0] || ev[1])  // events taken by the dispatch itself, around this kernel only
        hipExtLaunchKernelGGL((gemv_kernel<GATEUP, WB, TB, NW, KS, UB>), dim3((unsigned)blocks),
                              dim3(NW * kWave), lds, s, ev[0], ev[1], 0, a);
    else
        hipLaunchKernelGGL((gemv_kernel<GATEUP, WB, TB, NW, KS, UB>), dim3((unsigned)blocks),
                           dim3(NW * kWave), lds, s, a);
    return hipGetLastError();
}

// How a unit row is shared, by row length and by how many workgroups the
// pass has (few: spread each unit row over more waves; many: give each wave
// whole unit rows, so the activations staged per workgroup serve 4 of them):
//   rows of 1-3 units: 1 or 2 waves per unit row;
//   rows of 4-16 units: 4 waves of up to 4 units, or (many workgroups) one
//     wave per unit row with all its units;
//   longer rows: 4 waves of up to 12 units at a time; single tokens: 4
//     waves of 4 at a time, or (few workgroups, up to 48 units) 8 waves of 6.
struct GemvCfg {
    int nw, ks, ub;  // waves per workgroup, waves per unit row, units per batch
    bool is(int w, int k, int u) const { return nw == w && ks == k && ub == u; }
};

GemvCfg gemv_cfg(int epc, bool gateup, const Geo &g, int tb, int max_items)
{
    const int K = gateup ? g.d : g.f;
    const int rows = gateup ? g.f : g.d;
    const int n_kb = K / (4 * epc);
    const long long wgs = (long long)max_items * (rows / kUnitRows);
    const bool few = wgs < kFewWorkgroups;
    if (n_kb == 1) return {4, 1, 4};
    if (n_kb < 4) return {4, 2, 4};
    if (n_kb <= 16) {
        if (few) return {4, 4, 4};
        return n_kb <= 8 ? GemvCfg{4, 1, 8} : GemvCfg{4, 1, 16};
    }
    if (tb == 1 && n_kb <= 48 && few) return {8, 8, 6};
    if (tb == 1) return {4, 4, 4};
    return {4, 4, kUnitBatch};
}

template <bool GATEUP, int WB, int TB>
hipError_t run_ks(const GemvArgs &a, hipStream_t s)
{
    const GemvCfg c = gemv_cfg(Fmt<WB>::epc, GATEUP, a.f.g, TB, a.f.max_items);
    if (c.is(4, 1, 4)) return run_gemv<GATEUP, WB, TB, 4, 1, 4>(a, s);
    if (c.is(4, 2, 4)) return run_gemv<GATEUP, WB, TB, 4, 2, 4>(a, s);
    if (c.is(4, 4, 4)) return run_gemv<GATEUP, WB, TB, 4, 4, 4>(a, s);
    if (c.is(4, 1, 8)) return run_gemv<GATEUP, WB, TB, 4, 1, 8>(a, s);
    if (c.is(4, 1, 16)) return run_gemv<GATEUP, WB, TB, 4, 1, 16>(a, s);
    if (c.is(8, 8, 6)) return run_gemv<GATEUP, WB, TB, 8, 8, 6>(a, s);
    return run_gemv<GATEUP, WB, TB, 4, 4, kUnitBatch>(a, s);
}

template <bool GATEUP, int WB>
hipError_t run_tb(const GemvArgs &a, hipStream_t s)
{
    switch (a.f.tb) {
    case 1: return run_ks<GATEUP, WB, 1>(a, s);
    case 2: return run_ks<GATEUP, WB, 2>(a, s);
    case 4: return run_ks<GATEUP, WB, 4>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

int gemv_tokens_per_item(const Geo &g, int max_tokens)
{
    // the smallest of 1, 2, 4 that covers the largest group the GEMV pass
    // gets, within the LDS budget of staged activations for both passes
    int tb = max_tokens <= 1 ? 1 : (max_tokens <= 2 ? 2 : 4);
    const int nch = (g.d > g.f ? g.d : g.f) / g.epc;
    while (tb > 1 && tb * nch * stage_bytes(g.wbits) > kStageBudget) tb /= 2;
    return tb;
}

hipError_t launch_gateup(const Fwd &f, hipStream_t s, bool *x16_staged)
{
    *x16_staged = false;
    GemvArgs a;
    a.f = f;
    a.n_wg = 0;
    // a union of at most 64 experts is scanned inside the kernel when every
    // expert is on the GEMV pass; otherwise one planning workgroup builds the
    // work lists first
    const int max_union = f.A < f.g.E ? f.A : f.g.E;
    a.plan_here = max_union <= kWave && f.max_mitems == 0 && f.max_sitems == 0
                      ? (f.N <= f.tb ? 2 : 1)
                      : 0;
    if (f.route_in && (a.plan_here != 2 || f.N > 2)) return hipErrorInvalidValue;
    if (!a.plan_here) {
        if (f.max_mitems > 0 || f.max_sitems > 0) {
            // the matrix-core passes run: their x16 in the same launch
            const long long n8 = (long long)f.N * f.g.d / 8;
            const dim3 grid((unsigned)(1 + (n8 + kPlanThreads - 1) / kPlanThreads));
            if (f.g.wbits == 8)
                hipLaunchKernelGGL(plan_stage_kernel<8>, grid, dim3(kPlanThreads), 0, s, f, n8);
            else
                hipLaunchKernelGGL(plan_stage_kernel<4>, grid, dim3(kPlanThreads), 0, s, f, n8);
            *x16_staged = true;
        } else {
            hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, f);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return f.g.wbits == 4 ? run_tb<true, 4>(a, s) : run_tb<true, 8>(a, s);
}

hipError_t launch_down(const Fwd &f, hipStream_t s)
{
    GemvArgs a;
    a.f = f;
    a.n_wg = 0;
    a.plan_here = 0;
    return f.g.wbits == 4 ? run_tb<false, 4>(a, s) : run_tb<false, 8>(a, s);
}

hipError_t launch_combine(const float *o, const float *w, int N, int k, int d, int A,
                          int has_shared, float *y, hipStream_t s)
{
    const long long n = (long long)N * (d / 4);
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, o, w, N,
                       k, d, A, has_shared, y);
    return hipGetLastError();
}

hipError_t launch_residual_rmsnorm(float *h, const float *y, float *a, int N, int d, float eps,
                                   hipStream_t s)
{
    const bool al = (uintptr_t)h % 16 == 0 && (uintptr_t)y % 16 == 0 && (uintptr_t)a % 16 == 0;
    const int rv = al ? norm_vec_width(d) : 0;
    if (!rv) {
        hipLaunchKernelGGL(residual_rmsnorm_kernel, dim3(N), dim3(kNormThreads), 0, s, h, y, a, d,
                           eps);
        return hipGetLastError();
    }
    return with_norm_width(rv, [&](auto w) {
        hipLaunchKernelGGL(residual_rmsnorm_vec_kernel<decltype(w)::value>, dim3(N),
                           dim3(kNormThreads), 0, s, h, y, a, d, eps);
        return hipGetLastError();
    });
}

bool combine_norm_supported(int d, const float *h, const float *a)
{
    return norm_vec_width(d) > 0 && (uintptr_t)h % 16 == 0 && (uintptr_t)a % 16 == 0;
}

hipError_t launch_combine_norm(const float *o, const float *w, int N, int k, int d, int A,
                               int has_shared, float *h, float *a, float eps, hipStream_t s)
{
    if (!combine_norm_supported(d, h, a)) return hipErrorInvalidValue;
    return with_norm_width(norm_vec_width(d), [&](auto wd) {
        hipLaunchKernelGGL(combine_norm_kernel<decltype(wd)::value>, dim3(N), dim3(kNormThreads),
                           0, s, o, w, k, d, A, has_shared, h, a, eps);
        return hipGetLastError();
    });
}

}  // namespace moe
