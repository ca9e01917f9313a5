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
//  * codes are turned into float16 in registers by OR-ing them into the
//    mantissa of 1024.0 (offset-binary codes, so the value is 1024 + q + 8
//    exactly) and multiplied with float16 activations by v_dot2_f32_f16,
//    which accumulates in float32; 1032 (or 1152) times the activation sum
//    is taken off once per chunk;
//  * a work item's activations are staged once per workgroup in LDS, each
//    chunk as float16 scaled by the power of two that brings the chunk's
//    largest magnitude into [2^13, 2^14) (an exact scaling, undone on the
//    chunk's partial sum together with the group scale);
//  * partial sums of a row are added across its lanes with DPP and lane
//    reads, always in the same order.
#include <hip/hip_ext.h>

#include "internal.h"

namespace moe {
namespace {

typedef __fp16 h2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2_t as_h2(uint32_t v) { return __builtin_bit_cast(h2_t, v); }

constexpr uint32_t kMagic = 0x64006400u;  // two float16 1024.0

template <int WB> struct Fmt;
template <> struct Fmt<4> { static constexpr int epc = 32, xdw = 16; };
template <> struct Fmt<8> { static constexpr int epc = 16, xdw = 8; };

// The float16 pairs of one 16-byte chunk of offset-binary codes (1024 + code
// + offset in each half), in the order the staged activations use.
template <int WB>
__device__ __forceinline__ void extract_chunk(uint4 w, uint32_t *h)
{
    const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if constexpr (WB == 4) {
            const uint32_t d8 = d[q] >> 8;
            h[4 * q + 0] = (d[q] & 0x000F000Fu) | kMagic;
            h[4 * q + 1] = (d[q] & 0x00F000F0u) | kMagic;
            h[4 * q + 2] = (d8 & 0x000F000Fu) | kMagic;
            h[4 * q + 3] = (d8 & 0x00F000F0u) | kMagic;
        } else {
            h[2 * q + 0] = (d[q] & 0x00FF00FFu) | kMagic;
            h[2 * q + 1] = ((d[q] >> 8) & 0x00FF00FFu) | kMagic;
        }
    }
}

template <int N>
__device__ __forceinline__ float dot_halves(const uint32_t *h, const uint32_t *xs)
{
    float acc = 0.0f;
#pragma unroll
    for (int q = 0; q < N; ++q) acc = __builtin_amdgcn_fdot2(as_h2(h[q]), as_h2(xs[q]), acc, false);
    return acc;
}

// float -> float16 with values below the smallest normal float16 set to zero,
// so the dot product and the correction term see the same number
__device__ __forceinline__ __fp16 to_h(float v)
{
    return fabsf(v) < 6.103515625e-05f ? (__fp16)0.0f : (__fp16)v;
}

__device__ __forceinline__ uint32_t pack2(__fp16 lo, __fp16 hi)
{
    h2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Stage one chunk of activations (already scaled) for the dot product and
// return the correction 1032*sum(A) + 1152*sum(B) (int4) or 1152*sum (int8).
template <int WB>
__device__ __forceinline__ float stage_chunk(const float4 *src, float scale, uint32_t *xs)
{
    constexpr int epc = Fmt<WB>::epc;
    float v[epc];
#pragma unroll
    for (int q = 0; q < epc / 4; ++q) {
        const float4 f4 = src[q];
        v[4 * q + 0] = f4.x * scale;
        v[4 * q + 1] = f4.y * scale;
        v[4 * q + 2] = f4.z * scale;
        v[4 * q + 3] = f4.w * scale;
    }
    if constexpr (WB == 4) {
        float sa = 0.0f, sb = 0.0f;
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            const float *e = v + 8 * blk;
            __fp16 a0 = to_h(e[0]), a4 = to_h(e[4]), a2 = to_h(e[2]), a6 = to_h(e[6]);
            __fp16 b1 = to_h(e[1] * 0.0625f), b5 = to_h(e[5] * 0.0625f);
            __fp16 b3 = to_h(e[3] * 0.0625f), b7 = to_h(e[7] * 0.0625f);
            xs[4 * blk + 0] = pack2(a0, a4);
            xs[4 * blk + 1] = pack2(b1, b5);
            xs[4 * blk + 2] = pack2(a2, a6);
            xs[4 * blk + 3] = pack2(b3, b7);
            sa += ((float)a0 + (float)a4) + ((float)a2 + (float)a6);
            sb += ((float)b1 + (float)b5) + ((float)b3 + (float)b7);
        }
        return 1032.0f * sa + 1152.0f * sb;
    } else {
        float s = 0.0f;
#pragma unroll
        for (int dw = 0; dw < 4; ++dw) {
            const float *e = v + 4 * dw;
            __fp16 a0 = to_h(e[0]), a1 = to_h(e[1]), a2 = to_h(e[2]), a3 = to_h(e[3]);
            xs[2 * dw + 0] = pack2(a0, a2);
            xs[2 * dw + 1] = pack2(a1, a3);
            s += ((float)a0 + (float)a2) + ((float)a1 + (float)a3);
        }
        return 1152.0f * s;
    }
}

constexpr int kGemvThreads = 256;
constexpr int kGemvWaves = kGemvThreads / kWave;

// staged activations per token per row chunk: XDW dwords, the correction and
// the chunk's inverse scale
__host__ __device__ constexpr int stage_bytes(int wb) { return (wb == 4 ? 16 : 8) * 4 + 8; }

// rounds of (token, chunk) activation pairs loaded before the weight loads
constexpr int kPreRounds = 2;

// rows per wave per row block
__host__ __device__ constexpr int rows_of(bool gateup, int cpl)
{
    return gateup ? (cpl == 1 ? 2 : 1) : (cpl == 1 ? 4 : (cpl <= 3 ? 2 : 1));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                              0xF, 0xF, true));
}

__device__ __forceinline__ float lane_f(float v, int l)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// Sum over aligned groups of L lanes (L a power of two <= 64); the result is
// valid in the first lane of each group.
template <int L>
__device__ __forceinline__ float seg_sum(float v)
{
    if constexpr (L >= 2) v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
    if constexpr (L >= 4) v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
    if constexpr (L >= 8) v += dpp<0x141>(v);   // row_half_mirror
    if constexpr (L >= 16) v += dpp<0x140>(v);  // row_mirror
    if constexpr (L == 32) v += __shfl_xor(v, 16, kWave);
    if constexpr (L == 64) v = (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
    return v;
}

__device__ __forceinline__ float wave_max_dpp(float v)
{
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x141>(v));
    v = fmaxf(v, dpp<0x140>(v));
    return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

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
    int n_rbg;              // workgroups per item
    int iters;              // row blocks per workgroup
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

// One workgroup (4 waves) works on one item: up to TB tokens of one expert.
// The item's activations are staged once in LDS (float16, scaled by a power of
// two per chunk, in the order the dot product consumes them). Each wave then
// owns R rows (times 64/LPR rows that share a wave when rows are short) per
// row block; every lane reads CPL 16-byte chunks of each row, one 128-bit load
// per chunk, with the next block's loads issued before the current block is
// computed. Row sums are added across lanes with DPP and lane reads.
//
// gate/up pass with a union of at most 64 experts: the workgroup finds its
// item from the union itself (no separate planning launch) and records the
// item list for the down pass.
template <bool GATEUP, int WB, int CPL, int LPR, int TB>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(GemvArgs ga)
{
    constexpr int XDW = Fmt<WB>::xdw, EPC = Fmt<WB>::epc;
    constexpr int XQ = XDW / 4;              // uint4 per staged chunk
    constexpr int RPI = kWave / LPR;         // rows sharing a wave
    constexpr int NCH = CPL * LPR;           // chunks per row
    constexpr int R = rows_of(GATEUP, CPL);
    constexpr int ROWS = kGemvWaves * R * RPI;  // rows per row block
    constexpr int NM = GATEUP ? 2 : 1;          // gate and up, or down
    static_assert(CPL == 1 || LPR == kWave, "multi-chunk lanes need full-wave rows");

    extern __shared__ uint4 lds_x[];          // [TB][XQ][NCH] staged activations
    float2 *lds_ci = reinterpret_cast<float2 *>(lds_x + TB * XQ * NCH);  // [TB][NCH]
    __shared__ Item s_item;
    __shared__ int s_expert;

    const Fwd &f = ga.f;
    const Geo &g = f.g;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int item_idx = blockIdx.x / ga.n_rbg;
    const int rbg = blockIdx.x % ga.n_rbg;
    // The expert is needed first (the weight loads only depend on it); the
    // item's tokens are resolved after those loads are issued when possible.
    int expert;
    Item it;
    bool resolved = true;
    if (GATEUP && ga.plan_here == 2) {
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
                if (rbg == 0 && rel == 0) *f.n_items = nsh + nu;
            }
            __syncthreads();
            expert = s_expert;
            if (expert == -2) return;  // beyond the union: uniform exit
        }
    } else if (GATEUP && ga.plan_here == 1) {
        if (wave == 0) {
            const int total = find_item<TB>(f, item_idx, &s_item);
            if (lane == 0) {
                if (rbg == 0 && s_item.count > 0) f.items[item_idx] = s_item;
                // the first routed item's first workgroup publishes the total
                const int nsh = f.has_shared ? (f.N + TB - 1) / TB : 0;
                if (rbg == 0 && item_idx == nsh) *f.n_items = min(total, f.max_items);
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
    const uint8_t *blk = expert >= 0 ? f.pool + (size_t)expert * f.stride : f.shared;
    const int seg = lane / LPR, li = lane % LPR;
    const int cols = GATEUP ? g.d : g.f;
    const int rows = GATEUP ? g.f : g.d;
    const long long row_bytes = GATEUP ? g.row_gu : g.row_dn;
    const long long spr = GATEUP ? g.spr_gu : g.spr_dn;
    const uint8_t *q0 = blk + (GATEUP ? 0 : g.off_dn);
    const uint8_t *q1 = blk + g.off_up;
    const uint8_t *s0 = blk + (GATEUP ? g.off_gs : g.off_ds);
    const uint8_t *s1 = blk + g.off_us;
    const float *in = GATEUP ? f.x : f.h;
    float *out = GATEUP ? f.h : f.o;

    uint4 w[R][CPL][NM];
    float sc[R][CPL][NM];
    auto load_block = [&](int blk_idx, uint4 (&wv)[R][CPL][NM], float (&sv)[R][CPL][NM]) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const long long row = min(blk_idx * ROWS + (wave * R + r) * RPI + seg, rows - 1);
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const int c = li + j * LPR;
                const long long grp = g.group ? (long long)c * EPC / g.group : 0;
                wv[r][j][0] = *reinterpret_cast<const uint4 *>(q0 + row * row_bytes + c * 16);
                sv[r][j][0] = *reinterpret_cast<const float *>(s0 + (row * spr + grp) * 4);
                if (GATEUP) {
                    wv[r][j][NM - 1] = *reinterpret_cast<const uint4 *>(q1 + row * row_bytes + c * 16);
                    sv[r][j][NM - 1] = *reinterpret_cast<const float *>(s1 + (row * spr + grp) * 4);
                }
            }
        }
    };
    // ---- the item's tokens -----------------------------------------------------
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
        if (rbg == 0 && tid == 0 && it.count > 0) f.items[item_idx] = it;
        if (it.count <= 0) return;  // uniform: inconsistent offsets give no tokens
    }
    const int count = min(it.count, TB);

    // ---- stage the activations: loads first, then the weights ----------------
    // (token, chunk) pairs are spread over the threads; a round covers one
    // pair per thread. Each pair is staged on its own: float16 scaled by the
    // power of two that brings the chunk's largest magnitude into
    // [2^13, 2^14) (exact, undone per chunk with the group scale). The first
    // rounds are loaded before the weight loads are issued, so their data do
    // not wait behind the weights.
    constexpr int NPAIR = TB * NCH;
    constexpr int ROUNDS = (NPAIR + kGemvThreads - 1) / kGemvThreads;
    constexpr int PRE = ROUNDS < kPreRounds ? ROUNDS : kPreRounds;
    auto pair_src = [&](int q) -> const float * {
        const int i = q / NCH, c = q % NCH;
        if (i >= count) return nullptr;
        const int p = it.p0 + i;
        size_t r;
        if (!GATEUP)
            r = (size_t)p;
        else if (it.expert < 0)
            r = (size_t)(p - f.A);
        else  // values read from the permutation are clamped into range
            r = f.N == 1 ? 0 : (size_t)(min(max(f.perm[p], 0), f.A - 1) / f.k);
        return in + r * cols + (size_t)c * EPC;
    };
    float4 xv[PRE][EPC / 4];
#pragma unroll
    for (int r = 0; r < PRE; ++r) {
        const int q = tid + r * kGemvThreads;
        const float *src = q < NPAIR ? pair_src(q) : nullptr;
        if (src) {
#pragma unroll
            for (int v = 0; v < EPC / 4; ++v) xv[r][v] = reinterpret_cast<const float4 *>(src)[v];
        }
    }
    const int first_blk = rbg * ga.iters;
    load_block(first_blk, w, sc);
    auto stage_pair = [&](int q, const float4 (&v)[EPC / 4]) {
        const int i = q / NCH, c = q % NCH;
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
        const float corr = stage_chunk<WB>(v, ldexpf(1.0f, sh), xs);
        lds_ci[i * NCH + c] = make_float2(corr, ldexpf(1.0f, -sh));
#pragma unroll
        for (int u = 0; u < XQ; ++u)
            lds_x[(i * XQ + u) * NCH + c] = make_uint4(xs[4 * u], xs[4 * u + 1], xs[4 * u + 2],
                                                       xs[4 * u + 3]);
    };
#pragma unroll
    for (int r = 0; r < PRE; ++r) {
        const int q = tid + r * kGemvThreads;
        if (q < NPAIR && q / NCH < count) stage_pair(q, xv[r]);
    }
#pragma unroll 1
    for (int r = PRE; r < ROUNDS; ++r) {
        const int q = tid + r * kGemvThreads;
        const float *src = q < NPAIR ? pair_src(q) : nullptr;
        if (src) {
            float4 v[EPC / 4];
#pragma unroll
            for (int u = 0; u < EPC / 4; ++u) v[u] = reinterpret_cast<const float4 *>(src)[u];
            stage_pair(q, v);
        }
    }
    __syncthreads();
    int orow[TB];
#pragma unroll
    for (int i = 0; i < TB; ++i) {
        const int p = it.p0 + min(i, count - 1);
        orow[i] = (!GATEUP && it.expert >= 0) ? min(max(f.perm[p], 0), f.A - 1) : p;
    }

    // ---- stream the rows ------------------------------------------------------
    const int n_blk = (rows + ROWS - 1) / ROWS;
    const int last_blk = min(first_blk + ga.iters, n_blk);
    for (int b = first_blk; b < last_blk; ++b) {
        uint4 wn[R][CPL][NM];
        float sn[R][CPL][NM];
        if (b + 1 < last_blk) load_block(b + 1, wn, sn);
        float acc[R][TB][NM];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int i = 0; i < TB; ++i)
#pragma unroll
                for (int m = 0; m < NM; ++m) acc[r][i][m] = 0.0f;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = li + j * LPR;
            uint32_t hw[R][NM][XDW];
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < NM; ++m) extract_chunk<WB>(w[r][j][m], hw[r][m]);
#pragma unroll
            for (int i = 0; i < TB; ++i) {
                if (i >= count) break;
                uint32_t xs[XDW];
#pragma unroll
                for (int q = 0; q < XQ; ++q) {
                    const uint4 v = lds_x[(i * XQ + q) * NCH + c];
                    xs[4 * q] = v.x;
                    xs[4 * q + 1] = v.y;
                    xs[4 * q + 2] = v.z;
                    xs[4 * q + 3] = v.w;
                }
                const float2 ci = lds_ci[i * NCH + c];
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int m = 0; m < NM; ++m)
                        acc[r][i][m] = fmaf(sc[r][j][m] * ci.y,
                                            dot_halves<XDW>(hw[r][m], xs) - ci.x, acc[r][i][m]);
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = b * ROWS + (wave * R + r) * RPI + seg;
#pragma unroll
            for (int i = 0; i < TB; ++i) {
                if (i >= count) break;
                float v[NM];
#pragma unroll
                for (int m = 0; m < NM; ++m) v[m] = seg_sum<LPR>(acc[r][i][m]);
                if (li == 0 && row < rows) {
                    float o;
                    if (GATEUP) {
                        const float gv = v[0], uv = v[NM - 1];
                        o = gv / (1.0f + expf(-gv)) * uv;
                    } else {
                        o = v[0];
                    }
                    out[(size_t)orow[i] * rows + row] = o;
                }
            }
        }
        if (b + 1 < last_blk) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int j = 0; j < CPL; ++j)
#pragma unroll
                    for (int m = 0; m < NM; ++m) {
                        w[r][j][m] = wn[r][j][m];
                        sc[r][j][m] = sn[r][j][m];
                    }
        }
    }
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
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(Fwd f)
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
    const int pass = pass_of(f, T);
    const int sh_pass = f.has_shared ? pass_of(f, f.N) : -1;
    Item *const lists[3] = {f.items, f.mitems, f.sitems};
    int32_t *const counts[3] = {f.n_items, f.n_mitems, f.n_sitems};
    const int maxes[3] = {f.max_items, f.max_mitems, f.max_sitems};
    const int sizes[3] = {f.tb, kMfmaBigTokens, kMfmaSmallTokens};
#pragma unroll
    for (int l = 0; l < 3; ++l) {
        const int sz = sizes[l], mx = maxes[l];
        const int nsh = sh_pass == l ? (f.N + sz - 1) / sz : 0;
        const int nb = pass == l ? (T + sz - 1) / sz : 0;
        int tot;
        const int base = nsh + block_excl_scan(nb, tot);  // uniform call: every thread
        if (mx <= 0) continue;
        for (int b = u; b < nsh && b < mx; b += kPlanThreads) {
            Item it = {-1, f.A + b * sz, min(sz, f.N - b * sz), 0};
            lists[l][b] = it;
        }
        for (int b = 0; b < nb && base + b < mx; ++b) {
            Item it = {e, s0 + b * sz, min(sz, T - b * sz), 0};
            lists[l][base + b] = it;
        }
        if (u == 0) *counts[l] = min(nsh + tot, mx);
    }
}

// ---- combine and chaining ---------------------------------------------------

__global__ __launch_bounds__(256) void combine_kernel(
    const float *__restrict__ o, const float *__restrict__ w, int N, int k, int d, int A,
    int has_shared, float *__restrict__ y)
{
    const int nq = d / 4;
    const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long long)N * nq) return;
    const int t = (int)(idx / nq), q = (int)(idx % nq);
    float4 acc = has_shared ? reinterpret_cast<const float4 *>(o + (size_t)(A + t) * d)[q]
                            : make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
        const float wj = w[(size_t)t * k + j];
        const float4 v = reinterpret_cast<const float4 *>(o + ((size_t)t * k + j) * d)[q];
        acc.x = fmaf(wj, v.x, acc.x);
        acc.y = fmaf(wj, v.y, acc.y);
        acc.z = fmaf(wj, v.z, acc.z);
        acc.w = fmaf(wj, v.w, acc.w);
    }
    reinterpret_cast<float4 *>(y + (size_t)t * d)[q] = acc;
}

__global__ __launch_bounds__(256) void residual_rmsnorm_kernel(
    float *__restrict__ h, const float *__restrict__ y, float *__restrict__ a, int d, float eps)
{
    __shared__ float part[256 / kWave];
    const int t = blockIdx.x;
    float *ht = h + (size_t)t * d;
    float ss = 0.0f;
    for (int i = threadIdx.x; i < d; i += 256) {
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
    for (int i = threadIdx.x; i < d; i += 256) a[(size_t)t * d + i] = ht[i] * r;
}

// ---- dispatch -------------------------------------------------------------

template <bool GATEUP, int WB, int CPL>
constexpr int rows_per_block(int lpr)
{
    return kGemvWaves * rows_of(GATEUP, CPL) * (kWave / lpr);
}

struct Launch {
    int n_rbg, iters;
    long long blocks;
};

// Workgroups the device keeps resident at once for a kernel (a per-process
// cache of the occupancy query; 0 when the query fails).
template <typename K>
long long resident_blocks(K kernel, size_t lds)
{
    static long long cache[16] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) return 0;
    if (cache[dev] == 0) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kGemvThreads, lds) !=
                hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        cache[dev] = (long long)per_cu * cus;
    }
    return cache[dev];
}

Launch plan_launch(int rows, int rows_per_blk, int max_items, long long resident = 0)
{
    Launch L;
    const long long n_blk = (rows + rows_per_blk - 1) / rows_per_blk;
    // one workgroup per row block while the grid fits the chip in one
    // resident round; beyond that each workgroup takes several row blocks,
    // loading the next one while it computes the current one
    const long long cap = resident > 0 ? resident : 2048;
    long long iters = ((long long)max_items * n_blk + cap - 1) / cap;
    iters = iters < 1 ? 1 : (iters > 8 ? 8 : iters);
    L.iters = (int)iters;
    L.n_rbg = (int)((n_blk + iters - 1) / iters);
    L.blocks = (long long)max_items * L.n_rbg;
    return L;
}

template <bool GATEUP, int WB, int CPL, int LPR, int TB>
hipError_t run_gemv(GemvArgs a, hipStream_t s)
{
    constexpr int ROWS = kGemvWaves * rows_of(GATEUP, CPL) * (kWave / LPR);
    const size_t lds = (size_t)TB * CPL * LPR * stage_bytes(WB);
    const Launch L = plan_launch(GATEUP ? a.f.g.f : a.f.g.d, ROWS, a.f.max_items,
                                 resident_blocks(gemv_kernel<GATEUP, WB, CPL, LPR, TB>, lds));
    a.n_rbg = L.n_rbg;
    a.iters = L.iters;
    if (L.blocks <= 0) return hipSuccess;
    if (L.blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    const hipEvent_t *ev = GATEUP ? a.f.ev_gu : a.f.ev_dn;
    if (ev[0] || ev[1])  // events taken by the dispatch itself, around this kernel only
        hipExtLaunchKernelGGL((gemv_kernel<GATEUP, WB, CPL, LPR, TB>), dim3((unsigned)L.blocks),
                              dim3(kGemvThreads), lds, s, ev[0], ev[1], 0, a);
    else
        hipLaunchKernelGGL((gemv_kernel<GATEUP, WB, CPL, LPR, TB>), dim3((unsigned)L.blocks),
                           dim3(kGemvThreads), lds, s, a);
    return hipGetLastError();
}

template <bool GATEUP, int WB, int CPL, int LPR>
hipError_t run_tb(const GemvArgs &a, hipStream_t s)
{
    switch (a.f.tb) {
    case 1: return run_gemv<GATEUP, WB, CPL, LPR, 1>(a, s);
    case 2: return run_gemv<GATEUP, WB, CPL, LPR, 2>(a, s);
    case 4:
        if constexpr (4 * CPL * LPR * stage_bytes(WB) <= 65536)
            return run_gemv<GATEUP, WB, CPL, LPR, 4>(a, s);
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

template <bool GATEUP, int WB>
hipError_t dispatch_shape(int cpl, int lpr, const GemvArgs &a, hipStream_t s)
{
    if (lpr == kWave) {
        switch (cpl) {
        case 1: return run_tb<GATEUP, WB, 1, 64>(a, s);
        case 2: return run_tb<GATEUP, WB, 2, 64>(a, s);
        case 3: return run_tb<GATEUP, WB, 3, 64>(a, s);
        case 4: return run_tb<GATEUP, WB, 4, 64>(a, s);
        case 6: return run_tb<GATEUP, WB, 6, 64>(a, s);
        case 8: return run_tb<GATEUP, WB, 8, 64>(a, s);
        default: return hipErrorInvalidValue;
        }
    }
    if (cpl != 1) return hipErrorInvalidValue;
    switch (lpr) {
    case 2: return run_tb<GATEUP, WB, 1, 2>(a, s);
    case 4: return run_tb<GATEUP, WB, 1, 4>(a, s);
    case 8: return run_tb<GATEUP, WB, 1, 8>(a, s);
    case 16: return run_tb<GATEUP, WB, 1, 16>(a, s);
    case 32: return run_tb<GATEUP, WB, 1, 32>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

int gemv_tokens_per_item(const Geo &g, int n_tokens)
{
    // the smallest of 1, 2, 4 that covers the batch, within 64 KB of staged
    // activations for both passes (an expert has at most n_tokens tokens)
    int tb = n_tokens <= 1 ? 1 : (n_tokens <= 2 ? 2 : 4);
    const int worst = (g.gu_cpl * g.gu_lpr > g.dn_cpl * g.dn_lpr ? g.gu_cpl * g.gu_lpr
                                                                  : g.dn_cpl * g.dn_lpr) *
                      stage_bytes(g.wbits);
    while (tb > 1 && tb * worst > 65536) tb /= 2;
    return tb;
}

hipError_t launch_gateup(const Fwd &f, hipStream_t s)
{
    GemvArgs a;
    a.f = f;
    a.n_rbg = a.iters = 0;
    // a union of at most 64 experts is scanned inside the kernel when no
    // expert goes to the MFMA pass; otherwise one planning workgroup builds
    // both work lists first
    const int max_union = f.A < f.g.E ? f.A : f.g.E;
    a.plan_here = max_union <= kWave && f.max_mitems == 0 && f.max_sitems == 0
                      ? (f.N <= f.tb ? 2 : 1)
                      : 0;
    if (!a.plan_here) {
        hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, f);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return f.g.wbits == 4 ? dispatch_shape<true, 4>(f.g.gu_cpl, f.g.gu_lpr, a, s)
                          : dispatch_shape<true, 8>(f.g.gu_cpl, f.g.gu_lpr, a, s);
}

hipError_t launch_down(const Fwd &f, hipStream_t s)
{
    GemvArgs a;
    a.f = f;
    a.n_rbg = a.iters = 0;
    a.plan_here = 0;
    return f.g.wbits == 4 ? dispatch_shape<false, 4>(f.g.dn_cpl, f.g.dn_lpr, a, s)
                          : dispatch_shape<false, 8>(f.g.dn_cpl, f.g.dn_lpr, a, s);
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
    hipLaunchKernelGGL(residual_rmsnorm_kernel, dim3(N), dim3(256), 0, s, h, y, a, d, eps);
    return hipGetLastError();
}

}  // namespace moe
