// topk.h - the per-token top-k selection of the Route stage, shared by the
// top-k kernel and the fused route tail (top-k, union and counting in one
// workgroup).
//
// Colibri pages, "Public Colibri Observation and Revision Ledger", section
// "Exact Architecture and Data-Flow Reconstruction": sigmoid gate over all
// experts (n_group = 1), float32 gate parameters; the k best experts per token.
#pragma once

#include "internal.h"

namespace moe {

// most slices of the contraction the GEMM router splits into
constexpr int kMaxSlices = 16;
constexpr int kMaxPerLane = MOE_MAX_EXPERTS / kWave;  // 16

// 1 / (1 + e^-l) in float32. For l >= 0 it is taken as 1 - e / (1 + e) with
// e = e^-l: the small term keeps its relative precision and only the final
// subtraction rounds, so scores close to 1 (saturated logits) stay as far
// apart as their float32 values are; 1 / (1 + e) would round 1 + e first and
// merge scores up to 2^-23 apart. For l < 0 the quotient is already precise.
__device__ __forceinline__ float sigmoidf(float l)
{
    if (l >= 0.0f) {
        const float e = expf(-l);
        return 1.0f - e / (1.0f + e);
    }
    return 1.0f / (1.0f + expf(-l));
}

// Order-preserving map of float bits onto unsigned integers (NaN above +inf).
__device__ __forceinline__ uint32_t sortable(float v)
{
    uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// (bh, bl) = the larger of (bh, bl) and (oh, ol), compared as one 64-bit key
__device__ __forceinline__ void key_max(uint32_t &bh, uint32_t &bl, uint32_t oh, uint32_t ol)
{
    if (oh > bh || (oh == bh && ol > bl)) {
        bh = oh;
        bl = ol;
    }
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}

// The largest 64-bit key (bh, bl) of the wave, in every lane: within each
// row of 16 lanes by DPP moves (quad swaps, then the half-row and row
// mirrors), then over the four rows by lane reads. Every lane of the wave
// must be active.
__device__ __forceinline__ void wave_max_key(uint32_t &bh, uint32_t &bl)
{
    key_max(bh, bl, dpp_u32<0xB1>(bh), dpp_u32<0xB1>(bl));    // lanes i ^ 1
    key_max(bh, bl, dpp_u32<0x4E>(bh), dpp_u32<0x4E>(bl));    // lanes i ^ 2
    key_max(bh, bl, dpp_u32<0x141>(bh), dpp_u32<0x141>(bl));  // half-row mirror
    key_max(bh, bl, dpp_u32<0x140>(bh), dpp_u32<0x140>(bl));  // row mirror
    uint32_t h = __builtin_amdgcn_readlane(bh, 0), l = __builtin_amdgcn_readlane(bl, 0);
#pragma unroll
    for (int r = 1; r < 4; ++r)
        key_max(h, l, __builtin_amdgcn_readlane(bh, 16 * r), __builtin_amdgcn_readlane(bl, 16 * r));
    bh = h;
    bl = l;
}

// Opt-in router variant. sel (may be null): a bias that only steers the
// selection, the key of expert e being the float32 sum s + sel[e] while the
// weight stays the score; norm: each weight is divided by the sum of the k
// chosen scores (added in rank order); every weight is then multiplied by
// scale. top_p in (0, 1): a lossy cutoff, slot j kept when j == 0 or the
// float32 sum of the scores ranked before it is below top_p times the sum of
// all k (both summed in rank order); a dropped slot gets id -1 and weight 0.
// The default (sel null, norm 0, scale 1, top_p 0) keeps w = s.
struct TopkOpt {
    const float *sel = nullptr;
    int norm = 0;
    float scale = 1.0f;
    float top_p = 0.0f;
    bool any() const
    {
        return sel || norm || scale != 1.0f || (top_p > 0.0f && top_p < 1.0f);
    }
};

// One wave selects token t's k best experts: k rounds of a wave-wide max over
// 64-bit keys (sortable score, then inverted id so equal scores go to the
// lower id). With P == 1, `in` holds the scores [N][E]; with P > 1 it holds
// the router's raw partial sums [P][N][E] and the score is
// sigmoid(sum over slices in order + bias). The lane holding each round's
// winner writes ids/w[t * k + j] and, when lds_ids is not null,
// lds_ids[t * k + j].
// OPT false: the options are ignored (the default reading, compiled without
// them); true: they apply. PB: a bound of P known at compile time (the
// partial sums of 64 / PB experts per lane are loaded at a time).
// MPL: experts per lane the code is unrolled for (E <= 64 * MPL).
template <bool OPT, int PB, int MPL>
__device__ __forceinline__ void topk_wave_impl(const float *__restrict__ in, int P,
                                               const float *__restrict__ b, int N, int E, int k,
                                               int t, int32_t *__restrict__ ids,
                                               float *__restrict__ w, int32_t *lds_ids,
                                               TopkOpt opt)
{
    constexpr int kMaxPerLane = MPL;
    const int lane = threadIdx.x % kWave;
    uint32_t hi[kMaxPerLane];
    float sv[kMaxPerLane] = {};
    uint32_t taken = 0;
    if (P == 1) {
#pragma unroll
        for (int m = 0; m < kMaxPerLane; ++m) {
            const int e = lane + m * kWave;
            sv[m] = e < E ? in[(size_t)t * E + e] : 0.0f;
        }
    } else {
        // the partial sums of kGroup experts per lane at a time, every load
        // of a group issued together (slices past P and experts past E read
        // valid entries that are not used), then added in slice order
        constexpr int kSl = PB < kMaxSlices ? PB : kMaxSlices;
        constexpr int kGroup = (64 / kSl) < kMaxPerLane ? 64 / kSl : kMaxPerLane;
#pragma unroll
        for (int g = 0; g < kMaxPerLane; g += kGroup) {
            if (g * kWave >= E) break;
            float part[kGroup][kSl], bias[kGroup];
#pragma unroll
            for (int mm = 0; mm < kGroup; ++mm) {
                const int e = min(lane + (g + mm) * kWave, E - 1);
#pragma unroll
                for (int p = 0; p < kSl; ++p)
                    part[mm][p] = in[((size_t)min(p, P - 1) * N + t) * E + e];
                bias[mm] = b ? b[e] : 0.0f;
            }
#pragma unroll
            for (int mm = 0; mm < kGroup; ++mm) {
                const int e = lane + (g + mm) * kWave;
                float l = 0.0f;
#pragma unroll
                for (int p = 0; p < kSl; ++p)
                    if (p < P) l += part[mm][p];
                sv[g + mm] = e < E ? sigmoidf(l + bias[mm]) : 0.0f;
            }
        }
    }
#pragma unroll
    for (int m = 0; m < kMaxPerLane; ++m) {
        const int e = lane + m * kWave;
        float key = sv[m];
        if (OPT && opt.sel && e < E) key = sv[m] + opt.sel[e];  // one float32 rounding
        hi[m] = e < E ? sortable(key) : 0u;
        if (e >= E) taken |= 1u << m;
    }
    const bool cut = OPT && opt.top_p > 0.0f && opt.top_p < 1.0f;
    // with any option, lane j writes slot j after the rounds
    const bool post = OPT && (cut || opt.norm || opt.scale != 1.0f);
    // chosen scores in rank order: their sum, and lane j's round-j score, id
    // and the sum of the scores ranked before it
    float wsum = 0.0f, wmine = 0.0f, wbefore = 0.0f;
    int idmine = -1;
    for (int j = 0; j < k; ++j) {
        uint32_t bh = 0, bl = 0;  // best key of this lane: (hi, ~id)
        int bm = -1;
#pragma unroll
        for (int m = 0; m < kMaxPerLane; ++m) {
            if (taken & (1u << m)) continue;
            uint32_t lo = 0xFFFFFFFFu - (uint32_t)(lane + m * kWave);
            if (bm < 0 || hi[m] > bh || (hi[m] == bh && lo > bl)) { bh = hi[m]; bl = lo; bm = m; }
        }
        if (bm < 0) { bh = 0; bl = 0; }
        float bs = bm >= 0 ? sv[0] : 0.0f;
#pragma unroll
        for (int m = 1; m < kMaxPerLane; ++m)
            if (m == bm) bs = sv[m];
        wave_max_key(bh, bl);
        const int id = (int)(0xFFFFFFFFu - bl);
        if (bm >= 0 && lane + bm * kWave == id) {
            // the lane holding the winner records it
            taken |= 1u << bm;
            if (!post) {
                ids[(size_t)t * k + j] = id;
                w[(size_t)t * k + j] = bs;
                if (lds_ids) lds_ids[t * k + j] = id;
            }
        }
        if (post) {
            const float ws = __shfl(bs, id % kWave, kWave);  // the winner's score
            if (lane == j) {
                wmine = ws;
                idmine = id;
                wbefore = wsum;
            }
            wsum += ws;
        }
    }
    if (post && lane < k) {
        const bool keep = !cut || lane == 0 || wbefore < opt.top_p * wsum;
        const int idv = keep ? idmine : -1;
        ids[(size_t)t * k + lane] = idv;
        w[(size_t)t * k + lane] =
            !keep ? 0.0f : (opt.norm ? wmine / wsum * opt.scale : wmine * opt.scale);
        if (lds_ids) lds_ids[t * k + lane] = idv;
    }
}

template <bool OPT, int PB = kMaxSlices>
__device__ __forceinline__ void topk_wave(const float *__restrict__ in, int P,
                                          const float *__restrict__ b, int N, int E, int k, int t,
                                          int32_t *__restrict__ ids, float *__restrict__ w,
                                          int32_t *lds_ids, TopkOpt opt = TopkOpt())
{
    // up to 256 experts, each round scans four candidates per lane, not 16
    if (E <= 4 * kWave)
        topk_wave_impl<OPT, PB, 4>(in, P, b, N, E, k, t, ids, w, lds_ids, opt);
    else
        topk_wave_impl<OPT, PB, kMaxPerLane>(in, P, b, N, E, k, t, ids, w, lds_ids, opt);
}

}  // namespace moe
