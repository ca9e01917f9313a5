// expert_mfma.hip - expert math for token groups large enough to be a dense
// contraction (prefill, the shared expert of a batch, experts hit by several
// tokens).
//
// Colibri pages: "Public Colibri Observation and Revision Ledger", section
// "Exact Architecture and Data-Flow Reconstruction" (three-matrix expert MLP,
// always-on shared expert), README "Get started" (int4 experts with group
// scales).
//
// For one expert and up to MT of its tokens (MT = 128 for large groups, 32
// for small ones), a workgroup of 4 or 8 waves computes 128 or 256 output
// rows of gate and up (each), or 128 or 512 rows of down, over the full
// contraction:
//   gate/up:  h[p][r] = silu(sum_c Wg[r][c] x_t[c]) * (sum_c Wu[r][c] x_t[c])
//   down:     o[out(p)][r] = sum_c Wd[r][c] h[p][c]
// on v_mfma_f32_16x16x32_f16 (float16 products, float32 accumulation):
//  * the weights are read in their 1 KB units (16 rows x 128 int4 columns):
//    one 16-byte load per lane is one unit, and the lane's 32 codes are its
//    weight operand for four MFMA steps; they are expanded in registers: OR
//    into the mantissa of 1024 (exact, a constant bias per code position),
//    then the bias subtracted (exact) or, in the 32-token gate/up pass with
//    one scale per unit step, taken out by products of the activations with
//    a constant operand; where groups are finer than a unit step, times the
//    group scale (one float16 rounding);
//  * within each 8-column group the columns are taken in the order
//    0,4,1,5,2,6,3,7 on both operands, which lets one 32-bit word of codes
//    feed one MFMA operand without shuffles;
//  * activations come as float16 rows already in the operand's column order
//    (x converted once per call by plan_stage_kernel or stage_x16_kernel, h
//    written so by the gate/up epilogue; int4 high-nibble columns divided by
//    16) and are copied into LDS one unit step at a time, double-buffered;
//  * each wave owns two or four unit rows and all MT tokens; weight
//    loads run up to four steps ahead of the matrix cores.
// Workgroups are mapped so that those sharing an expert (and so its weights
// and its tokens) land on the same XCD and share its L2.
#include <hip/hip_ext.h>

#include <type_traits>

#include "internal.h"

namespace moe {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Waves per workgroup and unit rows per wave. 32-token items: 4 waves of 2
// unit rows. 128-token items: 8 waves (two per SIMD, so one wave's products
// overlap the other's operand work) of 2 unit rows for gate/up (two
// matrices) or 4 for down: 64 weight rows per wave, so each activation
// fragment read from LDS feeds 64 rows of products; the accumulators (128
// tokens x 64 rows, 128 registers) still fit two waves per SIMD. A workgroup
// covers 128 rows of gate/up or 128 of down (32-token items), 256 of gate/up
// or 512 of down (128-token items).
__host__ __device__ constexpr int waves_per_wg(int mf) { return mf < 8 ? 4 : 8; }
__host__ __device__ constexpr int tiles_per_wave(bool gateup, int mf)
{
    return mf < 8 ? 2 : (gateup ? 2 : 4);
}
__host__ __device__ constexpr int rows_per_wg(bool gateup, int mf)
{
    return waves_per_wg(mf) * tiles_per_wave(gateup, mf) * kUnitRows;
}
constexpr int kXcds = 8;

// Code format: a unit has UC columns (one step), NS k-steps of 32, and each
// lane's 16 bytes cover QW columns of its row (one quarter of the unit).
// Activations are loaded in NA parts per step.
template <int WB> struct MFmt;
template <> struct MFmt<4> { static constexpr int UC = 128, NS = 4, QW = 32, NA = 2; };
template <> struct MFmt<8> { static constexpr int UC = 64, NS = 2, QW = 16, NA = 1; };

__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

// The 8 codes of k-step s of a lane's 16 bytes as float16:
// int4: the codes of 32-bit word s (element j in bits 4j..4j+3), in the
//   column order 0,4,1,5,2,6,3,7;
// int8: the bytes of words 2s and 2s+1, in the column order 0,2,1,3,4,6,5,7.
// Codes are offset binary (u = q + 8, or q + 128). ORed into the mantissa of
// 1024 (one AND-OR per pair of codes, exact), a code in bits 0..3 of a half
// gives 1024 + u = 1032 + q, one in bits 4..7 gives 1024 + 16 u = 1152 + 16 q
// (its activation is stored divided by 16, so the product is (72 + q) x),
// an int8 code 1024 + u = 1152 + q. One shift per word brings the other
// half of the codes into place. DQ says what leaves:
//   kDqBiased: those biased values (the bias is taken out on the matrix
//     cores, by products with a constant operand: bias_operand);
//   kDqExact: q (16 q in bits 4..7), one packed subtraction per pair;
//   kDqScaled: that times the group scale, one float16 rounding.
constexpr int kDqBiased = 0, kDqExact = 1, kDqScaled = 2;

template <int WB, int DQ>
__device__ __forceinline__ half8_t dequant8(const uint4 &u, int s, half2_t s2)
{
    const uint32_t magic = 0x64006400u;
    const uint32_t d[4] = {u.x, u.y, u.z, u.w};
    uint32_t v[4];
    if constexpr (WB == 4) {
        const uint32_t w = d[s], w8 = w >> 8, lo = 0x000F000Fu, hi = 0x00F000F0u;
        v[0] = and_or(w, lo, magic);
        v[1] = and_or(w, hi, magic);
        v[2] = and_or(w8, lo, magic);
        v[3] = and_or(w8, hi, magic);
    } else {
        const uint32_t w0 = d[2 * s], w1 = d[2 * s + 1], m = 0x00FF00FFu;
        v[0] = and_or(w0, m, magic);
        v[1] = and_or(w0 >> 8, m, magic);
        v[2] = and_or(w1, m, magic);
        v[3] = and_or(w1 >> 8, m, magic);
    }
    half2_t p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        p[i] = as_h2(v[i]);
        if constexpr (DQ != kDqBiased) {
            const _Float16 off = (WB == 4 && (i & 1) == 0) ? (_Float16)1032.0f : (_Float16)1152.0f;
            p[i] = p[i] - half2_t{off, off};
        }
        if constexpr (DQ == kDqScaled) p[i] = p[i] * s2;
    }
    half8_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[2 * i] = p[i][0];
        r[2 * i + 1] = p[i][1];
    }
    return r;
}

// The weight operand whose products with the activations give minus the
// biases that kDqBiased leaves: -1032 at the low-nibble positions, -1152 at
// the others (int8: everywhere). Exact in float16. The product does not
// depend on the weight row, so one accumulator per token block carries it.
template <int WB>
__device__ __forceinline__ half8_t bias_operand()
{
    half8_t r;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        r[i] = (WB == 4 && (i & 2) == 0) ? (_Float16)-1032.0f : (_Float16)-1152.0f;
    return r;
}


struct MfmaArgs {
    Fwd f;
    int n_tiles;        // row tiles per item
    const Item *items;  // the work list of this pass
    const int32_t *n_items;
    int max_items;
};

// One workgroup: one MFMA item (<= MT tokens of one expert) x
// rows_per_wg(GATEUP, MF) rows; each wave owns 32 or 64 rows and all MT
// tokens. Weight loads run two (128-token items) or four (32-token items)
// unit steps ahead of the matrix cores (registers), activations are
// double-buffered in LDS.
// Where the scales are applied (SM):
//  kScaleCode: each code times its group's scale, rounded to float16, enters
//    the matrix cores (any group size);
//  kScaleStep: the codes enter unscaled (exact small integers, or exact
//    biased values whose biases the gate/up kernel takes out with its bias
//    chain) and each unit step's float32 products are scaled per row
//    afterwards (groups that cover whole unit steps): fewer vector
//    instructions per code, no float16 rounding of code x scale;
//  kScaleRow: one scale per row (group 0): the unscaled products accumulate
//    over the whole row and the float32 sums are scaled once, in the
//    epilogue (no per-step work at all).
constexpr int kScaleCode = 0, kScaleStep = 1, kScaleRow = 2;

// Workgroups per compute unit the register allocation must allow: the
// 32-token down kernels keep four (four waves per SIMD, 128 registers).
__host__ __device__ constexpr int min_wgs_per_cu(bool gateup, int mf)
{
    return (!gateup && mf <= 2) ? 4 : 1;
}

template <bool GATEUP, int WB, int MF, int SM>
__global__ __launch_bounds__(waves_per_wg(MF) * 64, min_wgs_per_cu(GATEUP, MF)) void mfma_kernel(
    MfmaArgs ma)
{
    constexpr int kThreads = waves_per_wg(MF) * 64;
    constexpr int MT = 16 * MF;  // tokens per item
    constexpr int NM = GATEUP ? 2 : 1;
    constexpr int TW = tiles_per_wave(GATEUP, MF);
    constexpr int kNT = rows_per_wg(GATEUP, MF);
    constexpr int kUC = MFmt<WB>::UC, NS = MFmt<WB>::NS, QW = MFmt<WB>::QW, NA = MFmt<WB>::NA;
    constexpr int kAStride = kUC + 8;  // LDS row stride (halves), padded
    __shared__ _Float16 As[2][MT][kAStride];
    __shared__ int s_src[MT];   // input row of each item token (-1: none)

    const Fwd &f = ma.f;
    const Geo &g = f.g;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;

    // XCD-aware order over the items that exist: workgroups are dealt to the
    // XCDs round robin, so give each XCD a contiguous range of (item, row
    // tile) pairs; tiles of one item share its tokens, items of one expert
    // are adjacent and share its weights
    const int n_items = min(*ma.n_items, ma.max_items);
    const int n_active = n_items * ma.n_tiles;
    const int b = blockIdx.x;
    if (b >= n_active) return;
    const int qx = n_active / kXcds, rem = n_active % kXcds;
    const int xcd = b % kXcds, i = b / kXcds;
    const int logical = xcd * qx + min(xcd, rem) + i;
    const int item_idx = logical / ma.n_tiles;
    const int ntile = logical % ma.n_tiles;
    const Item it = ma.items[item_idx];
    if (!in_phase(f, it.expert)) return;  // uniform: the other phase's item
    const int count = min(it.count, MT);
    const uint8_t *blk = it.expert >= 0 ? expert_block(f, it.expert) : f.shared;
    const int K = GATEUP ? g.d : g.f;       // contraction length
    const int rows = GATEUP ? g.f : g.d;    // output rows
    const int n_kb = K / kUC;               // steps = units per row
    const int ng = GATEUP ? g.ng_gu : g.ng_dn;
    const uint16_t *in = GATEUP ? f.x16 : f.h16;

    // input row of every item token
    if (tid < MT) {
        int src = -1;
        if (tid < count) {
            const int p = it.p0 + tid;
            if (GATEUP)
                src = it.expert >= 0 ? min(max(f.perm[p], 0), f.A - 1) / f.k : p - f.A;
            else
                src = p;
        }
        s_src[tid] = src;
    }
    __syncthreads();

    // weights: this wave's unit rows; lane slot = (row in unit, quarter)
    const int r16 = lane % kUnitRows, q = lane / kUnitRows;
    const int rt0 = ntile * (kNT / kUnitRows) + wave * TW;  // first unit row of the wave
    const int n_rt = rows / kUnitRows;
    const uint8_t *qb[TW][NM];
    const float *sb[TW][NM];
#pragma unroll
    for (int t = 0; t < TW; ++t) {
        const int rt = min(rt0 + t, n_rt - 1);  // rows past the end: loads stay in range
        const size_t u0 = (size_t)rt * n_kb * kUnitBytes + (size_t)lane * 16;
        const size_t s0 = (size_t)rt * ng * kUnitRows + r16;
        if (GATEUP) {
            qb[t][0] = blk + u0;
            qb[t][NM - 1] = blk + g.off_up + u0;
            sb[t][0] = reinterpret_cast<const float *>(blk + g.off_gs) + s0;
            sb[t][NM - 1] = reinterpret_cast<const float *>(blk + g.off_us) + s0;
        } else {
            qb[t][0] = blk + g.off_dn + u0;
            sb[t][0] = reinterpret_cast<const float *>(blk + g.off_ds) + s0;
        }
    }
    // scale group of unit step kb: one value for the whole wave when the
    // groups cover whole unit steps (or rows), else per lane quarter
    const int G = g.group;
    const bool grp_uniform = G == 0 || G % kUC == 0;
    auto load_b = [&](int kb, uint4 (&bw)[TW][NM], float (&bs)[TW][NM]) {
        int grp = 0;
        if (G) grp = grp_uniform ? (kb * kUC) / G : (kb * kUC + q * QW) / G;
#pragma unroll
        for (int t = 0; t < TW; ++t)
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                bw[t][m] = *reinterpret_cast<const uint4 *>(qb[t][m] + (size_t)kb * kUnitBytes);
                bs[t][m] = sb[t][m][grp * kUnitRows];
            }
    };

    f32x4_t acc[NM][TW][MF];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int t = 0; t < TW; ++t)
#pragma unroll
            for (int mb = 0; mb < MF; ++mb)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[m][t][mb][r] = 0.0f;
    // Codes scaled per unit step on the 32-token gate/up pass enter the
    // matrix cores biased (kDqBiased: four fewer vector instructions per
    // eight int4 codes); one more product per token block and k-step against
    // bias_operand sums minus the biases of the step in bacc, which is added
    // to the step's products before they are scaled. The other passes
    // subtract the biases in the vector units: down has one matrix, so the
    // bias products would be half as many again as its own and it measured
    // slower; carried over a whole row (one scale per row) the float32 sums
    // of the biased products and of the biases cancel too many bits; the
    // 128-token passes are bound by the matrix cores.
    constexpr bool BIAS = SM == kScaleStep && MF <= 2 && GATEUP;
    constexpr int DQ = SM == kScaleCode ? kDqScaled : (BIAS ? kDqBiased : kDqExact);
    f32x4_t bacc[BIAS ? MF : 1];
#pragma unroll
    for (int mb = 0; mb < (BIAS ? MF : 1); ++mb) bacc[mb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // weight stages in registers: 32-token items (short steps, fewer
    // accumulators) keep four steps in flight, 128-token items two
    constexpr int D = MF <= 2 ? 4 : 2;
    // The unit-step loop for NB active token blocks of 16: NB = MF, or 1 for a
    // 32-token item holding at most 16 tokens, whose empty block then costs
    // no products and no scaling (a choice made once per workgroup).
    auto main_loop = [&](auto nb_tag) {
        constexpr int NB = decltype(nb_tag)::value;
        // activation tile of a step: kRows token rows, loaded in kNA parts
        // (kHalf columns each): thread -> (token row, 16-byte chunks). A loop
        // with fewer token blocks than the item's tile stages only its own
        // rows when a step's columns then still split into whole chunks per
        // thread (int4 32-token items of at most 16 tokens: half the bytes).
        constexpr bool kFew = NB < MF && kUC / (kThreads / (16 * NB)) >= 8;
        constexpr int kRows = kFew ? 16 * NB : MT;
        constexpr int kNA = kFew ? 1 : NA;
        constexpr int kHalf = kUC / kNA;
        constexpr int kParts = kThreads / kRows;       // threads per token row
        constexpr int kCols = kHalf / kParts;          // columns per thread per part
        constexpr int kVec = kCols / 8;                // 16-byte chunks per thread
        static_assert(kVec >= 1, "at least one 16-byte chunk per thread");
        const int a_row = tid / kParts, a_q = tid % kParts;
        const int a_src = s_src[a_row];
        // rows past the item's tokens load token 0's row (every load is issued
        // on every path, so waits stay exact); their products land in
        // accumulator rows that are never stored
        const uint16_t *a_ptr = in + (size_t)(a_src >= 0 ? a_src : s_src[0]) * K + a_q * kCols;
        auto load_a = [&](int kb, int hf, uint4 (&av)[kVec]) {
#pragma unroll
            for (int c = 0; c < kVec; ++c)
                av[c] = reinterpret_cast<const uint4 *>(a_ptr + (size_t)kb * kUC + hf * kHalf)[c];
        };
        auto store_a = [&](int buf, int hf, const uint4 (&av)[kVec]) {
            uint4 *dst = reinterpret_cast<uint4 *>(&As[buf][a_row][hf * kHalf + a_q * kCols]);
#pragma unroll
            for (int c = 0; c < kVec; ++c) dst[c] = make_uint4(av[c].x, av[c].y, av[c].z, av[c].w);
        };
        // half of a unit step on LDS buffer `cur` and weights (bw, bs):
        // k-steps s_lo .. s_lo + NS/2 - 1 of 32, each lane's quarter q
        // covering columns QW q + 8s .. + 8
        constexpr bool POST = SM == kScaleStep;
        f32x4_t tmp[POST ? NM : 1][POST ? TW : 1][POST ? NB : 1];  // a step's unscaled products
        auto compute = [&](int cur, const uint4 (&bw)[TW][NM], const float (&bs)[TW][NM],
                           int s_lo) {
            half2_t s2[TW][NM];
#pragma unroll
            for (int t = 0; t < TW; ++t)
#pragma unroll
                for (int m = 0; m < NM; ++m)
                    s2[t][m] = half2_t{(_Float16)bs[t][m], (_Float16)bs[t][m]};
#pragma unroll
            for (int s = s_lo; s < s_lo + NS / 2; ++s) {
                half8_t bf[TW][NM];
#pragma unroll
                for (int t = 0; t < TW; ++t)
#pragma unroll
                    for (int m = 0; m < NM; ++m)
                        bf[t][m] = dequant8<WB, DQ>(bw[t][m], s, s2[t][m]);
#pragma unroll
                for (int mb = 0; mb < NB; ++mb) {
                    const half8_t af =
                        *reinterpret_cast<const half8_t *>(&As[cur][mb * 16 + r16][QW * q + 8 * s]);
                    if constexpr (BIAS) {
                        const f32x4_t c0 = {0.0f, 0.0f, 0.0f, 0.0f};
                        bacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            af, bias_operand<WB>(), s == 0 ? c0 : bacc[mb], 0, 0, 0);
                    }
#pragma unroll
                    for (int t = 0; t < TW; ++t)
#pragma unroll
                        for (int m = 0; m < NM; ++m) {
                            if constexpr (POST) {
                                // the step's first k-step starts from zero
                                const f32x4_t c0 = {0.0f, 0.0f, 0.0f, 0.0f};
                                tmp[m][t][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                    af, bf[t][m], s == 0 ? c0 : tmp[m][t][mb], 0, 0, 0);
                            } else {
                                acc[m][t][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                    af, bf[t][m], acc[m][t][mb], 0, 0, 0);
                            }
                        }
                }
                // 128-token items: one k-step's operands live at a time
                // (hoisting the next k-steps' dequantisation spills the
                // accumulators of 64 rows x 128 tokens)
                if constexpr (MF == 8) __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (POST) {
                if (s_lo + NS / 2 == NS) {
                    // the lane's accumulator column is its weight row (r16):
                    // one scale for its four tokens
#pragma unroll
                    for (int m = 0; m < NM; ++m)
#pragma unroll
                        for (int t = 0; t < TW; ++t)
#pragma unroll
                            for (int mb = 0; mb < NB; ++mb)
#pragma unroll
                                for (int r = 0; r < 4; ++r) {
                                    float v = tmp[m][t][mb][r];
                                    if constexpr (BIAS) v += bacc[mb][r];
                                    acc[m][t][mb][r] = fmaf(bs[t][m], v, acc[m][t][mb][r]);
                                }
                }
            }
        };

        // weights: a ring of D register stages (stage j holds the steps ks
        // with ks % D == j), each reloaded with the step D ahead right after
        // its products, so a load has D - 1 steps to arrive; activations: one
        // register stage of half a step, loaded during the current step's
        // products and stored to the other LDS buffer. D is even, so the LDS
        // buffer of step ks + j (ks a multiple of D) is j % 2.
        // activations: a ring of AD register stages (AD = 2 for 32-token
        // items but int8 down: each step's tile is loaded two steps ahead of
        // its products; the others load one step ahead: the int8 down kernel
        // measured slower with two, and so did 128-token items, whose steps
        // are long)
        constexpr int AD = (MF <= 2 && (GATEUP || WB == 4)) ? 2 : 1;
        uint4 ar[2][kNA][kVec];
        uint4 bwr[D][TW][NM];
        float bsr[D][TW][NM];
        if constexpr (AD == 2) {
            // the tiles of steps 0 and 1 in flight with the first weights
#pragma unroll
            for (int j = 0; j < AD; ++j) {
                load_a(min(j, n_kb - 1), 0, ar[j][0]);
                if constexpr (kNA == 2) load_a(min(j, n_kb - 1), 1, ar[j][kNA - 1]);
            }
#pragma unroll
            for (int j = 0; j < D; ++j) load_b(min(j, n_kb - 1), bwr[j], bsr[j]);
            store_a(0, 0, ar[0][0]);
            if constexpr (kNA == 2) store_a(0, 1, ar[0][kNA - 1]);
        } else {
            // one half of step 0's tile in registers at a time
            load_a(0, 0, ar[0][0]);
#pragma unroll
            for (int j = 0; j < D; ++j) load_b(min(j, n_kb - 1), bwr[j], bsr[j]);
            store_a(0, 0, ar[0][0]);
            if constexpr (kNA == 2) {
                load_a(0, 1, ar[0][0]);
                store_a(0, 1, ar[0][0]);
            }
        }
        __syncthreads();
        // one step: the tile of step ks + AD is loaded into the register
        // stage `a_far`, products on LDS buffer `cur`, then the tile of step
        // ks + 1 (`a_next`, loaded AD - 1 steps earlier) is stored to the
        // other buffer. Loads are issued on every step (past the end they
        // reload the last step, into a buffer no later step reads), so that
        // no load sits in a branch: each wait is then for the load it needs.
        auto step = [&](int ks, int cur, uint4 (&a_next)[kNA][kVec], uint4 (&a_far)[kNA][kVec],
                        const uint4 (&bw)[TW][NM], const float (&bs)[TW][NM]) {
            const int kf = min(ks + AD, n_kb - 1);
            load_a(kf, 0, a_far[0]);
            if constexpr (kNA == 2) load_a(kf, 1, a_far[kNA - 1]);
            __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the products
            compute(cur, bw, bs, 0);
            compute(cur, bw, bs, NS / 2);
            store_a(cur ^ 1, 0, a_next[0]);
            if constexpr (kNA == 2) store_a(cur ^ 1, 1, a_next[kNA - 1]);
            __syncthreads();
        };
        // AD = 2: the two stages alternate (D is even, so stage j % 2 holds
        // step ks + j's tile until it is stored); AD = 1: each step loads and
        // stores the next tile through registers of its own
        for (int ks = 0; ks < n_kb; ks += D) {
#pragma unroll
            for (int j = 0; j < D; ++j) {
                if (ks + j >= n_kb) break;
                if constexpr (AD == 2) {
                    step(ks + j, j & 1, ar[(j + 1) & 1], ar[j & 1], bwr[j], bsr[j]);
                } else {
                    // the tile lives in registers within the step only
                    uint4 at[kNA][kVec];
                    step(ks + j, j & 1, at, at, bwr[j], bsr[j]);
                }
                load_b(min(ks + j + D, n_kb - 1), bwr[j], bsr[j]);
            }
        }
    };
    if constexpr (MF == 2) {
        if (count <= 16)
            main_loop(std::integral_constant<int, 1>());
        else
            main_loop(std::integral_constant<int, 2>());
    } else {
        main_loop(std::integral_constant<int, MF>());
    }

    // epilogue: register r of block (t, mb) is token mb*16 + 4q + r, weight
    // row 16 (rt0 + t) + r16
#pragma unroll
    for (int t = 0; t < TW; ++t) {
        const int row = (rt0 + t) * kUnitRows + r16;
        if (rt0 + t >= n_rt) continue;
        if constexpr (SM == kScaleRow) {
            // the row's one scale per matrix, on the whole row's sums
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const float sc = sb[t][m][0];
#pragma unroll
                for (int mb = 0; mb < MF; ++mb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[m][t][mb][r] *= sc;
            }
        }
#pragma unroll
        for (int mb = 0; mb < MF; ++mb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tok = mb * 16 + 4 * q + r;
                if (tok >= count) continue;
                const int p = it.p0 + tok;
                if (GATEUP) {
                    // hidden value as the down pass's float16 operand: row
                    // `row` of this pass is column `row` of the down pass
                    const float gv = acc[0][t][mb][r], uv = acc[NM - 1][t][mb][r];
                    // (times act16_factor of its column in the down pass)
                    const _Float16 hv = (_Float16)(gv / (1.0f + expf(-gv)) * uv *
                                                   act16_factor<WB>(row & 7));
                    f.h16[(size_t)p * rows + (row & ~7) + perm8<WB>(row & 7)] =
                        __builtin_bit_cast(uint16_t, hv);
                } else {
                    const int orow = it.expert >= 0 ? min(max(f.perm[p], 0), f.A - 1) : p;
                    f.o[(size_t)orow * rows + row] = acc[0][t][mb][r];
                }
            }
        }
    }
}

template <int WB>
__global__ __launch_bounds__(256) void stage_x16_kernel(const float *__restrict__ x, long long n8,
                                                        uint16_t *__restrict__ x16)
{
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n8) stage_x16_group<WB>(x, i, x16);
}

}  // namespace

bool mfma_supported(const Geo &g)
{
    return (g.wbits == 4 && g.ucols == MFmt<4>::UC) || (g.wbits == 8 && g.ucols == MFmt<8>::UC);
}

template <bool GATEUP, int WB, int MF, int SM>
hipError_t run_mfma(const MfmaArgs &a, long long blocks, const hipEvent_t *ev, hipStream_t s)
{
    constexpr int kThreads = waves_per_wg(MF) * 64;
    const dim3 grid((unsigned)blocks);
    if (ev[0] || ev[1])  // events taken by the dispatch itself, around this kernel only
        hipExtLaunchKernelGGL((mfma_kernel<GATEUP, WB, MF, SM>), grid, dim3(kThreads), 0, s, ev[0], ev[1],
                              0, a);
    else
        hipLaunchKernelGGL((mfma_kernel<GATEUP, WB, MF, SM>), grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_stage_x16(const Fwd &f, hipStream_t s)
{
    const long long n8 = (long long)f.N * f.g.d / 8;
    const unsigned blocks = (unsigned)((n8 + 255) / 256);
    if (f.g.wbits == 8)
        hipLaunchKernelGGL(stage_x16_kernel<8>, dim3(blocks), dim3(256), 0, s, f.x, n8, f.x16);
    else
        hipLaunchKernelGGL(stage_x16_kernel<4>, dim3(blocks), dim3(256), 0, s, f.x, n8, f.x16);
    return hipGetLastError();
}

hipError_t launch_mfma(const Fwd &f, bool gateup, bool small, hipStream_t s)
{
    MfmaArgs a;
    a.f = f;
    a.items = small ? f.sitems : f.mitems;
    a.n_items = small ? f.n_sitems : f.n_mitems;
    a.max_items = small ? f.max_sitems : f.max_mitems;
    const int rows = gateup ? f.g.f : f.g.d;
    const int mf = (small ? kMfmaSmallTokens : kMfmaBigTokens) / 16;
    a.n_tiles = (rows + rows_per_wg(gateup, mf) - 1) / rows_per_wg(gateup, mf);
    const long long blocks = (long long)a.max_items * a.n_tiles;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    const hipEvent_t *ev = small ? (gateup ? f.ev_sgu : f.ev_sdn) : (gateup ? f.ev_mgu : f.ev_mdn);
    constexpr int kSmall = kMfmaSmallTokens / 16, kBig = kMfmaBigTokens / 16;
    // where the scales go: per row when a row has one scale (int8 layers:
    // the draft head's format), per unit step for 32-token items whose
    // groups cover whole steps, else per code
    const int G = f.g.group;
    const bool post = small && (G == 0 || G % f.g.ucols == 0);
    if (f.g.wbits == 8) {
        if (G == 0)
            return small ? (gateup ? run_mfma<true, 8, kSmall, kScaleRow>(a, blocks, ev, s)
                                   : run_mfma<false, 8, kSmall, kScaleRow>(a, blocks, ev, s))
                         : (gateup ? run_mfma<true, 8, kBig, kScaleRow>(a, blocks, ev, s)
                                   : run_mfma<false, 8, kBig, kScaleRow>(a, blocks, ev, s));
        if (post)
            return gateup ? run_mfma<true, 8, kSmall, kScaleStep>(a, blocks, ev, s)
                          : run_mfma<false, 8, kSmall, kScaleStep>(a, blocks, ev, s);
        if (small)
            return gateup ? run_mfma<true, 8, kSmall, kScaleCode>(a, blocks, ev, s)
                          : run_mfma<false, 8, kSmall, kScaleCode>(a, blocks, ev, s);
        return gateup ? run_mfma<true, 8, kBig, kScaleCode>(a, blocks, ev, s)
                      : run_mfma<false, 8, kBig, kScaleCode>(a, blocks, ev, s);
    }
    if (post)
        return gateup ? run_mfma<true, 4, kSmall, kScaleStep>(a, blocks, ev, s)
                      : run_mfma<false, 4, kSmall, kScaleStep>(a, blocks, ev, s);
    if (small)
        return gateup ? run_mfma<true, 4, kSmall, kScaleCode>(a, blocks, ev, s)
                      : run_mfma<false, 4, kSmall, kScaleCode>(a, blocks, ev, s);
    return gateup ? run_mfma<true, 4, kBig, kScaleCode>(a, blocks, ev, s)
                  : run_mfma<false, 4, kBig, kScaleCode>(a, blocks, ev, s);
}

}  // namespace moe
