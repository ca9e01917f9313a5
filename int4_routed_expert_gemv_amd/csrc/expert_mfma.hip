// expert_mfma.hip - expert math for token groups large enough to be a dense
// contraction (prefill, the shared expert of a large batch, hot experts).
//
// Colibri pages: "Public Colibri Observation and Revision Ledger", section
// "Exact Architecture and Data-Flow Reconstruction" (three-matrix expert MLP,
// always-on shared expert), README "Get started" (int4 experts with group
// scales).
//
// For one expert and up to MT of its tokens (MT = 128 for large groups, 32
// for small ones), a workgroup computes 128 output rows (of gate and up
// together, or of down) over the full contraction:
//   gate/up:  h[p][r] = silu(sum_c Wg[r][c] x_t[c]) * (sum_c Wu[r][c] x_t[c])
//   down:     o[out(p)][r] = sum_c Wd[r][c] h[p][c]
// on v_mfma_f32_32x32x16_f16 (float16 products, float32 accumulation):
//  * activations (x or h, float32) are converted to float16 and staged in LDS,
//    64 columns at a time, double-buffered;
//  * every lane reads its weights straight from HBM, 16 bytes (32 int4 codes
//    of one row) per step, and expands them in registers: OR into the
//    mantissa of 1024 (exact), subtract 1032 (exact), multiply by the group
//    scale (one float16 rounding);
//  * within each 8-column group the columns are taken in the order
//    0,4,1,5,2,6,3,7 on both operands, which lets one 32-bit word of codes
//    feed one MFMA operand without shuffles;
//  * each of the 4 waves owns 32 rows and all MT tokens (MT/32 blocks of
//    32 x 32); loads run two steps ahead of the matrix cores.
// Workgroups are mapped so that those sharing an expert (and so its weights
// and its tokens) land on the same XCD and share its L2.
#include <hip/hip_ext.h>

#include "internal.h"

namespace moe {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kNW = 32;             // rows per wave
constexpr int kNT = (kThreads / 64) * kNW;  // rows per workgroup
constexpr int kKB = 64;             // columns per step
constexpr int kAStride = kKB + 8;   // LDS row stride (halves), padded
constexpr int kXcds = 8;

__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

// 8 offset-binary int4 codes (element j in bits 4j..4j+3) times the scale,
// as float16 in the column order 0,4,1,5,2,6,3,7.
__device__ __forceinline__ half8_t dequant8(uint32_t w, half2_t s2)
{
    const half2_t off = {(_Float16)1032.0f, (_Float16)1032.0f};
    const uint32_t m = 0x000F000Fu, magic = 0x64006400u;
    const half2_t p0 = (as_h2((w & m) | magic) - off) * s2;
    const half2_t p1 = (as_h2(((w >> 4) & m) | magic) - off) * s2;
    const half2_t p2 = (as_h2(((w >> 8) & m) | magic) - off) * s2;
    const half2_t p3 = (as_h2(((w >> 12) & m) | magic) - off) * s2;
    half8_t r;
    r[0] = p0[0]; r[1] = p0[1];
    r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1];
    r[6] = p3[0]; r[7] = p3[1];
    return r;
}

struct MfmaArgs {
    Fwd f;
    int n_tiles;        // row tiles per item
    const Item *items;  // the work list of this pass
    const int32_t *n_items;
    int max_items;
};

// One workgroup: one MFMA item (<= MT tokens of one expert) x kNT rows;
// each wave owns 32 rows and all MT tokens. Loads run two 64-column steps
// ahead of the matrix cores (registers), activations are double-buffered in
// LDS.
template <bool GATEUP, int MT>
__global__ __launch_bounds__(kThreads, MT > 32 ? 1 : 2) void mfma_kernel(MfmaArgs ma)
{
    constexpr int NM = GATEUP ? 2 : 1;
    constexpr int MF = MT / 32;  // 32 x 32 blocks per wave
    __shared__ _Float16 As[2][MT][kAStride];
    __shared__ int s_src[MT];   // input row of each tile token (-1: none)

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
    const int q = n_active / kXcds, rem = n_active % kXcds;
    const int xcd = b % kXcds, i = b / kXcds;
    const int logical = xcd * q + min(xcd, rem) + i;
    const int item_idx = logical / ma.n_tiles;
    const int ntile = logical % ma.n_tiles;
    const Item it = ma.items[item_idx];
    const int count = min(it.count, MT);
    const uint8_t *blk = it.expert >= 0 ? f.pool + (size_t)it.expert * f.stride : f.shared;
    const int K = GATEUP ? g.d : g.f;       // contraction length
    const int rows = GATEUP ? g.f : g.d;    // output rows
    const float *in = GATEUP ? f.x : f.h;
    float *out = GATEUP ? f.h : f.o;

    // input row of every tile token
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

    // activation loads: thread -> (token row, part of the 64 columns)
    constexpr int kParts = kThreads / MT;           // threads per token row
    constexpr int kCols = kKB / kParts;             // columns per thread
    constexpr int kVec = kCols / 4;                 // float4 per thread
    const int a_row = tid / kParts, a_q = tid % kParts;
    const int a_src = s_src[a_row];
    const float *a_ptr = a_src >= 0 ? in + (size_t)a_src * K + a_q * kCols : nullptr;
    auto load_a = [&](int k0, float4 (&av)[kVec]) {
#pragma unroll
        for (int c = 0; c < kVec; ++c)
            av[c] = a_ptr ? reinterpret_cast<const float4 *>(a_ptr + k0)[c]
                          : make_float4(0.f, 0.f, 0.f, 0.f);
    };
    auto store_a = [&](int buf, const float4 (&av)[kVec]) {
        // groups of 8 columns, each written in the order 0,4,1,5,2,6,3,7
        const float *v = reinterpret_cast<const float *>(av);
        _Float16 *dst = &As[buf][a_row][a_q * kCols];
#pragma unroll
        for (int gi = 0; gi < kCols / 8; ++gi) {
            half8_t h;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                h[2 * j] = (_Float16)v[8 * gi + j];
                h[2 * j + 1] = (_Float16)v[8 * gi + 4 + j];
            }
            *reinterpret_cast<half8_t *>(dst + 8 * gi) = h;
        }
    };

    // weights: this lane's row and 32-column half of each 64-column step
    const int hh = lane / 32;
    const int row = ntile * kNT + wave * kNW + (lane % 32);
    const int row_c = min(row, rows - 1);
    const long long row_bytes = K / 2;
    const uint8_t *qb[NM];
    const float *sb[NM];
    const long long spr = g.group ? K / g.group : 1;
    if (GATEUP) {
        qb[0] = blk + (long long)row_c * row_bytes;
        qb[NM - 1] = blk + g.off_up + (long long)row_c * row_bytes;
        sb[0] = reinterpret_cast<const float *>(blk + g.off_gs) + (long long)row_c * spr;
        sb[NM - 1] = reinterpret_cast<const float *>(blk + g.off_us) + (long long)row_c * spr;
    } else {
        qb[0] = blk + g.off_dn + (long long)row_c * row_bytes;
        sb[0] = reinterpret_cast<const float *>(blk + g.off_ds) + (long long)row_c * spr;
    }
    auto load_b = [&](int k0, uint4 (&bw)[NM], float (&bs)[NM]) {
        const int col = k0 + 32 * hh;
        const long long grp = g.group ? col / g.group : 0;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            bw[m] = *reinterpret_cast<const uint4 *>(qb[m] + col / 2);
            bs[m] = sb[m][grp];
        }
    };

    f32x16_t acc[NM][MF];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int mf = 0; mf < MF; ++mf)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[m][mf][r] = 0.0f;

    // one 64-column step on LDS buffer `cur` and weights (bw, bs)
    auto compute = [&](int cur, const uint4 (&bw)[NM], const float (&bs)[NM]) {
        half2_t s2[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) s2[m] = half2_t{(_Float16)bs[m], (_Float16)bs[m]};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            half8_t bf[NM];
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const uint32_t w = s == 0 ? bw[m].x : (s == 1 ? bw[m].y : (s == 2 ? bw[m].z : bw[m].w));
                bf[m] = dequant8(w, s2[m]);
            }
#pragma unroll
            for (int mf = 0; mf < MF; ++mf) {
                const half8_t af =
                    *reinterpret_cast<const half8_t *>(&As[cur][mf * 32 + (lane % 32)][32 * hh + 8 * s]);
#pragma unroll
                for (int m = 0; m < NM; ++m)
                    acc[m][mf] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, bf[m], acc[m][mf], 0, 0, 0);
            }
        }
    };

    const int steps = K / kKB;
    // ring of two register stages: stage j holds step ks with ks % 2 == j
    float4 av0[kVec], av1[kVec];
    uint4 bw0[NM], bw1[NM];
    float bs0[NM], bs1[NM];
    load_a(0, av0);
    load_b(0, bw0, bs0);
    if (steps > 1) {
        load_a(kKB, av1);
        load_b(kKB, bw1, bs1);
    }
    store_a(0, av0);
    __syncthreads();
    for (int ks = 0; ks < steps; ks += 2) {
        // even step ks: LDS buffer 0, weights in stage 0
        {
            uint4 bw[NM];
            float bs[NM];
#pragma unroll
            for (int m = 0; m < NM; ++m) { bw[m] = bw0[m]; bs[m] = bs0[m]; }
            if (ks + 2 < steps) {
                load_a((ks + 2) * kKB, av0);
                load_b((ks + 2) * kKB, bw0, bs0);
            }
            compute(0, bw, bs);
            if (ks + 1 < steps) store_a(1, av1);
            __syncthreads();
        }
        if (ks + 1 >= steps) break;
        // odd step ks + 1: LDS buffer 1, weights in stage 1
        {
            uint4 bw[NM];
            float bs[NM];
#pragma unroll
            for (int m = 0; m < NM; ++m) { bw[m] = bw1[m]; bs[m] = bs1[m]; }
            if (ks + 3 < steps) {
                load_a((ks + 3) * kKB, av1);
                load_b((ks + 3) * kKB, bw1, bs1);
            }
            compute(1, bw, bs);
            if (ks + 2 < steps) store_a(0, av0);
            __syncthreads();
        }
    }

    // epilogue: lane holds column `row` of MF 32x32 blocks; register r of
    // block mf is token mf*32 + (r/4)*8 + (lane/32)*4 + r%4
    if (row >= rows) return;
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int tok = mf * 32 + (r / 4) * 8 + hh * 4 + (r % 4);
            if (tok >= count) continue;
            const int p = it.p0 + tok;
            if (GATEUP) {
                const float gv = acc[0][mf][r], uv = acc[NM - 1][mf][r];
                out[(size_t)p * rows + row] = gv / (1.0f + expf(-gv)) * uv;
            } else {
                const int orow = it.expert >= 0 ? min(max(f.perm[p], 0), f.A - 1) : p;
                out[(size_t)orow * rows + row] = acc[0][mf][r];
            }
        }
    }
}

}  // namespace

bool mfma_supported(const Geo &g)
{
    return g.wbits == 4 && g.d % kKB == 0 && g.f % kKB == 0;
}

template <bool GATEUP, int MT>
hipError_t run_mfma(const MfmaArgs &a, long long blocks, const hipEvent_t *ev, hipStream_t s)
{
    const dim3 grid((unsigned)blocks);
    if (ev[0] || ev[1])  // events taken by the dispatch itself, around this kernel only
        hipExtLaunchKernelGGL((mfma_kernel<GATEUP, MT>), grid, dim3(kThreads), 0, s, ev[0], ev[1],
                              0, a);
    else
        hipLaunchKernelGGL((mfma_kernel<GATEUP, MT>), grid, dim3(kThreads), 0, s, a);
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
    a.n_tiles = (rows + kNT - 1) / kNT;
    const long long blocks = (long long)a.max_items * a.n_tiles;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    const hipEvent_t *ev = small ? (gateup ? f.ev_sgu : f.ev_sdn) : (gateup ? f.ev_mgu : f.ev_mdn);
    if (small)
        return gateup ? run_mfma<true, kMfmaSmallTokens>(a, blocks, ev, s)
                      : run_mfma<false, kMfmaSmallTokens>(a, blocks, ev, s);
    return gateup ? run_mfma<true, kMfmaBigTokens>(a, blocks, ev, s)
                  : run_mfma<false, kMfmaBigTokens>(a, blocks, ev, s);
}

}  // namespace moe
