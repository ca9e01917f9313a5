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
//  * each token's activations are staged once per wave in registers, as
//    float16 scaled by a power of two that brings the token's largest value
//    into [2^13, 2^14) (an exact scaling, undone on the output);
//  * the group scale multiplies each chunk's float32 partial sum;
//  * partial sums of a row are added across its lanes with shuffles and
//    across the waves of a split row in LDS, always in the same order.
#include "internal.h"

namespace moe {
namespace {

typedef __fp16 h2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2_t as_h2(uint32_t v) { return __builtin_bit_cast(h2_t, v); }

constexpr uint32_t kMagic = 0x64006400u;  // two float16 1024.0

// 8 offset-binary int4 codes (element j in bits 4j..4j+3) against staged
// activations xs = {(x0,x4), (x1/16,x5/16), (x2,x6), (x3/16,x7/16)}.
__device__ __forceinline__ float dot8_i4(uint32_t w, const uint32_t *xs, float acc)
{
    const uint32_t w8 = w >> 8;
    acc = __builtin_amdgcn_fdot2(as_h2((w & 0x000F000Fu) | kMagic), as_h2(xs[0]), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2((w & 0x00F000F0u) | kMagic), as_h2(xs[1]), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2((w8 & 0x000F000Fu) | kMagic), as_h2(xs[2]), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2((w8 & 0x00F000F0u) | kMagic), as_h2(xs[3]), acc, false);
    return acc;
}

// 4 offset-binary int8 codes against xs = {(x0,x2), (x1,x3)}.
__device__ __forceinline__ float dot4_i8(uint32_t w, const uint32_t *xs, float acc)
{
    acc = __builtin_amdgcn_fdot2(as_h2((w & 0x00FF00FFu) | kMagic), as_h2(xs[0]), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(((w >> 8) & 0x00FF00FFu) | kMagic), as_h2(xs[1]), acc, false);
    return acc;
}

template <int WB> struct Fmt;
template <> struct Fmt<4> { static constexpr int epc = 32, xdw = 16; };
template <> struct Fmt<8> { static constexpr int epc = 16, xdw = 8; };

template <int WB>
__device__ __forceinline__ float dot_chunk(uint4 w, const uint32_t *xs, float acc)
{
    if constexpr (WB == 4) {
        acc = dot8_i4(w.x, xs + 0, acc);
        acc = dot8_i4(w.y, xs + 4, acc);
        acc = dot8_i4(w.z, xs + 8, acc);
        acc = dot8_i4(w.w, xs + 12, acc);
    } else {
        acc = dot4_i8(w.x, xs + 0, acc);
        acc = dot4_i8(w.y, xs + 2, acc);
        acc = dot4_i8(w.z, xs + 4, acc);
        acc = dot4_i8(w.w, xs + 6, acc);
    }
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
__device__ __forceinline__ float stage_chunk(const float *src, float scale, uint32_t *xs)
{
    constexpr int epc = Fmt<WB>::epc;
    float v[epc];
#pragma unroll
    for (int q = 0; q < epc / 4; ++q) {
        float4 f4 = reinterpret_cast<const float4 *>(src)[q];
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

struct GemvArgs {
    Geo g;
    const uint8_t *pool;
    size_t stride;
    const uint8_t *shared;
    const float *in;        // x [N][d] (gate/up) or h [P][f] (down)
    int k;
    const int32_t *perm;
    int A;
    int N;
    const Item *items;
    const int32_t *n_items;
    int n_rbg;              // row groups (workgroups) per item
    float *out;             // h [P][f] (gate/up) or o [P][d] (down)
};

constexpr int kTB = 4;      // tokens per item

// One workgroup = KS x RG waves working on ROWS = RG * R * (64/LPR) rows of
// one item. The KS waves of a row group split the row into KS slices of 64
// 16-byte chunks (rows of at most 64 chunks use KS = 1 and LPR lanes per
// row). Each wave stages the activations of its chunk for the item's tokens
// in registers, streams R rows with one 128-bit load per lane per row and
// matrix, adds partial sums across the row's lanes with shuffles and, for
// KS > 1, across the KS waves in LDS in slice order.
template <bool GATEUP, int WB, int KS, int LPR, int RG, int R>
__global__ __launch_bounds__(KS * RG * kWave) void gemv_kernel(GemvArgs a)
{
    constexpr int XDW = Fmt<WB>::xdw, EPC = Fmt<WB>::epc;
    constexpr int RPI = kWave / LPR;
    constexpr int NW = KS * RG;
    constexpr int ROWS = RG * R * RPI;
    constexpr int NM = GATEUP ? 2 : 1;  // matrices per row: gate and up, or down
    static_assert(KS == 1 || LPR == kWave, "row slices need full-wave rows");

    __shared__ float smax[kTB][NW];
    __shared__ float red[KS > 1 ? RG * R * kTB * KS * NM : 1];

    const Geo &g = a.g;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int ks = wave % KS, rg = wave / KS;
    const int item_idx = blockIdx.x / a.n_rbg;
    if (item_idx >= *a.n_items) return;  // uniform over the workgroup
    const int rbg = blockIdx.x % a.n_rbg;
    const Item it = a.items[item_idx];
    const uint8_t *blk = it.expert >= 0 ? a.pool + (size_t)it.expert * a.stride : a.shared;
    const int seg = lane / LPR, li = lane % LPR;
    const int c = ks * kWave + li;  // this lane's chunk of the row
    const int cols = GATEUP ? g.d : g.f;
    const int rows = GATEUP ? g.f : g.d;

    // tokens: input row and output row of each position
    const float *src[kTB];
    int orow[kTB];
#pragma unroll
    for (int i = 0; i < kTB; ++i) {
        const int p = it.p0 + min(i, it.count - 1);
        // values read from the permutation are clamped into range, so
        // inconsistent caller buffers cannot move an access out of bounds
        const int a_idx = it.expert >= 0 ? min(max(a.perm[p], 0), a.A - 1) : 0;
        if (GATEUP) {
            const int t = it.expert >= 0 ? a_idx / a.k : p - a.A;
            src[i] = a.in + (size_t)t * cols;
            orow[i] = p;
        } else {
            src[i] = a.in + (size_t)p * cols;
            orow[i] = it.expert >= 0 ? a_idx : p;
        }
    }

    // per-token power-of-two scale from the largest |value| of the row
#pragma unroll
    for (int i = 0; i < kTB; ++i) {
        if (i >= it.count) break;
        const float4 *s4 = reinterpret_cast<const float4 *>(src[i] + (size_t)c * EPC);
        float mx = 0.0f;
#pragma unroll
        for (int q = 0; q < EPC / 4; ++q) {
            const float4 f4 = s4[q];
            mx = fmaxf(mx, fmaxf(fmaxf(fabsf(f4.x), fabsf(f4.y)), fmaxf(fabsf(f4.z), fabsf(f4.w))));
        }
        mx = wave_max(mx);
        if (lane == 0) smax[i][wave] = mx;
    }
    __syncthreads();
    uint32_t xs[kTB][XDW];
    float corr[kTB], inv[kTB];
#pragma unroll
    for (int i = 0; i < kTB; ++i) {
        inv[i] = 0.0f;
        corr[i] = 0.0f;
        if (i < it.count) {
            float mx = smax[i][0];
#pragma unroll
            for (int w = 1; w < NW; ++w) mx = fmaxf(mx, smax[i][w]);
            int sh = 0;
            if (mx > 0.0f && mx <= 3.4e38f) {
                int ex;
                frexpf(mx, &ex);
                sh = min(126, max(-126, 14 - ex));
            }
            inv[i] = ldexpf(1.0f, -sh);
            corr[i] = stage_chunk<WB>(src[i] + (size_t)c * EPC, ldexpf(1.0f, sh), xs[i]);
        } else {
#pragma unroll
            for (int q = 0; q < XDW; ++q) xs[i][q] = 0u;
        }
    }

    // weights: R rows, one 16-byte chunk per lane per matrix, and its scale
    const int row0 = rbg * ROWS + rg * R * RPI;
    const long long grp = g.group ? (long long)c * EPC / g.group : 0;
    const long long row_bytes = GATEUP ? g.row_gu : g.row_dn;
    const long long spr = GATEUP ? g.spr_gu : g.spr_dn;
    const uint8_t *q0 = blk + (GATEUP ? 0 : g.off_dn) + (long long)c * 16;
    const uint8_t *q1 = blk + g.off_up + (long long)c * 16;
    const uint8_t *s0 = blk + (GATEUP ? g.off_gs : g.off_ds) + grp * 4;
    const uint8_t *s1 = blk + g.off_us + grp * 4;
    uint4 w[R][NM];
    float sc[R][NM];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const long long row = min(row0 + r * RPI + seg, rows - 1);
        w[r][0] = *reinterpret_cast<const uint4 *>(q0 + row * row_bytes);
        sc[r][0] = *reinterpret_cast<const float *>(s0 + row * spr * 4);
        if (GATEUP) {
            w[r][NM - 1] = *reinterpret_cast<const uint4 *>(q1 + row * row_bytes);
            sc[r][NM - 1] = *reinterpret_cast<const float *>(s1 + row * spr * 4);
        }
    }

#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int row = row0 + r * RPI + seg;
#pragma unroll
        for (int i = 0; i < kTB; ++i) {
            if (i >= it.count) break;
            float acc[NM];
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const float cm = dot_chunk<WB>(w[r][m], xs[i], 0.0f);
                acc[m] = segment_sum<LPR>(sc[r][m] * (cm - corr[i]));
            }
            if (KS == 1) {
                if (li == 0 && row < rows) {
                    float v;
                    if (GATEUP) {
                        const float gv = acc[0] * inv[i], uv = acc[NM - 1] * inv[i];
                        v = gv / (1.0f + expf(-gv)) * uv;
                    } else {
                        v = acc[0] * inv[i];
                    }
                    a.out[(size_t)orow[i] * rows + row] = v;
                }
            } else if (lane == 0) {
#pragma unroll
                for (int m = 0; m < NM; ++m)
                    red[(((rg * R + r) * kTB + i) * KS + ks) * NM + m] = acc[m];
            }
        }
    }
    if (KS > 1) {
        __syncthreads();
        // one thread per (row group, row, token): add the slices in order
        for (int idx = threadIdx.x; idx < RG * R * kTB; idx += NW * kWave) {
            const int i = idx % kTB, rr = idx / kTB;
            const int row = rbg * ROWS + rr;  // RPI == 1 here
            if (i >= it.count || row >= rows) continue;
            float acc[NM];
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                acc[m] = red[(idx * KS + 0) * NM + m];
#pragma unroll
                for (int q = 1; q < KS; ++q) acc[m] += red[(idx * KS + q) * NM + m];
            }
            float v;
            if (GATEUP) {
                const float gv = acc[0] * inv[i], uv = acc[NM - 1] * inv[i];
                v = gv / (1.0f + expf(-gv)) * uv;
            } else {
                v = acc[0] * inv[i];
            }
            a.out[(size_t)orow[i] * rows + row] = v;
        }
    }
}

// ---- work list -------------------------------------------------------------

constexpr int kPlanThreads = 1024;

__device__ int block_exclusive_scan(int v, int &total)
{
    __shared__ int wt[kPlanThreads / kWave];
    const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
    int incl = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        int u = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += u;
    }
    if (lane == kWave - 1) wt[wv] = incl;
    __syncthreads();
    if (wv == 0) {
        int s = lane < kPlanThreads / kWave ? wt[lane] : 0;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            int u = __shfl_up(s, o, kWave);
            if (lane >= o) s += u;
        }
        if (lane < kPlanThreads / kWave) wt[lane] = s;
    }
    __syncthreads();
    total = wt[kPlanThreads / kWave - 1];
    const int r = incl - v + (wv > 0 ? wt[wv - 1] : 0);
    __syncthreads();
    return r;
}

// Splits every union expert's slice of the permutation (and the shared
// expert's N tokens) into items of at most tb tokens, for both GEMV passes.
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(
    const int32_t *__restrict__ union_ids, const int32_t *__restrict__ n_union,
    const int32_t *__restrict__ offsets, int E, int A, int N, int has_shared, int tb_gu,
    int tb_dn, int max_gu, int max_dn, Item *__restrict__ items_gu, Item *__restrict__ items_dn,
    int32_t *__restrict__ n_items)
{
    const int u = threadIdx.x;
    const int nu = min(max(*n_union, 0), E);
    int e = -1, s0 = 0, T = 0;
    if (u < nu) {
        e = union_ids[u];
        if (e >= 0 && e < E) {
            s0 = min(max(offsets[e], 0), A);
            const int s1 = min(max(offsets[e + 1], s0), A);
            T = s1 - s0;
        } else {
            e = -1;
        }
    }
    for (int pass = 0; pass < 2; ++pass) {
        const int tb = pass == 0 ? tb_gu : tb_dn;
        const int cap = pass == 0 ? max_gu : max_dn;  // host bound of the item count
        Item *items = pass == 0 ? items_gu : items_dn;
        const int nb = (T + tb - 1) / tb;
        int total;
        const int base = block_exclusive_scan(nb, total);
        for (int b = 0; b < nb; ++b) {
            Item it;
            it.expert = e;
            it.p0 = s0 + b * tb;
            it.count = min(tb, T - b * tb);
            it.pad = 0;
            if (base + b < cap) items[base + b] = it;
        }
        const int nsh = has_shared ? (N + tb - 1) / tb : 0;
        for (int b = threadIdx.x; b < nsh; b += kPlanThreads) {
            Item it;
            it.expert = -1;
            it.p0 = A + b * tb;
            it.count = min(tb, N - b * tb);
            it.pad = 0;
            if (total + b < cap) items[total + b] = it;
        }
        if (threadIdx.x == 0) n_items[pass] = min(total + nsh, cap);
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

// rows per wave for each pass
constexpr int kRowsGateUp = 4;
constexpr int kRowsDown = 8;

template <bool GATEUP, int WB, int KS, int LPR>
hipError_t run_gemv(GemvArgs a, int max_items, hipStream_t s)
{
    constexpr int RG = KS >= 4 ? 1 : (KS == 1 ? 4 : 2);
    constexpr int R = GATEUP ? kRowsGateUp : kRowsDown;
    constexpr int ROWS = RG * R * (kWave / LPR);
    const int rows = GATEUP ? a.g.f : a.g.d;
    a.n_rbg = (rows + ROWS - 1) / ROWS;
    const long long blocks = (long long)max_items * a.n_rbg;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemv_kernel<GATEUP, WB, KS, LPR, RG, R>), dim3((unsigned)blocks),
                       dim3(KS * RG * kWave), 0, s, a);
    return hipGetLastError();
}

template <bool GATEUP, int WB>
hipError_t dispatch_shape(int cpl, int lpr, const GemvArgs &a, int max_items, hipStream_t s)
{
    if (lpr == kWave) {
        switch (cpl) {
        case 1: return run_gemv<GATEUP, WB, 1, 64>(a, max_items, s);
        case 2: return run_gemv<GATEUP, WB, 2, 64>(a, max_items, s);
        case 3: return run_gemv<GATEUP, WB, 3, 64>(a, max_items, s);
        case 4: return run_gemv<GATEUP, WB, 4, 64>(a, max_items, s);
        case 6: return run_gemv<GATEUP, WB, 6, 64>(a, max_items, s);
        case 8: return run_gemv<GATEUP, WB, 8, 64>(a, max_items, s);
        default: return hipErrorInvalidValue;
        }
    }
    if (cpl != 1) return hipErrorInvalidValue;
    switch (lpr) {
    case 2: return run_gemv<GATEUP, WB, 1, 2>(a, max_items, s);
    case 4: return run_gemv<GATEUP, WB, 1, 4>(a, max_items, s);
    case 8: return run_gemv<GATEUP, WB, 1, 8>(a, max_items, s);
    case 16: return run_gemv<GATEUP, WB, 1, 16>(a, max_items, s);
    case 32: return run_gemv<GATEUP, WB, 1, 32>(a, max_items, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_pass(bool gateup, const Geo &g, const uint8_t *pool, size_t stride,
                       const uint8_t *shared, const float *in, int k, const int32_t *perm, int A,
                       int N, const Item *items, const int32_t *n_items, int max_items, float *out,
                       hipStream_t s)
{
    GemvArgs a;
    a.g = g;
    a.pool = pool;
    a.stride = stride;
    a.shared = shared;
    a.in = in;
    a.k = k;
    a.perm = perm;
    a.A = A;
    a.N = N;
    a.items = items;
    a.n_items = n_items;
    a.n_rbg = 0;
    a.out = out;
    const int lpr = gateup ? g.gu_lpr : g.dn_lpr;
    const int cpl = gateup ? g.gu_cpl : g.dn_cpl;
    if (gateup)
        return g.wbits == 4 ? dispatch_shape<true, 4>(cpl, lpr, a, max_items, s)
                            : dispatch_shape<true, 8>(cpl, lpr, a, max_items, s);
    return g.wbits == 4 ? dispatch_shape<false, 4>(cpl, lpr, a, max_items, s)
                        : dispatch_shape<false, 8>(cpl, lpr, a, max_items, s);
}

}  // namespace

int tokens_per_item(int, int) { return kTB; }

hipError_t launch_plan(const int32_t *union_ids, const int32_t *n_union, const int32_t *offsets,
                       int E, int A, int N, int has_shared, int tb_gu, int tb_dn, int max_gu,
                       int max_dn, Item *items_gu, Item *items_dn, int32_t *n_items, hipStream_t s)
{
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, union_ids, n_union,
                       offsets, E, A, N, has_shared, tb_gu, tb_dn, max_gu, max_dn, items_gu,
                       items_dn, n_items);
    return hipGetLastError();
}

hipError_t launch_gateup(const Geo &g, const uint8_t *pool, size_t stride, const uint8_t *shared,
                         const float *x, int k, const int32_t *perm, int A, const Item *items,
                         const int32_t *n_items, int max_items, float *h, hipStream_t s)
{
    return launch_pass(true, g, pool, stride, shared, x, k, perm, A, A / k, items, n_items,
                       max_items, h, s);
}

hipError_t launch_down(const Geo &g, const uint8_t *pool, size_t stride, const uint8_t *shared,
                       const float *h, int k, const int32_t *perm, int A, const Item *items,
                       const int32_t *n_items, int max_items, float *o, hipStream_t s)
{
    return launch_pass(false, g, pool, stride, shared, h, k, perm, A, A / k, items, n_items,
                       max_items, o, s);
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
