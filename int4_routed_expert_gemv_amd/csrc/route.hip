// route.hip - Route stage: float32 sigmoid router and stable top-k.
//
// Colibri pages, "Public Colibri Observation and Revision Ledger", section
// "Exact Architecture and Data-Flow Reconstruction": a trained sigmoid gate
// scores all experts for every token of every MoE layer, with n_group = 1 (a
// plain top-k over all experts) and float32 gate parameters.
//
//   scores[t][e] = 1 / (1 + exp(-(b[e] + sum_i Wr[e][i] x[t][i])))  (float32)
//   top-k on the float32 score, ties to the lower expert id, ids in rank order.
#include "internal.h"
#include "topk.h"

namespace moe {
namespace {

constexpr int kRouterThreads = 256;
constexpr int kMaxRowVec = 16;  // row of Wr cached in registers up to 16 float4 per thread

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

// Sum over the wave (uniform result): DPP within rows of 16, then lane reads.
__device__ __forceinline__ float wave_sum_dpp(float v)
{
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    v += dpp<0x141>(v);
    v += dpp<0x140>(v);
    return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

// pairwise sum of W per-wave partial sums, always in the same order
template <int W>
__device__ __forceinline__ float tree_sum(const float *p)
{
    if constexpr (W == 1)
        return p[0];
    else
        return tree_sum<W / 2>(p) + tree_sum<W / 2>(p + W / 2);
}

constexpr int kTokGroup = 4;
// batches up to this many tokens use the one-workgroup-per-expert GEMV router
constexpr int kGemvMaxTokens = 16;

// Decode-sized batches: one workgroup per expert keeps its router row in
// registers (read from HBM once) and dots it with the tokens, four tokens per
// reduction round. Loads are issued unconditionally (past the row's end they
// read its last float4, weighted by zero), so each round's loads are all in
// flight before the first product waits.
template <int RV>  // float4 of the row per thread (RV * 1024 >= d)
__global__ __launch_bounds__(kRouterThreads) void router_gemv_kernel(
    const float *__restrict__ x, int N, int d, const float *__restrict__ wr,
    const float *__restrict__ b, int E, float *__restrict__ scores)
{
    __shared__ float part[kTokGroup][kRouterThreads / kWave];
    const int e = blockIdx.x;
    const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
    const int nq = d / 4;
    const float4 *row = reinterpret_cast<const float4 *>(wr + (size_t)e * d);
    int qi[RV];
    float4 w[RV];
#pragma unroll
    for (int m = 0; m < RV; ++m) {
        const int q = tid + m * kRouterThreads;
        qi[m] = min(q, nq - 1);
        w[m] = row[qi[m]];
        if (q >= nq) w[m] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const float bias = b ? b[e] : 0.0f;
    for (int t0 = 0; t0 < N; t0 += kTokGroup) {
        float acc[kTokGroup];
        float4 v[kTokGroup][RV];
#pragma unroll
        for (int i = 0; i < kTokGroup; ++i) {
            const float4 *xt = reinterpret_cast<const float4 *>(x + (size_t)min(t0 + i, N - 1) * d);
#pragma unroll
            for (int m = 0; m < RV; ++m) v[i][m] = xt[qi[m]];
        }
#pragma unroll
        for (int i = 0; i < kTokGroup; ++i) {
            acc[i] = 0.0f;
#pragma unroll
            for (int m = 0; m < RV; ++m) {
                acc[i] = fmaf(w[m].x, v[i][m].x, acc[i]);
                acc[i] = fmaf(w[m].y, v[i][m].y, acc[i]);
                acc[i] = fmaf(w[m].z, v[i][m].z, acc[i]);
                acc[i] = fmaf(w[m].w, v[i][m].w, acc[i]);
            }
        }
#pragma unroll
        for (int i = 0; i < kTokGroup; ++i) {
            const float s = wave_sum_dpp(acc[i]);
            if (lane == 0) part[i][wv] = s;
        }
        __syncthreads();
        if (tid < kTokGroup && t0 + tid < N) {
            const float l = tree_sum<kRouterThreads / kWave>(part[tid]);
            scores[(size_t)(t0 + tid) * E + e] = sigmoidf(l + bias);
        }
        __syncthreads();
    }
}

// Rows longer than the register cache: stream the row for every token.
__global__ __launch_bounds__(kRouterThreads) void router_gemv_stream_kernel(
    const float *__restrict__ x, int N, int d, const float *__restrict__ wr,
    const float *__restrict__ b, int E, float *__restrict__ scores)
{
    __shared__ float part[kRouterThreads / kWave];
    const int e = blockIdx.x;
    const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
    const int nq = d / 4;
    const float4 *row = reinterpret_cast<const float4 *>(wr + (size_t)e * d);
    const float bias = b ? b[e] : 0.0f;
    for (int t = 0; t < N; ++t) {
        const float4 *xt = reinterpret_cast<const float4 *>(x + (size_t)t * d);
        float acc = 0.0f;
        for (int q = tid; q < nq; q += kRouterThreads) {
            float4 w = row[q], v = xt[q];
            acc = fmaf(w.x, v.x, acc);
            acc = fmaf(w.y, v.y, acc);
            acc = fmaf(w.z, v.z, acc);
            acc = fmaf(w.w, v.w, acc);
        }
        acc = wave_sum(acc);
        if (lane == 0) part[wv] = acc;
        __syncthreads();
        if (tid == 0) {
            float l = part[0];
            for (int i = 1; i < kRouterThreads / kWave; ++i) l += part[i];
            scores[(size_t)t * E + e] = sigmoidf(l + bias);
        }
        __syncthreads();
    }
}

// Larger batches: a 64-token x 64-expert tile per workgroup over one K slice
// (of P), operands staged through LDS in K-steps of 32 (double-buffered, the
// next step's loads issued before the current step's products), 4x4
// outputs per thread, float32 FMA. With P == 1 the tile writes final scores;
// otherwise it writes raw partial sums [P][N][E] that the top-k kernel adds
// in slice order.
constexpr int kTM = 64, kTN = 64, kTK = 32;

__global__ __launch_bounds__(256) void router_gemm_kernel(
    const float *__restrict__ x, int N, int d, const float *__restrict__ wr,
    const float *__restrict__ b, int E, int P, float *__restrict__ out)
{
    __shared__ float xs[2][kTK][kTM + 4];
    __shared__ float ws[2][kTK][kTN + 4];
    const int t0 = blockIdx.x * kTM, e0 = blockIdx.y * kTN, p = blockIdx.z;
    const int tid = threadIdx.x;
    const int tr = tid / 16, tc = tid % 16;  // 16 x 16 threads, 4x4 each
    const int kper = d / P, kbeg = p * kper, steps = kper / kTK;
    // loader: 64 rows x 32 k = 512 float4 -> two per thread (rows lr, lr + 32);
    // rows past N or E read the last row (results dropped): every load issued
    const int lr = tid / 8, lk = (tid % 8) * 4;
    const float *xr0 = x + (size_t)min(t0 + lr, N - 1) * d + kbeg + lk;
    const float *xr1 = x + (size_t)min(t0 + lr + 32, N - 1) * d + kbeg + lk;
    const float *wr0 = wr + (size_t)min(e0 + lr, E - 1) * d + kbeg + lk;
    const float *wr1 = wr + (size_t)min(e0 + lr + 32, E - 1) * d + kbeg + lk;
    float4 xv0, xv1, wv0, wv1;
    auto load = [&](int st) {
        const int o = st * kTK;
        xv0 = *reinterpret_cast<const float4 *>(xr0 + o);
        xv1 = *reinterpret_cast<const float4 *>(xr1 + o);
        wv0 = *reinterpret_cast<const float4 *>(wr0 + o);
        wv1 = *reinterpret_cast<const float4 *>(wr1 + o);
    };
    auto store = [&](int buf) {
        const float xa[4] = {xv0.x, xv0.y, xv0.z, xv0.w}, xb[4] = {xv1.x, xv1.y, xv1.z, xv1.w};
        const float wa[4] = {wv0.x, wv0.y, wv0.z, wv0.w}, wb[4] = {wv1.x, wv1.y, wv1.z, wv1.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            xs[buf][lk + j][lr] = xa[j];
            xs[buf][lk + j][lr + 32] = xb[j];
            ws[buf][lk + j][lr] = wa[j];
            ws[buf][lk + j][lr + 32] = wb[j];
        }
    };
    float acc[4][4] = {};
    load(0);
    store(0);
    __syncthreads();
    for (int st = 0; st < steps; ++st) {
        const int cur = st & 1;
        if (st + 1 < steps) load(st + 1);
        // each K-step is summed on its own and then added, which keeps the
        // rounding error of the long dot products near that of a tree
        float part[4][4] = {};
#pragma unroll 4
        for (int kk = 0; kk < kTK; ++kk) {
            float a[4], c[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = xs[cur][kk][tr * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) c[j] = ws[cur][kk][tc * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) part[i][j] = fmaf(a[i], c[j], part[i][j]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] += part[i][j];
        if (st + 1 < steps) store(cur ^ 1);
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + tr * 4 + i;
        if (t >= N) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = e0 + tc * 4 + j;
            if (e >= E) continue;
            if (P == 1)
                out[(size_t)t * E + e] = sigmoidf(acc[i][j] + (b ? b[e] : 0.0f));
            else
                out[((size_t)p * N + t) * E + e] = acc[i][j];
        }
    }
}

// Larger batches, d a multiple of 128: the same product on the matrix cores in
// float32 (v_mfma_f32_16x16x4f32: exact float32 products, float32 sums). A
// workgroup of 4 waves computes a 32-token x 32-expert tile over one K slice
// (of P); each wave takes a quarter of the slice and the four partial tiles
// are added in LDS in wave order. Both operands come straight from memory,
// 16 bytes per lane: within each 16-column block lane l reads columns
// 4 (l / 16) .. + 3 of token row (or router row) l % 16, and k-step j of the
// block takes component j of every lane, so a step multiplies matching
// columns of x and Wr (a permutation of the contraction order, the same for
// every output). Loads run kRD blocks ahead of the products (kRD even, and
// every wave's column count a multiple of 32). Rows past N or E
// read the last row; their outputs are dropped. The output is as
// router_gemm_kernel's: final scores when P == 1, raw partial sums
// [P][N][E] otherwise.
constexpr int kRT = 32;      // tokens and experts per workgroup tile (the large one: 64)
constexpr int kRW = 4;       // waves per workgroup, each a quarter of the K slice
constexpr int kRD = 4;       // 16-column blocks of operands in flight per wave (large tile: 2)

typedef float rf32x4_t __attribute__((ext_vector_type(4)));

// RT x RT tiles (RT = 32, or 64 for batches that give at least 256 such
// tiles: each operand block then feeds twice the products, which halves the
// operand bytes per product), RD blocks of operands in flight.
template <int RT, int RD>
__global__ __launch_bounds__(kRW * kWave) void router_mfma_kernel(
    const float *__restrict__ x, int N, int d, const float *__restrict__ wr,
    const float *__restrict__ b, int E, int P, float *__restrict__ out)
{
    constexpr int NT = RT / 16;  // 16-row blocks per tile side
    __shared__ float red[kRW][RT][RT + 1];
    const int t0 = blockIdx.x * RT, e0 = blockIdx.y * RT, p = blockIdx.z;
    const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
    const int r = lane % 16, kq = lane / 16;
    const int kw = d / (P * kRW);                    // this wave's columns
    const int kbeg = p * (d / P) + wv * kw + 4 * kq;
    const int nb = kw / 16;                          // 16-column blocks
    const float *xr[NT], *wp[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        xr[i] = x + (size_t)min(t0 + 16 * i + r, N - 1) * d + kbeg;
        wp[i] = wr + (size_t)min(e0 + 16 * i + r, E - 1) * d + kbeg;
    }
    float4 xa[RD][NT], wb[RD][NT];
    auto load = [&](int blk, float4 (&xv)[NT], float4 (&wv4)[NT]) {
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            xv[i] = *reinterpret_cast<const float4 *>(xr[i] + (size_t)blk * 16);
            wv4[i] = *reinterpret_cast<const float4 *>(wp[i] + (size_t)blk * 16);
        }
    };
    rf32x4_t acc[NT][NT], part[NT][NT];
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = rf32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < RD; ++s) load(min(s, nb - 1), xa[s], wb[s]);
    // every load is issued on every path (past the end they reload the last
    // block into a stage no later step reads), so each wait is for one stage.
    // Each pair of blocks (32 columns) is summed from zero on its own and then
    // added to the running sum, which keeps the long dot products' rounding
    // error near that of a blocked sum (the running sum takes d / 32 adds,
    // not d / 4)
    for (int b0 = 0; b0 < nb; b0 += RD) {
#pragma unroll
        for (int s = 0; s < RD; ++s) {
            if (b0 + s >= nb) break;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int it = 0; it < NT; ++it)
#pragma unroll
                    for (int ie = 0; ie < NT; ++ie)
                        part[it][ie] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                            xa[s][it][j], wb[s][ie][j],
                            (s % 2 == 0 && j == 0) ? rf32x4_t{0.f, 0.f, 0.f, 0.f} : part[it][ie],
                            0, 0, 0);
            if (s % 2 == 1) {
#pragma unroll
                for (int it = 0; it < NT; ++it)
#pragma unroll
                    for (int ie = 0; ie < NT; ++ie) acc[it][ie] += part[it][ie];
            }
            load(min(b0 + s + RD, nb - 1), xa[s], wb[s]);
        }
    }
    // register v of block (it, ie): token 16 it + 4 kq + v, expert 16 ie + r
#pragma unroll
    for (int it = 0; it < NT; ++it)
#pragma unroll
        for (int ie = 0; ie < NT; ++ie)
#pragma unroll
            for (int v = 0; v < 4; ++v) red[wv][16 * it + 4 * kq + v][16 * ie + r] = acc[it][ie][v];
    __syncthreads();
    for (int o = tid; o < RT * RT; o += kRW * kWave) {
        const int tt = o / RT, ee = o % RT;
        const int t = t0 + tt, e = e0 + ee;
        if (t >= N || e >= E) continue;
        float v = red[0][tt][ee];
#pragma unroll
        for (int w = 1; w < kRW; ++w) v += red[w][tt][ee];
        if (P == 1)
            out[(size_t)t * E + e] = sigmoidf(v + (b ? b[e] : 0.0f));
        else
            out[((size_t)p * N + t) * E + e] = v;
    }
}

// One wave per token (the selection itself is topk_wave).
template <bool OPT, int PB>
__global__ __launch_bounds__(256) void topk_kernel(
    const float *__restrict__ in, int P, const float *__restrict__ b, int N, int E, int k,
    int32_t *__restrict__ ids, float *__restrict__ w, TopkOpt opt)
{
    const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (t >= N) return;
    topk_wave<OPT, PB>(in, P, b, N, E, k, t, ids, w, nullptr, opt);
}

}  // namespace

int router_slices_bound(int N, int E)
{
    // K slices so that the tiles and slices give about 512 workgroups (two
    // per compute unit), at most 16; none for the GEMV router
    if (N <= kGemvMaxTokens) return 1;
    const long long tiles = (long long)((N + kTM - 1) / kTM) * ((E + kTN - 1) / kTN);
    int p = 1;
    while (p < kMaxSlices && tiles * p * 2 <= 512) p *= 2;
    return p;
}

// whether launch_router takes the matrix-core router
bool router_on_mfma(int N, int d) { return N > kGemvMaxTokens && d % (kRW * 32) == 0; }

int router_slices(int N, int d, int E)
{
    if (N <= kGemvMaxTokens) return 1;
    const int bound = router_slices_bound(N, E);
    if (router_on_mfma(N, d)) {
        // K slices until the 32 x 32 tiles give 256 workgroups (one per
        // compute unit: each holds four waves on the matrix cores)
        const long long tiles = (long long)((N + kRT - 1) / kRT) * ((E + kRT - 1) / kRT);
        int p = 1;
        while (p < bound && tiles * p < 256 && d % (2 * p * kRW * 32) == 0) p *= 2;
        return p;
    }
    int p = bound;
    while (p > 1 && (d % (p * kTK)) != 0) p /= 2;
    return p;
}

hipError_t launch_router(const float *x, int N, int d, const float *wr, const float *b, int E,
                         float *out, hipStream_t s)
{
    if (N <= kGemvMaxTokens) {
        const int rv = (d / 4 + kRouterThreads - 1) / kRouterThreads;
        auto go = [&](auto kernel) {
            hipLaunchKernelGGL(kernel, dim3(E), dim3(kRouterThreads), 0, s, x, N, d, wr, b, E, out);
        };
        if (rv <= 1) go(router_gemv_kernel<1>);
        else if (rv <= 2) go(router_gemv_kernel<2>);
        else if (rv <= 4) go(router_gemv_kernel<4>);
        else if (rv <= 6) go(router_gemv_kernel<6>);
        else if (rv <= 8) go(router_gemv_kernel<8>);
        else if (rv <= 12) go(router_gemv_kernel<12>);
        else if (rv <= kMaxRowVec) go(router_gemv_kernel<kMaxRowVec>);
        else
            hipLaunchKernelGGL(router_gemv_stream_kernel, dim3(E), dim3(kRouterThreads), 0, s, x,
                               N, d, wr, b, E, out);
    } else if (router_on_mfma(N, d)) {
        const int P = router_slices(N, d, E);
        // one slice and at least 256 tiles of 64: the large tile
        const long long big = (long long)((N + 63) / 64) * ((E + 63) / 64);
        if (P == 1 && big >= 256) {
            dim3 grid((N + 63) / 64, (E + 63) / 64, 1);
            hipLaunchKernelGGL((router_mfma_kernel<64, 2>), grid, dim3(kRW * kWave), 0, s, x, N, d,
                               wr, b, E, P, out);
        } else {
            dim3 grid((N + kRT - 1) / kRT, (E + kRT - 1) / kRT, P);
            hipLaunchKernelGGL((router_mfma_kernel<kRT, kRD>), grid, dim3(kRW * kWave), 0, s, x, N,
                               d, wr, b, E, P, out);
        }
    } else {
        const int P = router_slices(N, d, E);
        dim3 grid((N + kTM - 1) / kTM, (E + kTN - 1) / kTN, P);
        hipLaunchKernelGGL(router_gemm_kernel, grid, dim3(256), 0, s, x, N, d, wr, b, E, P, out);
    }
    return hipGetLastError();
}

hipError_t launch_topk(const float *in, int P, const float *b, int N, int E, int k, int32_t *ids,
                       float *w, hipStream_t s, TopkOpt opt)
{
    const int per_block = 4;
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3((N + per_block - 1) / per_block), dim3(per_block * kWave), 0,
                           s, in, P, b, N, E, k, ids, w, opt);
        return hipGetLastError();
    };
    // the slice bound fixes how many partial sums each lane loads at a time
    const bool o = opt.any();
    if (P <= 1) return o ? go(topk_kernel<true, 1>) : go(topk_kernel<false, 1>);
    if (P <= 2) return o ? go(topk_kernel<true, 2>) : go(topk_kernel<false, 2>);
    if (P <= 4) return o ? go(topk_kernel<true, 4>) : go(topk_kernel<false, 4>);
    if (P <= 8) return o ? go(topk_kernel<true, 8>) : go(topk_kernel<false, 8>);
    if (P <= kMaxSlices) return o ? go(topk_kernel<true, kMaxSlices>) : go(topk_kernel<false, kMaxSlices>);
    return hipErrorInvalidValue;
}

}  // namespace moe
