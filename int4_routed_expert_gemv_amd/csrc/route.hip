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

namespace moe {
namespace {

constexpr int kRouterThreads = 256;
constexpr int kMaxRowVec = 16;  // row of Wr cached in registers up to 16 float4 per thread

__device__ __forceinline__ float sigmoidf(float l) { return 1.0f / (1.0f + expf(-l)); }

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

constexpr int kTokGroup = 4;

// Decode-sized batches: one workgroup per expert keeps its router row in
// registers (read from HBM once) and dots it with the tokens, four tokens per
// reduction round.
__global__ __launch_bounds__(kRouterThreads) void router_gemv_kernel(
    const float *__restrict__ x, int N, int d, const float *__restrict__ wr,
    const float *__restrict__ b, int E, float *__restrict__ scores)
{
    __shared__ float part[kTokGroup][kRouterThreads / kWave];
    const int e = blockIdx.x;
    const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
    const int nq = d / 4;
    const float4 *row = reinterpret_cast<const float4 *>(wr + (size_t)e * d);
    float4 w[kMaxRowVec];
#pragma unroll
    for (int m = 0; m < kMaxRowVec; ++m) {
        const int q = tid + m * kRouterThreads;
        w[m] = q < nq ? row[q] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const float bias = b ? b[e] : 0.0f;
    for (int t0 = 0; t0 < N; t0 += kTokGroup) {
        float acc[kTokGroup];
#pragma unroll
        for (int i = 0; i < kTokGroup; ++i) {
            acc[i] = 0.0f;
            if (t0 + i >= N) continue;
            const float4 *xt = reinterpret_cast<const float4 *>(x + (size_t)(t0 + i) * d);
#pragma unroll
            for (int m = 0; m < kMaxRowVec; ++m) {
                const int q = tid + m * kRouterThreads;
                if (q < nq) {
                    const float4 v = xt[q];
                    acc[i] = fmaf(w[m].x, v.x, acc[i]);
                    acc[i] = fmaf(w[m].y, v.y, acc[i]);
                    acc[i] = fmaf(w[m].z, v.z, acc[i]);
                    acc[i] = fmaf(w[m].w, v.w, acc[i]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < kTokGroup; ++i) {
            const float v = wave_sum_dpp(acc[i]);
            if (lane == 0) part[i][wv] = v;
        }
        __syncthreads();
        if (tid < kTokGroup && t0 + tid < N) {
            const float l = (part[tid][0] + part[tid][1]) + (part[tid][2] + part[tid][3]);
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

// Prefill-sized batches: a 64-token x 64-expert tile per workgroup, operands
// staged through LDS in K-steps of 16, 4x4 outputs per thread, float32 FMA.
constexpr int kTM = 64, kTN = 64, kTK = 16;

__global__ __launch_bounds__(256) void router_gemm_kernel(
    const float *__restrict__ x, int N, int d, const float *__restrict__ wr,
    const float *__restrict__ b, int E, float *__restrict__ scores)
{
    __shared__ float xs[kTK][kTM + 4];
    __shared__ float ws[kTK][kTN + 4];
    const int t0 = blockIdx.x * kTM, e0 = blockIdx.y * kTN;
    const int tid = threadIdx.x;
    const int tr = tid / 16, tc = tid % 16;  // 16 x 16 threads, 4x4 each
    float acc[4][4] = {};
    // loader: 64 rows x 16 k = 256 float4 -> one float4 per thread
    const int lr = tid / 4, lk = (tid % 4) * 4;
    for (int k0 = 0; k0 < d; k0 += kTK) {
        float4 xv = make_float4(0.f, 0.f, 0.f, 0.f), wv = xv;
        if (t0 + lr < N) xv = *reinterpret_cast<const float4 *>(x + (size_t)(t0 + lr) * d + k0 + lk);
        if (e0 + lr < E) wv = *reinterpret_cast<const float4 *>(wr + (size_t)(e0 + lr) * d + k0 + lk);
        xs[lk + 0][lr] = xv.x; xs[lk + 1][lr] = xv.y; xs[lk + 2][lr] = xv.z; xs[lk + 3][lr] = xv.w;
        ws[lk + 0][lr] = wv.x; ws[lk + 1][lr] = wv.y; ws[lk + 2][lr] = wv.z; ws[lk + 3][lr] = wv.w;
        __syncthreads();
        // each K-step is summed on its own and then added, which keeps the
        // rounding error of the 6144-term dot products near that of a tree
        float part[4][4] = {};
#pragma unroll
        for (int kk = 0; kk < kTK; ++kk) {
            float a[4], c[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = xs[kk][tr * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) c[j] = ws[kk][tc * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) part[i][j] = fmaf(a[i], c[j], part[i][j]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] += part[i][j];
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int t = t0 + tr * 4 + i;
        if (t >= N) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int e = e0 + tc * 4 + j;
            if (e < E) scores[(size_t)t * E + e] = sigmoidf(acc[i][j] + (b ? b[e] : 0.0f));
        }
    }
}

// Order-preserving map of float bits onto unsigned integers (NaN above +inf).
__device__ __forceinline__ uint32_t sortable(float v) {
    uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kMaxPerLane = MOE_MAX_EXPERTS / kWave;  // 16

// One wave per token: k rounds of a wave-wide max over 64-bit keys
// (sortable score, then inverted id so equal scores go to the lower id).
__global__ __launch_bounds__(256) void topk_kernel(
    const float *__restrict__ scores, int N, int E, int k, int32_t *__restrict__ ids,
    float *__restrict__ w)
{
    const int lane = threadIdx.x % kWave;
    const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (t >= N) return;
    const float *s = scores + (size_t)t * E;
    uint32_t hi[kMaxPerLane];
    uint32_t taken = 0;
#pragma unroll
    for (int m = 0; m < kMaxPerLane; ++m) {
        int e = lane + m * kWave;
        hi[m] = e < E ? sortable(s[e]) : 0u;
        if (e >= E) taken |= 1u << m;
    }
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
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            uint32_t oh = __shfl_xor(bh, o, kWave), ol = __shfl_xor(bl, o, kWave);
            if (oh > bh || (oh == bh && ol > bl)) { bh = oh; bl = ol; }
        }
        const int id = (int)(0xFFFFFFFFu - bl);
        if (bm >= 0 && lane + bm * kWave == id) taken |= 1u << bm;
        if (lane == 0) {
            ids[(size_t)t * k + j] = id;
            w[(size_t)t * k + j] = s[id];
        }
    }
}

}  // namespace

hipError_t launch_router(const float *x, int N, int d, const float *wr, const float *b, int E,
                         float *scores, hipStream_t s)
{
    if (N <= 512) {
        if (d <= 4 * kMaxRowVec * kRouterThreads)
            hipLaunchKernelGGL(router_gemv_kernel, dim3(E), dim3(kRouterThreads), 0, s, x, N, d,
                               wr, b, E, scores);
        else
            hipLaunchKernelGGL(router_gemv_stream_kernel, dim3(E), dim3(kRouterThreads), 0, s, x,
                               N, d, wr, b, E, scores);
    } else {
        dim3 grid((N + kTM - 1) / kTM, (E + kTN - 1) / kTN);
        hipLaunchKernelGGL(router_gemm_kernel, grid, dim3(256), 0, s, x, N, d, wr, b, E, scores);
    }
    return hipGetLastError();
}

hipError_t launch_topk(const float *scores, int N, int E, int k, int32_t *ids, float *w,
                       hipStream_t s)
{
    const int per_block = 4;
    hipLaunchKernelGGL(topk_kernel, dim3((N + per_block - 1) / per_block), dim3(per_block * kWave),
                       0, s, scores, N, E, k, ids, w);
    return hipGetLastError();
}

}  // namespace moe
