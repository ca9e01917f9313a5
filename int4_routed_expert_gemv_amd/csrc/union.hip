// union.hip - Union and Learn stages.
//
// Colibri pages, "Public Colibri Observation and Revision Ledger", section
// "Exact Architecture and Data-Flow Reconstruction": stage (2) Union merges the
// batch's requests so that each distinct expert is used once, and stage (5)
// Learn records which experts were used (per-expert hit counters). Same page,
// "Cache/Prefetch Design Comparison" (figure on async I/O and prefetch): the
// batch-union reads each unique expert once.
//
// Union also produces the token -> expert permutation that lets one pass over
// an expert's weights serve all of its tokens: a stable counting sort of the
// assignments a = t*k + j by expert id. Order comes from prefix sums and wave
// ballots, never from the order in which atomics land, so the permutation is
// the same on every run.
#include "internal.h"
#include "topk.h"

namespace moe {
namespace {

constexpr int kUnionThreads = 1024;
// s_waitcnt operand that waits for LDS operations only (lgkmcnt 0, vmcnt and
// expcnt at their maxima, gfx9 encoding)
constexpr int kLdsWait = 0xC07F;

__device__ __forceinline__ int wave_incl_scan_int(int v)
{
    const int lane = threadIdx.x % kWave;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int u = __shfl_up(v, o, kWave);
        if (lane >= o) v += u;
    }
    return v;
}

// waves of a union workgroup, each with its own chunk of the assignments
constexpr int kUnionWaves = kUnionThreads / kWave;

// Union and permutation by one workgroup of kUnionThreads threads. The
// assignments are cut into kUnionWaves contiguous chunks of whole 64-lane
// rounds, one per wave, in ascending order. ids may point to global or LDS
// memory; when stage is not null (LDS room for A ids) the ids are copied
// there as the histogram reads them and read back from there. hist: LDS of
// kUnionWaves * E ints (per-wave counts, then per-wave first positions); base:
// LDS of E ints. When counters is not null, counters[e] += expert e's count
// (the Learn stage's hit counts).
__device__ __forceinline__ void union_block(const int32_t *ids, int A, int E,
                                            int32_t *__restrict__ union_ids,
                                            int32_t *__restrict__ n_union,
                                            int32_t *__restrict__ offsets,
                                            int32_t *__restrict__ perm,
                                            unsigned long long *__restrict__ counters, int *hist,
                                            int *base, int *stage)
{
    const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
    const int C = ((A + kUnionWaves - 1) / kUnionWaves + kWave - 1) / kWave * kWave;
    const int a0 = min(A, wv * C), a1 = min(A, a0 + C);
    int *hw = hist + wv * E;  // this wave's counts, then its positions

    for (int i = tid; i < kUnionWaves * E; i += kUnionThreads) hist[i] = 0;
    __syncthreads();
    // per-wave integer histograms: the result does not depend on the order
    // of the adds
    for (int a = a0 + lane; a < a1; a += kWave) {
        const int e = ids[a];
        if (stage) stage[a] = e;
        if (e >= 0 && e < E) atomicAdd(&hw[e], 1);
    }
    __syncthreads();
    if (stage) ids = stage;

    // per expert (a thread each, E <= 1024): its count, and where each
    // wave's assignments start within the expert's slice (the counts of the
    // waves before it)
    int c = 0;
    if (tid < E) {
        for (int w = 0; w < kUnionWaves; ++w) {
            const int h = hist[w * E + tid];
            hist[w * E + tid] = c;
            c += h;
        }
    }
    // exclusive prefix sums over experts: counts -> offsets, and "used"
    // flags -> positions in union_ids
    const int used = c > 0 ? 1 : 0;
    // wave-level inclusive scans of (c, used) packed as c * 2048 + used
    // (c <= A < 2^20 is checked on the host, so the pack cannot overflow)
    long long v = (long long)c * 2048 + used;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        long long u = __shfl_up(v, o, kWave);
        if (lane >= o) v += u;
    }
    __shared__ long long wtot[kUnionWaves];
    if (lane == kWave - 1) wtot[wv] = v;
    __syncthreads();
    if (wv == 0) {
        long long x = lane < kUnionWaves ? wtot[lane] : 0;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            long long u = __shfl_up(x, o, kWave);
            if (lane >= o) x += u;
        }
        if (lane < kUnionWaves) wtot[lane] = x;  // inclusive
    }
    __syncthreads();
    long long incl = v + (wv > 0 ? wtot[wv - 1] : 0);
    long long excl = incl - ((long long)c * 2048 + used);
    const int off = (int)(excl / 2048), upos = (int)(excl % 2048);
    if (tid < E) {
        offsets[tid] = off;
        base[tid] = off;
        if (used) union_ids[upos] = tid;
        if (counters && used) atomicAdd(&counters[tid], (unsigned long long)c);
    }
    if (tid == kUnionThreads - 1) {
        const long long tot = wtot[kUnionWaves - 1];
        offsets[E] = (int)(tot / 2048);
        *n_union = (int)(tot % 2048);
    }
    __syncthreads();

    // stable scatter: every wave its own chunk, 64 assignments at a time in
    // ascending a; an assignment goes to its expert's offset + the earlier
    // waves' count + its rank among the earlier assignments of its wave with
    // the same expert (ballots on the bits of the expert id)
    const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    for (int r0 = a0; r0 < a1; r0 += kWave) {
        const int a = r0 + lane;
        int e = a < a1 ? ids[a] : -1;
        const bool valid = e >= 0 && e < E;
        if (!valid) e = -1;
        unsigned long long peers = __ballot(valid);
#pragma unroll
        for (int bit = 0; bit < 11; ++bit) {  // E <= 1024 < 2^11, and -1 stays apart
            const unsigned long long m = __ballot((e >> bit) & 1);
            peers &= ((e >> bit) & 1) ? m : ~m;
        }
        int rank = 0, bw = 0, bo = 0;
        if (valid) {
            rank = __popcll(peers & lt);
            bw = hw[e];
            bo = base[e];
        }
        // all reads of hw[] finish before any lane writes it back
        __builtin_amdgcn_s_waitcnt(kLdsWait);
        __builtin_amdgcn_wave_barrier();
        if (valid) {
            perm[bo + bw + rank] = a;
            const bool last = (peers >> lane) == 1ull;  // highest peer lane
            if (last) hw[e] = bw + rank + 1;
        }
        __builtin_amdgcn_s_waitcnt(kLdsWait);
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
}

// The same union, permutation and counts for at most 64 assignments, by one
// wave (wave 0 of the workgroup; no workgroup barrier): lane a holds
// assignment a; lane l owns experts l * PE .. l * PE + PE - 1 for the prefix
// sums (PE = ceil(E / 64) <= 16). Outputs equal union_block's; when counters
// is not null, counters[e] += expert e's count.
__device__ __forceinline__ void union_wave(const int32_t *ids, int A, int E,
                                           int32_t *__restrict__ union_ids,
                                           int32_t *__restrict__ n_union,
                                           int32_t *__restrict__ offsets,
                                           int32_t *__restrict__ perm,
                                           unsigned long long *__restrict__ counters, int *cnt)
{
    const int lane = threadIdx.x % kWave;
    constexpr int kMaxPE = MOE_MAX_EXPERTS / kWave;
    const int PE = (E + kWave - 1) / kWave;
    for (int e = lane; e < E; e += kWave) cnt[e] = 0;
    __builtin_amdgcn_s_waitcnt(kLdsWait);
    __builtin_amdgcn_wave_barrier();
    int e = lane < A ? ids[lane] : -1;
    const bool valid = e >= 0 && e < E;
    if (!valid) e = -1;
    if (valid) atomicAdd(&cnt[e], 1);
    __builtin_amdgcn_s_waitcnt(kLdsWait);
    __builtin_amdgcn_wave_barrier();
    // this lane's experts: counts, then exclusive sums over the lanes before
    int c[kMaxPE];
    int sc = 0, su = 0;
#pragma unroll
    for (int j = 0; j < kMaxPE; ++j) {
        const int ej = lane * PE + j;
        c[j] = (j < PE && ej < E) ? cnt[ej] : 0;
        sc += c[j];
        su += c[j] > 0 ? 1 : 0;
    }
    const int ic = wave_incl_scan_int(sc), iu = wave_incl_scan_int(su);
    int rc = ic - sc, ru = iu - su;
#pragma unroll
    for (int j = 0; j < kMaxPE; ++j) {
        const int ej = lane * PE + j;
        if (j < PE && ej < E) {
            offsets[ej] = rc;
            cnt[ej] = rc;  // from here on: the expert's first permutation position
            if (c[j] > 0) {
                union_ids[ru] = ej;
                if (counters) atomicAdd(&counters[ej], (unsigned long long)c[j]);
            }
            rc += c[j];
            ru += c[j] > 0 ? 1 : 0;
        }
    }
    if (lane == kWave - 1) {
        offsets[E] = ic;
        *n_union = iu;
    }
    __builtin_amdgcn_s_waitcnt(kLdsWait);
    __builtin_amdgcn_wave_barrier();
    // stable scatter: the rank among the lower lanes with the same expert,
    // from ballots on the bits of the expert id
    unsigned long long peers = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 11; ++bit) {  // E <= 1024 < 2^11, and -1 stays apart
        const unsigned long long m = __ballot((e >> bit) & 1);
        peers &= ((e >> bit) & 1) ? m : ~m;
    }
    if (valid) {
        const unsigned long long lt = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
        perm[cnt[e] + __popcll(peers & lt)] = lane;
    }
}

// ids of up to this many assignments are staged in LDS by union_kernel
constexpr int kUnionStage = 4096;

__global__ __launch_bounds__(kUnionThreads) void union_kernel(
    const int32_t *__restrict__ ids, int A, int E, int32_t *__restrict__ union_ids,
    int32_t *__restrict__ n_union, int32_t *__restrict__ offsets, int32_t *__restrict__ perm,
    unsigned long long *__restrict__ counters)
{
    __shared__ int hist[kUnionWaves * MOE_MAX_EXPERTS];
    __shared__ int base[MOE_MAX_EXPERTS];
    __shared__ int stage[kUnionStage];
    union_block(ids, A, E, union_ids, n_union, offsets, perm, counters, hist, base,
                A <= kUnionStage ? stage : nullptr);
}

// Route tail of a small batch (N <= kTailTokens): one wave per token selects
// its top k from the router's output, then the same workgroup forms the union
// and permutation of the N * k assignments and adds the per-expert counts to
// the hit counters (counters may be null). Outputs equal those of the top-k,
// union and hit-count kernels run in turn. With at most 64 assignments the
// workgroup is N waves and wave 0 does the union alone; otherwise it is
// kUnionThreads threads.
constexpr int kTailTokens = kUnionThreads / kWave;  // 16

template <bool OPT>
__global__ __launch_bounds__(kUnionThreads) void route_tail_kernel(
    const float *__restrict__ in, int P, const float *__restrict__ b, int N, int E, int k,
    int32_t *__restrict__ ids, float *__restrict__ w, int32_t *__restrict__ union_ids,
    int32_t *__restrict__ n_union, int32_t *__restrict__ offsets, int32_t *__restrict__ perm,
    unsigned long long *__restrict__ counters, TopkOpt opt)
{
    __shared__ int32_t s_ids[kTailTokens * MOE_MAX_K];
    __shared__ int cnt[MOE_MAX_EXPERTS];
    __shared__ int base[MOE_MAX_EXPERTS];
    __shared__ int hist[kUnionWaves * MOE_MAX_EXPERTS];
    const int tid = threadIdx.x, A = N * k;
    for (int a = tid; a < A; a += blockDim.x) s_ids[a] = -1;
    __syncthreads();
    const int t = tid / kWave;
    if (t < N) topk_wave<OPT>(in, P, b, N, E, k, t, ids, w, s_ids, opt);
    __syncthreads();
    if (A <= kWave) {  // one wave; the workgroup has one wave per token
        if (t == 0) union_wave(s_ids, A, E, union_ids, n_union, offsets, perm, counters, cnt);
        return;
    }
    union_block(s_ids, A, E, union_ids, n_union, offsets, perm, counters, hist, base, nullptr);
}

// ---- large batches: union, permutation and counts over several workgroups --
//
// The assignments are cut into G contiguous chunks, one workgroup each.
// 1. union_hist_kernel: per-chunk histograms hist[w][e] (scratch).
// 2. union_scan_kernel (one workgroup, a thread per expert): per expert the
//    exclusive sums over the chunks, the totals -> offsets, union_ids,
//    n_union and the hit counters; hist[w][e] becomes chunk w's first
//    position for expert e.
// 3. union_scatter_kernel: each chunk's assignments in ascending order, one
//    wave, ranks from ballots, at those positions.
// The result is the same stable counting sort as union_block's.
constexpr int kChunkThreads = 256;

__global__ __launch_bounds__(kChunkThreads) void union_hist_kernel(
    const int32_t *__restrict__ ids, int A, int E, int C, int32_t *__restrict__ hist)
{
    __shared__ int cnt[MOE_MAX_EXPERTS];
    const int w = blockIdx.x, tid = threadIdx.x;
    for (int e = tid; e < E; e += kChunkThreads) cnt[e] = 0;
    __syncthreads();
    const int a0 = w * C, a1 = min(A, a0 + C);
    for (int a = a0 + tid; a < a1; a += kChunkThreads) {
        const int e = ids[a];
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    for (int e = tid; e < E; e += kChunkThreads) hist[(size_t)w * E + e] = cnt[e];
}

__global__ __launch_bounds__(kUnionThreads) void union_scan_kernel(
    int E, int G, int32_t *__restrict__ hist, int32_t *__restrict__ union_ids,
    int32_t *__restrict__ n_union, int32_t *__restrict__ offsets,
    unsigned long long *__restrict__ counters)
{
    const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
    // per expert: the total over the chunks (16 loads in flight at a time)
    constexpr int kB = 16;
    int c = 0;
    if (tid < E) {
        for (int w0 = 0; w0 < G; w0 += kB) {
            int h[kB];
#pragma unroll
            for (int j = 0; j < kB; ++j) h[j] = w0 + j < G ? hist[(size_t)(w0 + j) * E + tid] : 0;
#pragma unroll
            for (int j = 0; j < kB; ++j) c += h[j];
        }
    }
    const int used = c > 0 ? 1 : 0;
    // exclusive sums over experts of (count, used), packed as in union_block
    long long v = (long long)c * 2048 + used;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        long long u = __shfl_up(v, o, kWave);
        if (lane >= o) v += u;
    }
    __shared__ long long wtot[kUnionThreads / kWave];
    if (lane == kWave - 1) wtot[wv] = v;
    __syncthreads();
    if (wv == 0) {
        long long x = lane < kUnionThreads / kWave ? wtot[lane] : 0;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            long long u = __shfl_up(x, o, kWave);
            if (lane >= o) x += u;
        }
        if (lane < kUnionThreads / kWave) wtot[lane] = x;
    }
    __syncthreads();
    const long long incl = v + (wv > 0 ? wtot[wv - 1] : 0);
    const long long excl = incl - ((long long)c * 2048 + used);
    const int off = (int)(excl / 2048), upos = (int)(excl % 2048);
    if (tid < E) {
        offsets[tid] = off;
        if (used) union_ids[upos] = tid;
        if (counters && c) atomicAdd(&counters[tid], (unsigned long long)c);
        // chunk w's first position for this expert: off + the counts of the
        // chunks before it
        int run = off;
        for (int w0 = 0; w0 < G; w0 += kB) {
            int h[kB];
#pragma unroll
            for (int j = 0; j < kB; ++j) h[j] = w0 + j < G ? hist[(size_t)(w0 + j) * E + tid] : 0;
#pragma unroll
            for (int j = 0; j < kB; ++j) {
                if (w0 + j < G) hist[(size_t)(w0 + j) * E + tid] = run;
                run += h[j];
            }
        }
    }
    if (tid == kUnionThreads - 1) {
        const long long tot = wtot[kUnionThreads / kWave - 1];
        offsets[E] = (int)(tot / 2048);
        *n_union = (int)(tot % 2048);
    }
}

__global__ __launch_bounds__(kWave) void union_scatter_kernel(
    const int32_t *__restrict__ ids, int A, int E, int C, const int32_t *__restrict__ hist,
    int32_t *__restrict__ perm)
{
    __shared__ int base[MOE_MAX_EXPERTS];
    const int w = blockIdx.x, lane = threadIdx.x;
    for (int e = lane; e < E; e += kWave) base[e] = hist[(size_t)w * E + e];
    __builtin_amdgcn_s_waitcnt(kLdsWait);
    __builtin_amdgcn_wave_barrier();
    const unsigned long long lt = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
    const int a0 = w * C, a1 = min(A, a0 + C);
    constexpr int kR = 8;  // rounds of 64 assignments whose ids are loaded together
    for (int r0 = a0; r0 < a1; r0 += kR * kWave) {
        int ev[kR];
#pragma unroll
        for (int j = 0; j < kR; ++j) {
            const int a = r0 + j * kWave + lane;
            ev[j] = a < a1 ? ids[a] : -1;
        }
#pragma unroll
        for (int j = 0; j < kR; ++j) {
            const int a = r0 + j * kWave + lane;
            int e = ev[j];
            const bool valid = e >= 0 && e < E;
            if (!valid) e = -1;
            unsigned long long peers = __ballot(valid);
#pragma unroll
            for (int bit = 0; bit < 11; ++bit) {
                const unsigned long long m = __ballot((e >> bit) & 1);
                peers &= ((e >> bit) & 1) ? m : ~m;
            }
            int pos = 0;
            if (valid) pos = base[e] + __popcll(peers & lt);
            __builtin_amdgcn_s_waitcnt(kLdsWait);
            __builtin_amdgcn_wave_barrier();
            if (valid) {
                perm[pos] = a;
                if ((peers >> lane) == 1ull) base[e] = pos + 1;  // highest peer lane
            }
            __builtin_amdgcn_s_waitcnt(kLdsWait);
            __builtin_amdgcn_wave_barrier();
        }
    }
}

constexpr int kHitThreads = 256;
constexpr int kHitPerBlock = 4096;

__global__ __launch_bounds__(kHitThreads) void hit_count_kernel(
    const int32_t *__restrict__ ids, int A, int E, unsigned long long *__restrict__ counters)
{
    __shared__ int hist[MOE_MAX_EXPERTS];
    for (int e = threadIdx.x; e < E; e += kHitThreads) hist[e] = 0;
    __syncthreads();
    const int a0 = blockIdx.x * kHitPerBlock;
    const int a1 = min(A, a0 + kHitPerBlock);
    for (int a = a0 + threadIdx.x; a < a1; a += kHitThreads) {
        int e = ids[a];
        if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kHitThreads)
        if (hist[e]) atomicAdd(&counters[e], (unsigned long long)hist[e]);
}

}  // namespace

hipError_t launch_union(const int32_t *ids, int A, int E, int32_t *union_ids, int32_t *n_union,
                        int32_t *offsets, int32_t *perm, uint64_t *counters, hipStream_t s)
{
    hipLaunchKernelGGL(union_kernel, dim3(1), dim3(kUnionThreads), 0, s, ids, A, E, union_ids,
                       n_union, offsets, perm, reinterpret_cast<unsigned long long *>(counters));
    return hipGetLastError();
}

int route_tail_max_tokens() { return kTailTokens; }

hipError_t launch_route_tail(const float *in, int P, const float *b, int N, int E, int k,
                             int32_t *ids, float *w, int32_t *union_ids, int32_t *n_union,
                             int32_t *offsets, int32_t *perm, uint64_t *counters, hipStream_t s,
                             TopkOpt opt)
{
    if (N < 1 || N > kTailTokens) return hipErrorInvalidValue;
    const int threads = N * k <= kWave ? N * kWave : kUnionThreads;
    hipLaunchKernelGGL(opt.any() ? route_tail_kernel<true> : route_tail_kernel<false>, dim3(1),
                       dim3(threads), 0, s, in, P, b, N, E, k,
                       ids, w, union_ids, n_union, offsets, perm,
                       reinterpret_cast<unsigned long long *>(counters), opt);
    return hipGetLastError();
}

int union_chunks(int A, int E, size_t scratch_bytes)
{
    // chunks of at least 512 assignments, at most 256 of them, within the scratch
    int G = (A + 511) / 512;
    if (G > 256) G = 256;
    while (G > 1 && (size_t)G * E * 4 > scratch_bytes) G /= 2;
    return G;
}

hipError_t launch_union_chunked(const int32_t *ids, int A, int E, int32_t *union_ids,
                                int32_t *n_union, int32_t *offsets, int32_t *perm,
                                uint64_t *counters, void *scratch, size_t scratch_bytes,
                                hipStream_t s)
{
    const int G = union_chunks(A, E, scratch_bytes);
    if (G < 1 || (size_t)G * E * 4 > scratch_bytes) return hipErrorInvalidValue;
    const int C = (A + G - 1) / G;
    int32_t *hist = static_cast<int32_t *>(scratch);
    hipLaunchKernelGGL(union_hist_kernel, dim3(G), dim3(kChunkThreads), 0, s, ids, A, E, C, hist);
    hipLaunchKernelGGL(union_scan_kernel, dim3(1), dim3(kUnionThreads), 0, s, E, G, hist, union_ids,
                       n_union, offsets, reinterpret_cast<unsigned long long *>(counters));
    hipLaunchKernelGGL(union_scatter_kernel, dim3(G), dim3(kWave), 0, s, ids, A, E, C, hist, perm);
    return hipGetLastError();
}

hipError_t launch_hit_count(const int32_t *ids, int A, int E, uint64_t *counters, hipStream_t s)
{
    hipLaunchKernelGGL(hit_count_kernel, dim3((A + kHitPerBlock - 1) / kHitPerBlock),
                       dim3(kHitThreads), 0, s, ids, A, E,
                       reinterpret_cast<unsigned long long *>(counters));
    return hipGetLastError();
}

}  // namespace moe
