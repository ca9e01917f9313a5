// probe.hip - measured ceilings of the machine, beside the published peaks:
// a plain streaming read (what one launch of a given size can pull from HBM)
// and a loop of independent float16 matrix-core products (what the matrix
// cores sustain). Neither is part of the layer step; bench.py reports them
// next to the roofline of the step's kernels.
#include <hip/hip_ext.h>

#include "internal.h"
#include "moe_probe.h"

namespace moe {
namespace {

// Each wave reads UB consecutive 1 KB units (one 16-byte load per lane per
// unit, all issued before the first use) and folds them into one word; the
// word is stored only if it equals a value the caller never plants, so the
// loads cannot be dropped and nothing is written in practice.
template <int UB>
__global__ void stream_read_kernel(const uint4 *__restrict__ buf, long long units,
                                   unsigned *__restrict__ sink)
{
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const long long first = ((long long)blockIdx.x * (blockDim.x / kWave) + wave) * UB;
    uint4 w[UB];
#pragma unroll
    for (int u = 0; u < UB; ++u) {
        const long long un = min(first + u, units - 1);
        w[u] = buf[un * kWave + lane];
    }
    unsigned acc = 0;
#pragma unroll
    for (int u = 0; u < UB; ++u) acc ^= w[u].x ^ w[u].y ^ w[u].z ^ w[u].w;
    if (acc == 0x9E3779B9u && first < units) sink[blockIdx.x] = acc;
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Four independent accumulation chains of v_mfma_f32_16x16x32_f16 per wave,
// iters rounds; operands stay in registers. One float per wave is stored.
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float seed, float *__restrict__ out)
{
    const int lane = threadIdx.x % kWave;
    f16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (_Float16)(seed * (float)(lane + i));
        b[i] = (_Float16)(seed * (float)(lane - i));
    }
    f32x4 c0 = {0, 0, 0, 0}, c1 = c0, c2 = c0, c3 = c0;
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c3, 0, 0, 0);
    }
    const f32x4 s = c0 + c1 + c2 + c3;
    if (lane == 0)
        out[blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave] = s[0] + s[1] + s[2] + s[3];
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

moe_status moe_probe_stream_read(const void *buf, size_t bytes, int units_per_wave,
                                 int waves_per_workgroup, unsigned *sink, size_t sink_words,
                                 hipEvent_t start, hipEvent_t end, hipStream_t stream)
{
    if (!buf || !sink || bytes < 1024 || bytes % 1024) return MOE_EINVAL;
    if ((uintptr_t)buf % 16) return MOE_EALIGN;
    if (waves_per_workgroup < 1 || waves_per_workgroup > 16) return MOE_EINVAL;
    const long long units = (long long)(bytes / 1024);
    const long long waves = (units + units_per_wave - 1) / units_per_wave;
    const long long blocks = (waves + waves_per_workgroup - 1) / waves_per_workgroup;
    if (blocks > 0x7FFFFFFFLL || (size_t)blocks > sink_words) return MOE_EINVAL;
    const dim3 grid((unsigned)blocks), block(waves_per_workgroup * kWave);
    const uint4 *b = static_cast<const uint4 *>(buf);
    auto go = [&](auto kernel) {
        hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, start, end, 0, b, units, sink);
    };
    switch (units_per_wave) {
    case 3: go(stream_read_kernel<3>); break;
    case 6: go(stream_read_kernel<6>); break;
    case 12: go(stream_read_kernel<12>); break;
    default: return MOE_EINVAL;
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

moe_status moe_probe_mfma_f16(float *out, int workgroups, int iters, hipEvent_t start,
                              hipEvent_t end, hipStream_t stream)
{
    if (!out || workgroups < 1 || iters < 1) return MOE_EINVAL;
    hipExtLaunchKernelGGL(mfma_loop_kernel, dim3(workgroups), dim3(256), 0, stream, start, end, 0,
                          iters, 1.0f / 4096.0f, out);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

}  // extern "C"
