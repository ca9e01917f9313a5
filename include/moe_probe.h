/*
 * moe_probe.h - measured ceilings of the GPU, reported beside the published
 * peaks (8 TB/s HBM, 2.5 PFLOP/s dense float16). Not part of the layer step:
 * the layer-step calls are in moe.h. Both calls enqueue one kernel on
 * `stream`, taking the optional events `start` and `end` (may be NULL) at the
 * kernel's own start and end, and return MOE_EINVAL / MOE_EALIGN for bad
 * arguments before any launch.
 */
#ifndef MOE_PROBE_H
#define MOE_PROBE_H

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * A plain streaming read of `bytes` (a multiple of 1024) at `buf` (device,
 * 16-byte aligned): each wave reads units_per_wave (3, 6 or 12) consecutive
 * 1 KB blocks with one 16-byte load per lane per block, workgroups of
 * waves_per_workgroup (1..16) waves. sink (device, sink_words >= the number
 * of workgroups, ceil(bytes / 1024 / units_per_wave / waves_per_workgroup))
 * receives a word only in a case that never happens for real data, so the
 * kernel reads `bytes` and writes nothing. The shape matches the expert
 * kernels' weight streams (one 1 KB unit per wave load instruction).
 */
moe_status moe_probe_stream_read(const void *buf, size_t bytes, int units_per_wave,
                                 int waves_per_workgroup, unsigned *sink, size_t sink_words,
                                 hipEvent_t start, hipEvent_t end, hipStream_t stream);

/*
 * `workgroups` workgroups of 4 waves; each wave runs `iters` rounds of four
 * independent v_mfma_f32_16x16x32_f16 products on register operands
 * (16 x 16 x 32 x 2 flops each), then stores one float to out[wave index]
 * (device, at least 4 * workgroups floats).
 * Flops per launch: workgroups * 4 * iters * 4 * 16384.
 */
moe_status moe_probe_mfma_f16(float *out, int workgroups, int iters, hipEvent_t start,
                              hipEvent_t end, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBE_H */
