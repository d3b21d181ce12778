/* Measurement probes for gfx950 (libsegpaged_probe.so): the rates the chip
 * sustains on the two resources the attention kernels are bound by, so that a
 * kernel's achieved rate can be reported against what is reachable as well as
 * against the published peak. Not part of the attention path; nothing in
 * libsegpaged.so uses them.
 *
 * Both entry points only enqueue a kernel on `stream` (a hipStream_t, NULL =
 * the null stream); the caller times them (e.g. with events) and owns every
 * buffer. Status codes are those of segpaged.h: SEGPAGED_OK, SEGPAGED_EINVAL
 * for a bad argument (checked before any launch), SEGPAGED_EHIP if the launch
 * fails. */
#ifndef SEGPAGED_PROBE_H
#define SEGPAGED_PROBE_H

#include <stdint.h>

#include "segpaged.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Dense bf16 matrix-core rate: `workgroups` workgroups of 8 waves (two per
 * SIMD); each wave issues iters x 8 v_mfma_f32_32x32x16_bf16 on four
 * independent accumulators, its operands cycling through values loaded from
 * `seed`, so they change every instruction. Work per launch:
 * workgroups * 8 * iters * 8 * 32768 flops.
 *   seed  device bf16 [32768] (64 KiB), e.g. N(0,1) values
 *   out   device fp32 [workgroups * 512] (written: accumulator sums, so the
 *         work cannot be elided)
 * EINVAL if a pointer is NULL or not 16-byte aligned, iters < 1 or
 * workgroups < 1. */
SEGPAGED_API int segpaged_probe_mfma_bf16(const void* seed, int32_t iters, int32_t workgroups,
                                          float* out, void* stream);

/* Streaming read rate: `workgroups` workgroups of 256 threads read `bytes`
 * bytes of `src` once with 16-byte non-temporal loads, `depth` (4, 8 or 16) in
 * flight per thread, and sum them as fp32.
 *   src   device, 16-byte aligned; bytes > 0 and a multiple of 16; read as fp32
 *   out   device fp32 [workgroups] (written: each workgroup's partial sum; their
 *         total is the fp32 sum of src, up to rounding order)
 * EINVAL if a pointer is NULL or misaligned, bytes is not a positive multiple of
 * 16, workgroups < 1 or depth is not 4, 8 or 16. */
SEGPAGED_API int segpaged_probe_hbm_read(const void* src, int64_t bytes, int32_t workgroups,
                                         int32_t depth, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SEGPAGED_PROBE_H */
