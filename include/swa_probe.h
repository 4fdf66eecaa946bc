/* swa_probe.h: measurement probes for the benchmark.
 *
 * Not part of the attention path.  They give the practical ceilings that the
 * benchmark reports beside the published MI355X peaks: what a plain streaming
 * read reaches on the HBM, and what a loop of nothing but bf16 MFMAs reaches on
 * the matrix cores, and what a plain copy (as many bytes written as read)
 * reaches.  Each result of the benchmark is then also stated as a fraction of
 * the probe that bounds it.
 *
 * All pointers are device pointers owned by the caller.  Argument errors are
 * returned before anything is enqueued; a failed launch returns SWA_E_HIP.
 */
#ifndef SWA_PROBE_H
#define SWA_PROBE_H

#include "swa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes of `buf` once with 16-byte loads (a grid-stride loop over
 * `grid` workgroups of 256 threads) and write one float per thread (a sum of
 * what it read, so the loads cannot be dropped) to out[grid * 256].
 *   buf    device, 16-aligned, bytes > 0 and a multiple of 16.
 *   grid   1 .. 65,535 workgroups.
 * Errors: SWA_E_ARG. */
swa_status_t swa_probe_read(const void *buf, size_t bytes, float *out, int32_t grid, hipStream_t stream);

/* Copy `bytes` bytes from src to dst with 16-byte loads and stores (a
 * grid-stride loop over `grid` workgroups of 256 threads): `bytes` read and
 * `bytes` written, the traffic mix of a kernel that streams one tensor in and
 * another out.
 *   src, dst  device, 16-aligned, not overlapping; bytes > 0 and a multiple of 16.
 *   grid      1 .. 65,535 workgroups.
 * Errors: SWA_E_ARG. */
swa_status_t swa_probe_copy(const void *src, void *dst, size_t bytes, int32_t grid, hipStream_t stream);

/* `grid` workgroups of 256 threads each run `iters` rounds of eight independent
 * v_mfma_f32_16x16x32_bf16 per wavefront (16,384 FLOPs each, so a launch does
 * grid * 4 * iters * 8 * 16,384 FLOPs) and write one float per thread to
 * out[grid * 256].
 *   grid   1 .. 65,535; iters >= 1.
 * Errors: SWA_E_ARG. */
swa_status_t swa_probe_mfma(float *out, int32_t grid, int32_t iters, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SWA_PROBE_H */
