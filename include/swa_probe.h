/*
 * swa_probe.h -- measurement kernels of libswa.so (not part of the attention
 * method): the two reference rates against which the attention kernels'
 * achieved figures are also stated, besides the MI355X datasheet peaks.
 *
 *  - swa_probe_mfma_bf16: a dense stream of v_mfma_f32_32x32x16_bf16 on
 *    register operands (no memory traffic in the loop), four independent
 *    accumulator chains per wave.  Work: swa_probe_mfma_bf16_flops(...) FLOP
 *    (32x32x16 multiply-adds, a multiply-add counted as 2 FLOP).
 *  - swa_probe_hbm_read: a streaming read of `bytes` bytes with 16-byte
 *    non-temporal loads, each workgroup reading one contiguous range as
 *    `streams` interleaved sub-ranges, 8 loads in flight per lane.  Work:
 *    `bytes` bytes read (nothing written but one word per workgroup).
 *
 * Both follow the conventions of swa.h: device pointers owned by the caller,
 * asynchronous on `stream`, arguments validated before anything is enqueued
 * (SWA_EINVAL, SWA_EALIGN; SWA_EHIP if the launch is rejected).
 */
#ifndef SWA_PROBE_H
#define SWA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* out: workgroups * 256 floats (a per-lane checksum that keeps the stream
 * live; its value is not meaningful).  workgroups >= 1, iters >= 1. */
int swa_probe_mfma_bf16(float *out, int workgroups, int iters, hipStream_t stream);
/* FLOP of one such launch: workgroups * 4 waves * iters * 4 MFMAs * 32768. */
double swa_probe_mfma_bf16_flops(int workgroups, int iters);

/* buf: bytes readable device bytes, 16-byte aligned; bytes a multiple of
 * 32768 * workgroups (each workgroup's range is whole rounds of 8 loads of
 * 16 bytes by 256 lanes); streams in {1, 2, 4, 8}; sink: workgroups words,
 * 4-byte aligned (written only if a checksum hits one fixed value). */
int swa_probe_hbm_read(const void *buf, size_t bytes, int workgroups, int streams, uint32_t *sink,
                       hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SWA_PROBE_H */
