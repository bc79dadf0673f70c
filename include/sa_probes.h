/*
 * sa_probes.h -- C ABI of libsa_probes.so: two microbenchmark kernels that re-measure, on the part
 * itself, the peaks the attention kernels' rooflines are quoted against (the bf16 MFMA rate and
 * the HBM read rate).  They are diagnostics for measurement, not part of the attention path, and
 * live in a library of their own.
 *
 * Conventions: device pointers from the caller; `stream` is a hipStream_t (NULL = default stream);
 * each call enqueues one kernel asynchronously and returns 0, 1 for a bad argument (nothing
 * enqueued) or 2 when the launch failed.  The caller times the kernels with events on `stream`.
 */
#ifndef SA_PROBES_H
#define SA_PROBES_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Work of one sa_probe_mfma_bf16 call, in flops: workgroups * 4 waves * iters * 4 chains *
 * 32768 (one v_mfma_f32_32x32x16_bf16 is 32 * 32 * 16 multiply-adds). */
double sa_probe_mfma_bf16_flops(int workgroups, int iters);

/* Matrix-core rate: `workgroups` workgroups of four waves, each wave running `iters` rounds of four
 * independent accumulation chains of v_mfma_f32_32x32x16_bf16 on register operands (no memory
 * traffic in the loop).  random_operands != 0: two sets of random bf16 operands alternate from
 * issue to issue (the switching power of real data, which lowers the sustained clock); 0: small
 * constant operands (the rate at the clock an idle-data load allows).  out: float
 * [workgroups * 256], written once at the end (keeps the chains live).  workgroups >= 1,
 * iters >= 1. */
int sa_probe_mfma_bf16(float* out, int workgroups, int iters, int random_operands, void* stream);

/* HBM read rate: reads every byte of buf[0, bytes) once, in 16 KiB contiguous chunks; workgroups of
 * eight waves, each wave keeping four chunks in flight.  bytes must be a positive multiple of
 * 16384 and buf 16-byte aligned; out: uint32 [workgroups * 512], written once at the end.  To
 * measure HBM rather than the 256 MB last-level cache, rotate over buffers whose total exceeds it. */
int sa_probe_read(const void* buf, size_t bytes, unsigned* out, int workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SA_PROBES_H */
