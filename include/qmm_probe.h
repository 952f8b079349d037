/*
 * qmm_probe.h -- measurement probes for the benchmark (libqmm_probe.so), not part of the product
 * path: they give the practically attainable HBM read rate and int8 matrix-core rate on the GPU
 * the benchmark runs on, so that measured kernels can be reported as a fraction of both the
 * datasheet peaks and these ceilings.  Same conventions as qmm.h: device pointers owned by the
 * caller, asynchronous on `stream`, a status (0 = OK, -1 argument error, -5 launch failure).
 */
#ifndef QMM_PROBE_H
#define QMM_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Loads-only streaming read of `bytes` bytes at `buf` (16-byte aligned, bytes a positive multiple
 * of 16): `wgs` workgroups of `threads` threads (64..1024, a multiple of 64) walk the buffer in a
 * grid stride of 16-byte streaming loads and fold what they read into one word per workgroup,
 * written to sink[workgroup] only when it equals a value no real data produces (so the loads
 * cannot be removed).  sink: at least `wgs` uint32 of device memory. */
int qmm_probe_read(const void *buf, uint64_t bytes, uint32_t *sink, int32_t wgs, int32_t threads, void *stream);

/* int8 matrix-core throughput: `wgs` workgroups of 256 threads, every wave runs `iters` rounds of
 * four independent v_mfma_i32_32x32x32_i8 (2 * 32 * 32 * 32 * 4 operations per round and wave)
 * on register operands; sink[0] is written only for an impossible result.  sink: one int32. */
int qmm_probe_mfma_i8(int32_t iters, int32_t wgs, int32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* QMM_PROBE_H */
