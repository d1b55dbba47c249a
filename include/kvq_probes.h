/*
 * kvq_probes.h -- measurement probes for MI355X (gfx950), built as
 * libkvq_probes.so beside the attention library.  They are not part of the
 * attention path: they measure the ceilings that the attention kernels are
 * reported against besides the published peaks (8 TB/s HBM3E; 2.5 PFLOP/s dense
 * bf16 MFMA).
 *
 * Each call launches one kernel on `stream` and returns at once: 0 on success,
 * 1 for an invalid argument (nothing launched), 2 for a HIP launch error.  The
 * caller owns every buffer and times the call with events on `stream`.
 */
#ifndef KVQ_PROBES_H
#define KVQ_PROBES_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read `bytes` of device memory at `src` once, with 128-bit loads (non-temporal
 * when `nontemporal` is 1), grid-stride over `blocks` workgroups of 256 threads.
 *   src   16-byte aligned; bytes a multiple of 16
 *   sink  uint32 [blocks * 256], written only under a condition the data never
 *         meets (it stops the reads from being optimized away)
 */
int kvq_probe_stream_read(const void *src, size_t bytes, int32_t blocks, int32_t nontemporal,
                          uint32_t *sink, hipStream_t stream);

/*
 * Workgroup b of `blocks` (256 threads) reads bytes [b * segment_bytes,
 * (b + 1) * segment_bytes) of `src` once, front to back, with 128-bit loads
 * (non-temporal when `nontemporal` is 1): the access shape of a split-KV read,
 * where each workgroup streams its own run of the cache.
 *   src   16-byte aligned, at least blocks * segment_bytes bytes; segment_bytes a
 *         multiple of 16
 *   sink  uint32 [blocks * 256], written only under a condition the data never meets
 */
int kvq_probe_segment_read(const void *src, size_t segment_bytes, int32_t blocks, int32_t nontemporal,
                           uint32_t *sink, hipStream_t stream);

/*
 * Dense bf16 matrix-core loop: `blocks` workgroups of 4 waves, each wave
 * issuing `iters` rounds of independent MFMAs with fp32 accumulation:
 *   shape 0: 8 x v_mfma_f32_16x16x32_bf16 per round,
 *   shape 1: 4 x v_mfma_f32_32x32x16_bf16 per round.
 *   sink  float [blocks * 256], written under a condition never met
 */
int kvq_probe_mfma_bf16(int32_t shape, int32_t iters, int32_t blocks, float *sink, hipStream_t stream);

/* (host) FLOPs one round of kvq_probe_mfma_bf16 performs over all its blocks. */
double kvq_probe_mfma_flops_per_iter(int32_t shape, int32_t blocks);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_PROBES_H */
