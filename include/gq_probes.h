/*
 * gq_probes.h -- measurement controls for the benchmark (libgq_probes.so).
 * Not part of the matmul path.  They give the same-run reference points a
 * kernel's time is read against: the device duration of an empty launch
 * (the per-launch floor) and a plain coalesced streaming read of a given
 * byte count (the achievable HBM rate at that size).  The pages recommend
 * pairing every measurement with controls taken on the same instance
 * ("Receipts-driven engineering", "What the discipline caught": baselines
 * differ between hosts, so ratios are taken on one machine).
 *
 * Pointers are device memory owned by the caller; work is enqueued on
 * `stream`.  Return 0, hipErrorInvalidValue for bad arguments, or the launch
 * error.
 */
#ifndef GQ_PROBES_H
#define GQ_PROBES_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One workgroup that does nothing. */
int gq_probe_empty(hipStream_t stream);

/* Reads `bytes` bytes (a multiple of 16, buffer 16-byte aligned) once with
 * 16-byte coalesced loads, `loads_per_thread` (1, 2, 4, 8 or 16) per thread
 * in workgroups of 256 threads, all issued before use; writes nothing
 * unless the xor of everything read equals 0x9E3779B9, in which case one
 * word goes to sink[0] (sink: >= 4 bytes).  Few loads per thread means many
 * workgroups; the benchmark takes the fastest shape at each size. */
int gq_probe_stream_read(const void* buf, int64_t bytes, int32_t loads_per_thread,
                         uint32_t* sink, hipStream_t stream);

/* Copies `bytes` bytes (a multiple of 16, both buffers 16-byte aligned, not
 * overlapping) with 16-byte coalesced loads and stores: a kernel of known
 * read and write size, the reference that scales HBM byte counters. */
int gq_probe_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream);

/* Matrix-instruction issue rate: `blocks` workgroups of 256 threads (4
 * waves); every wave runs `iters` (a multiple of 4) iterations of gq_probe_mfma_per_wave_iter()
 * independent matrix instructions on random finite operands (4 operand
 * sets in turn), then writes sink[0] only if the sum of its accumulators
 * has one particular bit pattern.  kind:
 *   0  v_mfma_f32_32x32x16_bf16
 *   1  v_mfma_scale_f32_32x32x64_f8f6f4, A e4m3, B e2m1 (scales 1.0)
 *   2  the same, A e2m1, B e2m1
 *   3  the same, A e4m3, B e4m3
 * Flops of one instruction: gq_probe_mfma_flops(kind) (-1 for a bad kind).
 * The block-scaled instruction and its formats are the gfx950 (CDNA4)
 * matrix-core operations for MX formats (OCP MX v1.0 e2m1 / e4m3 with e8m0
 * scales), the formats the MXFP4 weights are stored in. */
int gq_probe_mfma(int32_t kind, int64_t iters, int32_t blocks, uint32_t* sink,
                  hipStream_t stream);
int64_t gq_probe_mfma_flops(int32_t kind);
int32_t gq_probe_mfma_per_wave_iter(void);

#ifdef __cplusplus
}
#endif
#endif /* GQ_PROBES_H */
