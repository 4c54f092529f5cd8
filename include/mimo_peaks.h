/*
 * mimo_peaks.h — on-box peak measurements for the roofline (libmimo_peaks.so).
 *
 * Measurement only: the attention library (mimo_attn.h) does not use these.
 * The benchmark times them with HIP events and reports every attention kernel
 * against both the vendor peaks and what these loops reach on the same card.
 * All pointers are device pointers owned by the caller; `stream` is a
 * hipStream_t (NULL = default stream); each call enqueues one kernel and
 * returns a hipError_t value (0 = enqueued).
 */
#ifndef MIMO_PEAKS_H
#define MIMO_PEAKS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Waves the MFMA loop launches (two per SIMD of every CU). */
int mimo_peak_mfma_waves(void);

/*
 * bf16 MFMA throughput loop: every wave loads 16 operand fragments from
 * `operands` (n_elems >= 64 bf16 values; the caller picks their distribution,
 * e.g. N(0,1) like attention's operands) and issues iters * 64
 * v_mfma_f32_32x32x16_bf16 (32768 FLOP each) in 8 independent chains, the
 * operands changing from one MFMA to the next.  Total FLOP =
 * mimo_peak_mfma_waves() * iters * 64 * 32768.  sink: mimo_peak_mfma_waves()
 * floats, overwritten.
 */
int mimo_peak_mfma_bf16(const uint16_t *operands, int64_t n_elems, int32_t iters, float *sink, void *stream);

/* HBM copy of `bytes` (a multiple of 16) from src to dst: 2 * bytes of traffic. */
int mimo_peak_copy(const void *src, void *dst, int64_t bytes, void *stream);

/* HBM read of `bytes` (a multiple of 16); out: one uint32, practically never written. */
int mimo_peak_read(const void *src, int64_t bytes, uint32_t *out, void *stream);

/* HBM write of `bytes` (a multiple of 16): dst filled with the 32-bit `value`. */
int mimo_peak_write(void *dst, int64_t bytes, uint32_t value, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MIMO_PEAKS_H */
