/*
 * vlf_probe.h — C ABI of libvlf_probe.so: a measurement probe of the MI355X (gfx950) matrix
 * unit, kept apart from the attention library. It exists so that the forward's matrix rate can
 * be set against what the chip sustains for the same instruction at its running clock, beside
 * the 2516.6 TFLOP/s that the published figure (256 CUs x 2.4 GHz x 4096 FLOP per clock) gives.
 *
 * Status codes are those of vlf.h (0 = OK, -1 = bad argument, -3 = HIP error); a message is in
 * vlf_probe_last_error() for the calling thread.
 */
#ifndef VLF_PROBE_H
#define VLF_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Queue one launch of the matrix probe on `stream`: `blocks` workgroups of four waves, each wave
 * issuing 8 * iters v_mfma_f32_32x32x16_bf16 (32768 FLOP each) on four independent
 * accumulators, nothing else in its loop. Every workgroup's first wave records, into
 * record_dev[4 * b .. 4 * b + 3] (uint64), the shader-clock ticks (s_memtime) and the 100 MHz
 * constant-clock ticks (s_memrealtime) its loop took, a checksum of its accumulators (so the
 * products cannot be dropped) and the constant-clock tick at which its loop began. FLOP per
 * launch:
 * blocks * 4 * iters * 8 * 32768. With blocks a multiple of 256 x 2 every SIMD holds two such
 * waves. Asynchronous; allocates nothing.
 *   iters       1 .. 2^24.
 *   blocks      1 .. 2^20.
 *   record_dev  device, at least 32 * blocks bytes, 8-byte aligned.
 *   stream      hipStream_t (NULL = the null stream).
 * Errors: -1 (iters or blocks out of range, null or misaligned record_dev), -3 (launch).
 */
int vlf_probe_mfma(int32_t iters, int32_t blocks, uint64_t *record_dev, void *stream);

/* Message for the last non-OK status on the calling thread ("" if none). */
const char *vlf_probe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* VLF_PROBE_H */
