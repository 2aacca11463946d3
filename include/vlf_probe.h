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

/*
 * Queue one launch of the overlap probe: `blocks` workgroups of eight waves; waves 0-3 (one per
 * SIMD) run role `lo_role` and waves 4-7 (sharing those SIMDs) role `hi_role`, `iters` times:
 *   0 nothing;
 *   1 eight v_mfma_f32_32x32x16_bf16 on four independent accumulators (256 matrix clocks);
 *   2 32 v_exp_f32;  3 32 v_fma_f32 (eight independent chains each);
 *   4 the softmax of 32 scores per lane as the forward runs it: 32 fma, 32 exp, 32 add into a
 *     row sum, 16 conversions to bf16 pairs;
 *   5 roles 1 and 4 in one wave, with 16 products (one 32-row, 64-key attention step);
 *   6 role 5 with the 16 products' A operands read from LDS (16 KiB per step), each read as
 *     the compiler places it (just before its product);
 *   7 role 6 with all 16 reads issued one step ahead of their products;
 *   8 role 6 with each read issued four products ahead of its own;
 *   9 role 6's 16 LDS reads alone (16 KiB per wave and iteration);
 *  10 a 64-row step: role 8's 16 reads, each feeding two products (32 in all), and the softmax
 *     of 64 scores per lane.
 * Workgroup b records into record_dev[4b .. 4b + 3] (uint64): the shader-clock and 100 MHz
 * ticks from the common start to the end of its last wave, then wave 0's and wave 4's own loop
 * in shader clocks (a SIMD may run the older wave first, so one wave's loop alone does not show
 * the pair's cost); sink_dev[512 b + thread] receives a checksum. With blocks = the CU count
 * each CU runs one workgroup, so a pair of roles shares every SIMD. Asynchronous.
 *   sink_dev    device, 512 * blocks floats.   record_dev  device, 4 * blocks uint64.
 * Errors: -1 (a role outside 0 .. 10, iters or blocks out of range, null or misaligned
 * buffers), -3 (launch).
 */
int vlf_probe_overlap(int32_t lo_role, int32_t hi_role, int32_t iters, int32_t blocks,
                      float *sink_dev, uint64_t *record_dev, void *stream);

/*
 * Queue one launch of a phase-schedule probe of the forward's 32-row, 64-key wave step, one
 * workgroup per CU (`blocks` = the CU count), or of the matrix unit's toll on vector work.
 * Kinds 0-5 run `steps` steps per wave with the forward's dataflow (scores from a K image in LDS
 * and a query operand in registers, exp2 softmax with the row sum and bf16 pair conversions,
 * output product from a V image in LDS), groups of four waves (one per SIMD) rotating roles at a
 * barrier per phase, so that every SIMD holds one product wave and the rest softmax waves:
 *   0 three groups (12 waves): product, softmax of half the step's scores, the other half;
 *   1 kind 0 with the softmax phases left empty;   2 kind 0 with the products left empty;
 *   3 four groups (16 waves), the softmax in thirds;   4, 5 kind 3 emptied as 1, 2.
 *   record_dev[16 b] (uint64) gets workgroup b's shader clocks for the whole loop: per wave
 *   step that is record / (groups * steps) on each SIMD.
 * Kinds 6-9 run 12 waves per workgroup for `steps` iterations: waves 0-3 (one per SIMD) four
 * v_mfma_f32_32x32x16_bf16 per iteration (kinds 7, 9) or nothing (6, 8); waves 4-11 (two per
 * SIMD) 16 v_fma_f32 (6, 7) or v_exp_f32 (8, 9) on eight chains; record_dev[16 b + w] gets
 * wave w's own loop in shader clocks.
 * sink_dev receives checksums. Asynchronous; allocates nothing.
 *   kind        0 .. 9.   steps  a multiple of 4 in 4 .. 2^22.   blocks  1 .. 2^20.
 *   sink_dev    device, 1024 * blocks floats, 4-byte aligned.
 *   record_dev  device, 16 * blocks uint64, 8-byte aligned.
 * Errors: -1 (kind, steps or blocks out of range, null or misaligned buffers), -3 (launch).
 */
int vlf_probe_schedule(int32_t kind, int32_t steps, int32_t blocks, float *sink_dev,
                       uint64_t *record_dev, void *stream);

/* Message for the last non-OK status on the calling thread ("" if none). */
const char *vlf_probe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* VLF_PROBE_H */
