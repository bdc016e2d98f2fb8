/*
 * zl_calib.h — a measurement aid exported by libzl.so beside the attention
 * calls of zl.h. It is not part of the attention path.
 *
 * The matrix cores of a GPU whose clock is limited by power do not reach
 * their nominal rate on every operand: the clock the chip settles at under a
 * dense stream of matrix instructions depends on how much the operand bits
 * switch. zl_calib_mfma times such a stream on the calling GPU so that a
 * measured kernel rate can be set beside the rate this GPU attains on
 * operands of the same kind, as well as beside the nominal peak.
 *
 * Same conventions as zl.h: ZL_OK (0) or a negative ZL_ERR_* code, details
 * in zl_last_error().
 */
#ifndef ZL_CALIB_H_
#define ZL_CALIB_H_

#ifdef __cplusplus
extern "C" {
#endif

/* Operand kinds for zl_calib_mfma. */
enum zl_calib_operands {
  ZL_CALIB_RANDOM = 0,   /* bf16 values with random signs, exponents over a
                            range of 2^7 and random mantissas (a fixed
                            linear congruential sequence) */
  ZL_CALIB_CONSTANT = 1  /* every element 1.0 in bf16 */
};

/* Time `iters` rounds of 8 v_mfma_f32_32x32x16_bf16 per wave on one
 * workgroup of 8 waves per compute unit (two per SIMD), the operands held in
 * registers and cycled over four accumulators; no memory traffic inside the
 * timed loop.
 *   operands: ZL_CALIB_RANDOM or ZL_CALIB_CONSTANT.
 *   iters:    1 .. 2^24 rounds; ~400000 keep the loop near 0.1 s.
 *   tflops:   host pointer; receives 32768 * 8 * iters * waves flops over
 *             the time between two HIP events around the timed launch.
 *   stream:   hipStream_t (NULL = default stream). The call synchronizes on
 *             its events before it returns.
 * The call allocates and frees its own device buffers (1 MiB of operands and
 * one float per thread), runs one untimed launch of iters / 10 rounds first,
 * and then the timed one.
 * Errors: ZL_ERR_NULL (tflops NULL), ZL_ERR_ARG (operands or iters out of
 * range), ZL_ERR_HIP. */
int zl_calib_mfma(int operands, int iters, double* tflops, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ZL_CALIB_H_ */
