/*
 * gla_internal.h -- launch-plan overrides of libgla.so, for tests and tuning
 * sweeps only.  Not part of the operator's interface (gla.h): a program that
 * only computes the operator never needs it.
 *
 * Every call of the operator picks its kernels and launch sizes from the
 * shapes alone, with defaults chosen by measurement.  The tests use these
 * knobs to reach every kernel variant (the LDS-staged pass-1 kernel, the
 * one-head output kernel, RoPE rows from the global table, other chunk
 * counts) on shapes where the default plan would not.  The results of every
 * variant are the operator's results; only speed differs.
 *
 * The knobs are process-wide (all threads and devices).  Each operator call
 * reads all of them once when it starts, so a change affects calls that start
 * after gla_plan_override returns.  The library reads no environment
 * variable.
 */
#ifndef GLA_INTERNAL_H
#define GLA_INTERNAL_H

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GLA_PLAN_PASS1_GENERIC = 0,            /* > 0: LDS-staged pass-1 kernel instead of the register-
                                            accumulating one (bf16 and fp8 at d = 128) */
  GLA_PLAN_PASS1_WORKGROUPS = 1,         /* > 0: workgroups aimed for by pass 1 (chunks per segment
                                            follow from it, at most 64) */
  GLA_PLAN_PASS2_GENERIC = 2,            /* > 0: one head per workgroup in the output kernel and in the
                                            token-causal walk */
  GLA_PLAN_PASS2_WORKGROUPS = 3,         /* > 0: workgroups aimed for by the output kernel */
  GLA_PLAN_ROPE_GLOBAL = 4,              /* > 0: RoPE rows read from the global table instead of LDS */
  GLA_PLAN_TOKEN_CAUSAL_WORKGROUPS = 5,  /* > 0: (head, segment) units aimed for by the token-causal
                                            walk (segment length follows from it) */
  GLA_PLAN_PASS2_HEADS = 6,              /* > 0: at most this many heads per workgroup in the output
                                            kernel (1, 2 or 4; default 4 at d = 128) and in the
                                            token-causal walk (1 or 2; default 2) */
  GLA_PLAN_NUM_KNOBS = 7
} gla_plan_knob;

/*
 * Set knob `knob` to `value`; 0 restores the default plan for that knob.
 * Returns GLA_OK, or GLA_ERR_SHAPE (nothing changed) for an unknown knob or a
 * value outside [0, 2^24].
 */
int gla_plan_override(int knob, int value);

/*
 * The launch plan that a call with these shapes would use under the current
 * knobs, for tests: writes the first n of {tokens per segment, segments per
 * batch item, pass-1 chunks per segment, pass-1 tokens per chunk, pass-2
 * chunks per segment, pass-2 tokens per chunk, register-accumulating pass 1
 * (0 or 1), heads per pass-2 workgroup (0 for one head, 2 or 4), pass-1 RoPE
 * rows in LDS (0 or 1), pass-2 RoPE rows in LDS (0 or 1)} to out.  form: 0
 * bidirectional, 1 block-causal (block_frames frames per block), 2
 * token-causal.  Returns GLA_OK, or the status the operator call would return
 * for these shapes, dtype and head dim (GLA_ERR_SHAPE also for an empty grid
 * or an unknown form; GLA_ERR_NULL for out == NULL with n > 0).  Touches no
 * device.
 */
int gla_plan_describe(int form, int batch, int T, int H, int W, int heads, int d, int dtype, int block_frames,
                      int* out, int n);

#ifdef __cplusplus
}
#endif

#endif /* GLA_INTERNAL_H */
