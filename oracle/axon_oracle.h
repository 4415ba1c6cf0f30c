/*
 * CPU oracle of the Axon-SSM selective-scan hot path.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark load this code. The product path (libaxonscan) never links, loads or calls it, and
 * the two share no source, header or helper.
 *
 * Every value is widened to double on entry and every result is returned in double, so that
 * rounding in the oracle stays far below the tolerances it is compared against. The arithmetic
 * is the plain definition, evaluated one token at a time in the order the pages give it.
 */
#ifndef AXON_ORACLE_H_
#define AXON_ORACLE_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Variants (section 8(f) of the build's scope: next rows beyond the Axon-SSM layer):
 *   conv_act: ORACLE_CONV_NONE (Axon-SSM: u = conv(x)) or ORACLE_CONV_SILU (Mamba block:
 *             u = SiLU(conv(x)); the skip term D u uses the same u)
 *   disc:     ORACLE_DISC_FIRST_ORDER (Axon-SSM: Bbar = dt B) or ORACLE_DISC_ZOH (exact
 *             zero-order hold for a diagonal A: Bbar = (exp(dt A) - 1) / A * B) */
#define ORACLE_CONV_NONE 0
#define ORACLE_CONV_SILU 1
#define ORACLE_DISC_FIRST_ORDER 0
#define ORACLE_DISC_ZOH 1

/* One channel (one (b, e) pair) over L tokens.
 *   x, z, dt_raw : token t at [t * act_stride]
 *   Bm, Cm       : B_t,n at [t * bc_stride + n]
 *   A_log        : N values; conv_w: K values, conv_w[K-1] multiplies the current token
 *   win_in       : the K-1 x-branch inputs that precede token 0, oldest first; NULL = zeros
 *   h_in         : N initial states; NULL = zeros
 *   y            : output token t at [t * y_stride]
 *   win_out      : K-1 values, the last K-1 x-branch inputs of [win_in, x], oldest first
 *   h_out        : N final states
 *   u_out, dt_out: optional (may be NULL) per-token conv output and step size, [t * y_stride]
 *   mag_out      : optional (may be NULL) per-token size of the terms the output sums,
 *                  |SiLU(z_t)| * (sum_n |C_t,n h_t,n| + |D u_t|), [t * y_stride]; it bounds how
 *                  much rounding of those terms can move y_t (a diagnostic, not part of y)
 * Returns 0, or -1 for an invalid argument. */
int oracle_ssm_channel(int64_t L, int64_t N, int64_t K,
                       const float* x, const float* z, const float* dt_raw, int64_t act_stride,
                       const float* Bm, const float* Cm, int64_t bc_stride,
                       const float* A_log, double D, double dt_bias, const float* conv_w,
                       double conv_b, double dt_min, double dt_max, int conv_act, int disc,
                       const double* win_in, const double* h_in,
                       double* y, int64_t y_stride, double* win_out, double* h_out,
                       double* u_out, double* dt_out, double* mag_out);

/* Whole prefill over (B, L, E) tensors laid out as in libaxonscan's header:
 *   x, z, dt_raw (B,L,E); Bm, Cm (B,L,N); A_log (E,N); D, dt_bias, conv_b (E); conv_w (E,K);
 *   conv_cache_in (B,K-1,E) or NULL; ssm_state_in (B,E,N) or NULL;
 *   y (B,L,E); conv_cache_out (B,K-1,E); ssm_state_out (B,E,N); mag (B,L,E) or NULL (see
 *   mag_out above).
 * threads >= 1 splits the independent channels over that many POSIX threads. */
int oracle_ssm_prefill(int64_t Bsz, int64_t L, int64_t E, int64_t N, int64_t K,
                       const float* x, const float* z, const float* dt_raw,
                       const float* Bm, const float* Cm,
                       const float* A_log, const float* D, const float* dt_bias,
                       const float* conv_w, const float* conv_b, double dt_min, double dt_max,
                       int conv_act, int disc,
                       const double* conv_cache_in, const double* ssm_state_in,
                       double* y, double* conv_cache_out, double* ssm_state_out, double* mag,
                       int threads);

/* One decode step: x, z, dt_raw (B,E); Bm, Cm (B,N); conv_cache (B,K-1,E) and ssm_state (B,E,N)
 * are read and overwritten; y (B,E). */
int oracle_ssm_decode_step(int64_t Bsz, int64_t E, int64_t N, int64_t K,
                           const float* x, const float* z, const float* dt_raw,
                           const float* Bm, const float* Cm,
                           const float* A_log, const float* D, const float* dt_bias,
                           const float* conv_w, const float* conv_b, double dt_min, double dt_max,
                           int conv_act, int disc,
                           double* conv_cache, double* ssm_state, double* y, int threads);

#ifdef __cplusplus
}
#endif

#endif /* AXON_ORACLE_H_ */

#ifdef __cplusplus
extern "C" {
#endif

/* Mamba-2 state space duality (SSD) core, per batch row b and head hd (a further layer the pages
 * describe: "Selective State Space Models (Mamba)", pattern "Mamba-2 block"; the SSD article):
 *   dt_t = clip(softplus(dt_raw_t + dt_bias), dt_min, dt_max),  A = -exp(A_log)  (one scalar)
 *   h_t[p, n] = exp(dt_t A) h_{t-1}[p, n] + dt_t x_t[p] B_t[n]
 *   y_t[p]    = sum_n C_t[n] h_t[p, n] + D x_t[p]
 * x, y (B, L, H, P); dt_raw (B, L, H); Bm, Cm (B, L, N) shared by all heads; A_log, D, dt_bias
 * (H); state_in / state_out (B, H, P, N) (state_in NULL = zeros); mag (B, L, H, P) or NULL:
 * sum_n |C_t[n] h_t[p, n]| + |D x_t[p]|, the size of the terms y sums (for tolerances of
 * ill-conditioned outputs). Returns 0 or -1. */
int oracle_ssd_scan(int64_t Bsz, int64_t L, int64_t H, int64_t P, int64_t N,
                    const float* x, const float* dt_raw, const float* Bm, const float* Cm,
                    const float* A_log, const float* D, const float* dt_bias, double dt_min,
                    double dt_max, const double* state_in, double* y, double* state_out,
                    double* mag, int threads);

#ifdef __cplusplus
}
#endif
