/*
 * libaxonscan — C ABI of the selective-scan hot path of the Axon-SSM layer on AMD Instinct
 * MI355X (gfx950).
 *
 * What is computed. The pages cited below are:
 *   [AXON] "Axon-SSM: Selective State Space Model for Apple Silicon" (bit-axon docs).
 *   [WIKI] "Selective State Space Models (Mamba)" (wiki note, "Selective scan (toy)" and
 *          "1M context inference" patterns).
 *
 * For every batch row b and channel e (d_inner = E channels) the layer carries a state
 * h[b,e,0..N-1] and runs, for t = 0..L-1:
 *
 *   u_t   = conv_b[e] + sum_{k=0}^{K-1} conv_w[e,k] * xx[t-(K-1)+k]
 *             [AXON "Key contributions": causal depthwise conv1d, kernel size 4, before the scan;
 *              xx[s] = x[b,s,e] for s >= 0, taken from conv_cache for s < 0]
 *   dt_t  = min(max(softplus(dt_raw[b,t,e] + dt_bias[e]), dt_min), dt_max)
 *             [AXON "Selective mechanism": softplus of the raw step plus a bias, clipped to
 *              [eps, dt_max] with eps = 1e-4, dt_max = 100]
 *   A_n   = -exp(A_log[e,n])                       [AXON "Diagonal state matrix"]
 *   h_n  <- exp(dt_t * A_n) * h_n + dt_t * B[b,t,n] * u_t
 *             [AXON "ZOH discretization": first-order form, Abar = exp(dt A), Bbar = dt B]
 *   y_t   = sum_n C[b,t,n] * h_n + D[e] * u_t      [AXON "Continuous-time SSM", readout]
 *   out[b,t,e] = y_t * z_t * sigmoid(z_t)          [AXON "Gating": y times SiLU(z)]
 *
 * There is no activation between the convolution and the scan (the Axon-SSM page applies SiLU
 * only on the z branch). B, C and dt_raw arrive already projected; the projections W_in,
 * f_proj and W_out are the caller's.
 *
 * Layouts (all row-major, contiguous, innermost index last):
 *   x, z, dt_raw, y : (batch, seqlen, d_inner), activation dtype
 *   B, C            : (batch, seqlen, d_state), activation dtype
 *   A_log           : (d_inner, d_state) fp32
 *   D, dt_bias      : (d_inner) fp32
 *   conv_w          : (d_inner, d_conv) fp32; tap d_conv-1 multiplies the current token
 *   conv_b          : (d_inner) fp32
 *   conv_cache      : (batch, d_conv-1, d_inner) fp32; the last d_conv-1 x-branch inputs seen
 *                     (before the convolution), oldest first [AXON "Autoregressive decoding"]
 *   ssm_state       : (batch, d_inner, d_state) fp32 [AXON "Autoregressive decoding"]
 *
 * Supported shapes: d_state == 16, d_conv == 4 (the layer configuration table of [AXON]);
 * batch >= 1, d_inner >= 1, seqlen >= 0 (else AXON_ERR_INVALID_ARGUMENT);
 * batch <= 65535 and d_inner <= 2^23 (else AXON_ERR_UNSUPPORTED);
 * batch*seqlen*d_inner*d_state <= 2^40 (else AXON_ERR_INVALID_ARGUMENT).
 * Activation dtype: fp32 or bf16 (bf16 outputs are rounded to nearest even from fp32).
 * State, cache and parameters are always fp32; the state recurrence runs in fp32.
 *
 * Ownership and memory: every tensor pointer is device memory owned by the caller, 16-byte
 * aligned. The library allocates nothing and keeps no mutable global state; scratch memory
 * is a caller-provided workspace. Calls are asynchronous on the given stream (a hipStream_t
 * passed as void*; NULL = the default stream); nothing is synchronised on the host.
 *
 * Errors: every argument is checked on the host before anything is launched. On any error
 * code other than AXON_ERR_HIP nothing has been enqueued and no memory was written.
 * AXON_ERR_HIP means a launch failed (hipGetLastError); outputs are then unspecified.
 * The functions are thread-safe.
 */
#ifndef AXONSCAN_H_
#define AXONSCAN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  AXON_OK = 0,
  AXON_ERR_INVALID_ARGUMENT = 1,  /* null/misaligned pointer, bad size, forbidden aliasing */
  AXON_ERR_UNSUPPORTED = 2,       /* d_state != 16, d_conv != 4, unknown dtype, size limits */
  AXON_ERR_WORKSPACE_TOO_SMALL = 3,
  AXON_ERR_HIP = 4                /* a HIP launch or runtime call failed */
} axon_status;

typedef enum { AXON_F32 = 0, AXON_BF16 = 1 } axon_dtype;
/* Enumerated fields of the structs below are int32_t holding these values, so that any integer a
 * caller stores is a defined value that the checks can reject. */

typedef struct {
  int64_t batch;      /* B */
  int64_t seqlen;     /* L (ignored by the decode step) */
  int64_t d_inner;    /* E, channels */
  int64_t d_state;    /* N, must be 16 */
  int64_t d_conv;     /* K, must be 4 */
  int32_t act_dtype;  /* an axon_dtype value */
} axon_ssm_shape;

typedef struct {
  const float* A_log;    /* (E, N) */
  const float* D;        /* (E)    */
  const float* dt_bias;  /* (E)    */
  const float* conv_w;   /* (E, K) */
  const float* conv_b;   /* (E)    */
  float dt_min;          /* lower clip of dt; the Axon-SSM page uses 1e-4 */
  float dt_max;          /* upper clip of dt; the Axon-SSM page uses 100  */
  /* Variants; zero (the default of a zero-initialised struct) is the Axon-SSM layer.
   *   conv_activation: AXON_CONV_NONE, or AXON_CONV_SILU: u = SiLU(conv(x)) before the scan
   *     (the Mamba block of "Selective State Space Models (Mamba)", pattern "Mamba block"); the
   *     skip term D u uses the same u, and conv_cache still holds the raw inputs.
   *   discretization: AXON_DISC_FIRST_ORDER (Bbar = dt B, [AXON "ZOH discretization"]), or
   *     AXON_DISC_ZOH: the exact zero-order hold for the diagonal A that the same section
   *     states first, Bbar = expm1(dt A) / A * B.
   * Other values: AXON_ERR_UNSUPPORTED. */
  int32_t conv_activation;
  int32_t discretization;
} axon_ssm_params;

enum { AXON_CONV_NONE = 0, AXON_CONV_SILU = 1 };
enum { AXON_DISC_FIRST_ORDER = 0, AXON_DISC_ZOH = 1 };

/* Library version as 10000*major + 100*minor + patch. */
int axon_version(void);

/* Static description of a status code (any int; unknown codes give "unknown status"); never
 * NULL. */
const char* axon_status_string(int status);

/* Bytes of device workspace axon_ssm_prefill needs for this shape (0 is possible). A pure
 * function of the shape: no device is queried. Returns 0 for an invalid shape as well, so call
 * axon_ssm_prefill for the diagnosis. */
size_t axon_ssm_prefill_workspace_bytes(const axon_ssm_shape* shape);

/* Prefill: runs the layer over seqlen tokens for every (b, e), continuing from the given cache.
 *
 * conv_cache_in (B, K-1, E) and ssm_state_in (B, E, N) may be NULL, meaning zeros (a fresh
 * sequence, as with state = None in the streaming loop of [WIKI "1M context inference"]).
 * conv_cache_out and ssm_state_out receive the cache after the last token; they may be equal to
 * the corresponding inputs (in-place update) but must not partially overlap them. y must not
 * overlap any input. Prefill(L1) followed by prefill(L2) from its caches equals prefill(L1+L2)
 * up to rounding.
 * seqlen == 0 copies the caches in to out unchanged (zeros for NULL inputs) and writes no y.
 * The conv cache after the call holds exact copies (fp32, exact widening for bf16) of the last
 * K-1 x-branch inputs of the concatenation [cache_in, x].
 * workspace: device memory of at least axon_ssm_prefill_workspace_bytes(shape) bytes, 16-byte
 * aligned; may be NULL when that size is 0. Its contents need no initialisation. */
axon_status axon_ssm_prefill(const axon_ssm_shape* shape, const axon_ssm_params* params,
                             const void* x, const void* z, const void* dt_raw,
                             const void* B, const void* C,
                             const float* conv_cache_in, const float* ssm_state_in,
                             void* y, float* conv_cache_out, float* ssm_state_out,
                             void* workspace, size_t workspace_bytes, void* stream);

/* The same prefill without allocating and without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation). The time-chunked scan's workspace is a 64 MiB scratch array the library
 * holds on each GPU it runs on until the process ends; for shapes whose chunked plan would need
 * more, the plan takes fewer time chunks (same results to rounding, possibly slower), so every
 * shape axon_ssm_prefill accepts is accepted. Arguments, checks and results otherwise as
 * axon_ssm_prefill; the stream must belong to the current device. Calls on one GPU share its
 * scratch: calls that overlap in time on the same GPU race (serialise them, e.g. on one
 * stream). AXON_ERR_HIP if the scratch's device address cannot be obtained. */
axon_status axon_ssm_prefill_noalloc(const axon_ssm_shape* shape, const axon_ssm_params* params,
                                     const void* x, const void* z, const void* dt_raw,
                                     const void* B, const void* C, const float* conv_cache_in,
                                     const float* ssm_state_in, void* y, float* conv_cache_out,
                                     float* ssm_state_out, void* stream);

/* Decode step: one token per batch row, with the caches updated in place
 * [AXON "Autoregressive decoding": the cache pair carries the convolution padding and the
 * hidden state from one step to the next].
 * x, z, dt_raw, y: (B, E) activation dtype; B, C: (B, N) activation dtype;
 * conv_cache (B, K-1, E) and ssm_state (B, E, N) fp32, read and then overwritten.
 * shape->seqlen is ignored. y must not overlap any input or cache. Equivalent to
 * axon_ssm_prefill with seqlen = 1 and in-place caches. */
axon_status axon_ssm_decode_step(const axon_ssm_shape* shape, const axon_ssm_params* params,
                                 const void* x, const void* z, const void* dt_raw,
                                 const void* B, const void* C,
                                 float* conv_cache, float* ssm_state,
                                 void* y, void* stream);

/* ---- The layer around the path ---------------------------------------------------------------
 * The whole Axon-SSM layer on (B, L, D) activations [AXON "Gating", "Selective mechanism",
 * "Code mapping"]:
 *   (x_branch, z_branch) = split(W_in x)                  W_in (2E, D): rows 0..E-1 give x_branch
 *   u = conv(x_branch) (+ SiLU with AXON_CONV_SILU)        causal depthwise, K = 4, with the cache
 *   (B_t, C_t, dt_raw_t) = f_proj(u_t)                    W_f (2N + E, E): rows 0..N-1 give B_t,
 *                                                           N..2N-1 C_t, 2N..2N+E-1 dt_raw_t
 *   y = the selective scan of u with B, C, dt_raw, gated by SiLU(z_branch) (as axon_ssm_prefill)
 *   out = W_out y                                         W_out (D, E)
 * READING: f_proj is one full-rank linear map from the E conv outputs to [B, C, dt_raw] (the page
 * states a linear projection and no rank bottleneck), with no bias.
 * The projections are dense GEMMs (hipBLASLt, fp32 accumulation) in the activation dtype; every
 * intermediate (x_branch, z_branch, u, B, C, dt_raw, y) is stored in the activation dtype, the
 * conv cache and the state in fp32. seqlen = 1 with in-place caches is the layer's decode step.
 *
 * A context owns the GEMM library handle and its cached GEMM plans; create one per thread (a
 * context is not safe for concurrent use). The forward call allocates nothing: all scratch is
 * the caller's workspace. */
typedef struct axon_layer_ctx axon_layer_ctx;

typedef struct {
  int64_t batch;      /* B */
  int64_t seqlen;     /* L >= 1 */
  int64_t d_model;    /* D */
  int64_t d_inner;    /* E */
  int64_t d_state;    /* N, must be 16 */
  int64_t d_conv;     /* K, must be 4 */
  int32_t act_dtype;  /* an axon_dtype: x_in, out, the three projection weights and the
                        * intermediates */
} axon_layer_shape;

typedef struct {
  const void* W_in;   /* (2E, D) activation dtype, row-major (output feature major) */
  const void* W_f;    /* (2N + E, E) activation dtype */
  const void* W_out;  /* (D, E) activation dtype */
  axon_ssm_params ssm;  /* A_log, D, dt_bias, conv_w, conv_b (fp32), dt clips, variants */
} axon_layer_weights;

/* Create / destroy a context (AXON_ERR_HIP if the GEMM library cannot be initialised). */
axon_status axon_layer_create(axon_layer_ctx** ctx);
void axon_layer_destroy(axon_layer_ctx* ctx);

/* Bytes of device workspace axon_layer_forward needs (0 for an invalid shape). */
size_t axon_layer_workspace_bytes(const axon_layer_shape* shape);

/* Forward over seqlen tokens: x_in (B, L, D) -> out (B, L, D), continuing from the caches as
 * axon_ssm_prefill does (NULL inputs = zeros). Aliasing: out, the workspace, conv_cache_out and
 * ssm_state_out must not overlap x_in, a weight, a parameter array or one another; out and the
 * workspace also not the cache / state inputs; conv_cache_out may equal conv_cache_in and
 * ssm_state_out may equal ssm_state_in exactly (in place), never overlap them partly; the cache
 * output must not overlap the state input nor the state output the cache input. Any violation:
 * AXON_ERR_INVALID_ARGUMENT, nothing written. workspace: axon_layer_workspace_bytes(shape) bytes,
 * 16-byte aligned, contents need no initialisation. */
axon_status axon_layer_forward(axon_layer_ctx* ctx, const axon_layer_shape* shape,
                               const axon_layer_weights* weights, const void* x_in,
                               const float* conv_cache_in, const float* ssm_state_in, void* out,
                               float* conv_cache_out, float* ssm_state_out, void* workspace,
                               size_t workspace_bytes, void* stream);

/* The checks axon_layer_forward makes of its arguments before it launches anything (shape,
 * parameters, null and misaligned pointers, workspace size, aliasing), without a context and
 * without touching device memory: AXON_OK when the forward call with these arguments would run.
 * Pointers are only compared, never dereferenced. */
axon_status axon_layer_forward_check(const axon_layer_shape* shape,
                                     const axon_layer_weights* weights, const void* x_in,
                                     const float* conv_cache_in, const float* ssm_state_in,
                                     const void* out, const float* conv_cache_out,
                                     const float* ssm_state_out, const void* workspace,
                                     size_t workspace_bytes);

/* ---- Mamba-2 SSD core ------------------------------------------------------------------------
 * The state space duality (SSD) layer core of Mamba-2 ["Selective State Space Models (Mamba)",
 * pattern "Mamba-2 block": d_state 128, headdim 64; the SSD article, sections on the duality
 * with linear attention and on the chunked scan]. Heads of head_dim P channels share one scalar
 * decay; for every batch row b and head h, with a state h[p, n] (P x N), for t = 0..L-1:
 *
 *   dt_t      = min(max(softplus(dt_raw[b,t,h] + dt_bias[h]), dt_min), dt_max)
 *   A         = -exp(A_log[h])
 *   h[p, n]  <- exp(dt_t A) h[p, n] + dt_t x[b,t,h,p] B[b,t,n]
 *   y[b,t,h,p] = sum_n C[b,t,n] h[p, n] + D[h] x[b,t,h,p]
 *
 * READING: the first-order input term dt B and the step size of the Axon-SSM layer; B and C are
 * shared by all heads (one group); the convolution, gate and projections of the Mamba-2 block
 * are the caller's. The library computes it in chunks of 64 tokens: within a chunk as matrix
 * products on the matrix cores (the decay-masked C B^T times dt x, the chunk's state
 * contribution x^T diag(w) B and the readout of the incoming state C h^T), and across chunks as a
 * recurrence over the chunk states. fp32 arithmetic throughout (bf16 inputs are widened).
 *
 * Layouts (row-major, contiguous):
 *   x, y    : (batch, seqlen, n_heads, head_dim), activation dtype
 *   dt_raw  : (batch, seqlen, n_heads), activation dtype
 *   B, C    : (batch, seqlen, d_state), activation dtype
 *   A_log, D, dt_bias : (n_heads) fp32
 *   state   : (batch, n_heads, head_dim, d_state) fp32
 * Supported: head_dim == 64 and d_state == 128 (else AXON_ERR_UNSUPPORTED); batch and n_heads in
 * [1, 65535] (0 or negative: AXON_ERR_INVALID_ARGUMENT; larger: AXON_ERR_UNSUPPORTED);
 * seqlen >= 0; batch*seqlen*n_heads*head_dim <= 2^40. Pointers are device memory owned by the
 * caller, 16-byte aligned; errors as for axon_ssm_prefill. */
typedef struct {
  int64_t batch;     /* B */
  int64_t seqlen;    /* L */
  int64_t n_heads;   /* H */
  int64_t head_dim;  /* P, must be 64 */
  int64_t d_state;   /* N, must be 128 */
  int32_t act_dtype;  /* an axon_dtype value */
} axon_ssd_shape;

typedef struct {
  const float* A_log;    /* (H) */
  const float* D;        /* (H) */
  const float* dt_bias;  /* (H) */
  float dt_min;
  float dt_max;
} axon_ssd_params;

/* Bytes of device workspace axon_ssd_scan needs (0 for an invalid shape or seqlen == 0). */
size_t axon_ssd_scan_workspace_bytes(const axon_ssd_shape* shape);

/* Runs the SSD core over seqlen tokens. state_in (B, H, P, N) may be NULL (zeros); state_out
 * receives the state after the last token and may equal state_in (in place) but must not
 * partially overlap it. y must not overlap any input. seqlen == 0 copies state_in to state_out
 * (zeros for NULL) and writes no y. Running L1 tokens then L2 from the returned state equals
 * running L1 + L2 up to rounding. workspace: axon_ssd_scan_workspace_bytes(shape) bytes,
 * 16-byte aligned, no initialisation needed. */
axon_status axon_ssd_scan(const axon_ssd_shape* shape, const axon_ssd_params* params,
                          const void* x, const void* dt_raw, const void* B, const void* C,
                          const float* state_in, void* y, float* state_out, void* workspace,
                          size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AXONSCAN_H_ */
