/*
 * CPU oracle of the Axon-SSM selective-scan hot path — TEST INFRASTRUCTURE ONLY (see
 * axon_oracle.h). Plain sequential loops in double precision.
 *
 * Sources (page title, then section):
 *   [AXON] "Axon-SSM: Selective State Space Model for Apple Silicon"
 *   [WIKI] "Selective State Space Models (Mamba)", pattern "Selective scan (toy)"
 * Readings taken where the pages leave a step open are marked READING below.
 */
#include "axon_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* softplus(v) = log(1 + e^v). Written as max(v, 0) + log1p(e^-|v|): the same function, but it
 * neither overflows for large v nor loses the small result for very negative v.
 * [AXON "Selective mechanism"] READING: no beta / threshold parameter. */
static double softplus(double v) {
  double pos = v > 0.0 ? v : 0.0;
  return pos + log1p(exp(-fabs(v)));
}

/* SiLU(z) = z * sigmoid(z) = z / (1 + e^-z).  [AXON "Gating"] */
static double silu(double z) { return z / (1.0 + exp(-z)); }

int oracle_ssm_channel(int64_t L, int64_t N, int64_t K,
                       const float* x, const float* z, const float* dt_raw, int64_t act_stride,
                       const float* Bm, const float* Cm, int64_t bc_stride,
                       const float* A_log, double D, double dt_bias, const float* conv_w,
                       double conv_b, double dt_min, double dt_max, int conv_act, int disc,
                       const double* win_in, const double* h_in,
                       double* y, int64_t y_stride, double* win_out, double* h_out,
                       double* u_out, double* dt_out, double* mag_out) {
  if (L < 0 || N < 1 || K < 1 || N > 4096 || K > 64) return -1;
  if (L > 0 && (!x || !z || !dt_raw || !Bm || !Cm || !y)) return -1;
  if (!A_log || !conv_w || !win_out || !h_out) return -1;
  if (conv_act != ORACLE_CONV_NONE && conv_act != ORACLE_CONV_SILU) return -1;
  if (disc != ORACLE_DISC_FIRST_ORDER && disc != ORACLE_DISC_ZOH) return -1;

  /* Diagonal state matrix: A_n = -exp(A_log_n).  [AXON "Diagonal state matrix"] */
  double* A = (double*)malloc(sizeof(double) * (size_t)N);
  double* h = (double*)malloc(sizeof(double) * (size_t)N);
  /* win[0..K-2]: the K-1 most recent x-branch inputs before the current token, oldest first.
   * READING: the cache stores raw inputs of the convolution (not its outputs), so that the
   * causal window of the first new token is [cache, x_0]. [AXON "Autoregressive decoding"] */
  double* win = (double*)malloc(sizeof(double) * (size_t)(K > 1 ? K - 1 : 1));
  if (!A || !h || !win) { free(A); free(h); free(win); return -1; }
  for (int64_t n = 0; n < N; ++n) {
    A[n] = -exp((double)A_log[n]);
    h[n] = h_in ? h_in[n] : 0.0; /* READING: no initial state means zeros [WIKI toy scan]. */
  }
  for (int64_t k = 0; k < K - 1; ++k) win[k] = win_in ? win_in[k] : 0.0;

  for (int64_t t = 0; t < L; ++t) {
    const double xt = (double)x[t * act_stride];

    /* Causal depthwise convolution, kernel size K, with bias:
     * u_t = conv_b + sum_k w_k * xx[t-(K-1)+k]; w_{K-1} multiplies the current token.
     * [AXON "Key contributions", "Code mapping": _causal_conv1d]
     * READING: cross-correlation order with K-1 left padding (taken from the cache), and no
     * activation on u before the scan. */
    double u = conv_b;
    for (int64_t k = 0; k < K - 1; ++k) u += (double)conv_w[k] * win[k];
    u += (double)conv_w[K - 1] * xt;
    for (int64_t k = 0; k + 1 < K - 1; ++k) win[k] = win[k + 1];
    if (K > 1) win[K - 2] = xt;
    /* Mamba-block variant: SiLU on the convolution output before the scan.
     * ["Selective State Space Models (Mamba)", pattern "Mamba block" (mamba-ssm's block)] */
    if (conv_act == ORACLE_CONV_SILU) u = silu(u);

    /* Step size: dt = softplus(dt_raw + b_dt), clipped to [dt_min, dt_max].
     * [AXON "Selective mechanism"] */
    double dt = softplus((double)dt_raw[t * act_stride] + dt_bias);
    if (dt < dt_min) dt = dt_min;
    if (dt > dt_max) dt = dt_max;

    /* First-order discretisation Abar = exp(dt A), Bbar = dt B, then
     * h_t = Abar h_{t-1} + Bbar x_t and y_t = C h_t + D x_t, with the convolution output u_t as
     * the scan input x_t in both places. [AXON "ZOH discretization"; WIKI "Selective scan (toy)"]
     * READING: the skip term D uses the same u_t as the recurrence. */
    double acc = 0.0, mag = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      const double abar = exp(dt * A[n]);
      /* Exact zero-order hold for a diagonal A: Bbar = (dt A)^-1 (exp(dt A) - 1) dt B
       * = expm1(dt A) / A * B.  [AXON "ZOH discretization"; glossary "How SSMs work"] */
      const double bbar = disc == ORACLE_DISC_ZOH
                              ? expm1(dt * A[n]) / A[n] * (double)Bm[t * bc_stride + n]
                              : dt * (double)Bm[t * bc_stride + n];
      h[n] = abar * h[n] + bbar * u;
      acc += (double)Cm[t * bc_stride + n] * h[n];
      mag += fabs((double)Cm[t * bc_stride + n] * h[n]);
    }
    acc += D * u;
    mag += fabs(D * u);

    /* Gate: y * SiLU(z).  [AXON "Gating"] */
    const double gate = silu((double)z[t * act_stride]);
    y[t * y_stride] = acc * gate;
    if (u_out) u_out[t * y_stride] = u;
    if (dt_out) dt_out[t * y_stride] = dt;
    if (mag_out) mag_out[t * y_stride] = mag * fabs(gate);
  }

  for (int64_t k = 0; k < K - 1; ++k) win_out[k] = win[k];
  for (int64_t n = 0; n < N; ++n) h_out[n] = h[n];
  free(A);
  free(h);
  free(win);
  return 0;
}

/* ---- whole-tensor drivers: gather one channel, run it, scatter the results ---------------- */

typedef struct {
  int64_t Bsz, L, E, N, K;
  const float *x, *z, *dt_raw, *Bm, *Cm, *A_log, *D, *dt_bias, *conv_w, *conv_b;
  double dt_min, dt_max;
  int conv_act, disc;
  const double *cache_in, *state_in;
  double *y, *cache_out, *state_out, *mag;
  int64_t ch_begin, ch_end; /* channel index c = b * E + e */
  int status;
} prefill_job;

static void* prefill_worker(void* arg) {
  prefill_job* j = (prefill_job*)arg;
  const int64_t E = j->E, N = j->N, K = j->K, L = j->L;
  double win_in[64], win_out[64];
  double* h_out = (double*)malloc(sizeof(double) * (size_t)N);
  double* h_in = (double*)malloc(sizeof(double) * (size_t)N);
  if (!h_out || !h_in) { free(h_out); free(h_in); j->status = -1; return NULL; }
  j->status = 0;
  for (int64_t c = j->ch_begin; c < j->ch_end && j->status == 0; ++c) {
    const int64_t b = c / E, e = c % E;
    for (int64_t k = 0; k < K - 1; ++k)
      win_in[k] = j->cache_in ? j->cache_in[(b * (K - 1) + k) * E + e] : 0.0;
    for (int64_t n = 0; n < N; ++n)
      h_in[n] = j->state_in ? j->state_in[(b * E + e) * N + n] : 0.0;
    const int64_t off = b * L * E + e;
    const int has_tokens = L > 0;
    j->status = oracle_ssm_channel(
        L, N, K, has_tokens ? j->x + off : NULL, has_tokens ? j->z + off : NULL,
        has_tokens ? j->dt_raw + off : NULL, E, has_tokens ? j->Bm + b * L * N : NULL,
        has_tokens ? j->Cm + b * L * N : NULL, N, j->A_log + e * N, (double)j->D[e],
        (double)j->dt_bias[e], j->conv_w + e * K, (double)j->conv_b[e], j->dt_min, j->dt_max,
        j->conv_act, j->disc, win_in, h_in, has_tokens ? j->y + off : NULL, E, win_out, h_out, NULL, NULL,
        (has_tokens && j->mag) ? j->mag + off : NULL);
    for (int64_t k = 0; k < K - 1; ++k) j->cache_out[(b * (K - 1) + k) * E + e] = win_out[k];
    for (int64_t n = 0; n < N; ++n) j->state_out[(b * E + e) * N + n] = h_out[n];
  }
  free(h_out);
  free(h_in);
  return NULL;
}

static int run_jobs(prefill_job* proto, int threads) {
  const int64_t total = proto->Bsz * proto->E;
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  if ((int64_t)threads > total) threads = (int)(total > 0 ? total : 1);
  prefill_job jobs[256];
  pthread_t tids[256];
  int started[256];
  for (int i = 0; i < threads; ++i) {
    jobs[i] = *proto;
    jobs[i].ch_begin = total * i / threads;
    jobs[i].ch_end = total * (i + 1) / threads;
    started[i] = 0;
  }
  for (int i = 1; i < threads; ++i)
    started[i] = pthread_create(&tids[i], NULL, prefill_worker, &jobs[i]) == 0;
  prefill_worker(&jobs[0]);
  int status = jobs[0].status;
  for (int i = 1; i < threads; ++i) {
    if (started[i]) {
      pthread_join(tids[i], NULL);
    } else {
      prefill_worker(&jobs[i]); /* could not start a thread: do its share here */
    }
    if (jobs[i].status != 0) status = jobs[i].status;
  }
  return status;
}

int oracle_ssm_prefill(int64_t Bsz, int64_t L, int64_t E, int64_t N, int64_t K,
                       const float* x, const float* z, const float* dt_raw,
                       const float* Bm, const float* Cm,
                       const float* A_log, const float* D, const float* dt_bias,
                       const float* conv_w, const float* conv_b, double dt_min, double dt_max,
                       int conv_act, int disc,
                       const double* conv_cache_in, const double* ssm_state_in,
                       double* y, double* conv_cache_out, double* ssm_state_out, double* mag,
                       int threads) {
  if (Bsz < 1 || E < 1 || L < 0 || N < 1 || K < 1 || K > 64) return -1;
  if (!A_log || !D || !dt_bias || !conv_w || !conv_b || !conv_cache_out || !ssm_state_out)
    return -1;
  prefill_job proto;
  memset(&proto, 0, sizeof(proto));
  proto.Bsz = Bsz; proto.L = L; proto.E = E; proto.N = N; proto.K = K;
  proto.x = x; proto.z = z; proto.dt_raw = dt_raw; proto.Bm = Bm; proto.Cm = Cm;
  proto.A_log = A_log; proto.D = D; proto.dt_bias = dt_bias; proto.conv_w = conv_w;
  proto.conv_b = conv_b; proto.dt_min = dt_min; proto.dt_max = dt_max;
  proto.conv_act = conv_act; proto.disc = disc;
  proto.cache_in = conv_cache_in; proto.state_in = ssm_state_in;
  proto.y = y; proto.cache_out = conv_cache_out; proto.state_out = ssm_state_out;
  proto.mag = mag;
  return run_jobs(&proto, threads);
}

int oracle_ssm_decode_step(int64_t Bsz, int64_t E, int64_t N, int64_t K,
                           const float* x, const float* z, const float* dt_raw,
                           const float* Bm, const float* Cm,
                           const float* A_log, const float* D, const float* dt_bias,
                           const float* conv_w, const float* conv_b, double dt_min, double dt_max,
                           int conv_act, int disc,
                           double* conv_cache, double* ssm_state, double* y, int threads) {
  /* A decode step is the prefill body for a single token with the caches carried in place.
   * [AXON "Autoregressive decoding"] Each channel reads its own cache entries before writing
   * them, so passing the same arrays as input and output is safe. */
  return oracle_ssm_prefill(Bsz, 1, E, N, K, x, z, dt_raw, Bm, Cm, A_log, D, dt_bias, conv_w,
                            conv_b, dt_min, dt_max, conv_act, disc, conv_cache, ssm_state, y,
                            conv_cache,
                            ssm_state, NULL, threads);
}

/* ---- Mamba-2 SSD core -------------------------------------------------------------------------
 * ["Selective State Space Models (Mamba)", pattern "Mamba-2 block": d_state 128, headdim 64;
 * the SSD article: the same selective recurrence with one scalar decay per head, which makes it
 * a masked linear attention]. Plain sequential recurrence, one (b, head) at a time.
 * READING: first-order input term dt B (as the Axon-SSM layer), B and C shared by all heads
 * (one group), no convolution and no gate (those belong to the block around the core). */
typedef struct {
  int64_t Bsz, L, H, P, N;
  const float *x, *dt_raw, *Bm, *Cm, *A_log, *D, *dt_bias;
  double dt_min, dt_max;
  const double* state_in;
  double *y, *state_out, *mag;
  int64_t begin, end; /* (b, head) index range */
  int status;
} ssd_job;

static void* ssd_worker(void* arg) {
  ssd_job* j = (ssd_job*)arg;
  const int64_t L = j->L, H = j->H, P = j->P, N = j->N;
  double* h = (double*)malloc(sizeof(double) * (size_t)(P * N));
  if (!h) { j->status = -1; return NULL; }
  j->status = 0;
  for (int64_t bh = j->begin; bh < j->end; ++bh) {
    const int64_t b = bh / H, hd = bh % H;
    const double A = -exp((double)j->A_log[hd]);
    for (int64_t i = 0; i < P * N; ++i) h[i] = j->state_in ? j->state_in[bh * P * N + i] : 0.0;
    for (int64_t t = 0; t < L; ++t) {
      double dt = softplus((double)j->dt_raw[(b * L + t) * H + hd] + (double)j->dt_bias[hd]);
      if (dt < j->dt_min) dt = j->dt_min;
      if (dt > j->dt_max) dt = j->dt_max;
      const double a = exp(dt * A);
      const float* xt = j->x + ((b * L + t) * H + hd) * P;
      const float* Bt = j->Bm + (b * L + t) * N;
      const float* Ct = j->Cm + (b * L + t) * N;
      double* yt = j->y + ((b * L + t) * H + hd) * P;
      double* mt = j->mag ? j->mag + ((b * L + t) * H + hd) * P : NULL;
      for (int64_t p = 0; p < P; ++p) {
        double acc = 0.0, size = 0.0;
        for (int64_t n = 0; n < N; ++n) {
          h[p * N + n] = a * h[p * N + n] + dt * (double)xt[p] * (double)Bt[n];
          acc += (double)Ct[n] * h[p * N + n];
          size += fabs((double)Ct[n] * h[p * N + n]);
        }
        yt[p] = acc + (double)j->D[hd] * (double)xt[p];
        if (mt) mt[p] = size + fabs((double)j->D[hd] * (double)xt[p]);
      }
    }
    for (int64_t i = 0; i < P * N; ++i) j->state_out[bh * P * N + i] = h[i];
  }
  free(h);
  return NULL;
}

int oracle_ssd_scan(int64_t Bsz, int64_t L, int64_t H, int64_t P, int64_t N,
                    const float* x, const float* dt_raw, const float* Bm, const float* Cm,
                    const float* A_log, const float* D, const float* dt_bias, double dt_min,
                    double dt_max, const double* state_in, double* y, double* state_out,
                    double* mag, int threads) {
  if (Bsz < 1 || L < 0 || H < 1 || P < 1 || N < 1 || !A_log || !D || !dt_bias || !state_out)
    return -1;
  if (L > 0 && (!x || !dt_raw || !Bm || !Cm || !y)) return -1;
  const int64_t total = Bsz * H;
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  if ((int64_t)threads > total) threads = (int)total;
  ssd_job jobs[256];
  pthread_t tids[256];
  int started[256];
  for (int i = 0; i < threads; ++i) {
    ssd_job jb = {Bsz, L, H, P, N, x, dt_raw, Bm, Cm, A_log, D, dt_bias, dt_min, dt_max,
                  state_in, y, state_out, mag, total * i / threads, total * (i + 1) / threads,
                  0};
    jobs[i] = jb;
    started[i] = 0;
  }
  for (int i = 1; i < threads; ++i)
    started[i] = pthread_create(&tids[i], NULL, ssd_worker, &jobs[i]) == 0;
  ssd_worker(&jobs[0]);
  int status = jobs[0].status;
  for (int i = 1; i < threads; ++i) {
    if (started[i])
      pthread_join(tids[i], NULL);
    else
      ssd_worker(&jobs[i]);
    if (jobs[i].status != 0) status = jobs[i].status;
  }
  return status;
}
