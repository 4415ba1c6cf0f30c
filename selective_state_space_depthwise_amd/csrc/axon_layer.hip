// The whole Axon-SSM layer around the selective-scan path: the input projection split into the
// x and z branches, the causal depthwise convolution, the selection projection f_proj, the scan
// with its gate, and the output projection ("Axon-SSM: Selective State Space Model for Apple
// Silicon", sections "Gating", "Selective mechanism", "Code mapping").
//
// The projections are plain dense GEMMs and run on hipBLASLt (fp32 accumulation, MFMA). Each is
// issued as out = in * W^T on row-major operands, with W split into row blocks so that every
// intermediate is its own contiguous tensor: W_in into the x and z halves, W_f into the B, C and
// dt_raw rows. The convolution runs here, once, because f_proj reads its output; the scan then
// receives u with an identity convolution (taps 0, 0, 0, 1 and bias 0, which reproduce u
// exactly) and a throw-away conv cache, while the layer's conv cache is kept by this file.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <new>
#include <tuple>

#include "axon_device.h"
#include "axon_internal.h"

struct axon_layer_ctx {
  hipblasLtHandle_t blas = nullptr;
  // GEMM plans by (m, n, k, dtype): the algorithm hipBLASLt's heuristic picked and its workspace.
  std::map<std::tuple<int64_t, int64_t, int64_t, int>, hipblasLtMatmulHeuristicResult_t> plans;
};

namespace axon {
namespace {

constexpr size_t kGemmWorkspace = size_t(64) << 20;

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// u[b, t, e] = conv_b[e] + sum_k w[e, k] x~[b, t - 3 + k, e], x~ = [cache_in, x] (zeros without a
// cache), then SiLU for the Mamba-block variant; the same accumulation order as the prefill
// kernel's prologue.
// Vector of V consecutive activations (V = 4: one 16-byte fp32 or 8-byte bf16 access).
template <int V>
__device__ __forceinline__ void load_vec(const float* p, int64_t i, float (&v)[V]) {
  if constexpr (V == 4) {
    const float4 q = *reinterpret_cast<const float4*>(p + i);
    v[0] = q.x, v[1] = q.y, v[2] = q.z, v[3] = q.w;
  } else {
#pragma unroll
    for (int k = 0; k < V; ++k) v[k] = p[i + k];
  }
}
template <int V>
__device__ __forceinline__ void load_vec(const bf16_bits* p, int64_t i, float (&v)[V]) {
  if constexpr (V == 4) {
    const uint2 q = *reinterpret_cast<const uint2*>(p + i);
    v[0] = __uint_as_float(q.x << 16), v[1] = __uint_as_float(q.x & 0xFFFF0000u);
    v[2] = __uint_as_float(q.y << 16), v[3] = __uint_as_float(q.y & 0xFFFF0000u);
  } else {
#pragma unroll
    for (int k = 0; k < V; ++k) v[k] = bf16_to_f32(p[i + k]);
  }
}
template <int V>
__device__ __forceinline__ void store_vec(float* p, int64_t i, const float (&v)[V]) {
  if constexpr (V == 4) {
    *reinterpret_cast<float4*>(p + i) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
#pragma unroll
    for (int k = 0; k < V; ++k) p[i + k] = v[k];
  }
}
__device__ __forceinline__ uint32_t bf16_rne(float f) { return f32_to_bf16(f); }
template <int V>
__device__ __forceinline__ void store_vec(bf16_bits* p, int64_t i, const float (&v)[V]) {
  if constexpr (V == 4) {
    *reinterpret_cast<uint2*>(p + i) = make_uint2(bf16_rne(v[0]) | (bf16_rne(v[1]) << 16),
                                                  bf16_rne(v[2]) | (bf16_rne(v[3]) << 16));
  } else {
#pragma unroll
    for (int k = 0; k < V; ++k) store_act(p, i + k, v[k]);
  }
}

// Causal depthwise convolution of the x branch (with the variant's SiLU). Thread (channels
// e0 .. e0 + V - 1, tokens t0 .. t0 + tpt - 1 of batch row b): the taps slide along the tokens in
// registers, so each input is read once (plus a 3-token halo per run). The accumulation order
// (bias, then taps oldest to newest) is the scan prologue's. Grid (ceil(E / (256 V)),
// ceil(L / tpt), B); V = 4 needs E % 4 == 0.
template <typename Act, bool kSilu, int V>
__global__ __launch_bounds__(256) void conv_kernel(const Act* __restrict__ x,
                                                   const float* __restrict__ cache_in,
                                                   const float* __restrict__ w,
                                                   const float* __restrict__ bias,
                                                   Act* __restrict__ u, int64_t L, int64_t E,
                                                   int64_t tpt) {
  const int64_t e0 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * V;
  if (e0 >= E) return;
  const int64_t t0 = static_cast<int64_t>(blockIdx.y) * tpt;
  const int64_t b = blockIdx.z;
  float wk[V][kConv], bs[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    bs[v] = bias[e0 + v];
#pragma unroll
    for (int k = 0; k < kConv; ++k) wk[v][k] = w[(e0 + v) * kConv + k];
  }
  float win[kHalo][V];  // x[t - 3], x[t - 2], x[t - 1]
#pragma unroll
  for (int j = 0; j < kHalo; ++j) {
    const int64_t tt = t0 - kHalo + j;
    if (tt >= 0) {
      load_vec<V>(x, (b * L + tt) * E + e0, win[j]);
    } else {
#pragma unroll
      for (int v = 0; v < V; ++v)
        win[j][v] = cache_in ? cache_in[(b * kHalo + (tt + kHalo)) * E + e0 + v] : 0.0f;
    }
  }
  const int64_t tend = t0 + tpt < L ? t0 + tpt : L;
  for (int64_t t = t0; t < tend; ++t) {
    float xv[V], out[V];
    load_vec<V>(x, (b * L + t) * E + e0, xv);
#pragma unroll
    for (int v = 0; v < V; ++v) {
      float acc = bs[v];
      acc = fmaf(wk[v][0], win[0][v], acc);
      acc = fmaf(wk[v][1], win[1][v], acc);
      acc = fmaf(wk[v][2], win[2][v], acc);
      acc = fmaf(wk[v][3], xv[v], acc);
      if constexpr (kSilu) acc = silu(acc);
      out[v] = acc;
      win[0][v] = win[1][v];
      win[1][v] = win[2][v];
      win[2][v] = xv[v];
    }
    store_vec<V>(u, (b * L + t) * E + e0, out);
  }
}

// conv_cache_out[b, j, e] = x~[b, L + j, e] for j < K-1 (the last K-1 entries of [cache_in, x]),
// widened exactly to fp32. One thread per (b, e) reads all three before writing (in place).
template <typename Act>
__global__ __launch_bounds__(256) void cache_kernel(const Act* __restrict__ x,
                                                    const float* cache_in, float* cache_out,
                                                    int64_t B, int64_t L, int64_t E) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= B * E) return;
  const int64_t e = i % E;
  const int64_t b = i / E;
  float v[kHalo];
#pragma unroll
  for (int j = 0; j < kHalo; ++j) {
    const int64_t idx = L + j;  // position in [cache_in (3), x (L)]
    if (idx >= kHalo)
      v[j] = load_act(x, (b * L + (idx - kHalo)) * E + e);
    else
      v[j] = cache_in ? cache_in[(b * kHalo + idx) * E + e] : 0.0f;
  }
#pragma unroll
  for (int j = 0; j < kHalo; ++j) cache_out[(b * kHalo + j) * E + e] = v[j];
}

// Identity convolution for the scan: taps (0, 0, 0, 1), bias 0.
__global__ __launch_bounds__(256) void identity_conv_kernel(float* w, float* bias, int64_t E) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= E) return;
  w[e * kConv + 0] = 0.0f;
  w[e * kConv + 1] = 0.0f;
  w[e * kConv + 2] = 0.0f;
  w[e * kConv + 3] = 1.0f;
  bias[e] = 0.0f;
}

unsigned blocks_for(int64_t n) { return static_cast<unsigned>((n + 255) / 256); }

// Runs of 16 tokens per thread (longer when the sequence would need more than 65535 runs), four
// channels per thread when d_inner allows 16-byte / 8-byte accesses.
template <typename Act>
void launch_conv(const Act* x, const float* cache_in, const float* w, const float* bias, Act* u,
                 int64_t B, int64_t L, int64_t E, bool silu_conv, hipStream_t s) {
  int64_t tpt = 16;
  if ((L + tpt - 1) / tpt > 65535) tpt = (L + 65534) / 65535;
  const unsigned gy = static_cast<unsigned>((L + tpt - 1) / tpt);
  const dim3 blk(256);
  if (E % 4 == 0) {
    const dim3 grid(static_cast<unsigned>((E + 1023) / 1024), gy, static_cast<unsigned>(B));
    if (silu_conv)
      hipLaunchKernelGGL((conv_kernel<Act, true, 4>), grid, blk, 0, s, x, cache_in, w, bias, u, L,
                         E, tpt);
    else
      hipLaunchKernelGGL((conv_kernel<Act, false, 4>), grid, blk, 0, s, x, cache_in, w, bias, u,
                         L, E, tpt);
  } else {
    const dim3 grid(static_cast<unsigned>((E + 255) / 256), gy, static_cast<unsigned>(B));
    if (silu_conv)
      hipLaunchKernelGGL((conv_kernel<Act, true, 1>), grid, blk, 0, s, x, cache_in, w, bias, u, L,
                         E, tpt);
    else
      hipLaunchKernelGGL((conv_kernel<Act, false, 1>), grid, blk, 0, s, x, cache_in, w, bias, u,
                         L, E, tpt);
  }
}

// Row-major C (M x N) = A (M x K) * W^T, W (N x K): in column-major terms C^T = W^T' * A^T',
// i.e. op(A) = T on W stored K x N and op(B) = N on A stored K x M.
hipblasStatus_t gemm_rm(axon_layer_ctx* ctx, hipStream_t s, hipDataType type, int64_t M,
                        int64_t N, int64_t K, const void* A, const void* W, void* C, void* ws) {
  hipblasLtMatmulDesc_t op = nullptr;
  hipblasLtMatrixLayout_t lw = nullptr, la = nullptr, lc = nullptr;
  hipblasStatus_t st = hipblasLtMatmulDescCreate(&op, HIPBLAS_COMPUTE_32F, HIP_R_32F);
  if (st != HIPBLAS_STATUS_SUCCESS) return st;
  const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
  hipblasLtMatmulDescSetAttribute(op, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta));
  hipblasLtMatmulDescSetAttribute(op, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb));
  st = hipblasLtMatrixLayoutCreate(&lw, type, K, N, K);
  if (st == HIPBLAS_STATUS_SUCCESS) st = hipblasLtMatrixLayoutCreate(&la, type, K, M, K);
  if (st == HIPBLAS_STATUS_SUCCESS) st = hipblasLtMatrixLayoutCreate(&lc, type, N, M, N);
  const auto key = std::make_tuple(M, N, K, static_cast<int>(type));
  auto it = ctx->plans.find(key);
  if (st == HIPBLAS_STATUS_SUCCESS && it == ctx->plans.end()) {
    hipblasLtMatmulPreference_t pref = nullptr;
    st = hipblasLtMatmulPreferenceCreate(&pref);
    if (st == HIPBLAS_STATUS_SUCCESS) {
      const uint64_t cap = kGemmWorkspace;
      hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &cap,
                                            sizeof(cap));
      hipblasLtMatmulHeuristicResult_t res[1];
      int found = 0;
      st = hipblasLtMatmulAlgoGetHeuristic(ctx->blas, op, lw, la, lc, lc, pref, 1, res, &found);
      if (st == HIPBLAS_STATUS_SUCCESS && found < 1) st = HIPBLAS_STATUS_NOT_SUPPORTED;
      if (st == HIPBLAS_STATUS_SUCCESS) it = ctx->plans.emplace(key, res[0]).first;
      hipblasLtMatmulPreferenceDestroy(pref);
    }
  }
  if (st == HIPBLAS_STATUS_SUCCESS) {
    const float alpha = 1.0f, beta = 0.0f;
    st = hipblasLtMatmul(ctx->blas, op, &alpha, W, lw, A, la, &beta, C, lc, C, lc,
                         &it->second.algo, ws, it->second.workspaceSize, s);
  }
  if (lc) hipblasLtMatrixLayoutDestroy(lc);
  if (la) hipblasLtMatrixLayoutDestroy(la);
  if (lw) hipblasLtMatrixLayoutDestroy(lw);
  hipblasLtMatmulDescDestroy(op);
  return st;
}

struct LayerPlan {
  size_t xb, z, u, bm, cm, dtr, y, idw, idb, cache, scan, gemm, total;
  PrefillPlan scan_plan;
};

bool shape_ok(const axon_layer_shape* s) {
  return s && s->batch >= 1 && s->seqlen >= 1 && s->d_model >= 1 && s->d_inner >= 1 &&
         s->d_inner <= kMaxChannels && s->batch <= 65535 && s->d_state == kState &&
         s->d_conv == kConv && (s->act_dtype == AXON_F32 || s->act_dtype == AXON_BF16) &&
         s->seqlen <= (int64_t(1) << 31) && s->batch * s->seqlen <= (int64_t(1) << 31) &&
         s->d_model <= (int64_t(1) << 24);
}

LayerPlan plan_layer(const axon_layer_shape* s) {
  LayerPlan p{};
  const size_t elt = s->act_dtype == AXON_BF16 ? 2 : 4;
  const size_t M = static_cast<size_t>(s->batch * s->seqlen), E = static_cast<size_t>(s->d_inner);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  p.xb = take(M * E * elt);
  p.z = take(M * E * elt);
  p.u = take(M * E * elt);
  p.bm = take(M * kState * elt);
  p.cm = take(M * kState * elt);
  p.dtr = take(M * E * elt);
  p.y = take(M * E * elt);
  p.idw = take(E * kConv * sizeof(float));
  p.idb = take(E * sizeof(float));
  p.cache = take(static_cast<size_t>(s->batch) * kHalo * E * sizeof(float));
  p.scan_plan = plan_prefill(s->batch, s->seqlen, s->d_inner, SIZE_MAX);
  p.scan = take(p.scan_plan.workspace_bytes);
  p.gemm = take(kGemmWorkspace);
  p.total = off;
  return p;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace
}  // namespace axon

extern "C" {

axon_status axon_layer_create(axon_layer_ctx** ctx) {
  if (!ctx) return AXON_ERR_INVALID_ARGUMENT;
  *ctx = nullptr;
  axon_layer_ctx* c = new (std::nothrow) axon_layer_ctx();
  if (!c) return AXON_ERR_HIP;
  if (hipblasLtCreate(&c->blas) != HIPBLAS_STATUS_SUCCESS) {
    delete c;
    return AXON_ERR_HIP;
  }
  *ctx = c;
  return AXON_OK;
}

void axon_layer_destroy(axon_layer_ctx* ctx) {
  if (!ctx) return;
  if (ctx->blas) hipblasLtDestroy(ctx->blas);
  delete ctx;
}

size_t axon_layer_workspace_bytes(const axon_layer_shape* shape) {
  if (!axon::shape_ok(shape)) return 0;
  return axon::plan_layer(shape).total;
}

axon_status axon_layer_forward_check(const axon_layer_shape* shape,
                                     const axon_layer_weights* weights, const void* x_in,
                                     const float* conv_cache_in, const float* ssm_state_in,
                                     const void* out, const float* conv_cache_out,
                                     const float* ssm_state_out, const void* workspace,
                                     size_t workspace_bytes) {
  using namespace axon;
  if (!weights || !shape) return AXON_ERR_INVALID_ARGUMENT;
  if (shape->d_state != kState || shape->d_conv != kConv ||
      (shape->act_dtype != AXON_F32 && shape->act_dtype != AXON_BF16))
    return AXON_ERR_UNSUPPORTED;
  if (!shape_ok(shape)) return AXON_ERR_INVALID_ARGUMENT;
  const axon_status pst = validate_params(&weights->ssm);
  if (pst != AXON_OK) return pst;
  const void* ptrs[] = {weights->W_in, weights->W_f, weights->W_out, x_in, out, conv_cache_out,
                        ssm_state_out, workspace};
  for (const void* q : ptrs)
    if (!q || !aligned16(q)) return AXON_ERR_INVALID_ARGUMENT;
  if ((conv_cache_in && !aligned16(conv_cache_in)) || (ssm_state_in && !aligned16(ssm_state_in)))
    return AXON_ERR_INVALID_ARGUMENT;
  const LayerPlan lp = plan_layer(shape);
  if (workspace_bytes < lp.total) return AXON_ERR_WORKSPACE_TOO_SMALL;

  // Aliasing: out, the workspace and the cache / state outputs overlap nothing they must not.
  // A cache or state output may be its input exactly (in place), never partly.
  const size_t elt = shape->act_dtype == AXON_BF16 ? 2 : 4;
  const int64_t B = shape->batch, L = shape->seqlen, D = shape->d_model, E = shape->d_inner;
  const size_t tok = static_cast<size_t>(B * L);
  const Span s_x = span(x_in, tok * D * elt), s_out = span(out, tok * D * elt);
  const Span s_win = span(weights->W_in, static_cast<size_t>(2 * E * D) * elt);
  const Span s_wf = span(weights->W_f, static_cast<size_t>((2 * kState + E) * E) * elt);
  const Span s_wout = span(weights->W_out, static_cast<size_t>(D * E) * elt);
  const size_t cache_bytes = sizeof(float) * B * kHalo * E;
  const size_t state_bytes = sizeof(float) * B * E * kState;
  const Span s_cin = span(conv_cache_in, cache_bytes), s_sin = span(ssm_state_in, state_bytes);
  const Span s_cout = span(conv_cache_out, cache_bytes), s_sout = span(ssm_state_out, state_bytes);
  const Span s_ws = span(workspace, lp.total);
  Span prm[5];
  param_spans(&weights->ssm, E, prm);
  const Span reads[] = {s_x, s_win, s_wf, s_wout, prm[0], prm[1], prm[2], prm[3], prm[4]};
  for (const Span& r : reads) {
    if (overlaps(s_out, r) || overlaps(s_cout, r) || overlaps(s_sout, r) || overlaps(s_ws, r))
      return AXON_ERR_INVALID_ARGUMENT;
  }
  const Span others_of_out[] = {s_cin, s_sin, s_cout, s_sout, s_ws};
  for (const Span& o : others_of_out)
    if (overlaps(s_out, o)) return AXON_ERR_INVALID_ARGUMENT;
  const Span others_of_ws[] = {s_cin, s_sin, s_cout, s_sout};
  for (const Span& o : others_of_ws)
    if (overlaps(s_ws, o)) return AXON_ERR_INVALID_ARGUMENT;
  if (conv_cache_in != conv_cache_out && overlaps(s_cout, s_cin)) return AXON_ERR_INVALID_ARGUMENT;
  if (ssm_state_in != ssm_state_out && overlaps(s_sout, s_sin)) return AXON_ERR_INVALID_ARGUMENT;
  if (overlaps(s_cout, s_sout) || overlaps(s_cout, s_sin) || overlaps(s_sout, s_cin))
    return AXON_ERR_INVALID_ARGUMENT;
  return AXON_OK;
}

axon_status axon_layer_forward(axon_layer_ctx* ctx, const axon_layer_shape* shape,
                               const axon_layer_weights* weights, const void* x_in,
                               const float* conv_cache_in, const float* ssm_state_in, void* out,
                               float* conv_cache_out, float* ssm_state_out, void* workspace,
                               size_t workspace_bytes, void* stream) {
  using namespace axon;
  if (!ctx) return AXON_ERR_INVALID_ARGUMENT;
  const axon_status cst =
      axon_layer_forward_check(shape, weights, x_in, conv_cache_in, ssm_state_in, out,
                               conv_cache_out, ssm_state_out, workspace, workspace_bytes);
  if (cst != AXON_OK) return cst;
  const LayerPlan lp = plan_layer(shape);
  const bool bf16 = shape->act_dtype == AXON_BF16;
  const size_t elt = bf16 ? 2 : 4;
  const int64_t B = shape->batch, L = shape->seqlen, D = shape->d_model, E = shape->d_inner;
  const int64_t M = B * L;

  if (!ctx->blas) return AXON_ERR_INVALID_ARGUMENT;  // the context is used only past here

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const hipDataType t = bf16 ? HIP_R_16BF : HIP_R_32F;
  void* gws = ws + lp.gemm;
  const char* W_in = static_cast<const char*>(weights->W_in);
  const char* W_f = static_cast<const char*>(weights->W_f);
  auto fail = [](hipblasStatus_t st) { return st != HIPBLAS_STATUS_SUCCESS; };

  // Input projection, split into the x and z branches.
  if (fail(gemm_rm(ctx, s, t, M, E, D, x_in, W_in, ws + lp.xb, gws)) ||
      fail(gemm_rm(ctx, s, t, M, E, D, x_in, W_in + static_cast<size_t>(E * D) * elt, ws + lp.z,
                   gws)))
    return AXON_ERR_HIP;
  // Convolution (with the variant's SiLU), then the layer's conv cache.
  const float* cw = weights->ssm.conv_w;
  const float* cb = weights->ssm.conv_b;
  const bool silu_conv = weights->ssm.conv_activation == AXON_CONV_SILU;
  if (bf16) {
    const auto* xb = reinterpret_cast<const bf16_bits*>(ws + lp.xb);
    launch_conv(xb, conv_cache_in, cw, cb, reinterpret_cast<bf16_bits*>(ws + lp.u), B, L, E,
                silu_conv, s);
    hipLaunchKernelGGL((cache_kernel<bf16_bits>), dim3(blocks_for(B * E)), dim3(256), 0, s, xb,
                       conv_cache_in, conv_cache_out, B, L, E);
  } else {
    const auto* xb = reinterpret_cast<const float*>(ws + lp.xb);
    launch_conv(xb, conv_cache_in, cw, cb, reinterpret_cast<float*>(ws + lp.u), B, L, E,
                silu_conv, s);
    hipLaunchKernelGGL((cache_kernel<float>), dim3(blocks_for(B * E)), dim3(256), 0, s, xb,
                       conv_cache_in, conv_cache_out, B, L, E);
  }
  if (hipGetLastError() != hipSuccess) return AXON_ERR_HIP;
  // Selection projection: B_t, C_t and dt_raw_t from u_t.
  if (fail(gemm_rm(ctx, s, t, M, kState, E, ws + lp.u, W_f, ws + lp.bm, gws)) ||
      fail(gemm_rm(ctx, s, t, M, kState, E, ws + lp.u, W_f + static_cast<size_t>(kState * E) * elt,
                   ws + lp.cm, gws)) ||
      fail(gemm_rm(ctx, s, t, M, E, E, ws + lp.u,
                   W_f + static_cast<size_t>(2 * kState * E) * elt, ws + lp.dtr, gws)))
    return AXON_ERR_HIP;
  // The scan and its gate, on u through an identity convolution.
  float* idw = reinterpret_cast<float*>(ws + lp.idw);
  float* idb = reinterpret_cast<float*>(ws + lp.idb);
  hipLaunchKernelGGL(identity_conv_kernel, dim3(blocks_for(E)), dim3(256), 0, s, idw, idb, E);
  PrefillLaunch p{};
  p.batch = B;
  p.seqlen = L;
  p.d_inner = E;
  p.act_bf16 = bf16;
  p.x = ws + lp.u;
  p.z = ws + lp.z;
  p.dt_raw = ws + lp.dtr;
  p.B = ws + lp.bm;
  p.C = ws + lp.cm;
  p.A_log = weights->ssm.A_log;
  p.D = weights->ssm.D;
  p.dt_bias = weights->ssm.dt_bias;
  p.conv_w = idw;
  p.conv_b = idb;
  p.dt_min = weights->ssm.dt_min;
  p.dt_max = weights->ssm.dt_max;
  p.conv_silu = 0;  // applied by the convolution above
  p.zoh = weights->ssm.discretization == AXON_DISC_ZOH;
  p.conv_cache_in = nullptr;
  p.ssm_state_in = ssm_state_in;
  p.y = ws + lp.y;
  p.conv_cache_out = reinterpret_cast<float*>(ws + lp.cache);
  p.ssm_state_out = ssm_state_out;
  p.workspace = ws + lp.scan;
  if (launch_prefill(p, lp.scan_plan, stream) != 0) return AXON_ERR_HIP;
  // Output projection.
  if (fail(gemm_rm(ctx, s, t, M, D, E, ws + lp.y, weights->W_out, out, gws))) return AXON_ERR_HIP;
  return AXON_OK;
}

}  // extern "C"
