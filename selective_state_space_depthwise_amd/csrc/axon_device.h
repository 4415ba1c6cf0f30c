// Device helpers shared by the prefill and decode kernels (gfx950, fp32 arithmetic).
//
// Definitions follow "Axon-SSM: Selective State Space Model for Apple Silicon":
//   section "Selective mechanism":   dt = clip(softplus(dt_raw + dt_bias), dt_min, dt_max)
//   section "Diagonal state matrix": A_n = -exp(A_log_n)
//   section "ZOH discretization":    Abar = exp(dt A) (first-order form, Bbar = dt B)
//   section "Gating":                out = y * SiLU(z)
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace axon {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

using bf16_bits = uint16_t;

__device__ __forceinline__ float bf16_to_f32(bf16_bits v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

__device__ __forceinline__ float load_act(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_act(const bf16_bits* p, int64_t i) {
  return bf16_to_f32(p[i]);
}

// Wave-uniform reads of data no kernel writes (B_t / C_t rows): through the constant address
// space, so the compiler issues scalar loads and the values arrive in SGPRs.
__device__ __forceinline__ float load_uniform(const float* p, int64_t i) {
  return ((const __attribute__((address_space(4))) float*)p)[i];
}
__device__ __forceinline__ float load_uniform(const bf16_bits* p, int64_t i) {
  return bf16_to_f32(((const __attribute__((address_space(4))) bf16_bits*)p)[i]);
}

__device__ __forceinline__ void store_act(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store_act(bf16_bits* p, int64_t i, float v) {
  // round to nearest, ties to even
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  p[i] = static_cast<bf16_bits>(u >> 16);
}

// A_n * log2(e) with A_n = -exp(A_log_n), so that exp(dt A_n) = exp2(dt * rate).
__device__ __forceinline__ float decay_rate_log2(float a_log) { return -expf(a_log) * kLog2e; }

// softplus(v) = max(v, 0) + log1p(w), w = exp(-|v|) in (0, 1]. log1p(w) is log(u) for
// u = fl(1 + w), corrected by the rounding error of that sum: log1p(w) = log(u) - ((u-1) - w)/u;
// the 1/u factor of the correction is taken as 1 (the term matters only when w is small, where
// u is 1 to within w). Relative error about 1e-6 over the whole range.
__device__ __forceinline__ float softplus_f32(float v) {
  const float w = __builtin_amdgcn_exp2f(-fabsf(v) * kLog2e);
  const float u = 1.0f + w;
  const float err = (u - 1.0f) - w;
  return fmaxf(v, 0.0f) + fmaf(__builtin_amdgcn_logf(u), kLn2, -err);
}

__device__ __forceinline__ float step_size(float v, float lo, float hi) {
  return fminf(fmaxf(softplus_f32(v), lo), hi);
}

// SiLU(z) = z / (1 + exp(-z)); for very negative z the exponential overflows to +inf and the
// reciprocal to 0, giving -0.
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

}  // namespace axon
