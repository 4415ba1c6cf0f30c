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
// Registers that hold an element's bits as loaded (fp32: 32 bits; bf16: 16 bits, so the
// compiler never masks them), widened to fp32 by raw_to_f32 at use.
template <typename Act>
struct RawOf {
  using type = uint32_t;
};
template <>
struct RawOf<bf16_bits> {
  using type = uint16_t;
};
__device__ __forceinline__ uint32_t load_act_raw(const float* p, int64_t i) {
  return __float_as_uint(p[i]);
}
__device__ __forceinline__ uint16_t load_act_raw(const bf16_bits* p, int64_t i) { return p[i]; }

// Wave-uniform reads of data no kernel writes (B_t / C_t rows): through the constant address
// space, so the compiler issues scalar loads and the values arrive in SGPRs.
__device__ __forceinline__ float load_uniform(const float* p, int64_t i) {
  return ((const __attribute__((address_space(4))) float*)p)[i];
}
__device__ __forceinline__ float load_uniform(const bf16_bits* p, int64_t i) {
  return bf16_to_f32(((const __attribute__((address_space(4))) bf16_bits*)p)[i]);
}

__device__ __forceinline__ void store_act(float* p, int64_t i, float v) { p[i] = v; }
// fp32 -> bf16 with round to nearest, ties to even: one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ bf16_bits f32_to_bf16(float v) {
  return __builtin_bit_cast(bf16_bits, static_cast<__bf16>(v));
}
__device__ __forceinline__ void store_act(bf16_bits* p, int64_t i, float v) {
  p[i] = f32_to_bf16(v);
}

// Raw buffer access: a wave-uniform 128-bit resource (base address in SGPRs) plus a 32-bit
// per-lane byte offset. Stride 0 and num_records 0xFFFFFFFF make every 32-bit offset in range;
// the data-format field is set to 32 bit only because a zero format marks the resource invalid.
using rsrc_t = __amdgpu_buffer_rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, -1, 0x00020000);
}
// A resource whose range is the first `bytes` bytes at base: an access at a byte offset at or
// past the range is out of range, so a load returns 0 and a store is dropped by the hardware.
// Stores use it to mask lanes without a branch (offset kNoStore, or past the valid range).
constexpr uint32_t kNoStore = 0x80000000u;
__device__ __forceinline__ rsrc_t make_rsrc_bounded(void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, static_cast<int>(bytes), 0x00020000);
}

template <typename Act>
__device__ __forceinline__ float load_buf(rsrc_t r, uint32_t off);
template <>
__device__ __forceinline__ float load_buf<float>(rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
template <>
__device__ __forceinline__ float load_buf<bf16_bits>(rsrc_t r, uint32_t off) {
  return bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
}

// The same with a wave-uniform byte offset added (soffset).
template <typename Act>
__device__ __forceinline__ float load_buf_s(rsrc_t r, uint32_t off, uint32_t soff);
template <>
__device__ __forceinline__ float load_buf_s<float>(rsrc_t r, uint32_t off, uint32_t soff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0));
}
template <>
__device__ __forceinline__ float load_buf_s<bf16_bits>(rsrc_t r, uint32_t off, uint32_t soff) {
  return bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, off, soff, 0));
}

// The loaded bits without widening (fp32: the float's bits; bf16: the 16 bits zero-extended),
// and their value: callers that prefetch keep the raw bits until use.
template <typename Act>
__device__ __forceinline__ uint32_t load_raw_s(rsrc_t r, uint32_t off, uint32_t soff);
template <>
__device__ __forceinline__ uint32_t load_raw_s<float>(rsrc_t r, uint32_t off, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0);
}
template <>
__device__ __forceinline__ uint32_t load_raw_s<bf16_bits>(rsrc_t r, uint32_t off, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, soff, 0);
}
template <typename Act>
__device__ __forceinline__ float raw_to_f32(uint32_t v);
template <>
__device__ __forceinline__ float raw_to_f32<float>(uint32_t v) {
  return __uint_as_float(v);
}
template <>
__device__ __forceinline__ float raw_to_f32<bf16_bits>(uint32_t v) {
  return __uint_as_float(v << 16);
}
// The 16-bit form (RawOf<bf16_bits>): the shift drops whatever the register's upper half holds.
__device__ __forceinline__ float raw16_to_f32(uint16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}
template <typename Act>
__device__ __forceinline__ typename RawOf<Act>::type load_raw_t(rsrc_t r, uint32_t off);
template <>
__device__ __forceinline__ uint32_t load_raw_t<float>(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
template <>
__device__ __forceinline__ uint16_t load_raw_t<bf16_bits>(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ float widen(uint32_t v) { return __uint_as_float(v); }
__device__ __forceinline__ float widen(uint16_t v) { return raw16_to_f32(v); }

template <typename Act>
__device__ __forceinline__ void store_buf_s(rsrc_t r, uint32_t off, uint32_t soff, float v);
template <>
__device__ __forceinline__ void store_buf_s<float>(rsrc_t r, uint32_t off, uint32_t soff, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, soff, 0);
}
template <>
__device__ __forceinline__ void store_buf_s<bf16_bits>(rsrc_t r, uint32_t off, uint32_t soff,
                                                       float v) {
  __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v), r, off, soff, 0);
}

template <typename Act>
__device__ __forceinline__ void store_buf(rsrc_t r, uint32_t off, float v);
template <>
__device__ __forceinline__ void store_buf<float>(rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}
template <>
__device__ __forceinline__ void store_buf<bf16_bits>(rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v), r, off, 0, 0);
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
