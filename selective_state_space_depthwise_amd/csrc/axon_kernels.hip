// HIP kernels (gfx950) besides the prefill scan: the single-token decode step, the carry combine
// of the time-chunked prefill, the empty-sequence cache copy, and the prefill dispatch.
//
// What is computed follows "Axon-SSM: Selective State Space Model for Apple Silicon" (formulas in
// axon_device.h); the decode step is the section "Autoregressive decoding": one token per batch
// row, with the conv window (the last K-1 raw inputs) and the hidden state carried in place.
#include "axon_device.h"
#include "axon_internal.h"

namespace axon {
namespace {

// Carry combine of the time-chunked prefill: one thread per (b, e, n) walks the M chunks in
// order, H_0 = state_in, H_{c+1} = exp(A S_c) H_c + h_c, where S_c is the chunk's sum of dt
// (the product of the chunk's decays exp(dt A)) and h_c its local final state from zero. The
// carries are read in groups of eight chunks, the next group's loads issued before the current
// group is folded, so one memory latency covers sixteen steps of the recurrence.
constexpr int kCombineGroup = 8;

__global__ __launch_bounds__(256) void carry_combine_kernel(int64_t B, int64_t E, int64_t M,
                                                            const float* __restrict__ A_log,
                                                            const float* __restrict__ state_in,
                                                            const float* __restrict__ carry_h,
                                                            const float* __restrict__ carry_s,
                                                            float* __restrict__ carry_in) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t total = B * E * kState;
  if (idx >= total) return;
  const int64_t be = idx / kState;
  const int64_t e = be % E;
  const int64_t n = idx % kState;
  const float rate = decay_rate_log2(A_log[e * kState + n]);
  float H = state_in ? state_in[idx] : 0.0f;
  carry_in[idx] = H;
  // Chunks 0..M-2 carry into 1..M-1. Loads past the last carry re-read carry M-2 (never folded).
  auto load_group = [&](int64_t c0, float (&hc)[kCombineGroup], float (&sc)[kCombineGroup]) {
#pragma unroll
    for (int i = 0; i < kCombineGroup; ++i) {
      const int64_t c = c0 + i < M - 1 ? c0 + i : M - 2;
      hc[i] = carry_h[c * total + idx];
      sc[i] = carry_s[c * B * E + be];
    }
  };
  auto fold_group = [&](int64_t c0, const float (&hc)[kCombineGroup],
                        const float (&sc)[kCombineGroup]) {
#pragma unroll
    for (int i = 0; i < kCombineGroup; ++i) {
      if (c0 + i + 1 < M) {
        H = fmaf(__builtin_amdgcn_exp2f(rate * sc[i]), H, hc[i]);
        carry_in[(c0 + i + 1) * total + idx] = H;
      }
    }
  };
  if (M < 2) return;
  float ha[kCombineGroup], sa[kCombineGroup], hb[kCombineGroup], sb[kCombineGroup];
  load_group(0, ha, sa);
  for (int64_t c0 = 0; c0 + 1 < M; c0 += 2 * kCombineGroup) {
    load_group(c0 + kCombineGroup, hb, sb);
    fold_group(c0, ha, sa);
    load_group(c0 + 2 * kCombineGroup, ha, sa);
    fold_group(c0 + kCombineGroup, hb, sb);
  }
}

// dst = src (or zeros when src is null); used for an empty sequence.
__global__ __launch_bounds__(256) void copy_or_zero_kernel(const float* __restrict__ src,
                                                           float* __restrict__ dst, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.0f;
}

struct DecodeArgs {
  int64_t B, E;
  const void *x, *z, *dt_raw, *Bm, *Cm;
  const float *A_log, *D, *dt_bias, *conv_w, *conv_b;
  float dt_min, dt_max;
  int conv_silu, zoh;
  float *cache, *state;
  void* y;
};

// Four consecutive activations at element i (a multiple of 4), widened to fp32: one 16-byte
// (fp32) or 8-byte (bf16) load.
__device__ __forceinline__ float4 load4_act(const float* p, int64_t i) {
  return *reinterpret_cast<const float4*>(p + i);
}
__device__ __forceinline__ float4 load4_act(const bf16_bits* p, int64_t i) {
  const uint2 v = *reinterpret_cast<const uint2*>(p + i);
  return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u),
                     __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u));
}

// Decode: kLanes lanes per channel, each owning kSpl = 16 / kLanes of its states (16-byte loads
// and stores of the state, contiguous across the wave); the readout is summed over the channel's
// lanes. The lane's values of A_log, B and C and the channel's 4 conv taps are vector loads.
// Two lanes per channel: 15.5 us per step at 64 x 7680 fp32 (four lanes 16.3 us, one 20.5 us).
constexpr int kDecodeLanes = 2;

template <typename Act, int kLanes>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  constexpr int kSpl = kState / kLanes;
  constexpr int kChannels = 256 / kLanes;
  const int q = threadIdx.x % kLanes;
  const int64_t e_raw = static_cast<int64_t>(blockIdx.x) * kChannels + threadIdx.x / kLanes;
  const bool active = e_raw < a.E;
  const int64_t e = active ? e_raw : a.E - 1;  // inactive lanes mirror a valid channel
  const int64_t b = blockIdx.y;
  const Act* __restrict__ x = static_cast<const Act*>(a.x);
  const Act* __restrict__ zp = static_cast<const Act*>(a.z);
  const Act* __restrict__ dtr = static_cast<const Act*>(a.dt_raw);
  float Bv[kSpl], Cv[kSpl], alog[kSpl], h[kSpl];
  float4* sp = reinterpret_cast<float4*>(a.state + (b * a.E + e) * kState + kSpl * q);
#pragma unroll
  for (int k4 = 0; k4 < kSpl / 4; ++k4) {
    const float4 B4 = load4_act(static_cast<const Act*>(a.Bm), b * kState + kSpl * q + 4 * k4);
    const float4 C4 = load4_act(static_cast<const Act*>(a.Cm), b * kState + kSpl * q + 4 * k4);
    const float4 al4 =
        *reinterpret_cast<const float4*>(a.A_log + e * kState + kSpl * q + 4 * k4);
    const float4 h4 = sp[k4];
    Bv[4 * k4] = B4.x, Bv[4 * k4 + 1] = B4.y, Bv[4 * k4 + 2] = B4.z, Bv[4 * k4 + 3] = B4.w;
    Cv[4 * k4] = C4.x, Cv[4 * k4 + 1] = C4.y, Cv[4 * k4 + 2] = C4.z, Cv[4 * k4 + 3] = C4.w;
    alog[4 * k4] = al4.x, alog[4 * k4 + 1] = al4.y, alog[4 * k4 + 2] = al4.z,
    alog[4 * k4 + 3] = al4.w;
    h[4 * k4] = h4.x, h[4 * k4 + 1] = h4.y, h[4 * k4 + 2] = h4.z, h[4 * k4 + 3] = h4.w;
  }
  const float4 cw = *reinterpret_cast<const float4*>(a.conv_w + e * kConv);

  const float x0 = a.cache[(b * kHalo + 0) * a.E + e];
  const float x1 = a.cache[(b * kHalo + 1) * a.E + e];
  const float x2 = a.cache[(b * kHalo + 2) * a.E + e];
  const int64_t i = b * a.E + e;
  const float xv = load_act(x, i);
  float u = fmaf(cw.w, xv, fmaf(cw.z, x2, fmaf(cw.y, x1, fmaf(cw.x, x0, a.conv_b[e]))));
  if (a.conv_silu) u = silu(u);  // Mamba-block variant: SiLU on the convolution output
  const float dt = step_size(load_act(dtr, i) + a.dt_bias[e], a.dt_min, a.dt_max);
  const float dtu = dt * u;

  float p = 0.0f;
#pragma unroll
  for (int k = 0; k < kSpl; ++k) {
    const float abar = __builtin_amdgcn_exp2f(dt * decay_rate_log2(alog[k]));
    if (a.zoh) {
      // Exact zero-order hold: Bbar = expm1(dt A) / A * B, A = -exp(A_log).
      const float A = -expf(alog[k]);
      h[k] = fmaf(abar, h[k], (expm1f(dt * A) / A) * u * Bv[k]);
    } else {
      h[k] = fmaf(abar, h[k], dtu * Bv[k]);
    }
    p = fmaf(Cv[k], h[k], p);
  }
#pragma unroll
  for (int m = 1; m < kLanes; m <<= 1) p += __shfl_xor(p, m);
  if (active) {
#pragma unroll
    for (int k4 = 0; k4 < kSpl / 4; ++k4)
      sp[k4] = make_float4(h[4 * k4], h[4 * k4 + 1], h[4 * k4 + 2], h[4 * k4 + 3]);
    if (q == 0) {
      const float yv = fmaf(a.D[e], u, p) * silu(load_act(zp, i));
      store_act(static_cast<Act*>(a.y), i, yv);
    }
    // the window shifts by one: slots 0, 1, 2 receive x1, x2, x
#pragma unroll
    for (int j = q; j < kHalo; j += kLanes) {
      const float nv = (j == 0) ? x1 : ((j == 1) ? x2 : xv);
      a.cache[(b * kHalo + j) * a.E + e] = nv;
    }
  }
}

template <typename Act>
int launch_decode_t(const DecodeLaunch& p, hipStream_t s) {
  DecodeArgs a{};
  a.B = p.batch;
  a.E = p.d_inner;
  a.x = p.x;
  a.z = p.z;
  a.dt_raw = p.dt_raw;
  a.Bm = p.B;
  a.Cm = p.C;
  a.A_log = p.A_log;
  a.D = p.D;
  a.dt_bias = p.dt_bias;
  a.conv_w = p.conv_w;
  a.conv_b = p.conv_b;
  a.dt_min = p.dt_min;
  a.dt_max = p.dt_max;
  a.conv_silu = p.conv_silu;
  a.zoh = p.zoh;
  a.cache = p.conv_cache;
  a.state = p.ssm_state;
  a.y = p.y;
  constexpr int kChannels = 256 / kDecodeLanes;
  const unsigned gx = static_cast<unsigned>((p.d_inner + kChannels - 1) / kChannels);
  hipLaunchKernelGGL((decode_kernel<Act, kDecodeLanes>), dim3(gx, static_cast<unsigned>(p.batch)), dim3(256), 0,
                     s, a);
  return static_cast<int>(hipGetLastError());
}

}  // namespace

void launch_carry_combine(int64_t B, int64_t E, int64_t M, const float* A_log,
                          const float* state_in, const float* carry_h, const float* carry_s,
                          float* carry_in, hipStream_t s) {
  const int64_t total = B * E * kState;
  hipLaunchKernelGGL(carry_combine_kernel, dim3(static_cast<unsigned>((total + 255) / 256)),
                     dim3(256), 0, s, B, E, M, A_log, state_in, carry_h, carry_s, carry_in);
}

int launch_prefill(const PrefillLaunch& p, const PrefillPlan& plan, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.seqlen == 0) {
    const int64_t nc = p.batch * kHalo * p.d_inner;
    const int64_t ns = p.batch * p.d_inner * kState;
    if (p.conv_cache_in != p.conv_cache_out) {
      hipLaunchKernelGGL(copy_or_zero_kernel, dim3(static_cast<unsigned>((nc + 255) / 256)),
                         dim3(256), 0, s, p.conv_cache_in, p.conv_cache_out, nc);
    }
    if (p.ssm_state_in != p.ssm_state_out) {
      hipLaunchKernelGGL(copy_or_zero_kernel, dim3(static_cast<unsigned>((ns + 255) / 256)),
                         dim3(256), 0, s, p.ssm_state_in, p.ssm_state_out, ns);
    }
    return static_cast<int>(hipGetLastError());
  }
  return plan.kernel == kChanScan ? launch_chan_scan(p, plan, stream)
                                  : launch_row_scan(p, plan, stream);
}

int launch_decode(const DecodeLaunch& p, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  return p.act_bf16 ? launch_decode_t<bf16_bits>(p, s) : launch_decode_t<float>(p, s);
}

}  // namespace axon
