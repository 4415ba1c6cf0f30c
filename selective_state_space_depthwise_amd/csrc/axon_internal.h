// Internal interface between the C-ABI layer (axonscan_api.cpp, plain host C++) and the HIP
// launchers (axon_kernels.hip). Deliberately free of HIP headers: streams travel as void* and
// launch results as the integer value of hipError_t (0 = success).
#pragma once

#include <cstddef>
#include <cstdint>

#include "axonscan.h"

namespace axon {

constexpr int kState = 16;  // N, states per channel (the Axon-SSM layer configuration)
constexpr int kConv = 4;    // K, causal conv taps
constexpr int kHalo = kConv - 1;

// How a prefill is split. The scan kernel spreads each channel's 16 states over 4 * row_waves
// (lane row, wave) pairs. When even that leaves the GPU short of lanes, the sequence is also cut
// into chunks processed in parallel: a first pass scans every chunk but the last from a zero
// state and keeps its carry (sum of dt, local final state); a small combine pass turns the
// carries into each chunk's true initial state; the final pass re-scans each chunk from that
// state and writes the outputs.
enum PrefillKernel : int {
  kRowScan = 0,   // 16 states of a channel spread over lanes (axon_rowscan.hip)
  kChanScan = 1,  // one lane per channel, 16 states in its registers (axon_chanscan.hip)
};

struct PrefillPlan {
  int kernel = kRowScan;
  int row_waves = 2;      // W: waves per 16-channel group (states per lane = 4 / W)
  int64_t chunks = 1;     // M
  int64_t chunk_len = 0;  // T (tokens per chunk; the last chunk may be shorter)
  // Workspace regions (byte offsets, 256-byte aligned), used only when chunks > 1.
  size_t off_carry_h = 0;   // (M, B, E, N) fp32: local final state of each chunk from h = 0
  size_t off_carry_s = 0;   // (M, B, E) fp32: sum of dt over each chunk
  size_t off_carry_in = 0;  // (M, B, E, N) fp32: true initial state of each chunk
  size_t off_halo = 0;      // (B, K-1, E) fp32: copy of conv_cache_in for chunk 0
  size_t workspace_bytes = 0;
};

// A pure function of the shape (no device query), so the workspace size is known up front.
// With a workspace limit, the plan takes fewer time chunks until its workspace fits.
PrefillPlan plan_prefill(int64_t batch, int64_t seqlen, int64_t d_inner, size_t max_workspace);
PrefillPlan plan_prefill_uncapped(int64_t batch, int64_t seqlen, int64_t d_inner);

struct PrefillLaunch {
  int64_t batch, seqlen, d_inner;
  int act_bf16;  // 0 = fp32 activations, 1 = bf16
  const void *x, *z, *dt_raw, *B, *C;
  const float *A_log, *D, *dt_bias, *conv_w, *conv_b;
  float dt_min, dt_max;
  int conv_silu, zoh;  // variants: SiLU after the conv; exact zero-order hold
  const float *conv_cache_in, *ssm_state_in;  // may be null (zeros)
  void* y;
  float *conv_cache_out, *ssm_state_out;
  void* workspace;
};

struct DecodeLaunch {
  int64_t batch, d_inner;
  int act_bf16;
  const void *x, *z, *dt_raw, *B, *C;
  const float *A_log, *D, *dt_bias, *conv_w, *conv_b;
  float dt_min, dt_max;
  int conv_silu, zoh;
  float *conv_cache, *ssm_state;
  void* y;
};

// Byte ranges of device buffers, for the aliasing checks of the entry points.
struct Span {
  uintptr_t lo = 0, hi = 0;  // [lo, hi); empty when lo == hi
};
inline Span span(const void* p, size_t bytes) {
  Span s;
  if (p && bytes) {
    s.lo = reinterpret_cast<uintptr_t>(p);
    s.hi = s.lo + bytes;
  }
  return s;
}
inline bool overlaps(const Span& a, const Span& b) {
  return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}
// Byte spans of a parameter block's arrays (read-only inputs), for d_inner = E.
void param_spans(const axon_ssm_params* p, int64_t E, Span out[5]);

int launch_prefill(const PrefillLaunch& a, const PrefillPlan& plan, void* stream);
// Every check of axon_ssm_prefill (shape, parameters, pointers, workspace size, aliasing) and
// the launch description; nothing is launched. library_scratch: the workspace is the library's
// own scratch array (not checked for null or overlap with the caller's buffers).
axon_status prepare_prefill(const axon_ssm_shape* shape, const axon_ssm_params* params,
                            const void* x, const void* z, const void* dt_raw, const void* B,
                            const void* C, const float* conv_cache_in, const float* ssm_state_in,
                            void* y, float* conv_cache_out, float* ssm_state_out,
                            void* workspace, size_t workspace_bytes, bool library_scratch,
                            size_t max_workspace, PrefillLaunch* launch, PrefillPlan* plan);
// The C-ABI checks of a parameter block (pointers, alignment, clips, variants).
axon_status validate_params(const axon_ssm_params* p);
constexpr int64_t kMaxChannels = int64_t(1) << 23;  // d_inner limit of the prefill kernels
int launch_row_scan(const PrefillLaunch& a, const PrefillPlan& plan, void* stream);
int launch_chan_scan(const PrefillLaunch& a, const PrefillPlan& plan, void* stream);
int launch_decode(const DecodeLaunch& a, void* stream);

}  // namespace axon
