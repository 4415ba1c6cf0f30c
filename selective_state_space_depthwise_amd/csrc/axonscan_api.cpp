// C ABI of libaxonscan: argument checks, planning, dispatch. Plain host C++ (no HIP headers):
// every check runs before anything is launched, so an error return leaves device memory and the
// stream untouched. Semantics of the entry points are documented in include/axonscan.h.
#include "axonscan.h"

#include <cmath>
#include <cstdint>
#include <cstdlib>

#include "axon_internal.h"

namespace {

constexpr int kVersion = 300;  // 0.3.0: the Mamba-2 SSD core (axon_ssd_scan)
constexpr int64_t kMaxBatch = 65535;      // launch grid y dimension
constexpr int64_t kMaxElems = int64_t(1) << 40;
// The prefill kernels address a tile of (32 + 3) tokens x d_inner channels with byte offsets
// below 2^31 (offset 2^31 marks a masked store).
constexpr int64_t kMaxDInner = axon::kMaxChannels;

// Work split of the prefill (measured on MI355X, 1024 SIMDs):
//  - from kSinglePassChannels channels, one state per lane (W = 4 waves per 16 channels) gives
//    about two waves per SIMD without cutting the sequence: 7680 channels -> 1920 waves;
//  - from kTwoStateChannels channels, two states per lane (W = 2) is faster (more work per wave,
//    half the cross-wave traffic): 61440 channels -> 7680 waves;
//  - below kSinglePassChannels, two states per lane plus time chunks (a carry pass, a combine
//    and a final pass) up to about kTargetLanes lanes in the final pass (eight waves per SIMD,
//    run in rounds of the three the kernel's registers allow), with chunks of at least
//    kMinChunk tokens. More chunks than two waves per SIMD still pay: 2 x 65536 tokens x 2048
//    channels in bf16 takes 2.60 ms at 4 chunks, 2.20 ms at 16, 2.16 ms at 32; 1 x 16384 x 4096
//    fp32 0.669 ms at 4, 0.626 ms at 16 and 32, 0.666 ms at 64.
constexpr int64_t kSinglePassChannels = 6144;
constexpr int64_t kTwoStateChannels = 16384;
constexpr int64_t kTargetLanes = 524288;
constexpr int64_t kMinChunk = 256;
constexpr int64_t kMaxChunks = 64;
// Lane-per-channel scan: time chunks up to about kChanTargetLanes lanes in the final pass, with
// chunks of at least kChanMinChunk tokens.
#ifndef AXON_PLAN_KERNEL
#define AXON_PLAN_KERNEL 2
#endif
#ifndef AXON_CHAN_TARGET_LANES
#define AXON_CHAN_TARGET_LANES 524288
#endif
constexpr int kPlanKernel = AXON_PLAN_KERNEL;  // 0: row scan only, 1: lane per channel only, 2: by shape
constexpr int64_t kChanTargetLanes = AXON_CHAN_TARGET_LANES;
constexpr int64_t kChanMinChunk = 64;
constexpr int64_t kChanMaxChunks = 256;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

using axon::overlaps;
using axon::param_spans;
using axon::span;
using axon::Span;

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  return !__builtin_mul_overflow(a, b, out) && *out <= kMaxElems;
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

axon_status check_shape(const axon_ssm_shape* s, bool prefill) {
  if (!s) return AXON_ERR_INVALID_ARGUMENT;
  if (s->d_state != axon::kState || s->d_conv != axon::kConv) return AXON_ERR_UNSUPPORTED;
  if (s->act_dtype != AXON_F32 && s->act_dtype != AXON_BF16) return AXON_ERR_UNSUPPORTED;
  if (s->batch < 1 || s->d_inner < 1 || (prefill && s->seqlen < 0))
    return AXON_ERR_INVALID_ARGUMENT;
  if (s->batch > kMaxBatch || s->d_inner > kMaxDInner) return AXON_ERR_UNSUPPORTED;
  int64_t t = 0;
  const int64_t L = prefill ? s->seqlen : 1;
  if (!mul_ok(s->batch, L, &t) || !mul_ok(t, s->d_inner, &t) || !mul_ok(t, axon::kState, &t))
    return AXON_ERR_INVALID_ARGUMENT;
  if (!mul_ok(s->batch, s->d_inner, &t) || !mul_ok(t, axon::kState, &t))
    return AXON_ERR_INVALID_ARGUMENT;
  return AXON_OK;
}

axon_status check_params(const axon_ssm_params* p) {
  if (!p) return AXON_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {p->A_log, p->D, p->dt_bias, p->conv_w, p->conv_b};
  for (const void* q : ptrs)
    if (!q || !aligned16(q)) return AXON_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(p->dt_min) || !std::isfinite(p->dt_max) || p->dt_min < 0.0f ||
      p->dt_min > p->dt_max)
    return AXON_ERR_INVALID_ARGUMENT;
  if ((p->conv_activation != AXON_CONV_NONE && p->conv_activation != AXON_CONV_SILU) ||
      (p->discretization != AXON_DISC_FIRST_ORDER && p->discretization != AXON_DISC_ZOH))
    return AXON_ERR_UNSUPPORTED;
  return AXON_OK;
}

}  // namespace

namespace axon {

void param_spans(const axon_ssm_params* p, int64_t E, Span out[5]) {
  out[0] = span(p->A_log, sizeof(float) * E * kState);
  out[1] = span(p->D, sizeof(float) * E);
  out[2] = span(p->dt_bias, sizeof(float) * E);
  out[3] = span(p->conv_w, sizeof(float) * E * kConv);
  out[4] = span(p->conv_b, sizeof(float) * E);
}

axon_status validate_params(const axon_ssm_params* p) { return check_params(p); }

namespace {

void layout_workspace(PrefillPlan& plan, int64_t channels) {
  if (plan.chunks <= 1) return;
  const int64_t M = plan.chunks;
  const size_t be = static_cast<size_t>(channels);
  size_t off = 0;
  plan.off_carry_h = off;
  off = round_up(off + sizeof(float) * M * be * kState, 256);
  plan.off_carry_s = off;
  off = round_up(off + sizeof(float) * M * be, 256);
  plan.off_carry_in = off;
  off = round_up(off + sizeof(float) * M * be * kState, 256);
  plan.off_halo = off;
  off = round_up(off + sizeof(float) * be * kHalo, 256);
  plan.workspace_bytes = off;
}

// Chunk length for M chunks: whole unrolled steps (8 tokens) where the sequence allows.
void set_chunks(PrefillPlan& plan, int64_t seqlen, int64_t M, int64_t step) {
  if (M < 1) M = 1;
  int64_t T = (seqlen + M - 1) / M;
  T = (T + step - 1) / step * step;
  if (T < step) T = step;
  plan.chunks = (seqlen + T - 1) / T;
  if (plan.chunks < 1) plan.chunks = 1;
  plan.chunk_len = T;
}

}  // namespace

PrefillPlan plan_prefill(int64_t batch, int64_t seqlen, int64_t d_inner, size_t max_workspace) {
  PrefillPlan plan = plan_prefill_uncapped(batch, seqlen, d_inner);
  // Fewer chunks until the workspace fits (one chunk needs none).
  const int step = plan.kernel == kChanScan ? 8 : (plan.row_waves == 4 ? 32 : 16);
  for (int64_t M = plan.chunks - 1; plan.workspace_bytes > max_workspace && M >= 1; --M) {
    PrefillPlan p = plan;
    p.off_carry_h = p.off_carry_s = p.off_carry_in = p.off_halo = 0;
    p.workspace_bytes = 0;
    set_chunks(p, seqlen, M, step);
    layout_workspace(p, batch * d_inner);
    plan = p;
  }
  return plan;
}

PrefillPlan plan_prefill_uncapped(int64_t batch, int64_t seqlen, int64_t d_inner) {
  PrefillPlan plan;
  const int64_t channels = batch * d_inner;
  const bool chan = kPlanKernel == 1 || (kPlanKernel == 2 && channels < kSinglePassChannels);
  if (chan) {
    plan.kernel = kChanScan;
    int64_t M = (kChanTargetLanes + channels - 1) / channels;
    int64_t max_m = seqlen / kChanMinChunk;
    if (max_m < 1) max_m = 1;
    if (M > max_m) M = max_m;
    if (M > kChanMaxChunks) M = kChanMaxChunks;
    set_chunks(plan, seqlen, M, 8);
    layout_workspace(plan, channels);
    return plan;
  }
  const bool single_pass = channels >= kSinglePassChannels;
  plan.row_waves = single_pass && channels < kTwoStateChannels ? 4 : 2;
  const int64_t lanes = channels * 4 * plan.row_waves;
  int64_t M = 1;
  if (!single_pass) {
    M = (kTargetLanes + lanes - 1) / lanes;
    int64_t max_m = seqlen / kMinChunk;
    if (max_m < 1) max_m = 1;
    if (M > max_m) M = max_m;
    if (M > kMaxChunks) M = kMaxChunks;
  }
  // Chunks hold whole scan tiles (32 tokens with one state per lane, else 16).
  set_chunks(plan, seqlen, M, plan.row_waves == 4 ? 32 : 16);
  layout_workspace(plan, channels);
  return plan;
}

}  // namespace axon

namespace axon {

axon_status prepare_prefill(const axon_ssm_shape* shape, const axon_ssm_params* params,
                            const void* x, const void* z, const void* dt_raw, const void* B,
                            const void* C, const float* conv_cache_in, const float* ssm_state_in,
                            void* y, float* conv_cache_out, float* ssm_state_out,
                            void* workspace, size_t workspace_bytes, bool library_scratch,
                            size_t max_workspace, PrefillLaunch* launch, PrefillPlan* plan_out) {
  axon_status st = check_shape(shape, true);
  if (st != AXON_OK) return st;
  st = check_params(params);
  if (st != AXON_OK) return st;
  const int64_t Bsz = shape->batch, L = shape->seqlen, E = shape->d_inner;
  const size_t elt = shape->act_dtype == AXON_BF16 ? 2 : 4;

  if (L > 0) {
    const void* acts[] = {x, z, dt_raw, B, C, y};
    for (const void* q : acts)
      if (!q || !aligned16(q)) return AXON_ERR_INVALID_ARGUMENT;
  }
  if (!conv_cache_out || !ssm_state_out || !aligned16(conv_cache_out) ||
      !aligned16(ssm_state_out))
    return AXON_ERR_INVALID_ARGUMENT;
  if ((conv_cache_in && !aligned16(conv_cache_in)) || (ssm_state_in && !aligned16(ssm_state_in)))
    return AXON_ERR_INVALID_ARGUMENT;

  const PrefillPlan plan = plan_prefill(Bsz, L, E, max_workspace);
  const bool needs_ws = L > 0 && plan.workspace_bytes > 0;
  if (needs_ws) {
    if (workspace_bytes < plan.workspace_bytes) return AXON_ERR_WORKSPACE_TOO_SMALL;
    if (!library_scratch && (!workspace || !aligned16(workspace)))
      return AXON_ERR_INVALID_ARGUMENT;
  }

  const size_t act_bytes = elt * Bsz * L * E;
  const size_t bc_bytes = elt * Bsz * L * kState;
  const size_t cache_bytes = sizeof(float) * Bsz * kHalo * E;
  const size_t state_bytes = sizeof(float) * Bsz * E * kState;
  Span in_x = span(x, act_bytes), in_z = span(z, act_bytes), in_dt = span(dt_raw, act_bytes);
  Span in_b = span(B, bc_bytes), in_c = span(C, bc_bytes);
  Span in_cache = span(conv_cache_in, cache_bytes), in_state = span(ssm_state_in, state_bytes);
  Span out_y = span(y, act_bytes), out_cache = span(conv_cache_out, cache_bytes);
  Span out_state = span(ssm_state_out, state_bytes);
  // The library's own scratch is a separate allocation of the code object: no caller buffer
  // can overlap it.
  Span ws = needs_ws && !library_scratch ? span(workspace, plan.workspace_bytes) : Span{};
  Span prm[5];
  param_spans(params, E, prm);

  // y overlaps nothing.
  const Span others_of_y[] = {in_x, in_z, in_dt, in_b, in_c, in_cache, in_state,
                              out_cache, out_state, ws, prm[0], prm[1], prm[2], prm[3], prm[4]};
  for (const Span& o : others_of_y)
    if (overlaps(out_y, o)) return AXON_ERR_INVALID_ARGUMENT;
  // cache_out is cache_in (in place) or disjoint from it, and disjoint from everything else.
  if (conv_cache_in != conv_cache_out && overlaps(out_cache, in_cache))
    return AXON_ERR_INVALID_ARGUMENT;
  if (ssm_state_in != ssm_state_out && overlaps(out_state, in_state))
    return AXON_ERR_INVALID_ARGUMENT;
  const Span reads[] = {in_x, in_z, in_dt, in_b, in_c, prm[0], prm[1], prm[2], prm[3], prm[4]};
  for (const Span& r : reads) {
    if (overlaps(out_cache, r) || overlaps(out_state, r) || overlaps(ws, r))
      return AXON_ERR_INVALID_ARGUMENT;
  }
  if (overlaps(out_cache, out_state) || overlaps(out_cache, in_state) ||
      overlaps(out_state, in_cache))
    return AXON_ERR_INVALID_ARGUMENT;
  const Span rw[] = {in_cache, in_state, out_cache, out_state};
  for (const Span& r : rw)
    if (overlaps(ws, r)) return AXON_ERR_INVALID_ARGUMENT;

  PrefillLaunch& a = *launch;
  a = PrefillLaunch{};
  a.batch = Bsz;
  a.seqlen = L;
  a.d_inner = E;
  a.act_bf16 = shape->act_dtype == AXON_BF16;
  a.x = x;
  a.z = z;
  a.dt_raw = dt_raw;
  a.B = B;
  a.C = C;
  a.A_log = params->A_log;
  a.D = params->D;
  a.dt_bias = params->dt_bias;
  a.conv_w = params->conv_w;
  a.conv_b = params->conv_b;
  a.dt_min = params->dt_min;
  a.dt_max = params->dt_max;
  a.conv_silu = params->conv_activation == AXON_CONV_SILU;
  a.zoh = params->discretization == AXON_DISC_ZOH;
  a.conv_cache_in = conv_cache_in;
  a.ssm_state_in = ssm_state_in;
  a.y = y;
  a.conv_cache_out = conv_cache_out;
  a.ssm_state_out = ssm_state_out;
  a.workspace = needs_ws ? workspace : nullptr;
  *plan_out = plan;
  return AXON_OK;
}

}  // namespace axon

extern "C" {


int axon_version(void) { return kVersion; }

const char* axon_status_string(int status) {
  switch (status) {
    case AXON_OK: return "ok";
    case AXON_ERR_INVALID_ARGUMENT: return "invalid argument";
    case AXON_ERR_UNSUPPORTED: return "unsupported shape, dtype or variant";
    case AXON_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case AXON_ERR_HIP: return "HIP launch or runtime error";
  }
  return "unknown status";
}

size_t axon_ssm_prefill_workspace_bytes(const axon_ssm_shape* shape) {
  if (check_shape(shape, true) != AXON_OK) return 0;
  return axon::plan_prefill(shape->batch, shape->seqlen, shape->d_inner, SIZE_MAX).workspace_bytes;
}

axon_status axon_ssm_prefill(const axon_ssm_shape* shape, const axon_ssm_params* params,
                             const void* x, const void* z, const void* dt_raw, const void* B,
                             const void* C, const float* conv_cache_in,
                             const float* ssm_state_in, void* y, float* conv_cache_out,
                             float* ssm_state_out, void* workspace, size_t workspace_bytes,
                             void* stream) {
  axon::PrefillLaunch a;
  axon::PrefillPlan plan;
  const axon_status st = axon::prepare_prefill(
      shape, params, x, z, dt_raw, B, C, conv_cache_in, ssm_state_in, y, conv_cache_out,
      ssm_state_out, workspace, workspace_bytes, false, SIZE_MAX, &a, &plan);
  if (st != AXON_OK) return st;
  return axon::launch_prefill(a, plan, stream) == 0 ? AXON_OK : AXON_ERR_HIP;
}

axon_status axon_ssm_decode_step(const axon_ssm_shape* shape, const axon_ssm_params* params,
                                 const void* x, const void* z, const void* dt_raw, const void* B,
                                 const void* C, float* conv_cache, float* ssm_state, void* y,
                                 void* stream) {
  axon_status st = check_shape(shape, false);
  if (st != AXON_OK) return st;
  st = check_params(params);
  if (st != AXON_OK) return st;
  const void* ptrs[] = {x, z, dt_raw, B, C, conv_cache, ssm_state, y};
  for (const void* q : ptrs)
    if (!q || !aligned16(q)) return AXON_ERR_INVALID_ARGUMENT;
  const int64_t Bsz = shape->batch, E = shape->d_inner;
  const size_t elt = shape->act_dtype == AXON_BF16 ? 2 : 4;
  Span in_x = span(x, elt * Bsz * E), in_z = span(z, elt * Bsz * E);
  Span in_dt = span(dt_raw, elt * Bsz * E);
  Span in_b = span(B, elt * Bsz * axon::kState), in_c = span(C, elt * Bsz * axon::kState);
  Span cache = span(conv_cache, sizeof(float) * Bsz * axon::kHalo * E);
  Span state = span(ssm_state, sizeof(float) * Bsz * E * axon::kState);
  Span out_y = span(y, elt * Bsz * E);
  Span prm[5];
  param_spans(params, E, prm);
  const Span reads[] = {in_x, in_z, in_dt, in_b, in_c, prm[0], prm[1], prm[2], prm[3], prm[4]};
  for (const Span& r : reads) {
    if (overlaps(out_y, r) || overlaps(cache, r) || overlaps(state, r))
      return AXON_ERR_INVALID_ARGUMENT;
  }
  if (overlaps(out_y, cache) || overlaps(out_y, state) || overlaps(cache, state))
    return AXON_ERR_INVALID_ARGUMENT;

  axon::DecodeLaunch a{};
  a.batch = Bsz;
  a.d_inner = E;
  a.act_bf16 = shape->act_dtype == AXON_BF16;
  a.x = x;
  a.z = z;
  a.dt_raw = dt_raw;
  a.B = B;
  a.C = C;
  a.A_log = params->A_log;
  a.D = params->D;
  a.dt_bias = params->dt_bias;
  a.conv_w = params->conv_w;
  a.conv_b = params->conv_b;
  a.dt_min = params->dt_min;
  a.dt_max = params->dt_max;
  a.conv_silu = params->conv_activation == AXON_CONV_SILU;
  a.zoh = params->discretization == AXON_DISC_ZOH;
  a.conv_cache = conv_cache;
  a.ssm_state = ssm_state;
  a.y = y;
  return axon::launch_decode(a, stream) == 0 ? AXON_OK : AXON_ERR_HIP;
}

}  // extern "C"
