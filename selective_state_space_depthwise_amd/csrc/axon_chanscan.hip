// Lane-per-channel selective scan for gfx950: a second prefill kernel family.
//
// What is computed is the Axon-SSM layer of "Axon-SSM: Selective State Space Model for Apple
// Silicon" (per-token formulas in axon_device.h): causal depthwise conv, dt, the diagonal
// recurrence h = exp(dt A) h + dt B u, the readout C . h + D u and the SiLU(z) gate.
//
// Work split. One lane owns one channel and all 16 of its states in registers, so nothing is
// exchanged between lanes: the conv window slides in the lane's registers, dt and dt*u are the
// lane's own, and the readout is summed in the lane. B_t and C_t (N values per token, shared by
// every channel of a batch row) are the same for every lane: a workgroup stages the rows of a
// tile of 64 tokens in LDS (widened to fp32), loaded from memory one tile ahead, and every lane
// reads a token's rows with broadcast LDS reads, so a state update is five plain VALU
// instructions (dt * rate, v_exp_f32, B * dtu, the fma into h, the fma of C * h into the
// readout) with no cross-lane broadcast and no reduction. A wave covers 64 consecutive channels,
// so every activation load and output store of a token is one contiguous run.
//
// A lane per channel gives only B * E / 64 waves, so the sequence is cut into M chunks (the
// two-level scan of the "State space duality" article's chunked associative scan): a carry pass
// scans chunks 0..M-2 from a zero state and keeps (sum of dt, final state) per chunk; the
// combine (axon_kernels.hip) folds the carries into each chunk's initial state; the final pass
// scans every chunk from its initial state and writes the outputs. With M = 1 only the final
// pass runs.
//
// Workgroups of the same (batch row, chunk) read the same B / C rows; blocks are handed to the
// eight XCDs round robin, so when the number of (batch row, chunk) groups is a multiple of 8 the
// block index is remapped to keep each group on one XCD (its rows are then fetched into one L2).
#include "axon_device.h"
#include "axon_internal.h"

namespace axon {
namespace {

constexpr int kChanBlock = 256;  // channels (lanes) per workgroup
constexpr int kUnroll = 8;       // tokens per step; a step's activations are loaded one step ahead

struct ChanArgs {
  int64_t B, L, E, T;    // T: tokens per chunk
  int64_t pass_chunks;   // chunks this launch covers (M - 1 for the carry pass, M for the final)
  int64_t cblocks;       // workgroups per (batch row, chunk) group
  int xcd_remap;
  const void *x, *z, *dt_raw, *Bm, *Cm;
  const float *A_log, *D, *dt_bias, *conv_w, *conv_b;
  float dt_min, dt_max;
  const float* win_src;   // (B, 3, E) conv inputs before token 0, or null (zeros)
  const float* h_src;     // initial states, chunk c at h_src + c * h_chunk_stride, or null
  int64_t h_chunk_stride;
  int64_t chunks;         // M
  void* y;
  float *state_out, *cache_out;
  float *carry_h, *carry_s;  // carry pass outputs: (M, B, E, N) and (M, B, E)
  float* halo;               // carry pass: copy of the incoming conv window (B, 3, E)
};

constexpr int kTile = 64;  // tokens per LDS tile of B / C rows (a multiple of kUnroll)

// A token's B (or C) row as four float4, read from LDS (the same address in every lane).
struct Row {
  float v[kState];
};
__device__ __forceinline__ void read_row(const float4* p, Row& r) {
#pragma unroll
  for (int q = 0; q < kState / 4; ++q) {
    const float4 f = p[q];
    r.v[4 * q] = f.x, r.v[4 * q + 1] = f.y, r.v[4 * q + 2] = f.z, r.v[4 * q + 3] = f.w;
  }
}

// Eight consecutive B or C values for the tile staging, widened to fp32.
__device__ __forceinline__ void load8(const float* p, float4& lo, float4& hi) {
  lo = reinterpret_cast<const float4*>(p)[0];
  hi = reinterpret_cast<const float4*>(p)[1];
}
__device__ __forceinline__ void load8(const bf16_bits* p, float4& lo, float4& hi) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  lo = make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u),
                   __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u));
  hi = make_float4(__uint_as_float(v.z << 16), __uint_as_float(v.z & 0xFFFF0000u),
                   __uint_as_float(v.w << 16), __uint_as_float(v.w & 0xFFFF0000u));
}

// Per-token values computed ahead of the state updates (for several tokens at once, so that
// their dependent chains of conv, softplus and gate overlap): dt, dt*u (u itself for the exact
// hold, which scales it per state), the gate SiLU(z) and the skip term D u.
struct Pre {
  float dt, du, g, q;
};

template <bool kFinal, bool kSilu, bool kZoh>
__device__ __forceinline__ void prologue_token(float xm3, float xm2, float xm1, float x0,
                                               float dr, float zv, float w0, float w1, float w2,
                                               float w3, float cb, float dtb, float Dv,
                                               float dt_min, float dt_max, Pre& p, float& S) {
  float u = fmaf(w3, x0, fmaf(w2, xm1, fmaf(w1, xm2, fmaf(w0, xm3, cb))));
  if constexpr (kSilu) u = silu(u);
  p.dt = step_size(dr + dtb, dt_min, dt_max);
  p.du = kZoh ? u : p.dt * u;
  if constexpr (kFinal) {
    p.g = silu(zv);
    p.q = Dv * u;
  } else {
    S += p.dt;
  }
}

// The 16 state updates of one token: B row in registers (read ahead), C row read from its
// staged copy at the start (final pass), used by the readout after the updates; returns the
// gated output. The readout is summed in two halves to halve its dependent chain, the skip term
// starting the second.
template <bool kFinal, bool kZoh>
__device__ __forceinline__ float update_token(const Row& rb, const float4* crow, const Pre& p,
                                              const float (&rate)[kState],
                                              const float (&ia)[kState], float (&h)[kState]) {
  Row rc;
  if constexpr (kFinal) read_row(crow, rc);
  if constexpr (!kZoh) {
#pragma unroll
    for (int n = 0; n < kState; ++n) {
      const float a = __builtin_amdgcn_exp2f(p.dt * rate[n]);
      h[n] = fmaf(a, h[n], rb.v[n] * p.du);
    }
  } else {
    // Exact zero-order hold: the input coefficient is expm1(dt A_n) / A_n, from the series of
    // expm1(x) / x for |x| < 0.25 and from the decay itself above (as in the row scan).
    constexpr float k1 = 0.34657359027997264f, k2 = 0.08007550231970023f;
    constexpr float k3 = 0.013876027166205392f, k4 = 0.0019236258215256953f;
    constexpr float thr = -0.36067376022224085f;
#pragma unroll
    for (int n = 0; n < kState; ++n) {
      const float yy = p.dt * rate[n];
      const float a = __builtin_amdgcn_exp2f(yy);
      const float phi = fmaf(yy, fmaf(yy, fmaf(yy, fmaf(yy, k4, k3), k2), k1), 1.0f);
      const float q = yy > thr ? p.dt * phi : (a - 1.0f) * ia[n];
      h[n] = fmaf(a, h[n], q * (rb.v[n] * p.du));
    }
  }
  if constexpr (kFinal) {
    float a0 = rc.v[0] * h[0], a1 = fmaf(rc.v[1], h[1], p.q);
#pragma unroll
    for (int n = 2; n < kState; n += 2) {
      a0 = fmaf(rc.v[n], h[n], a0);
      a1 = fmaf(rc.v[n + 1], h[n + 1], a1);
    }
    return (a0 + a1) * p.g;
  } else {
    return 0.0f;
  }
}

template <typename Act, bool kFinal, bool kSilu, bool kZoh>
__global__ __launch_bounds__(kChanBlock) __attribute__((amdgpu_waves_per_eu(kFinal ? 3 : 4))) void chan_scan_kernel(ChanArgs a) {
  // Block -> (group = (batch row, chunk), channel block).
  const int64_t w = blockIdx.x;
  int64_t g, cbk;
  if (a.xcd_remap) {
    const int64_t xcd = w % 8, k = w / 8;
    g = (k / a.cblocks) * 8 + xcd;
    cbk = k % a.cblocks;
  } else {
    g = w / a.cblocks;
    cbk = w % a.cblocks;
  }
  const int64_t chunk = g % a.pass_chunks;
  const int64_t b = g / a.pass_chunks;
  const int64_t e_raw = cbk * kChanBlock + threadIdx.x;
  const bool valid = e_raw < a.E;
  const int64_t e = valid ? e_raw : a.E - 1;  // lanes past the end mirror the last channel
  const int64_t L = a.L, E = a.E;
  const int64_t tb = chunk * a.T;
  const int64_t te = tb + a.T < L ? tb + a.T : L;

  const Act* __restrict__ Bp = static_cast<const Act*>(a.Bm) + b * L * kState;
  const Act* __restrict__ Cp = static_cast<const Act*>(a.Cm) + b * L * kState;
  // Activations of a step go through wave-uniform buffer resources at the step's first token:
  // token t + j of this lane's channel is at byte offset voff + soff[j]. Output stores use a
  // resource spanning the step's tokens; lanes past the last channel store at an offset outside
  // it, which the hardware drops (no branch per token).
  const Act* __restrict__ xrow = static_cast<const Act*>(a.x) + b * L * E;
  const Act* __restrict__ zrow = static_cast<const Act*>(a.z) + b * L * E;
  const Act* __restrict__ drow = static_cast<const Act*>(a.dt_raw) + b * L * E;
  Act* __restrict__ yrow = static_cast<Act*>(a.y) + b * L * E;
  const uint32_t voff = static_cast<uint32_t>(e * sizeof(Act));
  const uint32_t yoff = valid ? voff : kNoStore;
  const uint32_t tok_bytes = static_cast<uint32_t>(E * sizeof(Act));
  auto store_y1 = [&](int64_t tt, float v) {
    store_buf<Act>(make_rsrc_bounded(yrow + tt * E, tok_bytes), yoff, v);
  };

  float rate[kState], ia[kState], h[kState];
  {
    const float4* al = reinterpret_cast<const float4*>(a.A_log + e * kState);
#pragma unroll
    for (int q = 0; q < kState / 4; ++q) {
      const float4 v = al[q];
      const float lv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        rate[4 * q + i] = decay_rate_log2(lv[i]);
        ia[4 * q + i] = kZoh ? -expf(-lv[i]) : 0.0f;
      }
    }
  }
  if (kFinal && a.h_src) {
    const float4* hs =
        reinterpret_cast<const float4*>(a.h_src + chunk * a.h_chunk_stride + (b * E + e) * kState);
#pragma unroll
    for (int q = 0; q < kState / 4; ++q) {
      const float4 v = hs[q];
      h[4 * q] = v.x, h[4 * q + 1] = v.y, h[4 * q + 2] = v.z, h[4 * q + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int n = 0; n < kState; ++n) h[n] = 0.0f;
  }
  const float4 cw = *reinterpret_cast<const float4*>(a.conv_w + e * kConv);
  const float cb = a.conv_b[e], dtb = a.dt_bias[e], Dv = a.D[e];

  // Conv window: the three inputs before the chunk's first token.
  float xm3, xm2, xm1;
  if (tb == 0) {
    const float* ws = a.win_src ? a.win_src + b * kHalo * E + e : nullptr;
    xm3 = ws ? ws[0] : 0.0f;
    xm2 = ws ? ws[E] : 0.0f;
    xm1 = ws ? ws[2 * E] : 0.0f;
    if (!kFinal && valid) {
      // Keep a copy of the incoming window for the final pass, so that the caller may update
      // the conv cache in place.
      float* hl = a.halo + b * kHalo * E + e;
      hl[0] = xm3;
      hl[E] = xm2;
      hl[2 * E] = xm1;
    }
  } else {
    xm3 = load_buf<Act>(make_rsrc(xrow + (tb - 3) * E), voff);
    xm2 = load_buf<Act>(make_rsrc(xrow + (tb - 2) * E), voff);
    xm1 = load_buf<Act>(make_rsrc(xrow + (tb - 1) * E), voff);
  }

  // B / C rows of a tile of kTile tokens, double-buffered: 128 bytes per token (B in float4 0..3,
  // C in 4..7). Thread i stages 8 values of token i / 4: B (i % 4 = 0, 1) or C (2, 3).
  __shared__ float4 s_rows[2][kTile][8];
  const int nt = static_cast<int>(te - tb);
  const int ntiles = (nt + kTile - 1) / kTile;
  const int st_tok = threadIdx.x / 4, st_part = threadIdx.x % 4;
  const bool st_on = kFinal || st_part < 2;  // the carry pass needs only B
  float4 pre_lo = make_float4(0.f, 0.f, 0.f, 0.f), pre_hi = pre_lo;
  auto stage_load = [&](int k) {
    int64_t tt = tb + static_cast<int64_t>(k) * kTile + st_tok;
    tt = tt < L ? tt : L - 1;
    const Act* src = (st_part < 2 ? Bp : Cp) + tt * kState + (st_part & 1) * 8;
    if (st_on) load8(src, pre_lo, pre_hi);
  };
  auto stage_store = [&](int buf) {
    if (st_on) {
      s_rows[buf][st_tok][2 * st_part] = pre_lo;
      s_rows[buf][st_tok][2 * st_part + 1] = pre_hi;
    }
  };
  stage_load(0);
  stage_store(0);
  __syncthreads();
  if (ntiles > 1) stage_load(1);

  float S = 0.0f;
  int t = 0;  // token index within the chunk
  // Steps of kUnroll tokens in two halves: the prologue of a half's four tokens, then their
  // state updates one token at a time. Each activation slot is reloaded with the next step's
  // token as soon as its prologue has consumed it (loads run kUnroll tokens ahead). The
  // scheduling barriers keep each token's LDS reads and stores in its own region.
  // The slots hold the raw loaded bits (bf16 is widened where the prologue reads it): a widening
  // next to the load would sit inside the load's scheduling region and wait for its data.
  uint32_t nx[kUnroll], nd[kUnroll], nz[kUnroll];
  auto slot_load = [&](rsrc_t rx, rsrc_t rd, rsrc_t rz, int j) {
    nx[j] = load_raw_s<Act>(rx, voff, j * tok_bytes);
    nd[j] = load_raw_s<Act>(rd, voff, j * tok_bytes);
    if constexpr (kFinal) nz[j] = load_raw_s<Act>(rz, voff, j * tok_bytes);
  };
  if (kUnroll <= nt) {
    const rsrc_t rx = make_rsrc(xrow + tb * E), rd = make_rsrc(drow + tb * E);
    const rsrc_t rz = make_rsrc(zrow + tb * E);
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) slot_load(rx, rd, rz, j);
  }
  for (int k = 0; k < ntiles; ++k) {
    const int buf = k & 1;
    const int t_end = (k + 1) * kTile < nt ? (k + 1) * kTile : nt;
    for (; t + kUnroll <= t_end; t += kUnroll) {
      // The next step's tokens (clamped to a whole step inside the chunk: loads past a partial
      // last step are never used).
      const int64_t tn = tb + (t + 2 * kUnroll <= nt ? t + kUnroll : nt - kUnroll);
      const rsrc_t rx = make_rsrc(xrow + tn * E), rd = make_rsrc(drow + tn * E);
      const rsrc_t rz = make_rsrc(zrow + tn * E);
      const rsrc_t ry = make_rsrc_bounded(yrow + (tb + t) * E, kUnroll * tok_bytes);
      const int row0 = t - k * kTile;
      Row rb_next;
#pragma unroll
      for (int half = 0; half < kUnroll / 4; ++half) {
        Pre pre[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = 4 * half + i;
          const float x0 = raw_to_f32<Act>(nx[j]);
          prologue_token<kFinal, kSilu, kZoh>(xm3, xm2, xm1, x0, raw_to_f32<Act>(nd[j]),
                                              kFinal ? raw_to_f32<Act>(nz[j]) : 0.0f, cw.x, cw.y,
                                              cw.z, cw.w, cb,
                                              dtb, Dv, a.dt_min, a.dt_max, pre[i], S);
          xm3 = xm2;
          xm2 = xm1;
          xm1 = x0;
          slot_load(rx, rd, rz, j);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = 4 * half + i;
          // B of this token was read by the token before it (the step's first token reads its
          // own); B of the next token of the step is read now, to arrive during the updates.
          if (j == 0) read_row(&s_rows[buf][row0][0], rb_next);
          const Row rb = rb_next;
          if (j + 1 < kUnroll) read_row(&s_rows[buf][row0 + j + 1][0], rb_next);
          const float yv = update_token<kFinal, kZoh>(rb, &s_rows[buf][row0 + j][4], pre[i], rate,
                                                      ia, h);
          if constexpr (kFinal) store_buf_s<Act>(ry, yoff, j * tok_bytes, yv);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // The chunk's last (fewer than kUnroll) tokens, one at a time.
    for (; t < t_end; ++t) {
      const int64_t tt = tb + t;
      const float x0 = load_buf<Act>(make_rsrc(xrow + tt * E), voff);
      const float dr = load_buf<Act>(make_rsrc(drow + tt * E), voff);
      const float zv = kFinal ? load_buf<Act>(make_rsrc(zrow + tt * E), voff) : 0.0f;
      Pre pre;
      prologue_token<kFinal, kSilu, kZoh>(xm3, xm2, xm1, x0, dr, zv, cw.x, cw.y, cw.z, cw.w, cb,
                                          dtb, Dv, a.dt_min, a.dt_max, pre, S);
      Row rb;
      read_row(&s_rows[buf][t - k * kTile][0], rb);
      const float yv =
          update_token<kFinal, kZoh>(rb, &s_rows[buf][t - k * kTile][4], pre, rate, ia, h);
      if constexpr (kFinal) store_y1(tt, yv);
      xm3 = xm2;
      xm2 = xm1;
      xm1 = x0;
    }
    if (k + 1 < ntiles) {
      stage_store(buf ^ 1);
      __syncthreads();
      if (k + 2 < ntiles) stage_load(k + 2);
    }
  }

  if (!valid) return;
  if constexpr (!kFinal) {
    const int64_t be = (chunk * a.B + b) * E + e;
    float4* ch = reinterpret_cast<float4*>(a.carry_h + be * kState);
#pragma unroll
    for (int q = 0; q < kState / 4; ++q)
      ch[q] = make_float4(h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]);
    a.carry_s[be] = S;
  } else if (chunk == a.chunks - 1) {
    float4* so = reinterpret_cast<float4*>(a.state_out + (b * E + e) * kState);
#pragma unroll
    for (int q = 0; q < kState / 4; ++q)
      so[q] = make_float4(h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]);
    // The window now holds the last three inputs of [conv window, x] (te = L here).
    a.cache_out[(b * kHalo + 0) * E + e] = xm3;
    a.cache_out[(b * kHalo + 1) * E + e] = xm2;
    a.cache_out[(b * kHalo + 2) * E + e] = xm1;
  }
}

}  // namespace

void launch_carry_combine(int64_t B, int64_t E, int64_t M, const float* A_log,
                          const float* state_in, const float* carry_h, const float* carry_s,
                          float* carry_in, hipStream_t s);

template <typename Act, bool kSilu, bool kZoh>
int launch_chan_scan_t(const PrefillLaunch& p, const PrefillPlan& plan, hipStream_t s) {
  ChanArgs a{};
  a.B = p.batch;
  a.L = p.seqlen;
  a.E = p.d_inner;
  a.T = plan.chunk_len;
  a.chunks = plan.chunks;
  a.cblocks = (p.d_inner + kChanBlock - 1) / kChanBlock;
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
  a.win_src = p.conv_cache_in;
  a.y = p.y;
  a.state_out = p.ssm_state_out;
  a.cache_out = p.conv_cache_out;
  const dim3 block(kChanBlock);
  auto grid_for = [&](int64_t pass_chunks) {
    a.pass_chunks = pass_chunks;
    const int64_t groups = pass_chunks * p.batch;
    a.xcd_remap = groups % 8 == 0 ? 1 : 0;
    return dim3(static_cast<unsigned>(groups * a.cblocks));
  };
  if (plan.chunks == 1) {
    a.h_src = p.ssm_state_in;
    a.h_chunk_stride = 0;
    hipLaunchKernelGGL((chan_scan_kernel<Act, true, kSilu, kZoh>), grid_for(1), block, 0, s, a);
    return static_cast<int>(hipGetLastError());
  }
  char* ws = static_cast<char*>(p.workspace);
  a.carry_h = reinterpret_cast<float*>(ws + plan.off_carry_h);
  a.carry_s = reinterpret_cast<float*>(ws + plan.off_carry_s);
  a.halo = reinterpret_cast<float*>(ws + plan.off_halo);
  float* carry_in = reinterpret_cast<float*>(ws + plan.off_carry_in);
  a.h_src = nullptr;
  hipLaunchKernelGGL((chan_scan_kernel<Act, false, kSilu, kZoh>), grid_for(plan.chunks - 1),
                     block, 0, s, a);
  launch_carry_combine(p.batch, p.d_inner, plan.chunks, p.A_log, p.ssm_state_in, a.carry_h,
                       a.carry_s, carry_in, s);
  // In the final pass chunk 0 reads the window while the last chunk's lanes write the conv cache
  // out, in no set order within the launch; it therefore reads the carry pass's copy.
  a.win_src = a.halo;
  a.h_src = carry_in;
  a.h_chunk_stride = p.batch * p.d_inner * kState;
  hipLaunchKernelGGL((chan_scan_kernel<Act, true, kSilu, kZoh>), grid_for(plan.chunks), block, 0,
                     s, a);
  return static_cast<int>(hipGetLastError());
}

template <typename Act>
int launch_chan_scan_v(const PrefillLaunch& p, const PrefillPlan& plan, hipStream_t s) {
  if (p.conv_silu)
    return p.zoh ? launch_chan_scan_t<Act, true, true>(p, plan, s)
                 : launch_chan_scan_t<Act, true, false>(p, plan, s);
  return p.zoh ? launch_chan_scan_t<Act, false, true>(p, plan, s)
               : launch_chan_scan_t<Act, false, false>(p, plan, s);
}

int launch_chan_scan(const PrefillLaunch& p, const PrefillPlan& plan, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  return p.act_bf16 ? launch_chan_scan_v<bf16_bits>(p, plan, s)
                    : launch_chan_scan_v<float>(p, plan, s);
}

}  // namespace axon
