// Row-split selective scan for gfx950: the prefill kernel.
//
// What is computed is the Axon-SSM layer of "Axon-SSM: Selective State Space Model for Apple
// Silicon" (per-token formulas in axon_device.h): causal depthwise conv, dt, the diagonal
// recurrence h = exp(dt A) h + dt B u, the readout C . h + D u and the SiLU(z) gate.
//
// Work split. A wave covers 16 channels (lane column c = lane % 16) and 4 lane rows
// (q = lane / 16); W waves share the same 16 channels, so a channel's 16 states are spread over
// the 4*W (row, wave) pairs, SPL = 4 / W states per lane. Shapes with few channels (1 x 7680) use
// W = 4: one state per lane and two waves per SIMD, without cutting the sequence into chunks
// (which would cost a second pass of exponentials); every exp(dt A) is evaluated exactly once.
//
// Per token and lane the state update is 5 VALU instructions per state: dt * rate, exp2, the
// input dtu * B (B broadcast within the lane row by DPP row_newbcast from a register holding
// 16 / SPL tokens x SPL states of B), the fma into h, and the readout product C * h (C broadcast
// the same way). The products of 4 tokens are summed over the 4 lane rows by a transpose-reduce
// with v_permlane32_swap / v_permlane16_swap (6 VALU instructions per 4 tokens), which leaves
// token 4k + q of the wave's partial output in row q of register R_k. The W waves add their
// partials through LDS; the wave that computed a token's prologue finishes it (skip term, gate,
// store).
//
// Per (token, channel) the prologue computes u (conv) and dt once and shares (dt, dt*u) through
// LDS. Inputs are prefetched into registers two tiles ahead.
//
// Inline assembly holds only VALU instructions (no memory access). Hazards are handled by
// instruction order: in every block at least two VALU instructions of the block precede the first
// DPP instruction, so every operand of a DPP instruction was written two or more instructions
// earlier whatever the compiler placed before the block; every v_exp result is consumed at least
// one instruction later. A token's readout products are computed one block late, so the state they
// read is old enough for DPP; the products of a tile's last token are taken after an s_nop 1, and
// that block ends with an s_nop 1 before any instruction the compiler places after it.
#include <type_traits>

#include "axon_device.h"
#include "axon_internal.h"

namespace axon {
namespace {

// 16-channel groups per workgroup. One where a lane holds one state: four-wave workgroups, two
// per CU, so the two waves of a SIMD belong to workgroups that meet their barriers independently
// (1 x 2048 x 7680 fp32: 1-1.5% faster per launch than two groups, 4% with inputs in the
// last-level cache). Two otherwise (8 x 4096 x 7680 bf16 with one group: 7% slower).
template <int W>
constexpr int groups() {
  return W == 4 ? 1 : 2;
}

// The wave's slot on its SIMD (bits 3:0 of the HW_ID hardware register).
__device__ __forceinline__ int wave_slot() {
  return static_cast<int>(__builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 4));
}

// Tokens per tile: 32 where a lane holds one state (more work between barriers), 16 otherwise
// (the register budget of 4 states per lane).
template <int W>
constexpr int tile_tokens() {
  return W == 4 ? 32 : 16;
}

struct RowArgs {
  int64_t B, L, E, T;
  int xcd_remap;  // gridDim.x is a multiple of 8: keep neighbouring channel blocks on one XCD
  const void *x, *z, *dt_raw, *Bm, *Cm;
  const float *A_log, *D, *dt_bias, *conv_w, *conv_b;
  float dt_min, dt_max;
  const float* win_src;     // (B, 3, E) conv inputs before token 0, or null (zeros)
  const float* h_src;       // initial states (see h_chunk_stride), or null (zeros)
  int64_t h_chunk_stride;   // elements between chunks in h_src
  int64_t chunks;
  void* y;
  float *state_out, *cache_out;
  float *carry_h, *carry_s, *halo;
};

// ---- token step ------------------------------------------------------------------------------
// Block for token tau, in this order:
//   A  an_i = dtn * rate_i             (decay argument of token tau+1, if any)
//   D  an_i = exp2(an_i)
//   B  b_i = dtu * bcast(RB, k_i)
//   C  pp_i = bcast(RCp, kp_i) * h_i   (readout products of token tau-1: h is its state)
//   E  b_i += a_i * h_i                (a: token tau's decay from the previous block; b is the
//                                       new state)
// Computing the decays one block ahead keeps the exp2 latency off the state chain.

#define AXON_BC(dst, src, mul, k)                                                             \
  "v_mul_f32_dpp %[" #dst "], %[" #src "], %[" #mul "] row_newbcast:%[" #k                   \
  "] row_mask:0xf bank_mask:0xf\n\t"
#define AXON_A1(i) "v_mul_f32 %[n" #i "], %[dtn], %[r" #i "]\n\t"
#define AXON_D1(i) "v_exp_f32 %[n" #i "], %[n" #i "]\n\t"
#define AXON_E1(i) "v_fmac_f32 %[b" #i "], %[a" #i "], %[h" #i "]\n\t"

#define AXON_AD1 AXON_A1(0) AXON_D1(0)
#define AXON_AD2 AXON_A1(0) AXON_A1(1) AXON_D1(0) AXON_D1(1)
#define AXON_AD4 AXON_A1(0) AXON_A1(1) AXON_A1(2) AXON_A1(3) AXON_D1(0) AXON_D1(1) AXON_D1(2) AXON_D1(3)
#define AXON_B1 AXON_BC(b0, RB, dtu, k0)
#define AXON_B2 AXON_BC(b0, RB, dtu, k0) AXON_BC(b1, RB, dtu, k1)
#define AXON_B4 AXON_BC(b0, RB, dtu, k0) AXON_BC(b1, RB, dtu, k1) AXON_BC(b2, RB, dtu, k2) AXON_BC(b3, RB, dtu, k3)
// Readout products of the previous token, summed in the lane: C multiplies the first state of
// each pair, CF adds the second with a DPP fmac after the block's state fmacs (so the fmac's
// accumulator is two instructions old). SPL = 4 keeps two partial sums (states 0 + 1, 2 + 3).
#define AXON_BCF(dst, src, mul, k)                                                            \
  "v_fmac_f32_dpp %[" #dst "], %[" #src "], %[" #mul "] row_newbcast:%[" #k                  \
  "] row_mask:0xf bank_mask:0xf\n\t"
#define AXON_C1 AXON_BC(p0, RCp, h0, kp0)
#define AXON_C2 AXON_BC(p0, RCp, h0, kp0)
#define AXON_C4 AXON_BC(p0, RCp, h0, kp0) AXON_BC(p1, RCp, h2, kp2)
#define AXON_CF1
#define AXON_CF2 AXON_BCF(p0, RCp, h1, kp1)
#define AXON_CF4 AXON_BCF(p0, RCp, h1, kp1) AXON_BCF(p1, RCp, h3, kp3)
#define AXON_E1S AXON_E1(0)
#define AXON_E2S AXON_E1(0) AXON_E1(1)
#define AXON_E4S AXON_E1(0) AXON_E1(1) AXON_E1(2) AXON_E1(3)

#define AXON_OUTB1 [b0] "=&v"(b[0])
#define AXON_OUTB2 [b0] "=&v"(b[0]), [b1] "=&v"(b[1])
#define AXON_OUTB4 [b0] "=&v"(b[0]), [b1] "=&v"(b[1]), [b2] "=&v"(b[2]), [b3] "=&v"(b[3])
#define AXON_OUTN1 , [n0] "=&v"(an[0])
#define AXON_OUTN2 , [n0] "=&v"(an[0]), [n1] "=&v"(an[1])
#define AXON_OUTN4 , [n0] "=&v"(an[0]), [n1] "=&v"(an[1]), [n2] "=&v"(an[2]), [n3] "=&v"(an[3])
#define AXON_OUTP1 , [p0] "=&v"(pp[0])
#define AXON_OUTP2 , [p0] "=&v"(pp[0])
#define AXON_OUTP4 , [p0] "=&v"(pp[0]), [p1] "=&v"(pp[1])
#define AXON_IN_COMMON [dtn] "v"(dtn), [dtu] "v"(dtu), [RB] "v"(RB), [RCp] "v"(RCp)
#define AXON_IN1 , [r0] "v"(r[0]), [a0] "v"(ac[0]), [h0] "v"(h[0]), [k0] "i"(K), [kp0] "i"(KP)
#define AXON_IN2                                                                          \
  , [r0] "v"(r[0]), [r1] "v"(r[1]), [a0] "v"(ac[0]), [a1] "v"(ac[1]), [h0] "v"(h[0]),    \
      [h1] "v"(h[1]), [k0] "i"(K), [k1] "i"(K + 1), [kp0] "i"(KP), [kp1] "i"(KP + 1)
#define AXON_IN4                                                                              \
  , [r0] "v"(r[0]), [r1] "v"(r[1]), [r2] "v"(r[2]), [r3] "v"(r[3]), [a0] "v"(ac[0]),         \
      [a1] "v"(ac[1]), [a2] "v"(ac[2]), [a3] "v"(ac[3]), [h0] "v"(h[0]), [h1] "v"(h[1]),     \
      [h2] "v"(h[2]), [h3] "v"(h[3]), [k0] "i"(K), [k1] "i"(K + 1), [k2] "i"(K + 2),         \
      [k3] "i"(K + 3), [kp0] "i"(KP), [kp1] "i"(KP + 1), [kp2] "i"(KP + 2), [kp3] "i"(KP + 3)

// One token. ac: this token's decays; an (out, kNext): the next token's decays from dtn.
// kPrev: also the readout products of the previous token. Every block starts with two or more
// VALU instructions before its first DPP instruction (the A/D pair, or an s_nop 1 without it).
template <int SPL, int K, int KP, bool kPrev, bool kNext>
__device__ __forceinline__ void step(float dtn, float dtu, const float (&r)[SPL],
                                     const float (&ac)[SPL], float RB, float RCp,
                                     float (&h)[SPL], float (&an)[SPL], float (&pp)[SPL]) {
  float b[SPL];
#define AXON_STEP(N)                                                                            \
  if constexpr (kNext && kPrev)                                                                 \
    asm(AXON_AD##N AXON_B##N AXON_C##N AXON_E##N##S AXON_CF##N                                  \
        : AXON_OUTB##N AXON_OUTN##N AXON_OUTP##N : AXON_IN_COMMON AXON_IN##N);                  \
  else if constexpr (kNext)                                                                     \
    asm(AXON_AD##N AXON_B##N AXON_E##N##S : AXON_OUTB##N AXON_OUTN##N : AXON_IN_COMMON AXON_IN##N); \
  else if constexpr (kPrev)                                                                     \
    asm("s_nop 1\n\t" AXON_B##N AXON_C##N AXON_E##N##S AXON_CF##N                               \
        : AXON_OUTB##N AXON_OUTP##N : AXON_IN_COMMON AXON_IN##N);                               \
  else                                                                                          \
    asm("s_nop 1\n\t" AXON_B##N AXON_E##N##S : AXON_OUTB##N : AXON_IN_COMMON AXON_IN##N);
  if constexpr (SPL == 1) {
    AXON_STEP(1)
  } else if constexpr (SPL == 2) {
    AXON_STEP(2)
  } else {
    AXON_STEP(4)
  }
#undef AXON_STEP
#pragma unroll
  for (int i = 0; i < SPL; ++i) h[i] = b[i];
}

// Decays of a tile's first token: exp2(dt * rate), in a block of its own.
template <int SPL>
__device__ __forceinline__ void first_decay(float dtn, const float (&r)[SPL], float (&an)[SPL]) {
  if constexpr (SPL == 1) {
    asm(AXON_AD1 : [n0] "=&v"(an[0]) : [dtn] "v"(dtn), [r0] "v"(r[0]));
  } else if constexpr (SPL == 2) {
    asm(AXON_AD2 : [n0] "=&v"(an[0]), [n1] "=&v"(an[1]) : [dtn] "v"(dtn), [r0] "v"(r[0]), [r1] "v"(r[1]));
  } else {
    asm(AXON_AD4
        : [n0] "=&v"(an[0]), [n1] "=&v"(an[1]), [n2] "=&v"(an[2]), [n3] "=&v"(an[3])
        : [dtn] "v"(dtn), [r0] "v"(r[0]), [r1] "v"(r[1]), [r2] "v"(r[2]), [r3] "v"(r[3]));
  }
}

// Readout products of a tile's last token (its state was written by the block just before).
template <int SPL, int KP>
__device__ __forceinline__ void flush(float RCp, const float (&h)[SPL], float (&pp)[SPL]) {
  if constexpr (SPL == 1) {
    asm("s_nop 1\n\t" AXON_C1 "s_nop 1"
        : [p0] "=&v"(pp[0]) : [RCp] "v"(RCp), [h0] "v"(h[0]), [kp0] "i"(KP));
  } else if constexpr (SPL == 2) {
    asm("s_nop 1\n\t" AXON_C2 "s_nop 0\n\t" AXON_CF2 "s_nop 1"
        : [p0] "=&v"(pp[0])
        : [RCp] "v"(RCp), [h0] "v"(h[0]), [h1] "v"(h[1]), [kp0] "i"(KP), [kp1] "i"(KP + 1));
  } else {
    asm("s_nop 1\n\t" AXON_C4 AXON_CF4 "s_nop 1"
        : [p0] "=&v"(pp[0]), [p1] "=&v"(pp[1])
        : [RCp] "v"(RCp), [h0] "v"(h[0]), [h1] "v"(h[1]), [h2] "v"(h[2]), [h3] "v"(h[3]),
          [kp0] "i"(KP), [kp1] "i"(KP + 1), [kp2] "i"(KP + 2), [kp3] "i"(KP + 3));
  }
}

// The lane's readout of one token from the block's (or flush's) pre-summed products.
template <int SPL>
__device__ __forceinline__ float readout_sum(const float (&pp)[SPL]) {
  if constexpr (SPL == 4) return pp[0] + pp[1];
  return pp[0];
}

template <int SPL>
__device__ __forceinline__ float lane_sum(const float (&pp)[SPL]) {
  float p = pp[0];
#pragma unroll
  for (int i = 1; i < SPL; ++i) p += pp[i];
  return p;
}

// The tokens of a tile. RB[j] / RC[j] hold B / C of tokens j*16/SPL .. (j+1)*16/SPL - 1 for
// this row's SPL states (lane position tau_local * SPL + i). dd holds (dt, dt*u) of the tile's
// tokens for this lane's channel, two tokens per float4. P[tau] receives the lane's readout
// product of token tau; ac carries the current token's decays from block to block.
template <int SPL, bool kCarry, int TAU, int kTile>
__device__ __forceinline__ void scan_tile_from(const float4 (&dd)[kTile / 2],
                                               const float (&rate)[SPL],
                                               const float (&RB)[kTile * SPL / 16],
                                               const float (&RC)[kTile * SPL / 16],
                                               float (&h)[SPL], float (&ac)[SPL],
                                               float (&P)[kTile], float& S) {
  constexpr int TPR = 16 / SPL;  // tokens per broadcast register
  constexpr int J = TAU / TPR;
  constexpr int K = (TAU % TPR) * SPL;
  constexpr int JP = (TAU > 0 ? TAU - 1 : 0) / TPR;
  constexpr int KP = ((TAU > 0 ? TAU - 1 : 0) % TPR) * SPL;
  constexpr int TN = TAU + 1 < kTile ? TAU + 1 : TAU;
  const float dtu = (TAU & 1) ? dd[TAU / 2].w : dd[TAU / 2].y;
  const float dtn = (TN & 1) ? dd[TN / 2].z : dd[TN / 2].x;
  if constexpr (TAU == 0) {
    const float dt0 = dd[0].x;
    first_decay<SPL>(dt0, rate, ac);
    if constexpr (kCarry) S += dt0;
  }
  if constexpr (kCarry && TAU + 1 < kTile) S += dtn;
  float pp[SPL], an[SPL];
  constexpr bool kPrev = !kCarry && TAU >= 1;
  constexpr bool kNext = TAU + 1 < kTile;
  step<SPL, K, KP, kPrev, kNext>(dtn, dtu, rate, ac, RB[J], RC[JP], h, an, pp);
  if constexpr (kPrev) P[TAU - 1] = readout_sum<SPL>(pp);
  if constexpr (kNext) {
#pragma unroll
    for (int i = 0; i < SPL; ++i) ac[i] = an[i];
    scan_tile_from<SPL, kCarry, TAU + 1, kTile>(dd, rate, RB, RC, h, ac, P, S);
  } else if constexpr (!kCarry) {
    flush<SPL, ((kTile - 1) % TPR) * SPL>(RC[kTile * SPL / 16 - 1], h, pp);
    P[kTile - 1] = readout_sum<SPL>(pp);
  }
}

// ---- exact zero-order hold (variant) ---------------------------------------------------------
// The input coefficient of a state becomes expm1(x) / A with x = dt A <= 0 instead of dt. With
// y = x / ln 2 (the exp2 argument the decay already needs):
//   |x| <  0.25: dt * phi, phi = expm1(x) / x = 1 + y (k1 + y (k2 + y (k3 + y k4))),
//                k_j = ln2^j / (j + 1)! (the series cut after x^4: relative error < 1.4e-6);
//   |x| >= 0.25: (a - 1) / A with a = exp(x), the decay itself (a - 1 no longer cancels).
struct ZohConst {
  float k1 = 0.34657359027997264f;    // ln 2 / 2
  float k2 = 0.08007550231970023f;    // ln^2 2 / 6
  float k3 = 0.013876027166205392f;   // ln^3 2 / 24
  float k4 = 0.0019236258215256953f;  // ln^4 2 / 120
  float thr = -0.36067376022224085f;  // y at x = -0.25
};

// One state of one token, exact zero-order hold, in this order:
//   A  yn = dtn * rate, D  an = exp2(yn)        (next token's argument and decay, if any)
//   P  p = dtc * phi(yc)                        (small-|x| coefficient of this token)
//   Q  q = (ac - 1) / A, q = yc > thr ? p : q   (large-|x| coefficient, then the choice)
//   B  b = bcast(RB, K) * uc                    (B of this token times its u)
//   C  pp = bcast(RCp, KP) * h                  (readout product of the previous token)
//   E  b = b * q + ac * h                       (the new state)
// At least eight VALU instructions precede the first DPP instruction of the block.
#define AXON_ZA "v_mul_f32 %[yn], %[dtn], %[r]\n\tv_exp_f32 %[an], %[yn]\n\t"
#define AXON_ZP                                                                              \
  "v_fma_f32 %[p], %[yc], %[k4], %[k3]\n\tv_fma_f32 %[p], %[yc], %[p], %[k2]\n\t"            \
  "v_fma_f32 %[p], %[yc], %[p], %[k1]\n\tv_fma_f32 %[p], %[yc], %[p], 1.0\n\t"               \
  "v_mul_f32 %[p], %[p], %[dtc]\n\t"                                                         \
  "v_fma_f32 %[q], %[ac], %[ia], -%[ia]\n\tv_cmp_lt_f32 vcc, %[thr], %[yc]\n\t"              \
  "v_cndmask_b32 %[q], %[q], %[p], vcc\n\t"
#define AXON_ZB AXON_BC(b, RB, uc, k)
#define AXON_ZC AXON_BC(pp, RCp, h, kp)
#define AXON_ZE "v_mul_f32 %[b], %[b], %[q]\n\tv_fmac_f32 %[b], %[ac], %[h]\n\t"
#define AXON_ZOUT [b] "=&v"(b), [an] "=&v"(an), [yn] "=&v"(yn), [pp] "=&v"(pp), [p] "=&v"(p), \
                  [q] "=&v"(q)
#define AXON_ZIN                                                                             \
  [dtn] "v"(dtn), [dtc] "v"(dtc), [uc] "v"(uc), [RB] "v"(RB), [RCp] "v"(RCp), [k1] "v"(zc.k1), \
      [k2] "v"(zc.k2), [k3] "v"(zc.k3), [k4] "v"(zc.k4), [thr] "v"(zc.thr), [r] "v"(r),        \
      [ac] "v"(ac), [yc] "v"(yc), [ia] "v"(ia), [h] "v"(h), [k] "i"(K), [kp] "i"(KP)

template <int K, int KP, bool kPrev, bool kNext>
__device__ __forceinline__ void step_zoh(float dtn, float dtc, float uc, float r, float ac,
                                         float yc, float ia, float RB, float RCp,
                                         const ZohConst& zc, float& h, float& an, float& yn,
                                         float& pp) {
  float b, p, q;
  if constexpr (kNext && kPrev)
    asm(AXON_ZA AXON_ZP AXON_ZB AXON_ZC AXON_ZE : AXON_ZOUT : AXON_ZIN : "vcc");
  else if constexpr (kNext)
    asm(AXON_ZA AXON_ZP AXON_ZB AXON_ZE : AXON_ZOUT : AXON_ZIN : "vcc");
  else if constexpr (kPrev)
    asm(AXON_ZP AXON_ZB AXON_ZC AXON_ZE : AXON_ZOUT : AXON_ZIN : "vcc");
  else
    asm(AXON_ZP AXON_ZB AXON_ZE : AXON_ZOUT : AXON_ZIN : "vcc");
  h = b;
}

// The tokens of a tile with the exact zero-order hold: as scan_tile_from, with dd holding
// (dt, u) pairs and the arguments yc carried from block to block beside the decays ac.
template <int SPL, bool kCarry, int TAU, int kTile>
__device__ __forceinline__ void scan_tile_zoh_from(
    const float4 (&dd)[kTile / 2], const float (&rate)[SPL], const float (&ia)[SPL],
    const ZohConst& zc, const float (&RB)[kTile * SPL / 16], const float (&RC)[kTile * SPL / 16],
    float (&h)[SPL], float (&ac)[SPL], float (&yc)[SPL], float (&P)[kTile], float& S) {
  constexpr int TPR = 16 / SPL;
  constexpr int J = TAU / TPR;
  constexpr int K = (TAU % TPR) * SPL;
  constexpr int JP = (TAU > 0 ? TAU - 1 : 0) / TPR;
  constexpr int KP = ((TAU > 0 ? TAU - 1 : 0) % TPR) * SPL;
  constexpr int TN = TAU + 1 < kTile ? TAU + 1 : TAU;
  const float dtc = (TAU & 1) ? dd[TAU / 2].z : dd[TAU / 2].x;
  const float uc = (TAU & 1) ? dd[TAU / 2].w : dd[TAU / 2].y;
  const float dtn = (TN & 1) ? dd[TN / 2].z : dd[TN / 2].x;
  if constexpr (TAU == 0) {
#pragma unroll
    for (int i = 0; i < SPL; ++i)
      asm("v_mul_f32 %[y], %[dt], %[r]\n\tv_exp_f32 %[a], %[y]"
          : [y] "=&v"(yc[i]), [a] "=&v"(ac[i]) : [dt] "v"(dtc), [r] "v"(rate[i]));
    if constexpr (kCarry) S += dtc;
  }
  if constexpr (kCarry && TAU + 1 < kTile) S += dtn;
  constexpr bool kPrev = !kCarry && TAU >= 1;
  constexpr bool kNext = TAU + 1 < kTile;
  float an[SPL], yn[SPL], pp[SPL];
  step_zoh<K, KP, kPrev, kNext>(dtn, dtc, uc, rate[0], ac[0], yc[0], ia[0], RB[J], RC[JP], zc,
                                h[0], an[0], yn[0], pp[0]);
  if constexpr (SPL == 2)
    step_zoh<K + 1, KP + 1, kPrev, kNext>(dtn, dtc, uc, rate[1], ac[1], yc[1], ia[1], RB[J],
                                          RC[JP], zc, h[1], an[1], yn[1], pp[1]);
  if constexpr (kPrev) P[TAU - 1] = lane_sum<SPL>(pp);
  if constexpr (kNext) {
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
      ac[i] = an[i];
      yc[i] = yn[i];
    }
    scan_tile_zoh_from<SPL, kCarry, TAU + 1, kTile>(dd, rate, ia, zc, RB, RC, h, ac, yc, P, S);
  } else if constexpr (!kCarry) {
    flush<SPL, ((kTile - 1) % TPR) * SPL>(RC[kTile * SPL / 16 - 1], h, pp);
    P[kTile - 1] = readout_sum<SPL>(pp);
  }
}

// Sum of four tokens' products over the 4 lane rows: on return, row q holds token q's sum.
__device__ __forceinline__ float rows_reduce4(float p0, float p1, float p2, float p3) {
  const auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p2),
                                                    false, false);
  const auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p1), __float_as_uint(p3),
                                                    false, false);
  const float a = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);
  const float b = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Inputs of one tile for this lane, loaded ahead of use. The lane's prologue / epilogue tokens
// are TPL consecutive ones, tau0 .. tau0 + TPL - 1 with tau0 = (4 w + q) TPL, so its conv window
// is TPL + 3 inputs. B / C registers are laid out as scan_tile_from reads them. The registers
// hold the loaded bits (bf16: zero-extended), widened to fp32 only where they are used, so a
// load in flight is never copied or waited for before its use.
template <int TPL, int NR, typename Raw>
struct TileIn {
  Raw xw[TPL + 3];  // x at tau0 - 3 .. tau0 + TPL - 1 (tile 0: unused, see x0)
  Raw dr[TPL];
  Raw zz[TPL];
  Raw RB[NR], RC[NR];
};

// kSilu: SiLU on the convolution output (Mamba-block variant); kZoh: exact zero-order hold.
// The two-states-per-lane final pass fits 128 VGPRs with no spill in its loop, which gives
// it 4 waves per SIMD instead of 3.
template <typename Act, int W, bool kCarry, bool kSilu, bool kZoh>
__global__ __launch_bounds__(64 * W * groups<W>()) __attribute__((
    amdgpu_waves_per_eu(W == 2 && !kCarry && !kZoh ? 4 : 1))) void row_scan_kernel(RowArgs a) {
  constexpr int SPL = 4 / W;  // states per lane
  constexpr int kTile = tile_tokens<W>();
  constexpr int kDtStride = 2 * kTile + 4;  // floats per channel in the dt / dtu tile (padded)
  constexpr int TPL = kTile / (4 * W);      // prologue / epilogue tokens per lane per tile
  constexpr int kGroups = groups<W>();
  constexpr int NW = W * kGroups;
  constexpr int TPR = 16 / SPL;         // tokens per B / C register
  constexpr int NR = kTile * SPL / 16;  // B / C registers per tile
  constexpr int NX = kTile / 16;        // groups of 16 readout products reduced together
  // Reduced outputs: token tau of channel c at tau * 16 + c + 16 * (tau / TPL): the gap of 16
  // floats after every group of TPL tokens puts the 4 lane rows of the epilogue (which read
  // tokens TPL apart) on distinct LDS banks.
  constexpr int kExStride = kTile * 16 + 16 * (kTile / TPL);
  static_assert(TPL >= 2 && TPL % 2 == 0, "prologue writes token pairs");
  __shared__ __attribute__((aligned(16))) float s_dt[2][kGroups * 16][kDtStride];
  __shared__ float s_ex[2][NW][kExStride];
  constexpr size_t kElt = sizeof(Act);

  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int grp = wid / W;
  const int w = wid % W;
  const int q = lane >> 4;
  const int c = lane & 15;
  const int slot = grp * 16 + c;
  const int64_t b = blockIdx.y;
  // Workgroups go to the eight XCDs round robin by linear id. When the channel blocks of a row
  // are a multiple of 8 the XCD is blockIdx.x mod 8, and each XCD is given a contiguous range of
  // channel blocks: the cache lines that two neighbouring blocks share (32 bf16 channels are half
  // a 128-byte line) are then fetched into one L2 instead of two (8 x 4096 x 7680 bf16: L2
  // fetches from 2.0x to 1.03x the bytes the scan reads).
  const int64_t bx = a.xcd_remap ? (blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8
                                 : blockIdx.x;
  const int64_t e_raw = bx * (kGroups * 16) + slot;
  const bool valid = e_raw < a.E;
  const int64_t e = valid ? e_raw : a.E - 1;
  const int g = w * 4 + q;  // this lane's state group: states g*SPL .. g*SPL + SPL - 1
  const int tau0 = g * TPL;  // first of this lane's prologue / epilogue tokens in a tile
  const int64_t chunk = blockIdx.z;
  const int wslot = wave_slot();
  const int64_t tb = chunk * a.T;
  const int64_t te = (tb + a.T < a.L) ? tb + a.T : a.L;
  const int64_t L = a.L, E = a.E;

  const Act* __restrict__ xp = static_cast<const Act*>(a.x);
  const Act* __restrict__ zp = static_cast<const Act*>(a.z);
  const Act* __restrict__ dtrp = static_cast<const Act*>(a.dt_raw);
  const Act* __restrict__ Bp = static_cast<const Act*>(a.Bm) + b * L * kState;
  const Act* __restrict__ Cp = static_cast<const Act*>(a.Cm) + b * L * kState;
  Act* __restrict__ yp = static_cast<Act*>(a.y);

  // Byte offsets of this lane's elements (the host bounds d_inner so that (kTile + 3) * d_inner
  // elements stay below 2^31 bytes): xoff[j] is token tau0 + j of channel e relative to a
  // tile-aligned base, used for x with the base 3 tokens before the tile (x taps tau0 - 3 + j)
  // and, for j < TPL, for dt_raw and z with the base at the tile's first token. yoff is the
  // same for y, or kNoStore for a lane past the last channel.
  const uint32_t E32 = static_cast<uint32_t>(E);
  uint32_t xoff[TPL + 3];  // token tau0 + j of channel e (x taps from a base 3 tokens back)
#pragma unroll
  for (int j = 0; j < TPL + 3; ++j)
    xoff[j] = (static_cast<uint32_t>(tau0 + j) * E32 + static_cast<uint32_t>(e)) * kElt;
  uint32_t xoff_t[TPL], yoff[TPL];
#pragma unroll
  for (int r = 0; r < TPL; ++r) {
    xoff_t[r] = xoff[r];
    yoff[r] = valid ? xoff[r] : kNoStore;
  }
  uint32_t bcoff[NR];  // B / C element (token j*TPR + c/SPL, state g*SPL + c%SPL)
#pragma unroll
  for (int j = 0; j < NR; ++j)
    bcoff[j] = static_cast<uint32_t>((j * TPR + c / SPL) * kState + g * SPL + (c % SPL)) * kElt;

  float rate[SPL], h[SPL], ia[SPL];  // ia: 1 / A_n (exact zero-order hold only)
  const ZohConst zc;
#pragma unroll
  for (int i = 0; i < SPL; ++i) {
    const int n = g * SPL + i;
    rate[i] = valid ? decay_rate_log2(a.A_log[e * kState + n]) : 0.0f;
    ia[i] = valid ? -expf(-a.A_log[e * kState + n]) : 0.0f;
    h[i] = (a.h_src && valid) ? a.h_src[chunk * a.h_chunk_stride + (b * E + e) * kState + n]
                              : 0.0f;
  }
  const float w0 = a.conv_w[e * kConv + 0], w1 = a.conv_w[e * kConv + 1];
  const float w2 = a.conv_w[e * kConv + 2], w3 = a.conv_w[e * kConv + 3];
  const float cb = a.conv_b[e], dtb = a.dt_bias[e], Dv = a.D[e];

  if constexpr (kCarry) {
    // Chunk 0 keeps a copy of the incoming conv window: the final pass reads it from the
    // workspace, so the caller may update conv_cache in place.
    if (chunk == 0 && w == 0 && q == 0 && valid) {
#pragma unroll
      for (int j = 0; j < kHalo; ++j)
        a.halo[(b * kHalo + j) * E + e] = a.win_src ? a.win_src[(b * kHalo + j) * E + e] : 0.0f;
    }
  }

  using Tile = TileIn<TPL, NR, typename RawOf<Act>::type>;
  auto load_x = [&](int64_t tt) -> float {
    if (tt < 0) return a.win_src ? a.win_src[(b * kHalo + (tt + kHalo)) * E + e] : 0.0f;
    return load_act(xp, (b * L + (tt < L ? tt : L - 1)) * E + e);
  };
  // The first two tiles: conv halo from the incoming window, tokens past the end clamped.
  // The first two tiles: tokens past the end clamped. Tile 0's conv window may reach into the
  // incoming window (fp32), so its x is read as values by the caller (x0); tile 1 starts at
  // kTile > 3 tokens past the chunk start, so its window lies in x.
  auto load_tile_first = [&](int64_t ts, Tile& in, bool with_x) {
    const int64_t t0 = ts + tau0;
    if (with_x) {
#pragma unroll
      for (int j = 0; j < TPL + 3; ++j) {
        const int64_t tt = t0 - 3 + j;
        in.xw[j] = load_act_raw(xp, (b * L + (tt < L ? tt : L - 1)) * E + e);
      }
    }
#pragma unroll
    for (int r = 0; r < TPL; ++r) {
      const int64_t tt = t0 + r < L ? t0 + r : L - 1;
      in.dr[r] = load_act_raw(dtrp, (b * L + tt) * E + e);
      if constexpr (!kCarry) in.zz[r] = load_act_raw(zp, (b * L + tt) * E + e);
    }
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      int64_t tt = ts + j * TPR + c / SPL;
      tt = tt < L ? tt : L - 1;
      const int n = g * SPL + (c % SPL);
      in.RB[j] = load_act_raw(Bp, tt * kState + n);
      if constexpr (!kCarry) in.RC[j] = load_act_raw(Cp, tt * kState + n);
    }
  };
  // Tiles loaded inside the loop start at ts >= tb + 2 kTile >= 3, so their conv halo is in x,
  // and at ts <= L - 1. Addresses are a wave-uniform buffer resource per tile plus fixed 32-bit
  // lane offsets. Each resource's range ends at the end of the batch row's sequence, so in a
  // tile that runs past it the hardware returns 0 for the missing tokens (they get dt = 0 and
  // no store); every tile issues the same loads into the same registers with no per-lane
  // branch, so the compiler's wait counts stay exact.
  // Per-tile addresses: the batch row's base plus one 64-bit product per tile (ts * E), shared
  // by the three activation streams.
  const Act* const xrow = xp + (b * L - 3) * E;
  const Act* const drow = dtrp + b * L * E;
  const Act* const zrow = zp + b * L * E;
  Act* const yrow = yp + b * L * E;
  const uint32_t tile_row = static_cast<uint32_t>(E * kElt);  // bytes per token of a stream
  auto load_tile = [&](int64_t ts, Tile& in) {
    const int64_t toff = ts * E;
    // Tokens of the tile inside the sequence (its offsets reach no further than kTile tokens
    // past its first, 3 more for x; the byte counts fit 32 bits as the host bounds d_inner).
    const uint32_t n = static_cast<uint32_t>(L - ts < kTile ? L - ts : kTile);
    const uint32_t bc_row = static_cast<uint32_t>(kState * kElt);
    const rsrc_t rx = make_rsrc_bounded(const_cast<Act*>(xrow + toff), (n + 3) * tile_row);
    const rsrc_t rd = make_rsrc_bounded(const_cast<Act*>(drow + toff), n * tile_row);
    const rsrc_t rz = make_rsrc_bounded(const_cast<Act*>(zrow + toff), n * tile_row);
    const rsrc_t rB = make_rsrc_bounded(const_cast<Act*>(Bp + ts * kState), n * bc_row);
    const rsrc_t rC = make_rsrc_bounded(const_cast<Act*>(Cp + ts * kState), n * bc_row);
#pragma unroll
    for (int j = 0; j < TPL + 3; ++j) in.xw[j] = load_raw_t<Act>(rx, xoff[j]);
#pragma unroll
    for (int r = 0; r < TPL; ++r) {
      in.dr[r] = load_raw_t<Act>(rd, xoff_t[r]);
      if constexpr (!kCarry) in.zz[r] = load_raw_t<Act>(rz, xoff_t[r]);
    }
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      in.RB[j] = load_raw_t<Act>(rB, bcoff[j]);
      if constexpr (!kCarry) in.RC[j] = load_raw_t<Act>(rC, bcoff[j]);
    }
  };
  // Tokens past the chunk end (and lanes past the last channel) get dt = 0: their state update
  // is the identity.
  auto prologue = [&](int64_t ts, const float (&xw)[TPL + 3], const Tile& in, int buf,
                      float (&u)[TPL]) {
    const int rem = static_cast<int>(te - ts < kTile ? te - ts : kTile);  // tokens in the chunk
    float pair[2 * TPL];
#pragma unroll
    for (int r = 0; r < TPL; ++r) {
      float uu = fmaf(w3, xw[r + 3], fmaf(w2, xw[r + 2], fmaf(w1, xw[r + 1], fmaf(w0, xw[r], cb))));
      if constexpr (kSilu) uu = silu(uu);
      const float keep = (valid && tau0 + r < rem) ? 1.0f : 0.0f;
      const float dt = step_size(widen(in.dr[r]) + dtb, a.dt_min, a.dt_max) * keep;
      pair[2 * r] = dt;
      pair[2 * r + 1] = kZoh ? uu : dt * uu;  // the exact hold scales u per state in the scan
      u[r] = uu;
    }
#pragma unroll
    for (int r = 0; r < TPL; r += 2)
      *reinterpret_cast<float4*>(&s_dt[buf][slot][2 * (tau0 + r)]) =
          make_float4(pair[2 * r], pair[2 * r + 1], pair[2 * r + 2], pair[2 * r + 3]);
  };
  auto ex_index = [&](int tau) { return tau * 16 + c + 16 * (tau / TPL); };
  // Token 4 x4 + q of the four-row sums goes to ex_index(q) plus a constant of x4 (TPL divides
  // 4 or 4 divides TPL), which the compiler folds into the LDS store's offset.
  static_assert(4 % TPL == 0 || TPL % 4 == 0, "reduced-token index split");
  const int ex_q = ex_index(q);

  const int64_t ntiles = (te - tb + kTile - 1) / kTile;
  const int64_t ts_last = tb + (ntiles - 1) * kTile;
  // Three register slots (a dynamically indexed register array would live in scratch memory):
  // while tile k is scanned, tile k+1's inputs wait for their prologue and tile k+2's are in
  // flight. The main loop handles whole triples of tiles with the slots' roles rotated, so
  // loaded registers are never copied (a copy would wait for its load).
  Tile ring0, ring1, ring2;
  float u_cur[TPL];
  float x0[TPL + 3];
#pragma unroll
  for (int j = 0; j < TPL + 3; ++j) x0[j] = load_x(tb + tau0 - 3 + j);
  load_tile_first(tb, ring0, false);
  if (ntiles > 1) load_tile_first(tb + kTile, ring1, true);
  prologue(tb, x0, ring0, 0, u_cur);
  __syncthreads();

  float S = 0.0f;
  // Tile k: scan with cur's B / C, prologue of tile k+1 from nxt, epilogue with cur's z; with
  // kLoad, tile k+2 (clamped to the last tile) is first loaded into fut.
  auto do_tile = [&](auto load_tag, int64_t k, const Tile& cur,
                     const Tile& nxt, Tile& fut) {
    constexpr bool kLoad = decltype(load_tag)::value;
    const int64_t ts = tb + k * kTile;
    const int buf = static_cast<int>(k & 1);
    // At equal priority a SIMD issues its oldest wave first: of two waves from different
    // workgroups the older then runs almost as if alone and the younger finishes ~25 us later,
    // alone (1 x 2048 x 7680 fp32). Raising the priority of the waves whose slot parity differs
    // from the tile's, tile by tile, makes them share the VALU evenly: 3-4% per launch.
    if (((k + wslot) & 1) != 0)
      __builtin_amdgcn_s_setprio(1);
    else
      __builtin_amdgcn_s_setprio(0);
    if constexpr (kLoad) load_tile(ts + 2 * kTile < ts_last ? ts + 2 * kTile : ts_last, fut);
    float4 dd[kTile / 2];
#pragma unroll
    for (int i = 0; i < kTile / 2; ++i)
      dd[i] = *reinterpret_cast<const float4*>(&s_dt[buf][slot][4 * i]);
    float P[kTile], ac[SPL], RB[NR], RC[NR];
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      RB[j] = widen(cur.RB[j]);
      RC[j] = kCarry ? 0.0f : widen(cur.RC[j]);
    }
    if constexpr (kZoh) {
      float yc[SPL];
      scan_tile_zoh_from<SPL, kCarry, 0, kTile>(dd, rate, ia, zc, RB, RC, h, ac, yc, P, S);
    } else {
      scan_tile_from<SPL, kCarry, 0, kTile>(dd, rate, RB, RC, h, ac, P, S);
    }

    float u_next[TPL];
    if (k + 1 < ntiles) {
      float xw[TPL + 3];
#pragma unroll
      for (int j = 0; j < TPL + 3; ++j) xw[j] = widen(nxt.xw[j]);
      prologue(ts + kTile, xw, nxt, buf ^ 1, u_next);
    }
    if constexpr (!kCarry) {
      // Row q of the reduced register for tokens 4x .. 4x+3 holds token 4x + q.
#pragma unroll
      for (int x4 = 0; x4 < 4 * NX; ++x4) {
        const float R = rows_reduce4(P[4 * x4], P[4 * x4 + 1], P[4 * x4 + 2], P[4 * x4 + 3]);
        s_ex[buf][wid][ex_q + 64 * x4 + 16 * (4 * x4 / TPL)] = R;
      }
    }
    __syncthreads();
    if constexpr (!kCarry) {
      // This wave finishes its prologue tokens: skip term, gate, store. Every lane issues its
      // stores; those of tokens past the chunk end fall outside the resource's range and those
      // of lanes past the last channel carry kNoStore, so the hardware drops them and no
      // branch is needed.
      const int64_t rem = te - ts < kTile ? te - ts : kTile;
      const rsrc_t ry = make_rsrc_bounded(yrow + ts * E, static_cast<uint32_t>(rem) * tile_row);
#pragma unroll
      for (int r = 0; r < TPL; ++r) {
        const int ix = ex_index(tau0 + r);
        float ysum = s_ex[buf][grp * W][ix];
#pragma unroll
        for (int v = 1; v < W; ++v) ysum += s_ex[buf][grp * W + v][ix];
        const float yv = fmaf(Dv, u_cur[r], ysum) * silu(widen(cur.zz[r]));
        store_buf<Act>(ry, yoff[r], yv);
      }
    }
#pragma unroll
    for (int r = 0; r < TPL; ++r) u_cur[r] = u_next[r];
  };
  using Load = std::true_type;
  using NoLoad = std::false_type;
  int64_t k = 0;
  for (; k + 3 <= ntiles; k += 3) {
    do_tile(Load{}, k, ring0, ring1, ring2);
    do_tile(Load{}, k + 1, ring1, ring2, ring0);
    do_tile(Load{}, k + 2, ring2, ring0, ring1);
  }
  // At most two tiles remain, whose inputs are already loaded (in ring0 and ring1).
  if (k < ntiles) do_tile(NoLoad{}, k, ring0, ring1, ring2);
  if (k + 1 < ntiles) do_tile(NoLoad{}, k + 1, ring1, ring2, ring0);

  if (!valid) return;
  if constexpr (kCarry) {
    const int64_t be = (chunk * a.B + b) * E + e;
#pragma unroll
    for (int i = 0; i < SPL; ++i) a.carry_h[be * kState + g * SPL + i] = h[i];
    if (w == 0 && q == 0) a.carry_s[be] = S;
  } else if (chunk == a.chunks - 1) {
#pragma unroll
    for (int i = 0; i < SPL; ++i) a.state_out[(b * E + e) * kState + g * SPL + i] = h[i];
    if (w == 0 && q == 0) {
      // Last K-1 inputs of [conv window, x]: read all three before writing (in-place caches).
      float cv[kHalo];
#pragma unroll
      for (int j = 0; j < kHalo; ++j) cv[j] = load_x(L - kHalo + j);
#pragma unroll
      for (int j = 0; j < kHalo; ++j) a.cache_out[(b * kHalo + j) * E + e] = cv[j];
    }
  }
}

}  // namespace

// Carry combine of the time-chunked prefill (axon_kernels.hip).
void launch_carry_combine(int64_t B, int64_t E, int64_t M, const float* A_log,
                          const float* state_in, const float* carry_h, const float* carry_s,
                          float* carry_in, hipStream_t s);

template <typename Act, int W, bool kSilu, bool kZoh>
int launch_row_scan_t(const PrefillLaunch& p, const PrefillPlan& plan, hipStream_t s) {
  constexpr int kGroups = groups<W>();
  RowArgs a{};
  a.B = p.batch;
  a.L = p.seqlen;
  a.E = p.d_inner;
  a.T = plan.chunk_len;
  a.chunks = plan.chunks;
  // Only where a workgroup's channels fill less than a 128-byte line (bf16): with fp32 the
  // remap shares nothing and measured no gain.
  a.xcd_remap = sizeof(Act) * kGroups * 16 < 128 &&
                (p.d_inner + kGroups * 16 - 1) / (kGroups * 16) % 8 == 0 ? 1 : 0;
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
  a.y = p.y;
  a.state_out = p.ssm_state_out;
  a.cache_out = p.conv_cache_out;
  const dim3 block(64 * W * kGroups);
  const unsigned gx = static_cast<unsigned>((p.d_inner + kGroups * 16 - 1) / (kGroups * 16));
  const unsigned gy = static_cast<unsigned>(p.batch);
  if (plan.chunks == 1) {
    a.win_src = p.conv_cache_in;
    a.h_src = p.ssm_state_in;
    a.h_chunk_stride = 0;
    hipLaunchKernelGGL((row_scan_kernel<Act, W, false, kSilu, kZoh>), dim3(gx, gy, 1), block, 0, s, a);
    return static_cast<int>(hipGetLastError());
  }
  char* ws = static_cast<char*>(p.workspace);
  a.carry_h = reinterpret_cast<float*>(ws + plan.off_carry_h);
  a.carry_s = reinterpret_cast<float*>(ws + plan.off_carry_s);
  a.halo = reinterpret_cast<float*>(ws + plan.off_halo);
  float* carry_in = reinterpret_cast<float*>(ws + plan.off_carry_in);
  a.win_src = p.conv_cache_in;
  a.h_src = nullptr;
  a.h_chunk_stride = 0;
  hipLaunchKernelGGL((row_scan_kernel<Act, W, true, kSilu, kZoh>),
                     dim3(gx, gy, static_cast<unsigned>(plan.chunks - 1)), block, 0, s, a);
  launch_carry_combine(p.batch, p.d_inner, plan.chunks, p.A_log, p.ssm_state_in, a.carry_h,
                       a.carry_s, carry_in, s);
  a.win_src = a.halo;
  a.h_src = carry_in;
  a.h_chunk_stride = p.batch * p.d_inner * kState;
  hipLaunchKernelGGL((row_scan_kernel<Act, W, false, kSilu, kZoh>),
                     dim3(gx, gy, static_cast<unsigned>(plan.chunks)), block, 0, s, a);
  return static_cast<int>(hipGetLastError());
}

template <typename Act, bool kSilu, bool kZoh>
int launch_row_scan_w(const PrefillLaunch& p, const PrefillPlan& plan, hipStream_t s) {
  return plan.row_waves == 4 ? launch_row_scan_t<Act, 4, kSilu, kZoh>(p, plan, s)
                             : launch_row_scan_t<Act, 2, kSilu, kZoh>(p, plan, s);
}

template <typename Act>
int launch_row_scan_v(const PrefillLaunch& p, const PrefillPlan& plan, hipStream_t s) {
  if (p.conv_silu)
    return p.zoh ? launch_row_scan_w<Act, true, true>(p, plan, s)
                 : launch_row_scan_w<Act, true, false>(p, plan, s);
  return p.zoh ? launch_row_scan_w<Act, false, true>(p, plan, s)
               : launch_row_scan_w<Act, false, false>(p, plan, s);
}

int launch_row_scan(const PrefillLaunch& p, const PrefillPlan& plan, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  // The planner picks W = 4 (one state per lane) or W = 2 (two states per lane); the variants
  // are compile-time so that the Axon-SSM kernel carries none of their code.
  return p.act_bf16 ? launch_row_scan_v<bf16_bits>(p, plan, s)
                    : launch_row_scan_v<float>(p, plan, s);
}

}  // namespace axon
