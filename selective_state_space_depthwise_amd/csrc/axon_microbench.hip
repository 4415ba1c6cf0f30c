// Microbenchmarks of the gfx950 features the scan kernels are built from: the issue cost of the
// VALU instructions in their inner loops (FMA, v_exp_f32, DPP row broadcast, the permlane swaps
// of the readout reduction), latency of dependent chains, co-issue of scalar and vector work from
// one wave, and the HBM bandwidth a plain streaming copy and read reach. Built as its own library
// (libaxonmicro.so) so the product library carries none of it.
//
// Every ALU kernel runs a loop of inline-asm VALU blocks on registers only (no memory access in
// the asm). DPP instructions read only registers the block never writes, or that were written at
// least two VALU instructions earlier, so no wait states are needed beyond those written.
#include <hip/hip_runtime.h>

#include <type_traits>

#include <cstddef>
#include <cstdint>

namespace {

enum Kind : int {
  kFma = 0,        // 8 independent v_fmac_f32 chains
  kExp = 1,        // 8 independent v_exp_f32
  kDpp = 2,        // 8 independent v_mul_f32_dpp row_newbcast
  kPerm32 = 3,     // 4 v_permlane32_swap (register pairs)
  kUpdate = 4,     // the scan's state update: mul, exp, DPP mul, fmac, DPP mul (8 chains)
  kExpFma = 5,     // 1 v_exp_f32 per 4 independent v_fmac_f32
  kFmaSalu = 6,    // 1 s_add_u32 per v_fmac_f32
  kFmaChain = 7,   // one dependent v_fmac_f32 chain (latency)
  kExpChain = 8,   // one dependent v_exp_f32 chain, one wait state between (latency)
  kPerm16 = 9,     // 4 v_permlane16_swap (register pairs)
  kExpFma1 = 10,   // 1 v_exp_f32 per v_fmac_f32
  kExpFma2 = 11,   // 1 v_exp_f32 per 2 v_fmac_f32
  kExpFma8 = 12,   // 1 v_exp_f32 per 8 v_fmac_f32
  kChanUpd = 13,   // the lane-per-channel update: mul, exp, mul, fma, fmac (8 states)
  kChanNoExp = 14, // the same with the exp replaced by a mul
  kBurst16 = 15,   // 16 v_exp_f32, then 48 v_fmac_f32 (the exps of a token grouped)
  kBurst8 = 16,    // 8 v_exp_f32, then 24 v_fmac_f32
  kBurst16v3 = 17, // 16 v_exp_f32, then 48 v_fma_f32 (VOP3)
  kFmaSgpr = 18,   // 8 independent v_fmac_f32 chains with one operand in an SGPR
  // One state chain per lane, 8 tokens per block (the row scan with one state per lane):
  kChainDpp = 19,    // per token: mul, exp, DPP input product, DPP readout product, fma
                     // (the exp's result read two instructions later)
  kChainAhead = 20,  // the same with the decay computed one token ahead (the kernel's order)
  kPhaseDpp = 21,    // the 8 tokens' mul and exp first, then their DPP products and fmas
  kPhasePlain = 22,  // the same with B and C as plain registers instead of DPP broadcasts
  kNumKinds = 23
};

// VALU instructions per loop iteration of each kind (the SALU of kFmaSalu not counted).
__host__ __device__ constexpr int instrs_per_iter(int kind) {
  return kind == kFma ? 64 : kind == kExp ? 64 : kind == kDpp ? 64 : kind == kPerm32 ? 64
       : kind == kUpdate ? 80 : kind == kExpFma ? 80 : kind == kFmaSalu ? 32
       : kind == kFmaChain ? 32 : kind == kExpChain ? 32 : kind == kPerm16 ? 64
       : kind == kExpFma1 ? 64 : kind == kExpFma2 ? 72 : kind == kExpFma8 ? 72
       : kind == kChanUpd ? 80 : kind == kChanNoExp ? 80 : kind == kBurst16 ? 64
       : kind == kBurst8 ? 64 : kind == kBurst16v3 ? 64 : kind == kFmaSgpr ? 64
       : kind >= kChainDpp && kind <= kPhasePlain ? 80 : 0;
}

#define F8(op) op(0) op(1) op(2) op(3) op(4) op(5) op(6) op(7)
#define FMA1(i) "v_fmac_f32 %[a" #i "], %[m], %[n]\n\t"
#define EXP1(i) "v_exp_f32 %[a" #i "], %[a" #i "]\n\t"
#define DPP1(i) "v_mul_f32_dpp %[a" #i "], %[m], %[n] row_newbcast:" #i " row_mask:0xf bank_mask:0xf\n\t"
#define OUT8 [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), \
             [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7])

// The instruction mix of the scan's state update (one state per lane), 8 independent states per
// block: per state i, v_mul n_i = dt * r, v_exp n_i, v_mul_dpp b_i = bcast(RB) * dtu,
// v_mul_dpp p_i = bcast(RC) * h_i, v_fmac h_i += n_i * b_i (the same five instructions and
// dependences on n; the state chain runs through h).
#define UPD_A(i) "v_mul_f32 %[n" #i "], %[dt], %[r]\n\t"
#define UPD_D(i) "v_exp_f32 %[n" #i "], %[n" #i "]\n\t"
#define UPD_B(i) "v_mul_f32_dpp %[b" #i "], %[RB], %[dtu] row_newbcast:" #i " row_mask:0xf bank_mask:0xf\n\t"
#define UPD_C(i) "v_mul_f32_dpp %[p" #i "], %[RC], %[h" #i "] row_newbcast:" #i " row_mask:0xf bank_mask:0xf\n\t"
#define UPD_E(i) "v_fmac_f32 %[h" #i "], %[n" #i "], %[b" #i "]\n\t"

template <int kKind>
__global__ __launch_bounds__(1024) void alu_kernel(int iters, float seed, float* sink,
                                                 unsigned long long* clocks) {
  float a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = seed * static_cast<float>(threadIdx.x + i);
  const float m = 0.999f + seed * 1e-6f, n = 1e-3f * seed;
  unsigned long long t0 = 0, r0 = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  float h[8], b[8], nn[8], p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h[i] = a[i];
    b[i] = 0.0f;
    nn[i] = 0.0f;
    p[i] = 0.0f;
  }
  for (int it = 0; it < iters; ++it) {
    if constexpr (kKind == kFma) {
      asm volatile(F8(FMA1) F8(FMA1) F8(FMA1) F8(FMA1) F8(FMA1) F8(FMA1) F8(FMA1) F8(FMA1)
                   : OUT8 : [m] "v"(m), [n] "v"(n));
    } else if constexpr (kKind == kFmaSgpr) {
#define FMAS1(i) "v_fmac_f32 %[a" #i "], %[s], %[n]\n\t"
      asm volatile(F8(FMAS1) F8(FMAS1) F8(FMAS1) F8(FMAS1) F8(FMAS1) F8(FMAS1) F8(FMAS1)
                   F8(FMAS1) : OUT8 : [s] "s"(seed), [n] "v"(n));
#undef FMAS1
    } else if constexpr (kKind == kExp) {
      asm volatile(F8(EXP1) F8(EXP1) F8(EXP1) F8(EXP1) F8(EXP1) F8(EXP1) F8(EXP1) F8(EXP1)
                   : OUT8);
    } else if constexpr (kKind == kDpp) {
      asm volatile(F8(DPP1) F8(DPP1) F8(DPP1) F8(DPP1) F8(DPP1) F8(DPP1) F8(DPP1) F8(DPP1)
                   : OUT8 : [m] "v"(m), [n] "v"(n));
    } else if constexpr (kKind == kPerm32 || kKind == kPerm16) {
      // 16 swaps of 4 register pairs = 64 instructions
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        asm volatile("" : OUT8);
        if constexpr (kKind == kPerm32) {
          asm volatile(
              "v_permlane32_swap_b32 %[a0], %[a1]\n\tv_permlane32_swap_b32 %[a2], %[a3]\n\t"
              "v_permlane32_swap_b32 %[a4], %[a5]\n\tv_permlane32_swap_b32 %[a6], %[a7]\n\t"
              "v_permlane32_swap_b32 %[a0], %[a1]\n\tv_permlane32_swap_b32 %[a2], %[a3]\n\t"
              "v_permlane32_swap_b32 %[a4], %[a5]\n\tv_permlane32_swap_b32 %[a6], %[a7]\n\t"
              "v_permlane32_swap_b32 %[a0], %[a1]\n\tv_permlane32_swap_b32 %[a2], %[a3]\n\t"
              "v_permlane32_swap_b32 %[a4], %[a5]\n\tv_permlane32_swap_b32 %[a6], %[a7]\n\t"
              "v_permlane32_swap_b32 %[a0], %[a1]\n\tv_permlane32_swap_b32 %[a2], %[a3]\n\t"
              "v_permlane32_swap_b32 %[a4], %[a5]\n\tv_permlane32_swap_b32 %[a6], %[a7]\n\t"
              : OUT8);
        } else {
          asm volatile(
              "v_permlane16_swap_b32 %[a0], %[a1]\n\tv_permlane16_swap_b32 %[a2], %[a3]\n\t"
              "v_permlane16_swap_b32 %[a4], %[a5]\n\tv_permlane16_swap_b32 %[a6], %[a7]\n\t"
              "v_permlane16_swap_b32 %[a0], %[a1]\n\tv_permlane16_swap_b32 %[a2], %[a3]\n\t"
              "v_permlane16_swap_b32 %[a4], %[a5]\n\tv_permlane16_swap_b32 %[a6], %[a7]\n\t"
              "v_permlane16_swap_b32 %[a0], %[a1]\n\tv_permlane16_swap_b32 %[a2], %[a3]\n\t"
              "v_permlane16_swap_b32 %[a4], %[a5]\n\tv_permlane16_swap_b32 %[a6], %[a7]\n\t"
              "v_permlane16_swap_b32 %[a0], %[a1]\n\tv_permlane16_swap_b32 %[a2], %[a3]\n\t"
              "v_permlane16_swap_b32 %[a4], %[a5]\n\tv_permlane16_swap_b32 %[a6], %[a7]\n\t"
              : OUT8);
        }
      }
    } else if constexpr (kKind == kUpdate) {
      // two rounds of 8 states: 80 instructions
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        asm volatile(F8(UPD_A) F8(UPD_D) F8(UPD_B) F8(UPD_C) F8(UPD_E)
                     : [n0] "+v"(nn[0]), [n1] "+v"(nn[1]), [n2] "+v"(nn[2]), [n3] "+v"(nn[3]),
                       [n4] "+v"(nn[4]), [n5] "+v"(nn[5]), [n6] "+v"(nn[6]), [n7] "+v"(nn[7]),
                       [b0] "+v"(b[0]), [b1] "+v"(b[1]), [b2] "+v"(b[2]), [b3] "+v"(b[3]),
                       [b4] "+v"(b[4]), [b5] "+v"(b[5]), [b6] "+v"(b[6]), [b7] "+v"(b[7]),
                       [p0] "+v"(p[0]), [p1] "+v"(p[1]), [p2] "+v"(p[2]), [p3] "+v"(p[3]),
                       [p4] "+v"(p[4]), [p5] "+v"(p[5]), [p6] "+v"(p[6]), [p7] "+v"(p[7]),
                       [h0] "+v"(h[0]), [h1] "+v"(h[1]), [h2] "+v"(h[2]), [h3] "+v"(h[3]),
                       [h4] "+v"(h[4]), [h5] "+v"(h[5]), [h6] "+v"(h[6]), [h7] "+v"(h[7])
                     : [dt] "v"(m), [r] "v"(n), [RB] "v"(a[0]), [RC] "v"(a[1]), [dtu] "v"(a[2]));
      }
    } else if constexpr (kKind == kExpFma) {
#define EF(i) EXP1(i) FMA1(0) FMA1(1) FMA1(2) FMA1(3)
      asm volatile(EF(4) EF(5) EF(6) EF(7) EF(4) EF(5) EF(6) EF(7)
                   EF(4) EF(5) EF(6) EF(7) EF(4) EF(5) EF(6) EF(7)
                   : OUT8 : [m] "v"(m), [n] "v"(n));
#undef EF
    } else if constexpr (kKind == kExpFma1) {
#define E1F(i) EXP1(i) FMA1(0)
      asm volatile(E1F(4) E1F(5) E1F(6) E1F(7) E1F(4) E1F(5) E1F(6) E1F(7)
                   E1F(4) E1F(5) E1F(6) E1F(7) E1F(4) E1F(5) E1F(6) E1F(7)
                   E1F(4) E1F(5) E1F(6) E1F(7) E1F(4) E1F(5) E1F(6) E1F(7)
                   E1F(4) E1F(5) E1F(6) E1F(7) E1F(4) E1F(5) E1F(6) E1F(7)
                   : OUT8 : [m] "v"(m), [n] "v"(n));
#undef E1F
    } else if constexpr (kKind == kExpFma2) {
#define E2F(i) EXP1(i) FMA1(0) FMA1(1)
      asm volatile(E2F(4) E2F(5) E2F(6) E2F(7) E2F(4) E2F(5) E2F(6) E2F(7)
                   E2F(4) E2F(5) E2F(6) E2F(7) E2F(4) E2F(5) E2F(6) E2F(7)
                   E2F(4) E2F(5) E2F(6) E2F(7) E2F(4) E2F(5) E2F(6) E2F(7)
                   : OUT8 : [m] "v"(m), [n] "v"(n));
#undef E2F
    } else if constexpr (kKind == kExpFma8) {
#define E8F(i) EXP1(i) FMA1(0) FMA1(1) FMA1(2) FMA1(3) FMA1(0) FMA1(1) FMA1(2) FMA1(3)
      asm volatile(E8F(4) E8F(5) E8F(6) E8F(7) E8F(4) E8F(5) E8F(6) E8F(7)
                   : OUT8 : [m] "v"(m), [n] "v"(n));
#undef E8F
    } else if constexpr (kKind == kChanUpd || kKind == kChanNoExp) {
      // per state i: n_i = dt * r; n_i = exp2(n_i); b_i = B * du; h_i = n_i * h_i + b_i;
      // p_i += C * h_i  (two rounds of 8 states: 80 instructions)
#define CU_A(i) "v_mul_f32 %[n" #i "], %[dt], %[r]\n\t"
#define CU_B(i) "v_mul_f32 %[b" #i "], %[RB], %[dtu]\n\t"
#define CU_E(i) "v_fma_f32 %[h" #i "], %[n" #i "], %[h" #i "], %[b" #i "]\n\t"
#define CU_R(i) "v_fmac_f32 %[p" #i "], %[RC], %[h" #i "]\n\t"
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if constexpr (kKind == kChanUpd) {
          asm volatile(F8(CU_A)
                       "v_exp_f32 %[n0], %[n0]\n\tv_exp_f32 %[n1], %[n1]\n\t"
                       "v_exp_f32 %[n2], %[n2]\n\tv_exp_f32 %[n3], %[n3]\n\t"
                       "v_exp_f32 %[n4], %[n4]\n\tv_exp_f32 %[n5], %[n5]\n\t"
                       "v_exp_f32 %[n6], %[n6]\n\tv_exp_f32 %[n7], %[n7]\n\t"
                       F8(CU_B) F8(CU_E) F8(CU_R)
                       : [n0] "+v"(nn[0]), [n1] "+v"(nn[1]), [n2] "+v"(nn[2]), [n3] "+v"(nn[3]),
                         [n4] "+v"(nn[4]), [n5] "+v"(nn[5]), [n6] "+v"(nn[6]), [n7] "+v"(nn[7]),
                         [b0] "+v"(b[0]), [b1] "+v"(b[1]), [b2] "+v"(b[2]), [b3] "+v"(b[3]),
                         [b4] "+v"(b[4]), [b5] "+v"(b[5]), [b6] "+v"(b[6]), [b7] "+v"(b[7]),
                         [p0] "+v"(p[0]), [p1] "+v"(p[1]), [p2] "+v"(p[2]), [p3] "+v"(p[3]),
                         [p4] "+v"(p[4]), [p5] "+v"(p[5]), [p6] "+v"(p[6]), [p7] "+v"(p[7]),
                         [h0] "+v"(h[0]), [h1] "+v"(h[1]), [h2] "+v"(h[2]), [h3] "+v"(h[3]),
                         [h4] "+v"(h[4]), [h5] "+v"(h[5]), [h6] "+v"(h[6]), [h7] "+v"(h[7])
                       : [dt] "v"(m), [r] "v"(n), [RB] "v"(a[0]), [RC] "v"(a[1]),
                         [dtu] "v"(a[2]));
        } else {
          asm volatile(F8(CU_A)
                       "v_mul_f32 %[n0], %[n0], %[dt]\n\tv_mul_f32 %[n1], %[n1], %[dt]\n\t"
                       "v_mul_f32 %[n2], %[n2], %[dt]\n\tv_mul_f32 %[n3], %[n3], %[dt]\n\t"
                       "v_mul_f32 %[n4], %[n4], %[dt]\n\tv_mul_f32 %[n5], %[n5], %[dt]\n\t"
                       "v_mul_f32 %[n6], %[n6], %[dt]\n\tv_mul_f32 %[n7], %[n7], %[dt]\n\t"
                       F8(CU_B) F8(CU_E) F8(CU_R)
                       : [n0] "+v"(nn[0]), [n1] "+v"(nn[1]), [n2] "+v"(nn[2]), [n3] "+v"(nn[3]),
                         [n4] "+v"(nn[4]), [n5] "+v"(nn[5]), [n6] "+v"(nn[6]), [n7] "+v"(nn[7]),
                         [b0] "+v"(b[0]), [b1] "+v"(b[1]), [b2] "+v"(b[2]), [b3] "+v"(b[3]),
                         [b4] "+v"(b[4]), [b5] "+v"(b[5]), [b6] "+v"(b[6]), [b7] "+v"(b[7]),
                         [p0] "+v"(p[0]), [p1] "+v"(p[1]), [p2] "+v"(p[2]), [p3] "+v"(p[3]),
                         [p4] "+v"(p[4]), [p5] "+v"(p[5]), [p6] "+v"(p[6]), [p7] "+v"(p[7]),
                         [h0] "+v"(h[0]), [h1] "+v"(h[1]), [h2] "+v"(h[2]), [h3] "+v"(h[3]),
                         [h4] "+v"(h[4]), [h5] "+v"(h[5]), [h6] "+v"(h[6]), [h7] "+v"(h[7])
                       : [dt] "v"(m), [r] "v"(n), [RB] "v"(a[0]), [RC] "v"(a[1]),
                         [dtu] "v"(a[2]));
        }
      }
#undef CU_A
#undef CU_B
#undef CU_E
#undef CU_R
    } else if constexpr (kKind == kBurst16 || kKind == kBurst8 || kKind == kBurst16v3) {
      // exps into b[] / p[] (16 registers), FMAs on the 8 a[] chains
#define BE(x) "v_exp_f32 %[" #x "], %[" #x "]\n\t"
#define BE8 BE(b0) BE(b1) BE(b2) BE(b3) BE(b4) BE(b5) BE(b6) BE(b7)
#define BE8P BE(p0) BE(p1) BE(p2) BE(p3) BE(p4) BE(p5) BE(p6) BE(p7)
#define V3(i) "v_fma_f32 %[a" #i "], %[m], %[n], %[a" #i "]\n\t"
#define BOUT [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), \
             [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), \
             [b0] "+v"(b[0]), [b1] "+v"(b[1]), [b2] "+v"(b[2]), [b3] "+v"(b[3]), \
             [b4] "+v"(b[4]), [b5] "+v"(b[5]), [b6] "+v"(b[6]), [b7] "+v"(b[7]), \
             [p0] "+v"(p[0]), [p1] "+v"(p[1]), [p2] "+v"(p[2]), [p3] "+v"(p[3]), \
             [p4] "+v"(p[4]), [p5] "+v"(p[5]), [p6] "+v"(p[6]), [p7] "+v"(p[7])
      if constexpr (kKind == kBurst16) {
        asm volatile(BE8 BE8P F8(FMA1) F8(FMA1) F8(FMA1) F8(FMA1) F8(FMA1) F8(FMA1)
                     : BOUT : [m] "v"(m), [n] "v"(n));
      } else if constexpr (kKind == kBurst8) {
        asm volatile(BE8 F8(FMA1) F8(FMA1) F8(FMA1) BE8P F8(FMA1) F8(FMA1) F8(FMA1)
                     : BOUT : [m] "v"(m), [n] "v"(n));
      } else {
        asm volatile(BE8 BE8P F8(V3) F8(V3) F8(V3) F8(V3) F8(V3) F8(V3)
                     : BOUT : [m] "v"(m), [n] "v"(n));
      }
#undef BOUT
#undef V3
#undef BE8P
#undef BE8
#undef BE
    } else if constexpr (kKind >= kChainDpp && kKind <= kPhasePlain) {
      // h[0] is the state, h[1] the input product, nn[] the decays, p[] the readout products,
      // b[] the plain B registers; B, C and dtu (a[0..2]) are never written.
#define CA(i) "v_mul_f32 %[n" #i "], %[dt], %[r]\n\t"
#define CE(i) "v_exp_f32 %[n" #i "], %[n" #i "]\n\t"
#define CB "v_mul_f32_dpp %[bb], %[RB], %[dtu] row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
#define CC(i) "v_mul_f32_dpp %[p" #i "], %[RC], %[h] row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
#define CF(i) "v_fma_f32 %[h], %[n" #i "], %[h], %[bb]\n\t"
#define PB(i) "v_mul_f32 %[bb], %[R" #i "], %[dtu]\n\t"
#define PC(i) "v_mul_f32 %[p" #i "], %[RC], %[h]\n\t"
#define CHAIN(i) CA(i) CE(i) CB CC(i) CF(i)
#define AHEAD(i, j) CA(j) CE(j) CB CC(i) CF(i)
#define PHD(i) CB CC(i) CF(i)
#define PHP(i) PB(i) PC(i) CF(i)
#define COUT [n0] "+v"(nn[0]), [n1] "+v"(nn[1]), [n2] "+v"(nn[2]), [n3] "+v"(nn[3]), \
             [n4] "+v"(nn[4]), [n5] "+v"(nn[5]), [n6] "+v"(nn[6]), [n7] "+v"(nn[7]), \
             [p0] "+v"(p[0]), [p1] "+v"(p[1]), [p2] "+v"(p[2]), [p3] "+v"(p[3]), \
             [p4] "+v"(p[4]), [p5] "+v"(p[5]), [p6] "+v"(p[6]), [p7] "+v"(p[7]), \
             [h] "+v"(h[0]), [bb] "+v"(h[1])
#define CIN [dt] "v"(m), [r] "v"(n), [RB] "v"(a[0]), [RC] "v"(a[1]), [dtu] "v"(a[2]), \
            [R0] "v"(b[0]), [R1] "v"(b[1]), [R2] "v"(b[2]), [R3] "v"(b[3]), [R4] "v"(b[4]), \
            [R5] "v"(b[5]), [R6] "v"(b[6]), [R7] "v"(b[7])
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if constexpr (kKind == kChainDpp) {
          asm volatile(CHAIN(0) CHAIN(1) CHAIN(2) CHAIN(3) CHAIN(4) CHAIN(5) CHAIN(6) CHAIN(7)
                       : COUT : CIN);
        } else if constexpr (kKind == kChainAhead) {
          asm volatile(AHEAD(0, 1) AHEAD(1, 2) AHEAD(2, 3) AHEAD(3, 4) AHEAD(4, 5) AHEAD(5, 6)
                       AHEAD(6, 7) AHEAD(7, 0) : COUT : CIN);
        } else if constexpr (kKind == kPhaseDpp) {
          asm volatile(F8(CA) F8(CE) "s_nop 1\n\t" PHD(0) PHD(1) PHD(2) PHD(3) PHD(4) PHD(5)
                       PHD(6) PHD(7) : COUT : CIN);
        } else {
          asm volatile(F8(CA) F8(CE) PHP(0) PHP(1) PHP(2) PHP(3) PHP(4) PHP(5) PHP(6) PHP(7)
                       : COUT : CIN);
        }
      }
#undef CIN
#undef COUT
#undef PHP
#undef PHD
#undef AHEAD
#undef CHAIN
#undef PC
#undef PB
#undef CF
#undef CC
#undef CB
#undef CE
#undef CA
    } else if constexpr (kKind == kFmaSalu) {
      unsigned s0 = it, s1 = it + 1;
#define FS(i) FMA1(i) "s_add_u32 %[s0], %[s0], %[s1]\n\t"
      asm volatile(F8(FS) F8(FS) F8(FS) F8(FS)
                   : OUT8, [s0] "+s"(s0) : [m] "v"(m), [n] "v"(n), [s1] "s"(s1));
#undef FS
      a[0] += static_cast<float>(s0 & 1u);
    } else if constexpr (kKind == kFmaChain) {
#define C1 "v_fmac_f32 %[a0], %[m], %[a0]\n\t"
#define C8 C1 C1 C1 C1 C1 C1 C1 C1
      asm volatile(C8 C8 C8 C8 : [a0] "+v"(a[0]) : [m] "v"(m));
#undef C8
#undef C1
    } else if constexpr (kKind == kExpChain) {
#define E1 "v_exp_f32 %[a0], %[a0]\n\ts_nop 0\n\t"
#define E8 E1 E1 E1 E1 E1 E1 E1 E1
      asm volatile(E8 E8 E8 E8 : [a0] "+v"(a[0]));
#undef E8
#undef E1
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += a[i] + h[i] + p[i] + nn[i];
  sink[static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    clocks[0] = __builtin_amdgcn_s_memtime() - t0;
    clocks[1] = __builtin_amdgcn_s_memrealtime() - r0;
  }
}

__global__ __launch_bounds__(256) void copy_kernel(const float4* __restrict__ src,
                                                   float4* __restrict__ dst, size_t n) {
  const size_t stride = static_cast<size_t>(gridDim.x) * 256;
  for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride)
    dst[i] = src[i];
}

__global__ __launch_bounds__(256) void read_kernel(const float4* __restrict__ src, float* sink,
                                                   size_t n) {
  const size_t stride = static_cast<size_t>(gridDim.x) * 256;
  float s = 0.0f;
  for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride) {
    const float4 v = src[i];
    s += v.x + v.y + v.z + v.w;
  }
  if (s == 12345.678f) sink[0] = s;  // keeps the loads; never true for the zero-filled input
}

// Reads a (T, E) fp32 matrix the way the row scan reads its activations: workgroups of 8 waves
// over 2 x 16 lanes x VEC channels, each lane row of 16 lanes reading one token's 16 x VEC
// contiguous channels (64, 128 or 256 bytes), two tokens per lane per 32-token tile, four tiles
// of loads in flight. T is a multiple of 128 and E of 32 * VEC.
template <int VEC>
__global__ __launch_bounds__(512) void segment_read_kernel(const float* __restrict__ src,
                                                           float* sink, int64_t T, int64_t E) {
  using V = typename std::conditional<VEC == 1, float,
            typename std::conditional<VEC == 2, float2, float4>::type>::type;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int grp = wid / 4, w = wid % 4, q = lane >> 4, c = lane & 15;
  const int64_t ch = static_cast<int64_t>(blockIdx.x) * 32 * VEC + (grp * 16 + c) * VEC;
  const int tau0 = (4 * w + q) * 2;
  float s = 0.0f;
  for (int64_t t = 0; t < T; t += 128) {
    V v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t tok = t + (j / 2) * 32 + tau0 + (j % 2);
      v[j] = *reinterpret_cast<const V*>(src + tok * E + ch);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float* f = reinterpret_cast<const float*>(&v[j]);
#pragma unroll
      for (int i = 0; i < VEC; ++i) s += f[i];
    }
  }
  if (s == 12345.678f) sink[0] = s;  // keeps the loads; never true for the zero-filled input
}

// LDS read / write throughput of one wave pattern: 16 ds_read_b128 (or ds_write_b128) per loop
// iteration per wave, lane addresses by kind: 0 every lane distinct (1 KB of distinct data per
// instruction), 1 distinct within a 16-lane row and equal across the 4 rows (the row scan's
// (dt, dt*u) reads), 2 every lane the same address, 3 ds_write_b128 with distinct lanes.
// Addresses stay within the 16 KB buffer.
constexpr int kLdsKinds = 4;
template <int KIND>
__global__ __launch_bounds__(256) void lds_kernel(int iters, float* sink) {
  __shared__ float4 buf[1024];
  const int lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < 1024; i += 256) buf[i] = make_float4(i, 1.0f, 2.0f, 3.0f);
  __syncthreads();
  const int idx = KIND == 1 ? (lane & 15) : KIND == 2 ? 0 : lane;
  float acc = 0.0f;
  for (int it = 0; it < iters; ++it) {
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if constexpr (KIND == 3) {
        buf[idx + j * 64] = make_float4(acc, acc, acc, acc);
      } else {
        const float4 v = buf[idx + j * 64];
        acc += (v.x + v.y) + (v.z + v.w);
      }
    }
    if constexpr (KIND == 3) acc += 1.0f;
  }
  __syncthreads();
  if constexpr (KIND == 3) acc += buf[(threadIdx.x * 7) & 1023].y;
  sink[static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x] = acc;
}


// Workgroup size of the ALU kinds (threads); the grid keeps 256 * 4 * wps waves in total.
int g_alu_wg_threads = 256;

template <int K>
hipError_t launch_alu(int wps, int iters, float* sink, unsigned long long* clocks,
                      hipStream_t s) {
  const int wg = g_alu_wg_threads;
  hipLaunchKernelGGL(alu_kernel<K>, dim3(256 * 256 * wps / wg), dim3(wg), 0, s, iters, 1.0f, sink,
                     clocks);
  return hipGetLastError();
}

}  // namespace

extern "C" {

// Number of ALU kinds, and the VALU instructions one loop iteration of a kind issues per wave.
int axon_micro_alu_kinds(void) { return kNumKinds; }
int axon_micro_alu_instrs_per_iter(int kind) { return instrs_per_iter(kind); }

// Runs ALU kind `kind` on 256 * 4 * waves_per_simd waves (workgroups of 4 waves, 256 per
// launch step) for `iters` loop iterations, after one untimed launch. out[0] = elapsed ms of the
// timed launch (hipEvents), out[1] = s_memtime ticks and out[2] = s_memrealtime ticks (100 MHz)
// of the first wave. Returns 0 or a hipError_t value.
// Workgroup size (64, 128, 256, 512 or 1024 threads) of the next axon_micro_alu runs; 256 by
// default. Returns 0, or hipErrorInvalidValue for another size.
int axon_micro_alu_set_wg(int threads) {
  if (threads != 64 && threads != 128 && threads != 256 && threads != 512 && threads != 1024)
    return static_cast<int>(hipErrorInvalidValue);
  g_alu_wg_threads = threads;
  return 0;
}

int axon_micro_alu(int kind, int waves_per_simd, int iters, double* out) {
  if (kind < 0 || kind >= kNumKinds || waves_per_simd < 1 || waves_per_simd > 8 || iters < 1 ||
      !out)
    return static_cast<int>(hipErrorInvalidValue);
  float* sink = nullptr;
  unsigned long long* clocks = nullptr;
  hipError_t e = hipMalloc(&sink, sizeof(float) * 256 * 256 * waves_per_simd);
  if (e != hipSuccess) return static_cast<int>(e);
  e = hipMalloc(&clocks, 2 * sizeof(unsigned long long));
  if (e != hipSuccess) {
    (void)hipFree(sink);
    return static_cast<int>(e);
  }
  hipEvent_t e0, e1;
  (void)hipEventCreate(&e0);
  (void)hipEventCreate(&e1);
  auto run = [&](int it) -> hipError_t {
    switch (kind) {
      case kFma: return launch_alu<kFma>(waves_per_simd, it, sink, clocks, nullptr);
      case kExp: return launch_alu<kExp>(waves_per_simd, it, sink, clocks, nullptr);
      case kDpp: return launch_alu<kDpp>(waves_per_simd, it, sink, clocks, nullptr);
      case kPerm32: return launch_alu<kPerm32>(waves_per_simd, it, sink, clocks, nullptr);
      case kUpdate: return launch_alu<kUpdate>(waves_per_simd, it, sink, clocks, nullptr);
      case kExpFma: return launch_alu<kExpFma>(waves_per_simd, it, sink, clocks, nullptr);
      case kFmaSalu: return launch_alu<kFmaSalu>(waves_per_simd, it, sink, clocks, nullptr);
      case kFmaChain: return launch_alu<kFmaChain>(waves_per_simd, it, sink, clocks, nullptr);
      case kExpChain: return launch_alu<kExpChain>(waves_per_simd, it, sink, clocks, nullptr);
      case kExpFma1: return launch_alu<kExpFma1>(waves_per_simd, it, sink, clocks, nullptr);
      case kExpFma2: return launch_alu<kExpFma2>(waves_per_simd, it, sink, clocks, nullptr);
      case kExpFma8: return launch_alu<kExpFma8>(waves_per_simd, it, sink, clocks, nullptr);
      case kChanUpd: return launch_alu<kChanUpd>(waves_per_simd, it, sink, clocks, nullptr);
      case kChanNoExp: return launch_alu<kChanNoExp>(waves_per_simd, it, sink, clocks, nullptr);
      case kBurst16: return launch_alu<kBurst16>(waves_per_simd, it, sink, clocks, nullptr);
      case kBurst8: return launch_alu<kBurst8>(waves_per_simd, it, sink, clocks, nullptr);
      case kBurst16v3: return launch_alu<kBurst16v3>(waves_per_simd, it, sink, clocks, nullptr);
      case kFmaSgpr: return launch_alu<kFmaSgpr>(waves_per_simd, it, sink, clocks, nullptr);
      case kChainDpp: return launch_alu<kChainDpp>(waves_per_simd, it, sink, clocks, nullptr);
      case kChainAhead: return launch_alu<kChainAhead>(waves_per_simd, it, sink, clocks, nullptr);
      case kPhaseDpp: return launch_alu<kPhaseDpp>(waves_per_simd, it, sink, clocks, nullptr);
      case kPhasePlain: return launch_alu<kPhasePlain>(waves_per_simd, it, sink, clocks, nullptr);
      default: return launch_alu<kPerm16>(waves_per_simd, it, sink, clocks, nullptr);
    }
  };
  e = run(iters);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) {
    (void)hipEventRecord(e0, nullptr);
    e = run(iters);
    (void)hipEventRecord(e1, nullptr);
  }
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.0f;
  unsigned long long ck[2] = {0, 0};
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  if (e == hipSuccess) e = hipMemcpy(ck, clocks, sizeof(ck), hipMemcpyDeviceToHost);
  out[0] = ms;
  out[1] = static_cast<double>(ck[0]);
  out[2] = static_cast<double>(ck[1]);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  (void)hipFree(sink);
  (void)hipFree(clocks);
  return static_cast<int>(e);
}

// Runs LDS kind `kind` (lds_kernel) on 256 * waves_per_simd workgroups of 4 waves for `iters`
// iterations after one untimed launch. out[0] = elapsed ms of the timed launch.
int axon_micro_lds_kinds(void) { return kLdsKinds; }
int axon_micro_lds(int kind, int waves_per_simd, int iters, double* out) {
  if (kind < 0 || kind >= kLdsKinds || waves_per_simd < 1 || waves_per_simd > 8 || iters < 1 ||
      !out)
    return static_cast<int>(hipErrorInvalidValue);
  float* sink = nullptr;
  hipError_t e = hipMalloc(&sink, sizeof(float) * 256 * 256 * waves_per_simd);
  if (e != hipSuccess) return static_cast<int>(e);
  auto run = [&](int it) -> hipError_t {
    const dim3 grid(256 * waves_per_simd), block(256);
    switch (kind) {
      case 0: hipLaunchKernelGGL(lds_kernel<0>, grid, block, 0, nullptr, it, sink); break;
      case 1: hipLaunchKernelGGL(lds_kernel<1>, grid, block, 0, nullptr, it, sink); break;
      case 2: hipLaunchKernelGGL(lds_kernel<2>, grid, block, 0, nullptr, it, sink); break;
      default: hipLaunchKernelGGL(lds_kernel<3>, grid, block, 0, nullptr, it, sink); break;
    }
    return hipGetLastError();
  };
  hipEvent_t e0, e1;
  (void)hipEventCreate(&e0);
  (void)hipEventCreate(&e1);
  e = run(iters);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) {
    (void)hipEventRecord(e0, nullptr);
    e = run(iters);
    (void)hipEventRecord(e1, nullptr);
  }
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.0f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  out[0] = ms;
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  (void)hipFree(sink);
  return static_cast<int>(e);
}

// Streams `bytes` (a multiple of 16) through HBM `reps` times after one untimed pass:
// kind 0 = copy (bytes read + bytes written per pass), kind 1 = read only. out[0] = mean ms per
// pass. Workgroups: 256 threads, `blocks` of them (grid-stride loop).
// Kinds 2, 3, 4: the row scan's access pattern (segment_read_kernel) with 64-, 128- and
// 256-byte segments per lane row, over E = 7680 x (1, 2, 4) channels and T = bytes / (4 E) tokens
// (bytes must make T a multiple of 128; `blocks` is unused: E / (32 x VEC) workgroups, 240).
int axon_micro_hbm(int kind, size_t bytes, int reps, int blocks, double* out) {
  if (kind < 0 || kind > 4 || bytes == 0 || bytes % 16 || reps < 1 || blocks < 1 || !out)
    return static_cast<int>(hipErrorInvalidValue);
  const int vec = kind == 2 ? 1 : kind == 3 ? 2 : 4;
  const int64_t seg_e = int64_t(7680) * vec;
  const int64_t seg_t = static_cast<int64_t>(bytes / 4) / seg_e;
  if (kind >= 2 && (static_cast<size_t>(seg_t * seg_e * 4) != bytes || seg_t % 128 || seg_t < 128))
    return static_cast<int>(hipErrorInvalidValue);
  void *src = nullptr, *dst = nullptr;
  hipError_t e = hipMalloc(&src, bytes);
  if (e != hipSuccess) return static_cast<int>(e);
  e = hipMalloc(&dst, kind == 0 ? bytes : 256);
  if (e != hipSuccess) {
    (void)hipFree(src);
    return static_cast<int>(e);
  }
  e = hipMemset(src, 0, bytes);
  const size_t n = bytes / 16;
  auto run = [&]() {
    const unsigned seg_blocks = static_cast<unsigned>(seg_e / (32 * vec));
    if (kind == 0)
      hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(256), 0, nullptr,
                         static_cast<const float4*>(src), static_cast<float4*>(dst), n);
    else if (kind == 2)
      hipLaunchKernelGGL(segment_read_kernel<1>, dim3(seg_blocks), dim3(512), 0, nullptr,
                         static_cast<const float*>(src), static_cast<float*>(dst), seg_t, seg_e);
    else if (kind == 3)
      hipLaunchKernelGGL(segment_read_kernel<2>, dim3(seg_blocks), dim3(512), 0, nullptr,
                         static_cast<const float*>(src), static_cast<float*>(dst), seg_t, seg_e);
    else if (kind == 4)
      hipLaunchKernelGGL(segment_read_kernel<4>, dim3(seg_blocks), dim3(512), 0, nullptr,
                         static_cast<const float*>(src), static_cast<float*>(dst), seg_t, seg_e);
    else
      hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(256), 0, nullptr,
                         static_cast<const float4*>(src), static_cast<float*>(dst), n);
    return hipGetLastError();
  };
  hipEvent_t e0, e1;
  (void)hipEventCreate(&e0);
  (void)hipEventCreate(&e1);
  if (e == hipSuccess) e = run();
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) {
    (void)hipEventRecord(e0, nullptr);
    for (int r = 0; r < reps && e == hipSuccess; ++r) e = run();
    (void)hipEventRecord(e1, nullptr);
  }
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.0f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  out[0] = ms / reps;
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  (void)hipFree(src);
  (void)hipFree(dst);
  return static_cast<int>(e);
}


}  // extern "C"
