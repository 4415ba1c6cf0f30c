// Mamba-2 SSD core on gfx950: the scalar-decay selective scan of "Selective State Space Models
// (Mamba)" (pattern "Mamba-2 block") computed in 64-token chunks, as the SSD article describes
// it: matrix products inside a chunk, a recurrence over chunk states between chunks.
//
// Per (batch b, head h) with a = dt * A (A = -exp(A_log[h]) < 0) and, inside chunk c, the
// inclusive cumulative sum cum_t = a_{t0} + ... + a_t (t0 = first token of the chunk):
//   chunk state   S_c[p, n]   = sum_s exp(cum_last - cum_s) dt_s x_s[p] B_s[n]
//   state entering chunk c:  H_c = exp(cum_last of c-1) H_{c-1} + S_{c-1},  H_0 = state_in
//   y_t[p] = exp(cum_t) sum_n C_t[n] H_c[p, n]                          (incoming state)
//          + sum_{s <= t} (C_t . B_s) exp(cum_t - cum_s) dt_s x_s[p]      (inside the chunk)
//          + D[h] x_t[p]
// The decays are kept as exp2 of base-2 cumulative sums; within one chunk every difference
// cum_t - cum_s with s <= t is <= 0, so nothing overflows. The sums are compensated (a head and
// a tail float per token): once a large step (dt near its upper clip) has pushed cum to
// thousands, a plain fp32 sum would carry an absolute error of its ulp (2.4e-4 at 2048) into
// every later difference, i.e. a relative error of that size in the decays.
//
// Four kernels, in stream order:
//   ssd_gram_kernel   G_c = C_c B_c^T (64 x 64, lower block triangle), shared by all heads.
//   ssd_state_kernel  S_c for every (b, h, c) and the chunk decay exp(cum_last).
//   ssd_carry_kernel  the recurrence over chunks with H_c held on chip, and for every chunk the
//                     incoming-state products C_t . H_c[p] (unscaled); the final state goes to
//                     state_out. H_c itself is never stored.
//   ssd_output_kernel y for every (b, h, c) from those products, G_c and x.
// The contractions run on v_mfma_f32_16x16x4f32 (fp32 in, fp32 accumulate). Operand layout of
// that instruction (wave64, lane l, g = l / 16, i = l % 16): A supplies A[i][k = g], B supplies
// B[k = g][i], and the 16 x 16 result sits as D[4 g + r][i] in the r-th of 4 accumulators. Any
// assignment of the contraction index to (k-step, g) works as long as A and B use the same one.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "axon_device.h"
#include "axonscan.h"

namespace axon {
namespace {

constexpr int kQ = 64;   // tokens per chunk
constexpr int kP = 64;   // head dim
constexpr int kN = 128;  // states
constexpr int kThreads = 256;

typedef float f4 __attribute__((ext_vector_type(4)));

struct SsdArgs {
  const void *x, *dt_raw, *B, *C;
  const float *A_log, *D, *dt_bias;
  float dt_min, dt_max;
  const float* state_in;
  void* y;
  float* state_out;
  float* states;  // (B, H, nc, P, N): S_c
  float* decay;   // (B, H, nc): exp(cum_last) of each chunk
  float* gram;    // (B, nc, Q, Q): C_c B_c^T
  float* yinter;  // (B, H, nc, Q, P): sum_n C_t[n] H_c[p, n]
                  // (before the exp2(cum_t) factor)
  int64_t seqlen, heads;
  int nchunks;
};

__device__ __forceinline__ f4 mfma4(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Four consecutive activations starting at element i (i a multiple of 4), widened to fp32.
__device__ __forceinline__ float4 load4(const float* p, int64_t i) {
  return *reinterpret_cast<const float4*>(p + i);
}
__device__ __forceinline__ float4 load4(const bf16_bits* p, int64_t i) {
  const uint2 v = *reinterpret_cast<const uint2*>(p + i);
  return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u),
                     __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u));
}

// Wave-wide: lane t of the wave is token t of the chunk. Returns dt_t (0 past the sequence end)
// and the inclusive base-2 cumulative sum of dt * A * log2(e) over the chunk up to t as
// hi + lo: every addition of the scan keeps its rounding error (Knuth's two-sum) in lo.
template <typename Act>
__device__ __forceinline__ void chunk_steps(const SsdArgs& a, int64_t b, int64_t h, int64_t tok0,
                                            int lane, float* dt_out, float* hi_out,
                                            float* lo_out) {
  const int64_t tok = tok0 + lane;
  float dt = 0.0f;
  if (tok < a.seqlen) {
    const float v = load_act(static_cast<const Act*>(a.dt_raw), (b * a.seqlen + tok) * a.heads + h);
    dt = step_size(v + a.dt_bias[h], a.dt_min, a.dt_max);
  }
  float hi = dt * decay_rate_log2(a.A_log[h]), lo = 0.0f;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float oh = __shfl_up(hi, d, 64), ol = __shfl_up(lo, d, 64);
    if (lane >= d) {
      const float s = hi + oh;
      const float bv = s - hi;
      const float err = (hi - (s - bv)) + (oh - bv);
      hi = s;
      lo = lo + ol + err;
    }
  }
  *dt_out = dt;
  *hi_out = hi;
  *lo_out = lo;
}

// exp2 of the difference of two compensated sums.
__device__ __forceinline__ float exp2_diff(float hi_a, float lo_a, float hi_b, float lo_b) {
  return __builtin_amdgcn_exp2f((hi_a - hi_b) + (lo_a - lo_b));
}

// Contraction over the 128 states in the gram and output kernels: k-step (jb, jj), jb = 0..7,
// jj = 0..3, lane group g takes n = 16 jb + 4 g + jj, so one 16-byte load per lane and jb gives
// a 16-lane row block 64 contiguous bytes per row.

// ---- G_c = C_c B_c^T -----------------------------------------------------------------------
// Grid (nc, B), 10 waves, one per 16 x 16 block of the lower block triangle: wave v takes row
// block w and column block st <= w (v = w (w + 1) / 2 + st). Its C and B rows are loaded together
// and the contraction over the 128 states runs as four independent accumulator chains (one per
// jj), so a wave waits for one round of loads and its matrix instructions do not wait for each
// other's results.
constexpr int kGramWaves = 10;

template <typename Act>
__global__ __launch_bounds__(64 * kGramWaves) void ssd_gram_kernel(SsdArgs a) {
  const int c = blockIdx.x;
  const int64_t b = blockIdx.y;
  const int lane = threadIdx.x & 63, v = threadIdx.x >> 6, g = lane >> 4, i = lane & 15;
  const int w = v < 1 ? 0 : v < 3 ? 1 : v < 6 ? 2 : 3;
  const int st = v - w * (w + 1) / 2;
  const int64_t tok0 = int64_t(c) * kQ;
  const Act* Cp = static_cast<const Act*>(a.C);
  const Act* Bp = static_cast<const Act*>(a.B);
  float4 crow[8], brow[8];
  {
    const int64_t tc = tok0 + 16 * w + i, tb = tok0 + 16 * st + i;
    const bool okc = tc < a.seqlen, okb = tb < a.seqlen;
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) {
      crow[jb] = okc ? load4(Cp, (b * a.seqlen + tc) * kN + 16 * jb + 4 * g) : float4{};
      brow[jb] = okb ? load4(Bp, (b * a.seqlen + tb) * kN + 16 * jb + 4 * g) : float4{};
    }
  }
  f4 acc[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) acc[jj] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int jb = 0; jb < 8; ++jb) {
    acc[0] = mfma4(crow[jb].x, brow[jb].x, acc[0]);
    acc[1] = mfma4(crow[jb].y, brow[jb].y, acc[1]);
    acc[2] = mfma4(crow[jb].z, brow[jb].z, acc[2]);
    acc[3] = mfma4(crow[jb].w, brow[jb].w, acc[3]);
  }
  float* G = a.gram + (b * a.nchunks + c) * int64_t(kQ * kQ);
#pragma unroll
  for (int r = 0; r < 4; ++r)
    G[(16 * w + 4 * g + r) * kQ + 16 * st + i] = (acc[0][r] + acc[1][r]) + (acc[2][r] + acc[3][r]);
}

// ---- S_c = x^T diag(w) B --------------------------------------------------------------------
// Grid (nc, H / HG, B), 4 HG waves: HG heads of one chunk share the staged B. The chunk's x and
// B are staged in LDS while wave 0 of each head computes its weights w_s = exp(cum_last - cum_s)
// dt_s (x is staged unscaled so that its loads need not wait for them). Wave w of a head computes
// S^T for the head channels p = 16 w .. 16 w + 15 against all 8 blocks of 16 states, A operand
// B^T (rows n), B operand x scaled by w_s as it is read (columns p), contraction index
// s = 4 j + g; the result D[n][p] leaves every lane 4 consecutive states of one channel, stored
// as one 16-byte write. Row strides of 80 and 144 floats put the four lane groups of one LDS read
// in disjoint banks.
constexpr int kXS = kP + 16;
constexpr int kBS = kN + 16;

template <typename Act, int HG>
__global__ __launch_bounds__(kThreads * HG) void ssd_state_kernel(SsdArgs a) {
  __shared__ float xs[HG][kQ * kXS];
  __shared__ float bs[kQ * kBS];
  __shared__ float wsh[HG][kQ];
  const int c = blockIdx.x;
  const int64_t b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, i = lane & 15;
  const int hg = tid >> 8;        // head of this thread within the group
  const int w = (tid >> 6) & 3;  // wave within the head
  const int64_t h = int64_t(blockIdx.y) * HG + hg;
  const int64_t tok0 = int64_t(c) * kQ;
  const int64_t bh = b * a.heads + h;
  if (w == 0) {
    float dt, hi, lo;
    chunk_steps<Act>(a, b, h, tok0, lane, &dt, &hi, &lo);
    const float last_hi = __shfl(hi, 63, 64), last_lo = __shfl(lo, 63, 64);
    wsh[hg][lane] = exp2_diff(last_hi, last_lo, hi, lo) * dt;
    if (lane == 63) a.decay[bh * a.nchunks + c] = __builtin_amdgcn_exp2f(hi + lo);
  }
  const Act* Bp = static_cast<const Act*>(a.B);
  {
    // B (shared by the group's heads): thread -> token tid / (4 HG), 32 / HG states
    constexpr int kPer = 32 / HG;
    const int t = tid / (4 * HG), q = tid % (4 * HG);
    const int64_t tok = tok0 + t;
    const bool ok = tok < a.seqlen;
#pragma unroll
    for (int j = 0; j < kPer; j += 4) {
      const float4 v = ok ? load4(Bp, (b * a.seqlen + tok) * kN + kPer * q + j) : float4{};
      *reinterpret_cast<float4*>(&bs[t * kBS + kPer * q + j]) = v;
    }
  }
  {
    const Act* xp = static_cast<const Act*>(a.x);
    const int t = (tid & 255) >> 2, q = tid & 3;
    const int64_t tok = tok0 + t;
    const bool ok = tok < a.seqlen;
#pragma unroll
    for (int j = 0; j < 16; j += 4) {
      const float4 v = ok ? load4(xp, ((b * a.seqlen + tok) * a.heads + h) * kP + 16 * q + j)
                          : float4{};
      *reinterpret_cast<float4*>(&xs[hg][t * kXS + 16 * q + j]) = v;
    }
  }
  __syncthreads();  // wsh, x and B ready
  f4 acc[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) acc[nt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
  for (int j = 0; j < 16; ++j) {
    const int s = 4 * j + g;
    const float xv = xs[hg][s * kXS + 16 * w + i] * wsh[hg][s];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[nt] = mfma4(bs[s * kBS + 16 * nt + i], xv, acc[nt]);
  }
  float* S = a.states + (bh * a.nchunks + c) * int64_t(kP * kN) + (16 * w + i) * kN + 4 * g;
#pragma unroll
  for (int nt = 0; nt < 8; ++nt)
    *reinterpret_cast<float4*>(S + 16 * nt) =
        make_float4(acc[nt][0], acc[nt][1], acc[nt][2], acc[nt][3]);
}

// ---- recurrence over chunks and the incoming-state products -------------------------------
// Grid (P / 16, H, B), 8 waves. A workgroup owns head channels p0 .. p0 + 15 of one (b, h) and
// walks the chunks in order with that block of the state in registers: waves 0-3 hold states
// 0 .. 63, waves 4-7 states 64 .. 127 (half = 0, 1; n0 = 64 half). Every wave of a half keeps
// that half's whole block (lane (g, i): channel p0 + i, states n0 + 16 k + 4 g .. + 3 for
// k = 0..3). For chunk c, wave w of a half contracts the C rows of tokens 16 w .. 16 w + 15 with
// H_c over the half's 64 states (A operand C, B operand H^T, contraction index n0 + 16 k + 4 g + q
// at k-step (k, q), one accumulator per q: a 16-byte load per lane and k reads 64 contiguous
// bytes of each row) and advances the state: H_{c+1} = exp(cum_last of c) H_c + S_c. The upper
// half leaves its products in LDS; after the chunk's barrier the lower half adds them to its own
// and stores the sum, so the workspace holds one product per output. The next chunk's C rows and
// S slice are loaded while the current chunk is contracted (two register sets, chunks taken in
// pairs).
template <typename Act>
__global__ __launch_bounds__(2 * kThreads) void ssd_carry_kernel(SsdArgs a) {
  const int64_t h = blockIdx.y, b = blockIdx.z;
  const int p0 = 16 * static_cast<int>(blockIdx.x);
  const int tid = threadIdx.x, half = tid >> 8, ht = tid & 255, n0 = 64 * half;
  const int lane = tid & 63, w = ht >> 6, g = lane >> 4, i = lane & 15;
  const int64_t bh = b * a.heads + h;
  const Act* Cp = static_cast<const Act*>(a.C);
  const int64_t srow = (bh * kP + p0 + i) * kN + n0 + 4 * g;  // this lane's part of a state
  float hs[16];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float4 v = a.state_in ? *reinterpret_cast<const float4*>(a.state_in + srow + 16 * k)
                                : float4{0.0f, 0.0f, 0.0f, 0.0f};
    hs[4 * k] = v.x, hs[4 * k + 1] = v.y, hs[4 * k + 2] = v.z, hs[4 * k + 3] = v.w;
  }
  // Every wave has read its state before the first wave of each half may write state_out (which
  // may be state_in).
  __syncthreads();
  // S_c is read from memory once per workgroup: thread t of a half loads 16 bytes of row
  // p0 + t / 16 of the half's block and stores them in LDS where lane (g, i) of every wave of the
  // half reads its k-th float4 (slot 64 k + lane), two chunk buffers alternating. (C rows go
  // straight to registers: staged through LDS as well they took 64 us instead of 43 us at
  // 1 x 2048 x 64 heads.)
  __shared__ float4 ssh[2][2][4 * 64];
  // The upper half's products of a chunk, [chunk parity][wave][r][lane].
  __shared__ float ysh[2][4][4][64];
  const int prow = ht >> 4, pch = ht & 15;
  const float* Sg = a.states + bh * a.nchunks * int64_t(kP * kN) + (p0 + prow) * kN + n0 + 4 * pch;
  const int sdst = (pch >> 2) * 64 + 16 * (pch & 3) + prow;
  float* Y0 = a.yinter + bh * a.nchunks * int64_t(kQ * kP) + (16 * w + 4 * g) * kP + p0 + i;
  float yown[4];  // the lower half's products of the last chunk, until the upper half's are in
  const float* dec = a.decay + bh * a.nchunks;
  // A chunk's inputs: its C rows, this thread's part of its S block and its decay, loaded a chunk
  // ahead of use (the decay with them: loaded next to its use, its wait would also wait for the
  // prefetch).
  auto load = [&](int c, float4 (&cr)[4], float4& sg, float& d) {
    // S first: its LDS store at the end of the current chunk then waits for it alone.
    d = dec[c];
    sg = *reinterpret_cast<const float4*>(Sg + int64_t(c) * (kP * kN));
    // Tokens past the sequence end take the last token's C row (their products are never read),
    // so every lane issues the same loads and the compiler's wait counts stay exact.
    const int64_t tok = int64_t(c) * kQ + 16 * w + i;
    const int64_t row = (b * a.seqlen + (tok < a.seqlen ? tok : a.seqlen - 1)) * kN + n0 + 4 * g;
#pragma unroll
    for (int k = 0; k < 4; ++k) cr[k] = load4(Cp, row + 16 * k);
  };
  auto chunk = [&](const float4 (&cr)[4], float d, const float4* sb, int buf) {
    float4 sr[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) sr[k] = sb[64 * k + lane];
    f4 acc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc[0] = mfma4(cr[k].x, hs[4 * k], acc[0]);
      acc[1] = mfma4(cr[k].y, hs[4 * k + 1], acc[1]);
      acc[2] = mfma4(cr[k].z, hs[4 * k + 2], acc[2]);
      acc[3] = mfma4(cr[k].w, hs[4 * k + 3], acc[3]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = (acc[0][r] + acc[1][r]) + (acc[2][r] + acc[3][r]);
      if (half)
        ysh[buf][w][r][lane] = v;
      else
        yown[r] = v;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      hs[4 * k] = fmaf(d, hs[4 * k], sr[k].x);
      hs[4 * k + 1] = fmaf(d, hs[4 * k + 1], sr[k].y);
      hs[4 * k + 2] = fmaf(d, hs[4 * k + 2], sr[k].z);
      hs[4 * k + 3] = fmaf(d, hs[4 * k + 3], sr[k].w);
    }
  };
  // After the barrier that follows chunk c: the lower half stores the chunk's products.
  auto finish = [&](int c, int buf) {
    if (half == 0) {
      float* Y = Y0 + int64_t(c) * (kQ * kP);
#pragma unroll
      for (int r = 0; r < 4; ++r) Y[r * kP] = yown[r] + ysh[buf][w][r][lane];
    }
  };
  float4 c0[4], c1[4], g0, g1;
  float d0, d1;
  // Prefetches past the last chunk reload the last chunk (unused), so no load sits behind a
  // branch; the scheduling barriers keep each prefetch ahead of the chunk it overlaps. Each
  // chunk's S block is in LDS before the chunk starts; the barrier after a buffer is filled also
  // orders the previous reads of that buffer before its next fill. The same barriers order the
  // upper half's products (ysh[c & 1]) before the lower half reads them, and that read before
  // the upper half refills the buffer two chunks later.
  const int last = a.nchunks - 1;
  load(0, c0, g0, d0);
  ssh[0][half][sdst] = g0;
  __syncthreads();
  for (int c = 0; c < a.nchunks; c += 2) {
    load(c + 1 < last ? c + 1 : last, c1, g1, d1);
    __builtin_amdgcn_sched_barrier(0);
    chunk(c0, d0, ssh[0][half], 0);
    ssh[1][half][sdst] = g1;
    __syncthreads();
    finish(c, 0);
    if (c + 1 > last) break;
    load(c + 2 < last ? c + 2 : last, c0, g0, d0);
    __builtin_amdgcn_sched_barrier(0);
    chunk(c1, d1, ssh[1][half], 1);
    ssh[0][half][sdst] = g0;
    __syncthreads();
    finish(c + 1, 1);
  }
  if (w == 0) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      *reinterpret_cast<float4*>(a.state_out + srow + 16 * k) =
          make_float4(hs[4 * k], hs[4 * k + 1], hs[4 * k + 2], hs[4 * k + 3]);
  }
}

// state_out = state_in (or zeros) for an empty sequence.
__global__ __launch_bounds__(kThreads) void ssd_copy_state_kernel(const float* in, float* out,
                                                                   int64_t n4) {
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= n4) return;
  reinterpret_cast<float4*>(out)[i] =
      in ? reinterpret_cast<const float4*>(in)[i] : float4{0.0f, 0.0f, 0.0f, 0.0f};
}

// ---- outputs ---------------------------------------------------------------------------------
// Grid (nc, H, B), 4 waves; wave w owns tokens 16 w .. 16 w + 15 of the chunk and all 64 head
// channels (4 column blocks). Intra-chunk term: contraction over s = 16 st + 4 g + j for the
// column blocks st <= w, the A operand being G scaled by the decay mask, the B operand x from
// LDS (row stride 68 floats: the four lane groups, 4 rows apart, hit disjoint banks).
// Incoming-state term: the carry kernel's products C_t . H_c[p], scaled by exp2(cum_t).
constexpr int kXO = kP + 4;

template <typename Act>
__global__ __launch_bounds__(kThreads) void ssd_output_kernel(SsdArgs a) {
  __shared__ float xs[kQ * kXO];
  __shared__ float cum_hi[kQ];
  __shared__ float cum_lo[kQ];
  __shared__ float dts[kQ];
  const int c = blockIdx.x;
  const int64_t h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, i = lane & 15;
  const int64_t tok0 = int64_t(c) * kQ;
  const int64_t bh = b * a.heads + h;
  const Act* xp = static_cast<const Act*>(a.x);
  if (w == 0) {
    float dt, hi, lo;
    chunk_steps<Act>(a, b, h, tok0, lane, &dt, &hi, &lo);
    dts[lane] = dt;
    cum_hi[lane] = hi;
    cum_lo[lane] = lo;
  }
  {
    const int t = tid >> 2, q = tid & 3;
    const int64_t tok = tok0 + t;
    const bool ok = tok < a.seqlen;
#pragma unroll
    for (int j = 0; j < 16; j += 4) {
      const float4 v = ok ? load4(xp, ((b * a.seqlen + tok) * a.heads + h) * kP + 16 * q + j)
                          : float4{};
      *reinterpret_cast<float4*>(&xs[t * kXO + 16 * q + j]) = v;
    }
  }
  // The incoming-state products of this lane's outputs (token 16 w + 4 g + r, channel 16 pt + i).
  float yin[4][4];
  {
    const float* Yi = a.yinter + (bh * a.nchunks + c) * int64_t(kQ * kP) +
                      (16 * w + 4 * g) * kP + i;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
        yin[r][pt] = Yi[r * kP + 16 * pt];
  }
  __syncthreads();  // xs, cum_hi, cum_lo, dts ready
  f4 acc[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = 16 * w + 4 * g + r;
    const float e = __builtin_amdgcn_exp2f(cum_hi[t] + cum_lo[t]);
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) acc[pt][r] = e * yin[r][pt];
  }
  {
    const int t = 16 * w + i;  // A-operand row
    const float hi_t = cum_hi[t], lo_t = cum_lo[t];
    const float* G = a.gram + (b * a.nchunks + c) * int64_t(kQ * kQ) + t * kQ;
    for (int st = 0; st <= w; ++st) {
      const int s0 = 16 * st + 4 * g;
      const float4 gv = *reinterpret_cast<const float4*>(G + s0);
      const float gj[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int s = s0 + j;
        const float m =
            s <= t ? gj[j] * exp2_diff(hi_t, lo_t, cum_hi[s], cum_lo[s]) * dts[s] : 0.0f;
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc[pt] = mfma4(m, xs[s * kXO + 16 * pt + i], acc[pt]);
      }
    }
  }
  Act* yp = static_cast<Act*>(a.y);
  const float Dh = a.D[h];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = 16 * w + 4 * g + r;
    const int64_t tok = tok0 + t;
    if (tok >= a.seqlen) continue;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const int p = 16 * pt + i;
      store_act(yp, ((b * a.seqlen + tok) * a.heads + h) * kP + p,
                fmaf(Dh, xs[t * kXO + p], acc[pt][r]));
    }
  }
}

// ---- host side -------------------------------------------------------------------------------
constexpr int64_t kMaxGrid = 65535;
constexpr int64_t kMaxElems = int64_t(1) << 40;

struct SsdPlan {
  int64_t nchunks = 0;
  size_t off_states = 0, off_decay = 0, off_gram = 0, off_yinter = 0, bytes = 0;
};

size_t round_up(size_t v, size_t m) { return (v + m - 1) / m * m; }

bool shape_valid(const axon_ssd_shape* s, axon_status* why) {
  *why = AXON_ERR_INVALID_ARGUMENT;
  if (!s) return false;
  if (s->batch < 1 || s->n_heads < 1 || s->seqlen < 0) return false;
  *why = AXON_ERR_UNSUPPORTED;
  if (s->head_dim != kP || s->d_state != kN) return false;
  if (s->act_dtype != AXON_F32 && s->act_dtype != AXON_BF16) return false;
  if (s->batch > kMaxGrid || s->n_heads > kMaxGrid) return false;
  *why = AXON_ERR_INVALID_ARGUMENT;
  int64_t t = 0;
  if (__builtin_mul_overflow(s->batch, s->seqlen, &t) ||
      __builtin_mul_overflow(t, s->n_heads * kP, &t) || t > kMaxElems)
    return false;
  if ((s->seqlen + kQ - 1) / kQ > (int64_t(1) << 30)) return false;
  *why = AXON_OK;
  return true;
}

SsdPlan plan_ssd(const axon_ssd_shape* s) {
  SsdPlan p;
  p.nchunks = (s->seqlen + kQ - 1) / kQ;
  if (p.nchunks == 0) return p;
  const size_t BH = size_t(s->batch) * size_t(s->n_heads);
  p.off_states = 0;
  p.off_decay = round_up(p.off_states + sizeof(float) * BH * p.nchunks * kP * kN, 256);
  p.off_gram = round_up(p.off_decay + sizeof(float) * BH * p.nchunks, 256);
  p.off_yinter = round_up(p.off_gram + sizeof(float) * size_t(s->batch) * p.nchunks * kQ * kQ, 256);
  p.bytes = round_up(p.off_yinter + sizeof(float) * BH * p.nchunks * kQ * kP, 256);
  return p;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
  uintptr_t lo = 0, hi = 0;
};
Span span(const void* p, size_t bytes) {
  Span s;
  if (p && bytes) s.lo = reinterpret_cast<uintptr_t>(p), s.hi = s.lo + bytes;
  return s;
}
bool overlaps(const Span& x, const Span& y) {
  return x.lo < x.hi && y.lo < y.hi && x.lo < y.hi && y.lo < x.hi;
}

template <typename Act>
void launch_all(const SsdArgs& a, int64_t batch, hipStream_t st) {
  const dim3 blk(kThreads);
  const unsigned nc = static_cast<unsigned>(a.nchunks);
  const unsigned H = static_cast<unsigned>(a.heads), B = static_cast<unsigned>(batch);
  hipLaunchKernelGGL(ssd_gram_kernel<Act>, dim3(nc, B), dim3(64 * kGramWaves), 0, st, a);
  // Two heads per workgroup where the head count allows (37.6 us against 44.8 us for one and
  // 41.0 us for four at 1 x 2048 x 64 heads: LDS then holds two workgroups per CU).
  if (H % 2 == 0)
    hipLaunchKernelGGL((ssd_state_kernel<Act, 2>), dim3(nc, H / 2, B), dim3(2 * kThreads), 0, st,
                       a);
  else
    hipLaunchKernelGGL((ssd_state_kernel<Act, 1>), dim3(nc, H, B), blk, 0, st, a);
  hipLaunchKernelGGL(ssd_carry_kernel<Act>, dim3(kP / 16, H, B), dim3(2 * kThreads), 0, st, a);
  hipLaunchKernelGGL(ssd_output_kernel<Act>, dim3(nc, H, B), blk, 0, st, a);
}

}  // namespace
}  // namespace axon

extern "C" {

size_t axon_ssd_scan_workspace_bytes(const axon_ssd_shape* shape) {
  axon_status why;
  if (!axon::shape_valid(shape, &why)) return 0;
  return axon::plan_ssd(shape).bytes;
}

axon_status axon_ssd_scan(const axon_ssd_shape* shape, const axon_ssd_params* params,
                          const void* x, const void* dt_raw, const void* B, const void* C,
                          const float* state_in, void* y, float* state_out, void* workspace,
                          size_t workspace_bytes, void* stream) {
  using namespace axon;
  axon_status why;
  if (!shape_valid(shape, &why)) return why;
  if (!params) return AXON_ERR_INVALID_ARGUMENT;
  const float* pp[] = {params->A_log, params->D, params->dt_bias};
  for (const float* q : pp)
    if (!q || !aligned16(q)) return AXON_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(params->dt_min) || !std::isfinite(params->dt_max) || params->dt_min < 0.0f ||
      params->dt_min > params->dt_max)
    return AXON_ERR_INVALID_ARGUMENT;
  if (!state_out || !aligned16(state_out) || (state_in && !aligned16(state_in)))
    return AXON_ERR_INVALID_ARGUMENT;
  const int64_t Bsz = shape->batch, L = shape->seqlen, H = shape->n_heads;
  const size_t es = shape->act_dtype == AXON_BF16 ? 2 : 4;
  const size_t state_bytes = sizeof(float) * size_t(Bsz * H) * kP * kN;
  const SsdPlan plan = plan_ssd(shape);
  Span in_state = span(state_in, state_bytes), out_state = span(state_out, state_bytes);
  if (state_in != state_out && overlaps(in_state, out_state)) return AXON_ERR_INVALID_ARGUMENT;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (L == 0) {
    if (state_in == state_out) return AXON_OK;
    const int64_t n4 = int64_t(state_bytes / 16);
    hipLaunchKernelGGL(ssd_copy_state_kernel, dim3(unsigned((n4 + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, st, state_in, state_out, n4);
    return hipGetLastError() == hipSuccess ? AXON_OK : AXON_ERR_HIP;
  }
  const void* act_in[] = {x, dt_raw, B, C, y};
  for (const void* q : act_in)
    if (!q || !aligned16(q)) return AXON_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < plan.bytes) return AXON_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace || !aligned16(workspace)) return AXON_ERR_INVALID_ARGUMENT;
  const size_t tok = size_t(Bsz) * size_t(L);
  const Span in_x = span(x, es * tok * H * kP), in_dt = span(dt_raw, es * tok * H),
             in_b = span(B, es * tok * kN), in_c = span(C, es * tok * kN),
             out_y = span(y, es * tok * H * kP), ws = span(workspace, plan.bytes);
  const Span par[] = {span(params->A_log, 4 * H), span(params->D, 4 * H),
                      span(params->dt_bias, 4 * H)};
  const Span reads[] = {in_x, in_dt, in_b, in_c, in_state, par[0], par[1], par[2]};
  for (const Span& r : reads) {
    if (overlaps(out_y, r) || overlaps(ws, r)) return AXON_ERR_INVALID_ARGUMENT;
    if (state_out != state_in && overlaps(out_state, r)) return AXON_ERR_INVALID_ARGUMENT;
  }
  if (overlaps(out_y, out_state) || overlaps(out_y, ws) || overlaps(out_state, ws))
    return AXON_ERR_INVALID_ARGUMENT;
  if (state_in == state_out) {
    // In place: only the state itself may be shared.
    const Span others[] = {in_x, in_dt, in_b, in_c, par[0], par[1], par[2]};
    for (const Span& r : others)
      if (overlaps(out_state, r)) return AXON_ERR_INVALID_ARGUMENT;
  }
  SsdArgs a;
  a.x = x, a.dt_raw = dt_raw, a.B = B, a.C = C;
  a.A_log = params->A_log, a.D = params->D, a.dt_bias = params->dt_bias;
  a.dt_min = params->dt_min, a.dt_max = params->dt_max;
  a.state_in = state_in, a.y = y, a.state_out = state_out;
  char* w = static_cast<char*>(workspace);
  a.states = reinterpret_cast<float*>(w + plan.off_states);
  a.decay = reinterpret_cast<float*>(w + plan.off_decay);
  a.gram = reinterpret_cast<float*>(w + plan.off_gram);
  a.yinter = reinterpret_cast<float*>(w + plan.off_yinter);
  a.seqlen = L, a.heads = H, a.nchunks = static_cast<int>(plan.nchunks);
  if (shape->act_dtype == AXON_BF16)
    launch_all<bf16_bits>(a, Bsz, st);
  else
    launch_all<float>(a, Bsz, st);
  return hipGetLastError() == hipSuccess ? AXON_OK : AXON_ERR_HIP;
}

}  // extern "C"
