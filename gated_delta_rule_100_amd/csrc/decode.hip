// decode.hip -- one-token gated delta rule step on gfx950.
//
// Per (sequence, head) the fp32 state S (dv x dk, dk contiguous) is read once
// and written once; that stream is the whole cost (64 KiB each way per head at
// dk = dv = 128), so the kernel is an HBM stream:
//   * rows are independent, so each 256-thread workgroup takes 32 rows of one
//     (sequence, head) (16 KiB): many small workgroups keep the stream
//     smoother than one 64 KiB workgroup per head (measured 6.2 against
//     5.8 TB/s on the decode shape, with bitwise-equal results);
//   * 16 lanes per state row, each lane holding dk/16 columns as 16-byte
//     vectors, so one wave-wide load covers four contiguous row segments of
//     256 bytes -- fully used 128-byte lines;
//   * every load of the state is issued before any arithmetic, non-temporal
//     (the state is touched once), the rank-1 update happens in registers and
//     the rows are stored back in place; no LDS (the state has no reuse -- the
//     register-direct load of the FlashInfer PR #7156 page, code analysis 1);
//   * the two row dot products (s.k before the update, s'.q after) are
//     16-lane DPP reductions.
// Row i, with a = s_i . k:   u_i = beta (v_i - alpha a),  s_i' = alpha s_i + u_i k,
// o_i = s_i' . q  -- the recurrence S' = alpha S (I - beta k k^T) + beta v k^T,
// o = S' q written out per row.
#include "gdr_device.h"
#include "launch.h"
#include "mfma_planes.h"

namespace gdr {
namespace {

constexpr int kDecodeThreads = 256;
constexpr int kDecodeRowsPerThread = 2;  // 32 state rows per workgroup

// Rows per thread at dv (at most dv / 16 row groups' worth).
template <int DV>
constexpr int decode_rows_per_thread() {
  return kDecodeRowsPerThread < DV / (kDecodeThreads / 16) ? kDecodeRowsPerThread
                                                           : DV / (kDecodeThreads / 16);
}

// One state row of the decode step, shared by every decode-type kernel so that
// their results agree bit for bit: a = s.k, u = beta (v - alpha a),
// s' = alpha s + u k in place, returns s'.q (both dots reduced over the row's
// 16 lanes).  Contraction into fused multiply-adds is switched off and the
// fused operations are written out, so the instruction sequence does not
// depend on how the compiler schedules the surrounding kernel.
template <int VEC>
__device__ __forceinline__ float update_row(floatx4 (&st)[VEC], const float (&kk)[VEC][4],
                                            const float (&qq)[VEC][4], float alpha, float b,
                                            float v) {
#pragma clang fp contract(off)
  float a = 0.f;
#pragma unroll
  for (int j = 0; j < VEC; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) a = __builtin_fmaf(st[j][e], kk[j][e], a);
  a = row16_sum(a);
  const float u = b * __builtin_fmaf(-alpha, a, v);
  float p = 0.f;
#pragma unroll
  for (int j = 0; j < VEC; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = __builtin_fmaf(alpha, st[j][e], u * kk[j][e]);
      st[j][e] = x;
      p = __builtin_fmaf(x, qq[j][e], p);
    }
  return row16_sum(p);
}

template <int DK, int DV, Dt IN, Dt OUT, int RPT>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, float* __restrict__ state,
    void* __restrict__ o, int NH) {
  constexpr int LPR = 16;               // lanes per state row
  constexpr int CPL = DK / LPR;         // columns per lane (8 or 4)
  constexpr int VEC = CPL / 4;          // float4 per lane per row
  constexpr int RG = kDecodeThreads / LPR;  // row groups (16)
  constexpr int ROWS = RG * RPT;        // state rows per workgroup
  constexpr int WPP = DV / ROWS;        // workgroups per (sequence, head)
  static_assert(CPL % 4 == 0 && DV % ROWS == 0, "shape");

  const int pair = blockIdx.x / WPP, r0 = (blockIdx.x % WPP) * ROWS;
  if (pair >= NH) return;
  const int lane16 = threadIdx.x & (LPR - 1);
  const int rg = threadIdx.x / LPR;

  floatx4* S = reinterpret_cast<floatx4*>(state + static_cast<size_t>(pair) * DV * DK);

  // Issue every state load first.  The state is touched exactly once, so the
  // loads and stores are non-temporal (they do not displace reusable lines).
  floatx4 st[RPT][VEC];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = r0 + rg + RG * i;
#pragma unroll
    for (int j = 0; j < VEC; ++j)
      st[i][j] = __builtin_nontemporal_load(&S[(row * DK + 4 * lane16 + 64 * j) / 4]);
  }

  float kk[VEC][4], qq[VEC][4], vv[RPT];
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    load_vec<IN, 4>(k, static_cast<size_t>(pair) * DK + 4 * lane16 + 64 * j, kk[j]);
    load_vec<IN, 4>(q, static_cast<size_t>(pair) * DK + 4 * lane16 + 64 * j, qq[j]);
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    vv[i] = load_scalar<IN>(v, static_cast<size_t>(pair) * DV + r0 + rg + RG * i);
  const float alpha = expf(g[pair]);
  const float b = beta[pair];

  float oi[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) oi[i] = update_row<VEC>(st[i], kk, qq, alpha, b, vv[i]);

#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = r0 + rg + RG * i;
#pragma unroll
    for (int j = 0; j < VEC; ++j)
      __builtin_nontemporal_store(st[i][j], &S[(row * DK + 4 * lane16 + 64 * j) / 4]);
  }
  // lane i of each row group writes the output of its i-th row
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    if (lane16 == i) store_scalar<OUT>(o, static_cast<size_t>(pair) * DV + r0 + rg + RG * i, oi[i]);
}

// Multi-token decode: T tokens per (sequence, head) applied in order to a state
// that stays in registers, so the state is read once and written once whatever
// T is.  Token t of sequence n is row n*T + t of q, k, v, g, beta and o (a
// packed batch of N sequences of T tokens).  Optionally the state after every
// token is written to `inter` (for rolling back rejected draft tokens), and the
// final state to `state_out` (which may be the input state; NULL keeps the
// input state as it is).  The per-token arithmetic is that of decode_kernel.
template <int DK, int DV, Dt IN, Dt OUT, int RPT>
__global__ __launch_bounds__(kDecodeThreads) void mtp_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const float* state_in,
    float* state_out, void* __restrict__ o, float* __restrict__ inter, int NH, int H, int T) {
  constexpr int LPR = 16;
  constexpr int CPL = DK / LPR;
  constexpr int VEC = CPL / 4;
  constexpr int RG = kDecodeThreads / LPR;
  constexpr int ROWS = RG * RPT;        // state rows per workgroup
  constexpr int WPP = DV / ROWS;        // workgroups per (sequence, head)
  static_assert(CPL % 4 == 0 && DV % ROWS == 0, "shape");

  const int pair = blockIdx.x / WPP, r0 = (blockIdx.x % WPP) * ROWS;
  if (pair >= NH) return;
  const int n = pair / H, h = pair % H;
  const int lane16 = threadIdx.x & (LPR - 1);
  const int rg = threadIdx.x / LPR;

  const floatx4* Sin = reinterpret_cast<const floatx4*>(state_in + static_cast<size_t>(pair) * DV * DK);
  floatx4 st[RPT][VEC];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = r0 + rg + RG * i;
#pragma unroll
    for (int j = 0; j < VEC; ++j)
      st[i][j] = __builtin_nontemporal_load(&Sin[(row * DK + 4 * lane16 + 64 * j) / 4]);
  }

  // inputs of token t, loaded one token ahead
  float kk[VEC][4], qq[VEC][4], vv[RPT], gg, bb;
  auto load_token = [&](int t, float (&k_)[VEC][4], float (&q_)[VEC][4], float (&v_)[RPT],
                        float& g_, float& b_) {
    const size_t row = static_cast<size_t>(n) * T + t;  // token row
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      load_vec<IN, 4>(k, (row * H + h) * DK + 4 * lane16 + 64 * j, k_[j]);
      load_vec<IN, 4>(q, (row * H + h) * DK + 4 * lane16 + 64 * j, q_[j]);
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) v_[i] = load_scalar<IN>(v, (row * H + h) * DV + r0 + rg + RG * i);
    g_ = g[row * H + h];
    b_ = beta[row * H + h];
  };
  load_token(0, kk, qq, vv, gg, bb);

  for (int t = 0; t < T; ++t) {
    float nk[VEC][4], nq[VEC][4], nv[RPT], ng, nb;
    load_token(t + 1 < T ? t + 1 : t, nk, nq, nv, ng, nb);
    const float alpha = expf(gg);
    const size_t orow = ((static_cast<size_t>(n) * T + t) * H + h) * DV;
    float oi[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) oi[i] = update_row<VEC>(st[i], kk, qq, alpha, bb, vv[i]);
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      if (lane16 == i) store_scalar<OUT>(o, orow + r0 + rg + RG * i, oi[i]);
    if (inter) {
      floatx4* I = reinterpret_cast<floatx4*>(inter + orow * DK);
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int row = r0 + rg + RG * i;
#pragma unroll
        for (int j = 0; j < VEC; ++j) I[(row * DK + 4 * lane16 + 64 * j) / 4] = st[i][j];
      }
    }
#pragma unroll
    for (int j = 0; j < VEC; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kk[j][e] = nk[j][e];
        qq[j][e] = nq[j][e];
      }
#pragma unroll
    for (int i = 0; i < RPT; ++i) vv[i] = nv[i];
    gg = ng;
    bb = nb;
  }

  if (state_out) {
    floatx4* Sout = reinterpret_cast<floatx4*>(state_out + static_cast<size_t>(pair) * DV * DK);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = r0 + rg + RG * i;
#pragma unroll
      for (int j = 0; j < VEC; ++j)
        __builtin_nontemporal_store(st[i][j], &Sout[(row * DK + 4 * lane16 + 64 * j) / 4]);
    }
  }
}

// Multi-token decode on the matrix cores (T >= 2 tokens, no per-token states;
// the kernel itself takes any T >= 1).  The tokens of a (sequence, head) go in
// chunks of 8 (the last may be shorter), each one chunk of the chunked form of
// the recurrence applied to the state, which stays in registers from the
// first chunk to the last.  For a chunk of T tokens (derived from the
// recurrence: G_t = g_1 + ... + g_t, gamma_t = e^{G_t}, D_t = e^{G_T - G_t},
// A_ts = beta_t e^{G_t - G_s} k_t.k_s for s < t, Tinv = (I + A)^{-1},
// P_ts = e^{G_t - G_s} q_t.k_s for s <= t):
//   Z = S K^T, Y = S Q^T                         (one product: [K; Q] stacked)
//   U = (diag(beta) (V - diag(gamma) Z)) Tinv^T  per state row
//   O = diag(gamma) Y + U P^T                    (o_t = S_t q_t for every t)
//   S <- gamma_T S + U diag(D) K
// in fp32 on v_mfma_f32_16x16x4_f32 (with bf16 inputs, [Z | Y] and the state
// update on the bf16 matrix cores, their fp32 operand as two bf16 planes).
// A workgroup holds 64 state rows, a
// wave 16: lane (c, g) holds S[row c][16 kt + 4 g + e], which is at once the A
// operand of S K^T (the contraction index permuted the same way in both
// operands) and the accumulator layout of S^T <- gamma_T S^T + K^T diag(D) U^T,
// so the state is never moved between lanes.  The T x T factors are formed by
// every workgroup of a head (they are small).
constexpr int kMtpWaves = 4;               // 16 state rows each
constexpr int kMtpMaxT = 8;
// From this many tokens on the chunked kernel is the faster: it costs about
// the same for any T <= 8 (on 64 sequences x 32 heads, d = 128, bf16, four
// states in rotation: 47-48 us at T = 2 to 6, against 48, 53, 60 and 49 us
// token by token at T = 2, 3, 4 and 5); T = 1 stays token by token, which is
// the decode step bit for bit.
constexpr int kMtpChunkMinT = 2;

// Waves (16 state rows each) of a workgroup at dv.
template <int DV>
constexpr int mtp_waves() {
  return DV / 16 < kMtpWaves ? DV / 16 : kMtpWaves;
}

__device__ __forceinline__ floatx4 mfma4(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// MULTI: T > 8 (more than one chunk; the chunk loop holds the state in
// registers through the factor phase of every later chunk, which needs
// registers for four waves per SIMD instead of five).
template <int DK, int DV, Dt IN, Dt OUT, bool MULTI>
// (one chunk: at least 5 waves per SIMD, which keeps the accumulators out of
// a second register file; 4 waves by default were slower)
__global__ __launch_bounds__(64 * kMtpWaves, MULTI ? 4 : 5) void mtp_chunk_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const float* state_in,
    float* state_out, void* __restrict__ o, int NH, int H, int T) {
  constexpr int NW = mtp_waves<DV>(), kMtpThreads = 64 * NW, kMtpRows = 16 * NW;
  constexpr int WPP = DV / kMtpRows;  // workgroups per (sequence, head)
  constexpr int KT = DK / 16;         // 16-column tiles of the state
  constexpr int LDK = DK + 4;         // padded row of the token matrix (floats)
  constexpr int TPT = 16 * DK / kMtpThreads;  // token-matrix elements per thread
  constexpr int XLD = 9;              // row stride of the per-wave R / U exchange
  // factor region offsets (floats)
  constexpr int F_GRAW = 0, F_B = 8, F_G = 16, F_GAM = 24, F_D = 32, F_TINV = 40, F_P = 104,
                F_DOT = 168, F_A = 296, F_N = 360;
  static_assert(DV % kMtpRows == 0 && DK % 16 == 0, "shape");
  static_assert(kMtpThreads >= 128, "the factor step gives one thread to each entry of A and P");
  __shared__ __align__(16) float sKQ[16 * LDK];  // rows 0-7: k_t, rows 8-15: q_t (zero past the chunk)
  __shared__ __align__(16) float sF[F_N];
  __shared__ __align__(16) float sX[NW][16 * XLD];
  constexpr int TLD = 68;  // padded row of the per-wave state staging (floats)
  __shared__ __align__(16) float sT[NW][16 * TLD];
  // MULTI: the next chunk's k and q rows ([16][DK]) and v rows of this
  // workgroup ([8 tokens][kMtpRows]) as stored in memory, copied in while the
  // current chunk is applied (1 KiB per copy instruction)
  constexpr int ESZ = IN == Dt::BF16 ? 2 : 4;
  constexpr int KQ_BYTES = 16 * DK * ESZ, V_BYTES = kMtpMaxT * kMtpRows * ESZ;
  static_assert(KQ_BYTES % 1024 == 0 && V_BYTES % 1024 == 0, "copy tiling");
  __shared__ __align__(1024) unsigned char sStage[MULTI ? KQ_BYTES + V_BYTES : 1024];

  const int pair = blockIdx.x / WPP, r0 = (blockIdx.x % WPP) * kMtpRows;
  if (pair >= NH) return;
  const int n = pair / H, h = pair % H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c = lane & 15, gq = lane >> 4;
  const int rbase = r0 + 16 * wave;  // first state row of this wave
  const size_t seq0 = static_cast<size_t>(n) * T;  // the sequence's first token

  // The inputs of the Tc tokens from token tok0 on (a chunk of at most 8):
  // k and q rows, gates, and v of this lane's four rows at token c (lanes
  // c < Tc of the first 8).
  float tk[TPT], gv, bv, vv[4];
  auto load_tokens = [&](size_t tok0, int Tc) {
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int idx = tid + kMtpThreads * i, rr = idx / DK, col = idx % DK, t = rr & 7;
      tk[i] = t < Tc ? load_scalar<IN>(rr < 8 ? k : q, ((tok0 + t) * H + h) * DK + col) : 0.f;
    }
    gv = 0.f;
    bv = 0.f;
    if (tid < kMtpMaxT && tid < Tc) {
      gv = g[(tok0 + tid) * H + h];
      bv = beta[(tok0 + tid) * H + h];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      vv[e] = c < Tc ? load_scalar<IN>(v, ((tok0 + c) * H + h) * DV + rbase + 4 * gq + e) : 0.f;
  };
  // The first chunk's inputs first (a wait for them then does not wait for
  // the state).
  load_tokens(seq0, T < kMtpMaxT ? T : kMtpMaxT);
  // The state arrives in 256-byte row pieces (an instruction covers 4 rows x
  // 256 B: register j holds row 4 (j % 4) + lane / 16, columns
  // 64 (j / 4) + 4 (lane % 16)); the wave's own LDS rows turn it into the
  // matrix-core layout below, S[row c][16 kt + 4 gq + e], which read straight
  // from memory covers only 16 rows x 64 B per instruction.
  const floatx4* Sin = reinterpret_cast<const floatx4*>(state_in + static_cast<size_t>(pair) * DV * DK);
  floatx4 ld[KT];
#pragma unroll
  for (int j = 0; j < KT; ++j)
    ld[j] = __builtin_nontemporal_load(
        &Sin[((rbase + 4 * (j & 3) + (lane >> 4)) * DK + 64 * (j >> 2) + 4 * (lane & 15)) / 4]);

  // MULTI: the rows of the Tc tokens from token tok0 on into sStage (rows of
  // tokens t >= Tc repeat the last token; they are zeroed on the way to sKQ),
  // and their gates into gv, bv.
  auto stage_tokens = [&](size_t tok0, int Tc) {
    constexpr int NI = (KQ_BYTES + V_BYTES) / 1024;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
    for (int x = 0; x < (NI + NW - 1) / NW; ++x) {
      const int i = wv + NW * x;
      if (i >= NI) break;  // wave-uniform
      const int b = 1024 * i + 16 * lane;
      const char* src;
      if (b < KQ_BYTES) {
        const int r = b / (DK * ESZ), cb = b % (DK * ESZ), t = r & 7;
        const size_t tt = tok0 + (t < Tc ? t : Tc - 1);
        src = static_cast<const char*>(r < 8 ? k : q) + (tt * H + h) * DK * ESZ + cb;
      } else {
        const int bv_ = b - KQ_BYTES, t = bv_ / (kMtpRows * ESZ), cb = bv_ % (kMtpRows * ESZ);
        const size_t tt = tok0 + (t < Tc ? t : Tc - 1);
        src = static_cast<const char*>(v) + (tt * H + h) * DV * ESZ + r0 * ESZ + cb;
      }
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src),
                                       (__attribute__((address_space(3))) void*)(sStage + 1024 * i),
                                       16, 0, 0);
    }
    gv = 0.f;
    bv = 0.f;
    if (tid < kMtpMaxT && tid < Tc) {
      gv = g[(tok0 + tid) * H + h];
      bv = beta[(tok0 + tid) * H + h];
    }
  };
  auto staged = [&](int byte) -> float {
    if constexpr (IN == Dt::BF16)
      return bf16_bits_to_f32(*reinterpret_cast<const uint16_t*>(sStage + byte));
    else
      return *reinterpret_cast<const float*>(sStage + byte);
  };

  float* W = sT[wave];
  floatx4 st[KT];
  // The chunk of Tc tokens from token tok0 on: its k and q rows and gates into
  // LDS (from the registers load_tokens filled, or for later chunks from
  // sStage), its gate prefix, dots, A, P and Tinv.
  auto setup_chunk = [&](int Tc, auto lean) {
    if constexpr (decltype(lean)::value) {
#pragma unroll
      for (int i = 0; i < TPT; ++i) {
        const int idx = tid + kMtpThreads * i, rr = idx / DK, col = idx % DK;
        sKQ[rr * LDK + col] = (rr & 7) < Tc ? staged((rr * DK + col) * ESZ) : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        vv[e] = c < Tc ? staged(KQ_BYTES + (c * kMtpRows + 16 * wave + 4 * gq + e) * ESZ) : 0.f;
    } else {
#pragma unroll
      for (int i = 0; i < TPT; ++i) {
        const int idx = tid + kMtpThreads * i;
        sKQ[(idx / DK) * LDK + idx % DK] = tk[i];
      }
    }
    if (tid < kMtpMaxT) {
      sF[F_GRAW + tid] = gv;
      sF[F_B + tid] = bv;
    }
    lds_barrier();  // the state loads stay in flight

    // Gate prefix (fixed order; padding adds g = 0, so G_7 = G_T) and the dot
    // products k_t.k_s (slots 8 t + s) and q_t.k_s (slots 64 + 8 t + s), t, s < 8.
    if (tid < kMtpMaxT) {
      float G = 0.f, Gt = 0.f;
      for (int s = 0; s < kMtpMaxT; ++s) {
        G += sF[F_GRAW + s];
        if (s == tid) Gt = G;
      }
      sF[F_G + tid] = Gt;
      sF[F_GAM + tid] = expf(Gt);
      sF[F_D + tid] = tid < Tc ? expf(G - Gt) : 0.f;
    }
    if (wave == 1) {
      // [K; Q] K^T on the matrix cores (one wave, beside the gate prefix):
      // D[r][s] = k_r.k_s (r < 8) or q_{r-8}.k_s, s < 8; B is A's first eight
      // rows (zero beyond), the contraction index in the same order in both.
      const float* row = sKQ + c * LDK;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (IN == Dt::BF16) {
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) {
          const floatx4 x0 = *reinterpret_cast<const floatx4*>(row + 32 * kb + 8 * gq);
          const floatx4 x1 = *reinterpret_cast<const floatx4*>(row + 32 * kb + 8 * gq + 4);
          float xs[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            xs[e] = x0[e];
            xs[4 + e] = x1[e];
          }
          bf16x8 a[1];
          split8<1>(xs, a);  // exact: bf16 inputs
          const bf16x8 b = c < kMtpMaxT ? a[0] : bf16x8{};
          acc = mfma16x16x32(a[0], b, acc);
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < DK / 16; ++kk) {
          const floatx4 x = *reinterpret_cast<const floatx4*>(row + 16 * kk + 4 * gq);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc = mfma4(x[e], c < kMtpMaxT ? x[e] : 0.f, acc);
        }
      }
      // lane (c, gq) holds D[4 gq + e][c]; the dot of row r and token s goes to
      // slot 8 r + s
      if (c < kMtpMaxT) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sF[F_DOT + 8 * (4 * gq + e) + c] = acc[e];
      }
    }
    lds_barrier();
    // A (threads 0-63) and P (64-127), one element each
    if (tid < 128) {
      const int t = (tid >> 3) & 7, s = tid & 7;
      const float decay = expf(sF[F_G + t] - sF[F_G + s]);
      if (tid < 64)
        sF[F_A + 8 * t + s] = s < t ? sF[F_B + t] * decay * sF[F_DOT + tid] : 0.f;
      else
        sF[F_P + 8 * t + s] = s <= t ? decay * sF[F_DOT + tid] : 0.f;
    }
    lds_barrier();
    // Tinv = (I + A)^{-1} by forward substitution (thread j: column j)
    if (tid < kMtpMaxT) {
      const int j = tid;
      float x[kMtpMaxT];
#pragma unroll
      for (int t = 0; t < kMtpMaxT; ++t) {
        // later chunks: row t's reads are not hoisted above the rows before it
        if constexpr (decltype(lean)::value) __builtin_amdgcn_sched_barrier(0);
        float acc = t == j ? 1.f : 0.f;
#pragma unroll
        for (int s = 0; s < t; ++s) acc = fmaf(-sF[F_A + 8 * t + s], x[s], acc);
        x[t] = acc;
      }
#pragma unroll
      for (int t = 0; t < kMtpMaxT; ++t) sF[F_TINV + 8 * t + j] = x[t];
    }
    lds_barrier();
  };
  int t0 = 0;
  setup_chunk(T < kMtpMaxT ? T : kMtpMaxT, std::false_type{});
  // the next chunk's rows, in flight while this one is applied
  if constexpr (MULTI) {
    if (kMtpMaxT < T) stage_tokens(seq0 + kMtpMaxT, T - kMtpMaxT < kMtpMaxT ? T - kMtpMaxT : kMtpMaxT);
  }
  // 64 columns at a time through the wave's staging rows (its own; LDS
  // accesses of a wave complete in order)
#pragma unroll
  for (int v = 0; v < KT / 4; ++v) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<floatx4*>(W + (4 * i + (lane >> 4)) * TLD + 4 * (lane & 15)) = ld[4 * v + i];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      st[4 * v + t] = *reinterpret_cast<const floatx4*>(W + c * TLD + 16 * t + 4 * gq);
  }
  // The tokens in chunks of 8 (the last may be shorter); the state stays in
  // registers from the first chunk to the last.
  for (;;) {
    const int Tc = T - t0 < kMtpMaxT ? T - t0 : kMtpMaxT;
    const size_t tok0 = seq0 + t0;

    // [Z | Y] = S [K; Q]^T: lane (c, gq) ends with row 4 gq + e of the wave and
    // column c (token c of Z for c < 8, token c - 8 of Y for c >= 8).
    floatx4 zy0 = {0.f, 0.f, 0.f, 0.f}, zy1 = {0.f, 0.f, 0.f, 0.f};
    if constexpr (IN == Dt::BF16) {
      // bf16 inputs: S as two bf16 planes against the exact bf16 rows of K and
      // Q on the 16x16x32 matrix cores (8 products instead of 32 fp32 ones).
      // Block kb contracts columns 32 kb + 4 gq + e and 32 kb + 16 + 4 gq + e in
      // the slots of lane group gq, the same order in both operands, which is
      // where the state already is (st[2 kb], st[2 kb + 1]).
#pragma unroll
      for (int kb = 0; kb < KT / 2; ++kb) {
        const floatx4 k0 = *reinterpret_cast<const floatx4*>(sKQ + c * LDK + 32 * kb + 4 * gq);
        const floatx4 k1 = *reinterpret_cast<const floatx4*>(sKQ + c * LDK + 32 * kb + 16 + 4 * gq);
        float xs[8], xk[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xs[e] = st[2 * kb][e];
          xs[4 + e] = st[2 * kb + 1][e];
          xk[e] = k0[e];
          xk[4 + e] = k1[e];
        }
        bf16x8 sp[2], kp[1];
        split8<2>(xs, sp);
        split8<1>(xk, kp);  // exact: the rows are bf16 inputs
        floatx4& acc = (kb & 1) ? zy1 : zy0;
        acc = mfma16x16x32(sp[1], kp[0], acc);  // the low plane first
        acc = mfma16x16x32(sp[0], kp[0], acc);
      }
    } else {
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const floatx4 kc = *reinterpret_cast<const floatx4*>(sKQ + c * LDK + 16 * kt + 4 * gq);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (kt & 1) zy1 = mfma4(st[kt][e], kc[e], zy1);
          else zy0 = mfma4(st[kt][e], kc[e], zy0);
        }
      }
    }
    const floatx4 zy = zy0 + zy1;

    // R = beta (v - gamma Z) on lanes c < 8, exchanged through LDS as [row][t]
    float* X = sX[wave];
    if (c < kMtpMaxT) {
      const float bt = sF[F_B + c], gt = sF[F_GAM + c];
#pragma unroll
      for (int e = 0; e < 4; ++e) X[(4 * gq + e) * XLD + c] = bt * (vv[e] - gt * zy[e]);
    }
    wave_lds_sync();
    // U = R Tinv^T: A[row c][t] = R, B[t][t' = c] = Tinv[c][t]
    floatx4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int t = 4 * ks + gq;
      const float a = X[c * XLD + t];
      const float b = c < kMtpMaxT ? sF[F_TINV + 8 * c + t] : 0.f;
      u = mfma4(a, b, u);
    }
    wave_lds_sync();
    if (c < kMtpMaxT) {
#pragma unroll
      for (int e = 0; e < 4; ++e) X[(4 * gq + e) * XLD + c] = u[e];
    }
    wave_lds_sync();
    // U in the A layout (row c, token 4 ks + gq), for O and (scaled by D) the update
    float ua[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) ua[ks] = X[c * XLD + 4 * ks + gq];

    // O = gamma Y + U P^T on lanes c >= 8 (token c - 8, rows 4 gq + e)
    floatx4 pu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const float b = c >= kMtpMaxT ? sF[F_P + 8 * (c - kMtpMaxT) + 4 * ks + gq] : 0.f;
      pu = mfma4(ua[ks], b, pu);
    }
    if (c >= kMtpMaxT && c - kMtpMaxT < Tc) {
      const int t = c - kMtpMaxT;
      const float gt = sF[F_GAM + t];
      const size_t ob = ((tok0 + t) * H + h) * DV + rbase + 4 * gq;
#pragma unroll
      for (int e = 0; e < 4; ++e) store_scalar<OUT>(o, ob + e, fmaf(gt, zy[e], pu[e]));
    }

    // S^T <- gamma_T S^T + K^T diag(D) U^T, tile by tile: A[j][t] = K[t][16 kt + j],
    // B[t][row c] = D_t U[c][t]; the output lands on lane (c, gq), element e =
    // S[row c][16 kt + 4 gq + e], where the state already is.
    const float gam_end = sF[F_GAM + kMtpMaxT - 1];
    if constexpr (IN == Dt::BF16) {
      // 16x16x16 products over the tokens (8, padded to 16 with zeros in lane
      // groups 2 and 3): A[j][t] = K[t][16 kt + j] (exact bf16), B[t][row c] =
      // D_t U[c][t] as two bf16 planes (lane group gq: tokens 4 gq .. 4 gq + 3)
      shortx4 ubp[2] = {shortx4{0, 0, 0, 0}, shortx4{0, 0, 0, 0}};
      if (gq < 2) {
        floatx4 du;
#pragma unroll
        for (int e = 0; e < 4; ++e) du[e] = sF[F_D + 4 * gq + e] * X[c * XLD + 4 * gq + e];
        split4<2>(du, ubp);
      }
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        shortx4 ka[1] = {shortx4{0, 0, 0, 0}};
        if (gq < 2) {
          floatx4 kk;
#pragma unroll
          for (int e = 0; e < 4; ++e) kk[e] = sKQ[(4 * gq + e) * LDK + 16 * kt + c];
          split4<1>(kk, ka);  // exact
        }
        floatx4 acc = st[kt] * gam_end;
        acc = mfma16x16x16(ka[0], ubp[1], acc);
        acc = mfma16x16x16(ka[0], ubp[0], acc);
        st[kt] = acc;
      }
    } else {
      float ub[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) ub[ks] = sF[F_D + 4 * ks + gq] * ua[ks];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        floatx4 acc = st[kt] * gam_end;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) acc = mfma4(sKQ[(4 * ks + gq) * LDK + 16 * kt + c], ub[ks], acc);
        st[kt] = acc;
      }
    }
    t0 += kMtpMaxT;
    if (!MULTI || t0 >= T) break;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of the next chunk
    lds_barrier();  // every wave's have landed, and is done with this chunk's K, Q and factors
    setup_chunk(T - t0 < kMtpMaxT ? T - t0 : kMtpMaxT, std::true_type{});
    if (t0 + kMtpMaxT < T)
      stage_tokens(seq0 + t0 + kMtpMaxT,
                   T - t0 - kMtpMaxT < kMtpMaxT ? T - t0 - kMtpMaxT : kMtpMaxT);
  }
  if (state_out) {
    // back through the staging rows, leaving as it arrived: each store
    // instruction covers 4 rows x 256 B, where the matrix-core layout covers
    // 16 rows x 64 B (about 60% of the write rate in an in-place copy of the
    // same bytes)
    floatx4* Sout = reinterpret_cast<floatx4*>(state_out + static_cast<size_t>(pair) * DV * DK);
#pragma unroll
    for (int v = 0; v < KT / 4; ++v) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        *reinterpret_cast<floatx4*>(W + c * TLD + 16 * t + 4 * gq) = st[4 * v + t];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * i + (lane >> 4), col = 4 * (lane & 15);
        const floatx4 x = *reinterpret_cast<const floatx4*>(W + row * TLD + col);
        __builtin_nontemporal_store(x, &Sout[((rbase + row) * DK + 64 * v + col) / 4]);
      }
    }
  }
}

template <int DK, int DV, Dt IN, Dt OUT>
hipError_t launch_mtp_chunk_t(const void* q, const void* k, const void* v, const float* g,
                              const float* beta, const float* state_in, float* state_out, void* o,
                              int NH, int H, int T, hipStream_t stream) {
  const int64_t groups = static_cast<int64_t>(NH) * (DV / (16 * mtp_waves<DV>()));
  if (groups > INT32_MAX) return hipErrorInvalidConfiguration;
  if (T > kMtpMaxT)
    hipLaunchKernelGGL((mtp_chunk_kernel<DK, DV, IN, OUT, true>), dim3(static_cast<unsigned>(groups)),
                       dim3(64 * mtp_waves<DV>()), 0, stream, q, k, v, g, beta, state_in, state_out,
                       o, NH, H, T);
  else
    hipLaunchKernelGGL((mtp_chunk_kernel<DK, DV, IN, OUT, false>),
                       dim3(static_cast<unsigned>(groups)), dim3(64 * mtp_waves<DV>()), 0, stream, q,
                       k, v, g, beta, state_in, state_out, o, NH, H, T);
  return hipGetLastError();
}

template <int DK, int DV, Dt IN, Dt OUT>
hipError_t launch_mtp_t(const void* q, const void* k, const void* v, const float* g,
                        const float* beta, const float* state_in, float* state_out, void* o,
                        float* inter, int NH, int H, int T, hipStream_t stream) {
  constexpr int RPT = decode_rows_per_thread<DV>();
  const int64_t groups = static_cast<int64_t>(NH) * (DV / (RPT * (kDecodeThreads / 16)));
  if (groups > INT32_MAX) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((mtp_kernel<DK, DV, IN, OUT, RPT>), dim3(static_cast<unsigned>(groups)),
                     dim3(kDecodeThreads), 0, stream, q, k, v, g, beta, state_in, state_out, o,
                     inter, NH, H, T);
  return hipGetLastError();
}

template <int DK, int DV, Dt IN, Dt OUT>
hipError_t launch_decode_t(const void* q, const void* k, const void* v, const float* g,
                           const float* beta, float* state, void* o, int NH,
                           hipStream_t stream) {
  constexpr int RPT = decode_rows_per_thread<DV>();
  const int64_t groups = static_cast<int64_t>(NH) * (DV / (RPT * (kDecodeThreads / 16)));
  if (groups > INT32_MAX) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((decode_kernel<DK, DV, IN, OUT, RPT>), dim3(static_cast<unsigned>(groups)),
                     dim3(kDecodeThreads), 0, stream, q, k, v, g, beta, state, o, NH);
  return hipGetLastError();
}

template <int DK, int DV>
hipError_t dispatch_dtypes(const void* q, const void* k, const void* v, const float* g,
                           const float* beta, float* state, void* o, int NH, int in_dtype,
                           int out_dtype, hipStream_t stream) {
  if (in_dtype == 0 && out_dtype == 0)
    return launch_decode_t<DK, DV, Dt::BF16, Dt::BF16>(q, k, v, g, beta, state, o, NH, stream);
  if (in_dtype == 0 && out_dtype == 1)
    return launch_decode_t<DK, DV, Dt::BF16, Dt::F32>(q, k, v, g, beta, state, o, NH, stream);
  if (in_dtype == 1 && out_dtype == 0)
    return launch_decode_t<DK, DV, Dt::F32, Dt::BF16>(q, k, v, g, beta, state, o, NH, stream);
  return launch_decode_t<DK, DV, Dt::F32, Dt::F32>(q, k, v, g, beta, state, o, NH, stream);
}

}  // namespace

hipError_t launch_decode(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, float* state, void* o, int NH, int dk, int dv,
                         int in_dtype, int out_dtype, hipStream_t stream) {
  if (dk == 128 && dv == 128)
    return dispatch_dtypes<128, 128>(q, k, v, g, beta, state, o, NH, in_dtype, out_dtype, stream);
  return dispatch_dtypes<64, 64>(q, k, v, g, beta, state, o, NH, in_dtype, out_dtype, stream);
}

hipError_t launch_mtp(const void* q, const void* k, const void* v, const float* g,
                      const float* beta, const float* state_in, float* state_out, void* o,
                      float* inter, int N, int T, int H, int dk, int dv, int in_dtype,
                      int out_dtype, hipStream_t stream) {
  (void)dv;
  const int NH = N * H;
  // 2 or more tokens without per-token states: the chunked form on the matrix
  // cores; otherwise (and for T = 1, which then equals the decode step bit for
  // bit) the token-by-token kernel.
  const bool chunked = inter == nullptr && T >= kMtpChunkMinT;
#define GDR_MTP(D_, IN_, OUT_)                                                                \
  return chunked ? launch_mtp_chunk_t<D_, D_, IN_, OUT_>(q, k, v, g, beta, state_in, state_out, \
                                                         o, NH, H, T, stream)                    \
                 : launch_mtp_t<D_, D_, IN_, OUT_>(q, k, v, g, beta, state_in, state_out, o,     \
                                                   inter, NH, H, T, stream)
  if (dk == 128) {
    if (in_dtype == 0 && out_dtype == 0) GDR_MTP(128, Dt::BF16, Dt::BF16);
    if (in_dtype == 0) GDR_MTP(128, Dt::BF16, Dt::F32);
    if (out_dtype == 0) GDR_MTP(128, Dt::F32, Dt::BF16);
    GDR_MTP(128, Dt::F32, Dt::F32);
  }
  if (in_dtype == 0 && out_dtype == 0) GDR_MTP(64, Dt::BF16, Dt::BF16);
  if (in_dtype == 0) GDR_MTP(64, Dt::BF16, Dt::F32);
  if (out_dtype == 0) GDR_MTP(64, Dt::F32, Dt::BF16);
  GDR_MTP(64, Dt::F32, Dt::F32);
#undef GDR_MTP
}

}  // namespace gdr
