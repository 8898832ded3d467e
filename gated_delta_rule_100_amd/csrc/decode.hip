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
#define GDR_MTP(D_, IN_, OUT_)                                                                \
  return launch_mtp_t<D_, D_, IN_, OUT_>(q, k, v, g, beta, state_in, state_out, o, inter, NH, H, \
                                         T, stream)
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
