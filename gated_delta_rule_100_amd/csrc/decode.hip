// decode.hip -- one-token gated delta rule step on gfx950.
//
// Per (sequence, head) the fp32 state S (dv x dk, dk contiguous) is read once
// and written once; that stream is the whole cost (64 KiB each way per head at
// dk = dv = 128), so the kernel is an HBM stream:
//   * one 256-thread workgroup per (sequence, head);
//   * 16 lanes per state row, each lane holding dk/16 columns as 16-byte
//     vectors, so one wave-wide load covers four contiguous row segments of
//     256 bytes -- fully used 128-byte lines;
//   * every load of the state is issued before any arithmetic (64 KiB per
//     workgroup in flight), non-temporal (the state is touched once), the
//     rank-1 update happens in registers and the rows are stored back in
//     place; no LDS (the state has no reuse -- the
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

template <int DK, int DV, Dt IN, Dt OUT>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, float* __restrict__ state,
    void* __restrict__ o, int NH) {
  constexpr int LPR = 16;               // lanes per state row
  constexpr int CPL = DK / LPR;         // columns per lane (8 or 4)
  constexpr int VEC = CPL / 4;          // float4 per lane per row
  constexpr int RG = kDecodeThreads / LPR;  // row groups (16)
  constexpr int RPT = DV / RG;          // rows per thread (8 or 4)
  static_assert(CPL % 4 == 0 && DV % RG == 0, "shape");

  const int pair = blockIdx.x;
  if (pair >= NH) return;
  const int lane16 = threadIdx.x & (LPR - 1);
  const int rg = threadIdx.x / LPR;

  floatx4* S = reinterpret_cast<floatx4*>(state + static_cast<size_t>(pair) * DV * DK);

  // Issue every state load first.  The state is touched exactly once, so the
  // loads and stores are non-temporal (they do not displace reusable lines).
  floatx4 st[RPT][VEC];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg + RG * i;
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
    vv[i] = load_scalar<IN>(v, static_cast<size_t>(pair) * DV + rg + RG * i);
  const float alpha = expf(g[pair]);
  const float b = beta[pair];

  float oi[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    float a = 0.f;
#pragma unroll
    for (int j = 0; j < VEC; ++j)
      a += st[i][j][0] * kk[j][0] + st[i][j][1] * kk[j][1] + st[i][j][2] * kk[j][2] +
           st[i][j][3] * kk[j][3];
    a = row16_sum(a);
    const float u = b * (vv[i] - alpha * a);
    float p = 0.f;
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      floatx4 s = st[i][j];
#pragma unroll
      for (int e = 0; e < 4; ++e) s[e] = alpha * s[e] + u * kk[j][e];
      st[i][j] = s;
      p += s[0] * qq[j][0] + s[1] * qq[j][1] + s[2] * qq[j][2] + s[3] * qq[j][3];
    }
    oi[i] = row16_sum(p);
  }

#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg + RG * i;
#pragma unroll
    for (int j = 0; j < VEC; ++j)
      __builtin_nontemporal_store(st[i][j], &S[(row * DK + 4 * lane16 + 64 * j) / 4]);
  }
  // lane i of each row group writes the output of its i-th row
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    if (lane16 == i) store_scalar<OUT>(o, static_cast<size_t>(pair) * DV + rg + RG * i, oi[i]);
}

template <int DK, int DV, Dt IN, Dt OUT>
hipError_t launch_decode_t(const void* q, const void* k, const void* v, const float* g,
                           const float* beta, float* state, void* o, int NH,
                           hipStream_t stream) {
  hipLaunchKernelGGL((decode_kernel<DK, DV, IN, OUT>), dim3(NH), dim3(kDecodeThreads), 0, stream,
                     q, k, v, g, beta, state, o, NH);
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

}  // namespace gdr
