// fixup.hip -- inter-chunk state fixup and final-state copy on gfx950.
//
// fixed[c] = fixed[c-1] M_c + L_c is a chain of dependent matrix products per
// (sequence, head); the rows of the state are independent (row i of the
// result only needs row i of the previous state), so the work is split over
// workgroups of R state rows.  Each workgroup walks its sequence's chunks in
// order, the way run_simt_fixup_loop on the FlashInfer PR #3866 page does
// ("CP delta-rule precompute optimisation for ultra-low parallelism", code
// changes 2): it keeps its R rows in LDS, each thread owns one output column
// and one half of the contraction, loads its column of M_c straight into
// registers, and preloads chunk c+1's M and L columns while chunk c is
// accumulated.  The two half-contractions meet in LDS, the new rows are
// published to LDS and to fixed[c].  Start (init_state_tile on the same page):
// with an initial state the scan begins at the sequence's first chunk; without
// one the first fixed state is L of that chunk and the scan begins at the next.
// All arithmetic is fp32 FMA.
#include "gdr_device.h"
#include "launch.h"

namespace gdr {
namespace {

constexpr int kFixupRows = 4;

template <int DK, int DV, int R>
__global__ __launch_bounds__(2 * DK) void fixup_kernel(const float* __restrict__ L,
                                                       const float* __restrict__ M,
                                                       const float* __restrict__ state_in,
                                                       const int32_t* __restrict__ offs,
                                                       float* __restrict__ fixed, int n_chunks,
                                                       int H) {
  constexpr int KH = DK / 2;  // contraction half owned by a thread
  const int row0 = blockIdx.x * R;
  const int h = blockIdx.y;
  const int n = blockIdx.z;
  const int col = threadIdx.x % DK;
  const int kh = threadIdx.x / DK;

  int c_end = offs[n + 1];
  int c_begin = offs[n];
  c_end = c_end < n_chunks ? c_end : n_chunks;
  c_begin = c_begin < 0 ? 0 : c_begin;
  if (c_begin >= c_end) return;

  __shared__ float s_lds[R][DK];
  __shared__ float part[R][DK];

  auto l_at = [&](int c, int i) -> size_t {
    return ((static_cast<size_t>(c) * H + h) * DV + row0 + i) * DK + col;
  };
  auto m_base = [&](int c) -> size_t { return (static_cast<size_t>(c) * H + h) * DK * DK; };

  int start;
  if (state_in != nullptr) {
    if (kh == 0) {
#pragma unroll
      for (int i = 0; i < R; ++i)
        s_lds[i][col] = state_in[((static_cast<size_t>(n) * H + h) * DV + row0 + i) * DK + col];
    }
    start = c_begin;
  } else {
    if (kh == 0) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const float x = L[l_at(c_begin, i)];
        s_lds[i][col] = x;
        fixed[l_at(c_begin, i)] = x;
      }
    }
    start = c_begin + 1;
  }
  __syncthreads();
  if (start >= c_end) return;

  float m_cur[KH], l_cur[R];
  {
    const float* Mc = M + m_base(start) + static_cast<size_t>(kh) * KH * DK + col;
#pragma unroll
    for (int kk = 0; kk < KH; ++kk) m_cur[kk] = Mc[static_cast<size_t>(kk) * DK];
#pragma unroll
    for (int i = 0; i < R; ++i) l_cur[i] = kh == 0 ? L[l_at(start, i)] : 0.f;
  }

  for (int c = start; c < c_end; ++c) {
    const bool more = c + 1 < c_end;
    float m_nxt[KH], l_nxt[R];
    if (more) {
      const float* Mc = M + m_base(c + 1) + static_cast<size_t>(kh) * KH * DK + col;
#pragma unroll
      for (int kk = 0; kk < KH; ++kk) m_nxt[kk] = Mc[static_cast<size_t>(kk) * DK];
#pragma unroll
      for (int i = 0; i < R; ++i) l_nxt[i] = kh == 0 ? L[l_at(c + 1, i)] : 0.f;
    }

    float acc[R];
#pragma unroll
    for (int i = 0; i < R; ++i) acc[i] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KH; kk += 4) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const float4 s = *reinterpret_cast<const float4*>(&s_lds[i][kh * KH + kk]);
        acc[i] = fmaf(s.x, m_cur[kk + 0], acc[i]);
        acc[i] = fmaf(s.y, m_cur[kk + 1], acc[i]);
        acc[i] = fmaf(s.z, m_cur[kk + 2], acc[i]);
        acc[i] = fmaf(s.w, m_cur[kk + 3], acc[i]);
      }
    }
    if (kh == 1) {
#pragma unroll
      for (int i = 0; i < R; ++i) part[i][col] = acc[i];
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const float x = (acc[i] + part[i][col]) + l_cur[i];
        fixed[l_at(c, i)] = x;
        s_lds[i][col] = x;
      }
    }
    __syncthreads();
    if (more) {
#pragma unroll
      for (int kk = 0; kk < KH; ++kk) m_cur[kk] = m_nxt[kk];
#pragma unroll
      for (int i = 0; i < R; ++i) l_cur[i] = l_nxt[i];
    }
  }
}

__global__ __launch_bounds__(256) void final_state_kernel(const float* __restrict__ state_in,
                                                          const float* __restrict__ fixed,
                                                          const int32_t* __restrict__ offs,
                                                          int H, int elems, int n_chunks,
                                                          float* state_out) {
  const int pair = blockIdx.x;  // n * H + h
  const int n = pair / H;
  const int h = pair % H;
  int c_end = offs[n + 1];
  int c_begin = offs[n];
  c_end = c_end < n_chunks ? c_end : n_chunks;
  c_begin = c_begin < 0 ? 0 : c_begin;
  const float* src = nullptr;
  if (c_begin < c_end) {
    src = fixed + (static_cast<size_t>(c_end - 1) * H + h) * elems;
  } else if (state_in != nullptr) {
    src = state_in + static_cast<size_t>(pair) * elems;
  }
  float4* dst = reinterpret_cast<float4*>(state_out + static_cast<size_t>(pair) * elems);
  if (src == reinterpret_cast<const float*>(dst)) return;  // in place, nothing to move
  for (int e = threadIdx.x; e < elems / 4; e += blockDim.x)
    dst[e] = src ? reinterpret_cast<const float4*>(src)[e] : make_float4(0.f, 0.f, 0.f, 0.f);
}

}  // namespace

hipError_t launch_fixup(const float* L, const float* M, const float* state_in,
                        const int32_t* chunk_offsets, int N, float* fixed, int n_chunks, int H,
                        int dk, int dv, hipStream_t stream) {
  if (dk == 128 && dv == 128) {
    hipLaunchKernelGGL((fixup_kernel<128, 128, kFixupRows>), dim3(128 / kFixupRows, H, N),
                       dim3(256), 0, stream, L, M, state_in, chunk_offsets, fixed, n_chunks, H);
  } else {
    hipLaunchKernelGGL((fixup_kernel<64, 64, kFixupRows>), dim3(64 / kFixupRows, H, N),
                       dim3(128), 0, stream, L, M, state_in, chunk_offsets, fixed, n_chunks, H);
  }
  return hipGetLastError();
}

hipError_t launch_final_state(const float* state_in, const float* fixed,
                              const int32_t* chunk_offsets, int N, int H, int dk, int dv,
                              int n_chunks, float* state_out, hipStream_t stream) {
  hipLaunchKernelGGL(final_state_kernel, dim3(N * H), dim3(256), 0, stream, state_in, fixed,
                     chunk_offsets, H, dk * dv, n_chunks, state_out);
  return hipGetLastError();
}

}  // namespace gdr
