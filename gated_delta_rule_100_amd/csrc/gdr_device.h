// gdr_device.h -- small device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

enum class Dt { BF16 = 0, F32 = 1 };

// bf16 <-> fp32.  bf16 -> fp32 is exact (the 16 bits are the high half of an
// IEEE binary32).  fp32 -> bf16 rounds to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// gfx950 converts with v_cvt_pk_bf16_f32 (round to nearest even).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS accesses
// (lgkmcnt) but not for global loads still in flight, which __syncthreads()
// also drains (its release fence covers global memory).  The s_waitcnt
// immediate leaves vmcnt and expcnt at their maxima (no constraint) and sets
// lgkmcnt to zero; the empty asm statements keep the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Exchange point for the lanes of one wave through LDS, with no barrier:
// waits for the wave's LDS accesses (in order, so another lane's earlier
// write is then visible) and keeps the compiler from carrying a value read
// before the point past it -- for a lane whose own write was skipped, reusing
// its earlier read of the same address would be legal for threads that do
// not synchronise, and wrong here.
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
}

// Sum over the 16 lanes of a DPP row (lanes 16r .. 16r+15); every lane of the
// row receives the same bits.  Each stage adds the value of a partner lane
// whose partner is the lane itself (quad_perm [1,0,3,2] and [2,3,0,1] within
// a quad, row_half_mirror between the two quads of a half row, row_ror:8
// between the halves), so both lanes of a pair add the same two numbers and
// the total does not depend on the lane that reads it.
__device__ __forceinline__ float row16_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
           0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
           0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
           0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
           0, __builtin_bit_cast(int, x), 0x128, 0xF, 0xF, true));
  return x;
}

// Load N consecutive input elements (bf16 or fp32) starting at element `idx`
// and widen them to fp32.  N is 4 or 8; the address must be 8-byte aligned
// for bf16 x4, 16-byte aligned otherwise.
template <Dt D, int N>
__device__ __forceinline__ void load_vec(const void* base, size_t idx, float* out) {
  if constexpr (D == Dt::F32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      float4 t = p[i];
      out[4 * i + 0] = t.x; out[4 * i + 1] = t.y; out[4 * i + 2] = t.z; out[4 * i + 3] = t.w;
    }
  } else {
    const uint16_t* src = static_cast<const uint16_t*>(base) + idx;
    if constexpr (N == 4) {
      uint2 t = *reinterpret_cast<const uint2*>(src);
      out[0] = __uint_as_float(t.x << 16); out[1] = __uint_as_float(t.x & 0xffff0000u);
      out[2] = __uint_as_float(t.y << 16); out[3] = __uint_as_float(t.y & 0xffff0000u);
    } else {
#pragma unroll
      for (int i = 0; i < N / 8; ++i) {
        uint4 t = reinterpret_cast<const uint4*>(src)[i];
        uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          out[8 * i + 2 * j + 0] = __uint_as_float(w[j] << 16);
          out[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
        }
      }
    }
  }
}

template <Dt D>
__device__ __forceinline__ float load_scalar(const void* base, size_t idx) {
  if constexpr (D == Dt::F32) {
    return static_cast<const float*>(base)[idx];
  } else {
    return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[idx]);
  }
}

template <Dt D>
__device__ __forceinline__ void store_scalar(void* base, size_t idx, float x) {
  if constexpr (D == Dt::F32) {
    static_cast<float*>(base)[idx] = x;
  } else {
    static_cast<uint16_t*>(base)[idx] = f32_to_bf16_bits(x);
  }
}

}  // namespace gdr
