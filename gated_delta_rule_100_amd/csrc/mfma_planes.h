// mfma_planes.h -- bf16 "plane" arithmetic on gfx950 matrix cores.
//
// The dense contractions of the chunked form run on v_mfma_f32_16x16x32_bf16
// (16x16 output tile, 32-deep contraction, fp32 accumulate).  An fp32 operand
// x is carried as P bf16 planes x = p0 + p1 + ... (p0 = RNE(x), p1 = RNE(x - p0),
// ...): two planes keep ~16 significant bits, three keep all 24.  A product
// of a PA-plane and a PB-plane operand issues the plane pairs (i, j) with
// i + j < max(PA, PB), smallest terms first; the dropped pairs are below the
// kept precision.  Operands that are exactly bf16 (the bf16 inputs q, k, v)
// use one plane.
//
// Lane layout of the 16x16x32 instruction (wave64; c = lane % 16, g = lane / 16):
//   A fragment: A[c][8g .. 8g+7]        (row c of the 16-row tile)
//   B fragment: B[8g .. 8g+7][c]        (column c), i.e. row c of B^T
//   D tile:     D[4g + e][c], e = 0..3  (floatx4 per lane)
// The contraction index only has to agree between A and B; when an operand
// comes straight from a D tile (rows 4g+e of two stacked 16-row tiles), the
// other operand is read with the matching slot order (see load_*_perm).
#pragma once

#include "gdr_device.h"

namespace gdr {

typedef unsigned short ushort8 __attribute__((ext_vector_type(8)));
typedef unsigned short ushort4 __attribute__((ext_vector_type(4)));

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ floatx4 mfma16x16x32(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// fp16 operands (same lane layout): 11-bit significands for operands that are
// not exact bf16 inputs and whose range fp16 holds.
__device__ __forceinline__ floatx4 mfma16x16x32(halfx8 a, halfx8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// fp16 bit pattern of x (round to nearest even).
__device__ __forceinline__ uint16_t f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

// 16x16x16 variant (lane (c, g): A[c][4g .. 4g+3], B[4g .. 4g+3][c]); its
// B operand has exactly the layout of a D tile, so an output tile feeds the
// next product without leaving registers.
__device__ __forceinline__ floatx4 mfma16x16x16(shortx4 a, shortx4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

template <int PA, int PB>
__device__ __forceinline__ void mma16_planes(floatx4& acc, const shortx4 (&a)[PA],
                                             const shortx4 (&b)[PB]) {
  constexpr int PM = PA > PB ? PA : PB;
#pragma unroll
  for (int s = PM - 1; s >= 0; --s) {
#pragma unroll
    for (int i = 0; i < PA; ++i) {
      const int j = s - i;
      if (j >= 0 && j < PB) acc = mfma16x16x16(a[i], b[j], acc);
    }
  }
}

// Two fp32 values as P planes of bf16 pairs (value a in the low half): one
// v_cvt_pk_bf16_f32 (round to nearest even) per plane, and the residual taken
// against the rounded pair read back as fp32 (a shift and a mask).  Equal bit
// for bit to rounding each value on its own.
template <int P>
__device__ __forceinline__ void split2(float a, float b, uint32_t (&out)[P]) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2v));
    out[p] = h;
    if (p + 1 < P) {
      a = a - __uint_as_float(h << 16);
      b = b - __uint_as_float(h & 0xffff0000u);
    }
  }
}

// Split 4 fp32 values (a D tile's floatx4) into P planes of 4 bf16.
template <int P>
__device__ __forceinline__ void split4(const floatx4& x, shortx4 (&out)[P]) {
  uint32_t lo[P], hi[P];
  split2<P>(x[0], x[1], lo);
  split2<P>(x[2], x[3], hi);
#pragma unroll
  for (int p = 0; p < P; ++p) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    out[p] = __builtin_bit_cast(shortx4, u32x2{lo[p], hi[p]});
  }
}

// 4 consecutive bf16 of each plane from LDS (8-byte aligned).
template <int P>
__device__ __forceinline__ void load_lds4(const uint16_t* base, int plane_stride,
                                          shortx4 (&out)[P]) {
#pragma unroll
  for (int p = 0; p < P; ++p)
    out[p] = *reinterpret_cast<const shortx4*>(base + p * plane_stride);
}

// Chunk permutation for row-major bf16 tiles that are read with 16-bit
// transpose reads (read_tr4): the 8 rows a half-wave's transpose read touches
// get distinct pairs of 16-byte chunks, so the read is free of bank conflicts.
// ch = 16-byte chunks per row (8 or 16); the result is even.
__device__ __forceinline__ int swz_tr(int row, int ch) {
  return 2 * ((row * ch / 16) & (ch / 2 - 1));
}

// Transposed 4-element read with gfx950's ds_read_b64_tr_b16.  Within each
// 16-lane group that instruction hands output lane m element e of input lane
// 4e + m/4 (that lane's element m % 4).  With the addresses formed here, lane
// (c, g) receives X[r0 + 4g + e][col0 + c], e = 0..3, of a row-major bf16 tile
// X (ld elements per row, 16-byte chunks permuted by swz_tr), i.e. a column
// slice of four consecutive rows: the 16x16x16 A/B fragment of X^T, or half of
// a slot-permuted 16x16x32 fragment.  col0 is a multiple of 16.
__device__ __forceinline__ shortx4 read_tr4(const uint16_t* tile, int ld, int ch, int r0, int col0,
                                            int c16, int g4) {
  const int r = r0 + 4 * g4 + (c16 >> 2);
  const int col = col0 + 4 * (c16 & 3);
  const uint16_t* p = tile + r * ld + 8 * ((col >> 3) ^ swz_tr(r, ch)) + (col & 7);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) shortx4*)p);
}

template <int PA, int PB>
__device__ __forceinline__ void mma_planes(floatx4& acc, const bf16x8 (&a)[PA],
                                           const bf16x8 (&b)[PB]) {
  constexpr int PM = PA > PB ? PA : PB;
#pragma unroll
  for (int s = PM - 1; s >= 0; --s) {
#pragma unroll
    for (int i = 0; i < PA; ++i) {
      const int j = s - i;
      if (j >= 0 && j < PB) acc = mfma16x16x32(a[i], b[j], acc);
    }
  }
}

// Split one fp32 value into P bf16 planes (bit patterns).
template <int P>
__device__ __forceinline__ void split_planes(float x, uint16_t (&out)[P]) {
  float r = x;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const __bf16 hb = static_cast<__bf16>(r);
    out[p] = __builtin_bit_cast(uint16_t, hb);
    r = r - static_cast<float>(hb);
  }
}

// Two fp32 values as P planes of fp16 pairs (value a in the low half): each
// plane rounds the residual of the planes before it to nearest even; two
// planes keep ~22 significant bits.
template <int P>
__device__ __forceinline__ void split2_h(float a, float b, uint32_t (&out)[P]) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const f16x2 h = __builtin_convertvector(f32x2{a, b}, f16x2);
    out[p] = __builtin_bit_cast(uint32_t, h);
    if (p + 1 < P) {
      a = a - static_cast<float>(h[0]);
      b = b - static_cast<float>(h[1]);
    }
  }
}

// Split 8 fp32 values into P fp16x8 fragments.
template <int P>
__device__ __forceinline__ void split8_h(const float (&x)[8], halfx8 (&out)[P]) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  uint32_t w[4][P];
#pragma unroll
  for (int i = 0; i < 4; ++i) split2_h<P>(x[2 * i], x[2 * i + 1], w[i]);
#pragma unroll
  for (int p = 0; p < P; ++p) out[p] = __builtin_bit_cast(halfx8, u32x4{w[0][p], w[1][p], w[2][p], w[3][p]});
}

// Split 8 fp32 values into P bf16x8 fragments.
template <int P>
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8 (&out)[P]) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  uint32_t w[4][P];
#pragma unroll
  for (int i = 0; i < 4; ++i) split2<P>(x[2 * i], x[2 * i + 1], w[i]);
#pragma unroll
  for (int p = 0; p < P; ++p) out[p] = __builtin_bit_cast(bf16x8, u32x4{w[0][p], w[1][p], w[2][p], w[3][p]});
}

// 8 consecutive bf16 of each plane from LDS (16-byte aligned).
template <int P>
__device__ __forceinline__ void load_lds8(const uint16_t* base, int plane_stride,
                                          bf16x8 (&out)[P]) {
#pragma unroll
  for (int p = 0; p < P; ++p)
    out[p] = *reinterpret_cast<const bf16x8*>(base + p * plane_stride);
}

// Slot-permuted read: elements [0..3] and [16..19] from `base` (8-byte
// aligned), matching a D-tile operand made of two stacked 16-row tiles.
template <int P>
__device__ __forceinline__ void load_lds8_perm(const uint16_t* base, int plane_stride,
                                               bf16x8 (&out)[P]) {
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const ushort4 lo = *reinterpret_cast<const ushort4*>(base + p * plane_stride);
    const ushort4 hi = *reinterpret_cast<const ushort4*>(base + p * plane_stride + 16);
    const ushort8 w = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    out[p] = __builtin_bit_cast(bf16x8, w);
  }
}

// 8 consecutive input elements from global memory as P planes (zeros when
// !valid).  bf16 inputs are exact in one plane; fp32 inputs are split.
template <Dt IN, int P>
__device__ __forceinline__ void load_global8(const void* base, size_t idx, bool valid,
                                             bf16x8 (&out)[P]) {
  if constexpr (IN == Dt::BF16) {
    static_assert(P == 1, "bf16 inputs use one plane");
    uint4 w = valid ? *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx)
                    : make_uint4(0, 0, 0, 0);
    out[0] = __builtin_bit_cast(bf16x8, w);
  } else {
    float x[8];
    if (valid) {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
      const float4 a = p[0], b = p[1];
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
      x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
    }
    split8<P>(x, out);
  }
}

}  // namespace gdr
