// Shared pieces of the MFMA (matrix-core) ResidualAttention kernels for gfx950 (bf16
// storage, d = 128, r = 16, page size 16): operand types, MFMA wrappers, packed
// conversions and rotations with one fixed rounding sequence, cross-lane maxima, and the
// dimension permutation of the key reconstruction tiles.  Included by the decode and the
// prefill kernel sources; everything here has internal linkage.
//
// MFMA lane layouts used (checked on gfx950): for a 16x16xK instruction lane l supplies
// A[l % 16][kpl * (l / 16) + e] and B[kpl * (l / 16) + e][l % 16] (kpl = K / 4) and
// receives D[4 * (l / 16) + i][l % 16].
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <type_traits>

#include "forkkv_internal.h"

namespace forkkv {
namespace {

typedef short s4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef __bf16 bf8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f4 __attribute__((__vector_size__(4 * sizeof(float))));

constexpr int kD = 128;       // head dim
constexpr int kR = 16;        // rank
constexpr double kTwoPi = 6.283185307179586476925286766559;
constexpr double kInvTwoPi = 0.15915494309189533576888376337251;

__device__ __forceinline__ f4 mfma16(s4 a, s4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mfma32(bf8 a, bf8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
typedef _Float16 h8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f4 mfma32h(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
union H8 {
  h2 p[4];
  h8 v;
  uint4 u;
};
// Two floats -> fp16 pair, round to nearest even (v_cvt_pk_f16_f32).
__device__ __forceinline__ h2 pack_f16x2(float lo, float hi) {
  const float2 f = {lo, hi};
  typedef float fv2 __attribute__((ext_vector_type(2)));
  return __builtin_convertvector(fv2{f.x, f.y}, h2);
}
// a * b - c * d and a * b + c * d with one fixed rounding sequence (c * d rounded, then one
// fused multiply-add), so every instantiation of the kernels rounds the same way.
__device__ __forceinline__ h2 mul_sub2(h2 a, h2 b, h2 c, h2 d) {
#pragma clang fp contract(off)
  const h2 t = c * d;
  return __builtin_elementwise_fma(a, b, -t);
}
__device__ __forceinline__ h2 mul_add2(h2 a, h2 b, h2 c, h2 d) {
#pragma clang fp contract(off)
  const h2 t = c * d;
  return __builtin_elementwise_fma(a, b, t);
}
__device__ __forceinline__ float mul_sub(float a, float b, float c, float d) {
#pragma clang fp contract(off)
  const float t = c * d;
  return __builtin_fmaf(a, b, -t);
}
__device__ __forceinline__ float mul_add(float a, float b, float c, float d) {
#pragma clang fp contract(off)
  const float t = c * d;
  return __builtin_fmaf(a, b, t);
}
// Zero residual page, read in place of a page a sequence does not have.
__device__ __align__(16) uint16_t g_zero_res[2 * kPage * kR];

typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef float fl2 __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const fl2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf2));
}

__device__ __forceinline__ float shfl_xor(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}
// max(a, b) for values that are finite or -inf: one median-of-three against the largest
// finite float (fmaxf would first quiet possible signalling NaNs, one extra instruction per
// operand, and a bound of +inf is folded back into fmaxf by the compiler)
__device__ __forceinline__ float max2(float a, float b) {
  return __builtin_amdgcn_fmed3f(a, b, 3.402823466e38f);
}
// max over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one query column's rows): two
// butterfly steps with the cross-row lane swaps (no LDS round trip)
__device__ __forceinline__ float max_over_rows(float v) {
  const uint32_t x = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  v = max2(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t y = __float_as_uint(v);
  const auto b = __builtin_amdgcn_permlane32_swap(y, y, false, false);
  return max2(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

union U4 {
  uint4 u;
  bf8 b;
};
union U2 {
  uint2 u;
  s4 s;
};

// Dimension held by reconstruction tile T, row m (a permutation of 0..127 chosen so that
// (a) tiles T and T + 4 hold the RoPE partners j and j + 64 at the same row, and (b) the
// lane that receives rows 4g..4g+3 of tiles 2c, 2c+1 holds dims 32c + 8g .. 32c + 8g + 7,
// i.e. exactly the natural-order K slice it must supply to the 16x16x32 score MFMA.
__device__ __forceinline__ int perm_dim(int T, int m) {
  return 32 * (T >> 1) + 8 * (m >> 2) + 4 * (T & 1) + (m & 3);
}

}  // namespace
}  // namespace forkkv
