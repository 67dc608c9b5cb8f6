// Device-side helpers shared by the gfx950 attention kernels: vector types, the bf16
// MFMA wrappers, LDS transpose reads, cross-lane reductions and bf16 conversion.
//
// Lane layouts used throughout (CDNA4, wave64), as checked on the hardware:
//  * v_mfma_f32_32x32x16_bf16  C[32x32] += A[32x16] * B[16x32]:
//      A: lane l holds A[l % 32][8 * (l / 32) + p],  p = 0..7
//      B: lane l holds B[8 * (l / 32) + p][l % 32]
//      C: lane l, register r holds C[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32]
//  * ds_read_b64_tr_b16 (per group of 16 lanes): result lane j, element e is element
//      j % 4 of the 8 bytes loaded by lane 4 * e + j / 4 of the same group.  So if lane L
//      of a group loads row (k0 + L / 4), columns (n0 + 4 * (L % 4)) .. +3 of a row-major
//      [k][n] bf16 matrix, lane j receives column n0 + j, rows k0 .. k0 + 3.
//  * v_permlane32_swap(x, x): lane l < 32 gets (x[l], x[l + 32]); lane l >= 32 gets
//      (x[l - 32], x[l]) -- both halves of a lane pair (l, l ^ 32) in one instruction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Finite stand-in for -inf in the running maximum: exp2(kNegBig - m) is exactly 0 for any
// finite score m, and exp2(kNegBig - kNegBig) = 1 only while a row has seen no visible key,
// a state that a later visible key multiplies away (its rescale factor is 0).
constexpr float kNegBig = -1.0e30f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Round-to-nearest-even float -> bf16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16 to_bf16(float x) { return (bf16)x; }
__device__ __forceinline__ float from_bf16(bf16 x) { return (float)x; }

__device__ __forceinline__ bf16x8 pack8(const f32x16& v, int base) {
  bf16x8 r;
#pragma unroll
  for (int p = 0; p < 8; ++p) r[p] = (bf16)v[base + p];
  return r;
}

// Two transposing LDS reads (rows k0..k0+3 and k1..k1+3) glued into one MFMA operand.
__device__ __forceinline__ bf16x8 tr_read_pair(const bf16* p0, const bf16* p1) {
  i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0);
  i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p1);
  union {
    struct { i16x4 lo, hi; } s;
    bf16x8 v;
  } u;
  u.s.lo = a;
  u.s.hi = b;
  return u.v;
}

// max / sum over the lane pair (l, l ^ 32).
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <typename T>
__device__ __forceinline__ T ld16(const void* p) {
  return *reinterpret_cast<const T*>(p);
}

// Angle p * base^(-2i/D) reduced to [-pi, pi] in double precision, then its cosine and sine
// in single precision.
__device__ __forceinline__ void rope_cos_sin(int pos, int i, int D, double log2_base, float* c,
                                            float* s) {
  const double w = exp2(-(2.0 * i / D) * log2_base);
  double a = (double)pos * w;
  const double two_pi = 6.283185307179586;
  a -= two_pi * rint(a / two_pi);
  sincosf((float)a, s, c);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

}  // namespace attn
