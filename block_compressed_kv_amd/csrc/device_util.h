// Device helpers shared by the liblbca kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lbca {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct bf16_t {  // storage tag for bfloat16 bit patterns
  uint16_t bits;
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32; a in the low half
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2_t));
}

// 8 consecutive elements <-> 8 floats
__device__ __forceinline__ void load8(const float* p, float* f) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}
__device__ __forceinline__ void load8(const bf16_t* p, float* f) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  f[0] = lo_bf16(u.x); f[1] = hi_bf16(u.x); f[2] = lo_bf16(u.y); f[3] = hi_bf16(u.y);
  f[4] = lo_bf16(u.z); f[5] = hi_bf16(u.z); f[6] = lo_bf16(u.w); f[7] = hi_bf16(u.w);
}
__device__ __forceinline__ void store8(float* p, const float* f) {
  *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(f[4], f[5], f[6], f[7]);
}
__device__ __forceinline__ void store8(bf16_t* p, const float* f) {
  uint4 u;
  u.x = pack_bf16x2(f[0], f[1]); u.y = pack_bf16x2(f[2], f[3]);
  u.z = pack_bf16x2(f[4], f[5]); u.w = pack_bf16x2(f[6], f[7]);
  *reinterpret_cast<uint4*>(p) = u;
}

// Rotation angle pos * base^(-2k/r) in turns (angle / 2pi), reduced to
// [-1/2, 1/2] in double precision so that positions up to 2^40 keep an exact
// phase; the hardware sine/cosine (argument in turns) then act on the small
// reduced value.  Returns cos and sin.
__device__ __forceinline__ double rope_turns_per_pos(int k, int r, double log2_base) {
  const double inv_two_pi = 0.15915494309189533576888376337251;
  return exp2(-(2.0 * (double)k / (double)r) * log2_base) * inv_two_pi;
}
__device__ __forceinline__ void rope_cos_sin_turns(double turns, float* c, float* s) {
  const float f = (float)(turns - rint(turns));
  *c = __builtin_amdgcn_cosf(f);
  *s = __builtin_amdgcn_sinf(f);
}
__device__ __forceinline__ void rope_cos_sin(double pos, int k, int r, double log2_base, float* c,
                                             float* s) {
  rope_cos_sin_turns(pos * rope_turns_per_pos(k, r, log2_base), c, s);
}

template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
template <int WIDTH>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// a / b for a >= 0, b >= 1: 32-bit division when both fit (the 64-bit one is a
// long software sequence on this ISA).
__device__ __forceinline__ int64_t div_nonneg(int64_t a, int64_t b) {
  if (((a | b) >> 31) == 0) return (int64_t)((uint32_t)a / (uint32_t)b);
  return a / b;
}

// Visibility rule on the device (same definition as lbca_visible_range).
__device__ __forceinline__ void visible_range(int64_t t, int64_t m, int64_t W, int mode,
                                              int64_t* n_pooled, int64_t* raw_begin) {
  if (mode == 0) {
    int64_t x = t + 1 - W;
    *n_pooled = x > 0 ? div_nonneg(x, m) : 0;
    *raw_begin = *n_pooled * m;
  } else {
    *n_pooled = div_nonneg(t + 1, m);
    int64_t rb = t - W + 1;
    *raw_begin = rb > 0 ? rb : 0;
  }
}

// Cross-row reductions with the gfx950 lane swaps: after a 32-lane (16-lane)
// swap of x with itself, the two results hold x[l] and x[l^32] (x[l^16]) in
// some order on every lane.
__device__ __forceinline__ float xor32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 2^x on the hardware exp unit (inputs here are <= 0 or -inf; results that
// would be denormal flush to zero, which only drops weights below 2^-126).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// ds_read_b64_tr_b16: in each 16-lane group the lanes' 8-byte chunks form 64
// elements in source order e = 4*lane + i; lane i receives e = i, 16+i, 32+i,
// 48+i.  With lane (j, g) pointing at row 4g + j/4, column c0 + 4*(j%4) of a
// row-major tile, lane (j, g) receives rows 4g..4g+3 of column c0 + j: the
// A operand of v_mfma_f32_16x16x16_bf16 for O^T = V^T P^T.
__device__ __forceinline__ s16x4 lds_read_tr16(const bf16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)((__attribute__((address_space(3))) uint16_t*)(p)));
}

typedef __attribute__((address_space(1))) const void gbl_void;
typedef __attribute__((address_space(3))) void lds_void;

// 16-byte load from a global-memory byte address (global, not flat: a flat
// access would also count against the LDS wait counter).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 gbl_u32x4;
__device__ __forceinline__ uint4 ldg16(uintptr_t a) {
  return __builtin_bit_cast(uint4, *reinterpret_cast<gbl_u32x4*>(a));
}

}  // namespace lbca
