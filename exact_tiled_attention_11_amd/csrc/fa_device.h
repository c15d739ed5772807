// Device-side helpers shared by the libfa355 kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;

#define FA_LDS(T) __attribute__((address_space(3))) T

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Matrix-core products. One 32x32 fp32 accumulator block per call.
//  * 16-bit inputs: v_mfma_f32_32x32x16_{bf16,f16}; lane l supplies
//    A[l%32][8*(l/32) + 0..7] and B[8*(l/32) + 0..7][l%32].
//  * fp32 inputs:   v_mfma_f32_32x32x2_f32; lane l supplies A[l%32][l/32]
//    and B[l/32][l%32].
//  The accumulator holds C[8*(r/4) + 4*(l/32) + r%4][l%32] in element r.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16_t mma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mma(f16x8_t a, f16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mma(float a, float b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Per-element-type facts used by the kernels.
template <typename T> struct Elem;
template <> struct Elem<__bf16> {
  using frag = bf16x8_t;                // one MFMA operand per lane
  static constexpr int kStep = 16;      // contraction depth of one MFMA
  static constexpr int kBytes = 2;
};
template <> struct Elem<_Float16> {
  using frag = f16x8_t;
  static constexpr int kStep = 16;
  static constexpr int kBytes = 2;
};
template <> struct Elem<float> {
  using frag = float;
  static constexpr int kStep = 2;
  static constexpr int kBytes = 4;
};

// Values of the two 32-lane halves of a wave, combined per column: after the
// swap every lane holds its own value and the one 32 lanes away.
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Same for lanes 16 apart within each 32-lane half.
__device__ __forceinline__ float quarter_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float quarter_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Round-to-nearest-even conversions of fp32 pairs to 16-bit types, packed.
__device__ __forceinline__ unsigned pack2(float a, float b, __bf16*) {
  bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(unsigned, v);
}
__device__ __forceinline__ unsigned pack2(float a, float b, _Float16*) {
  f16x2_t v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(unsigned, v);
}

// Two packed fp16 values of a 32-bit word.  The word is taken by value: a
// bit cast applied directly to a vector element expression reads element 0.
__device__ __forceinline__ f16x2_t as_f16x2(unsigned w) { return __builtin_bit_cast(f16x2_t, w); }

// 16-bit element -> fp32 (exact).
__device__ __forceinline__ float lo_bf16(unsigned u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_bf16(unsigned u) { return __uint_as_float(u & 0xffff0000u); }

}  // namespace fa
