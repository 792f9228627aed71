// Device helpers shared by the gfx950 matrix-core kernels (forward and gradients).
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx4 __attribute__((ext_vector_type(4)));

// 8- and 4-element vectors of a 16-bit element type (bf16 or fp16).
template <typename E> struct Vec;
template <> struct Vec<__bf16> { typedef bf16x8 v8; typedef bf16x4 v4; };
template <> struct Vec<_Float16> { typedef halfx8 v8; typedef halfx4 v4; };

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))
// Word 3 of a raw buffer resource on gfx9-family GPUs (32-bit data format, no swizzle).
constexpr int kBufferWord3 = 0x00020000;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// v_mfma_f32_32x32x16_bf16: C(32x32) += A(32x16) B(16x32). Lane l holds row (l mod 32)
// of A and column (l mod 32) of B, k = 8*(l/32) .. +7 of each; accumulator register r
// of lane l is C[8*(r/4) + 4*(l/32) + r%4][l mod 32].
__device__ __forceinline__ floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// v_mfma_f32_32x32x16_f16: the same shapes and register layout with fp16 operands.
__device__ __forceinline__ floatx16 mfma32(halfx8 a, halfx8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Two fp32 values rounded to the nearest 16-bit float (ties to even), packed with the first
// in the low half. Written as asm so that each conversion is issued where the code places
// it: as plain conversions the compiler sinks all of a tile's conversions next to the first
// use of the packed vectors, which keeps every fp32 value live until then (the forward
// kernel with a bias and d = dv = 128 then spilled 91 registers).
template <typename E>
__device__ __forceinline__ unsigned cvt_pk(float a, float b);
template <>
__device__ __forceinline__ unsigned cvt_pk<__bf16>(float a, float b) {
  unsigned r;
  asm volatile("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
template <>
__device__ __forceinline__ unsigned cvt_pk<_Float16>(float a, float b) {
  unsigned r;
  asm volatile("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// Elements 2j and 2j+1 of an 8-element 16-bit vector set from a packed word.
template <typename V8>
__device__ __forceinline__ void set_pair(V8& v, int j, unsigned w) {
  u32x4 u = __builtin_bit_cast(u32x4, v);
  u[j] = w;
  v = __builtin_bit_cast(V8, u);
}

// Compile-time loop: f(integral_constant<int, I>) for I = I0 .. N-1.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

}  // namespace fa
