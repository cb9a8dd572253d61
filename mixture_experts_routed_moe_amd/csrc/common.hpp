// Internal helpers shared by the HIP kernels of libmoe_routed (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kF16 = 0;
constexpr int kBF16 = 1;
constexpr int kF32 = 2;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_float(uint32_t b) {
  return __uint_as_float(b << 16);
}

// fp32 -> bfloat16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t float_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float f16_to_float(uint32_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
}

// fp32 -> binary16 with the hardware conversion (round to nearest even).
__device__ __forceinline__ uint32_t float_to_f16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

template <int DT>
__device__ __forceinline__ float to_float(uint32_t bits16) {
  if constexpr (DT == kBF16) return bf16_to_float(bits16);
  else return f16_to_float(bits16);
}

template <int DT>
__device__ __forceinline__ uint32_t from_float(float v) {
  if constexpr (DT == kBF16) return float_to_bf16(v);
  else return float_to_f16(v);
}

}  // namespace moe
