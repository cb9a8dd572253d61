// Internal helpers shared by the HIP kernels of libmoe_routed (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace moe {

constexpr int kF16 = 0;
constexpr int kBF16 = 1;
constexpr int kF32 = 2;
constexpr int kFP8 = 3;   // OCP FP8 E4M3 ("fn": no infinities, max 448)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_float(uint32_t b) {
  return __uint_as_float(b << 16);
}

// fp32 -> bfloat16, round to nearest even, with gfx950's conversion
// instruction (v_cvt_pk_bf16_f32; one instruction where the integer form
// --- add 0x7fff plus the kept bit's lowest, shift, NaN select --- takes six,
// a measurable share of the GEMM epilogues). Checked on MI355X against that
// integer form on all 2^32 inputs: identical bits for every non-NaN input,
// and NaN stays NaN.
__device__ __forceinline__ uint32_t float_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ float f16_to_float(uint32_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
}

// fp32 -> binary16 with the hardware conversion (round to nearest even).
__device__ __forceinline__ uint32_t float_to_f16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// fp32 -> FP8 E4M3 (OCP "fn"), round to nearest even, saturating to +-448
// (infinities included); NaN -> 0x7f with the sign kept.
__device__ __forceinline__ uint32_t float_to_fp8e4m3(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(f);
  if (a != a) return sign | 0x7fu;
  if (a >= 448.0f) return sign | 0x7eu;
  if (a < 0.015625f) {                       // below 2^-6: q * 2^-9, q in [0, 8]
    return sign | static_cast<uint32_t>(rintf(a * 512.0f));
  }
  const uint32_t ua = __float_as_uint(a);
  int e = static_cast<int>(ua >> 23) - 127;  // in [-6, 8]
  uint32_t keep = (ua >> 20) & 7u;
  const uint32_t rest = ua & 0xfffffu;
  if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) keep += 1u;
  if (keep == 8u) {
    keep = 0u;
    e += 1;
  }
  return sign | (static_cast<uint32_t>(e + 7) << 3) | keep;
}

// Four floats to the E4M3 codes float_to_fp8e4m3 gives, packed a, b, c, d
// from the low byte up, with gfx950's packed conversion (v_cvt_pk_fp8_f32:
// OCP E4M3, round to nearest even): magnitudes are clamped to 448 first
// (med3, so that the conversion never sees an out-of-range value and
// infinities saturate), and a NaN input takes its code (sign | 0x7f) by a
// select afterwards.
__device__ __forceinline__ uint32_t pk4_fp8e4m3(float a, float b, float c, float d) {
  const float ca = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  const float cb = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  const float cc = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
  const float cd = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
  int q = __builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false);
  q = __builtin_amdgcn_cvt_pk_fp8_f32(cc, cd, q, true);
  uint32_t u = static_cast<uint32_t>(q);
  const float v[4] = {a, b, c, d};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (v[i] != v[i]) {
      const uint32_t code = ((__float_as_uint(v[i]) >> 24) & 0x80u) | 0x7fu;
      u = (u & ~(0xffu << (8 * i))) | (code << (8 * i));
    }
  }
  return u;
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

template <int N>
using int_c = std::integral_constant<int, N>;

// Calls f(int_c<0>{}), ..., f(int_c<N-1>{}): a loop whose index is a
// compile-time constant in every iteration (register-ring slots stay static).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(int_c<I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// SiLU(g) = g / (1 + e^-g), in fp32.
__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// v_mfma_f32_32x32x16_{bf16,f16}: c += A (32 x 16) * B (16 x 32). Lane l
// supplies A row l % 32 and B column l % 32, reduction elements
// 8 * (l / 32) .. + 7 of the 16; the result lane l holds column l % 32 and,
// in register i, row 8 * (i / 4) + 4 * (l / 32) + i % 4.
template <int DT>
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (DT == kBF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

// s_waitcnt vmcnt(N) lgkmcnt(0): this wave's vector loads but the newest N
// are complete, and so are its LDS accesses.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  // gfx9 s_waitcnt: vmcnt in bits [3:0] and [15:14], expcnt [6:4] (7 = no
  // wait), lgkmcnt [11:8] (0 = wait for all).
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

// A workgroup barrier that waits for no memory counter (the caller issues
// the s_waitcnt it needs first) but is a compiler-level memory fence: no LDS
// or global access is moved across it.
__device__ __forceinline__ void barrier_no_wait() { asm volatile("s_barrier" ::: "memory"); }

// Wait for this wave's outstanding LDS (and scalar memory) operations only:
// s_waitcnt lgkmcnt(0) with vmcnt and expcnt at their "no wait" values.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xc07f); }

}  // namespace moe
