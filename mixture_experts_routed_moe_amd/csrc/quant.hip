// Per-row FP8 E4M3 quantisation of expert weights (the FP8 weight format of
// grouped_gemm_w8.hip): for each row r of `cols` values,
//   amax = max_k |w[r, k]|,  s[r] = amax / 448 (1 for an all-zero row),
//   q[r, k] = FP8(w[r, k] / s[r])  (fp32 division, correctly rounded; round
//                                    to nearest even, saturating at +-448).
// One wave per row: a strided pass for the wave-wide maximum, a second pass
// (served by the cache: a row is at most a few tens of KB) for the codes.
// The same call quantises activations on the W8A8 forward path (x per token,
// h per routed row): 16-bit rows of a multiple of 8 values on 16-byte
// aligned bases take a vectorised form (16-byte loads, every load of a row
// in flight at once, 8 codes per 8-byte store).

#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

template <int DT>
__device__ __forceinline__ float load_w(const void* w, int64_t i) {
  if constexpr (DT == kF32) {
    return static_cast<const float*>(w)[i];
  } else {
    return to_float<DT>(static_cast<const uint16_t*>(w)[i]);
  }
}

template <int DT>
__global__ __launch_bounds__(256) void quantize_fp8_rows_kernel(const void* __restrict__ w,
                                                                int64_t rows, int cols,
                                                                uint8_t* __restrict__ q,
                                                                float* __restrict__ scales) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;                 // whole wave exits together
  const int lane = threadIdx.x & 63;
  const int64_t base = r * cols;
  float amax = 0.0f;
  for (int k = lane; k < cols; k += 64) amax = fmaxf(amax, fabsf(load_w<DT>(w, base + k)));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  if (lane == 0) scales[r] = s;
  for (int k = lane; k < cols; k += 64) {
    q[base + k] = static_cast<uint8_t>(float_to_fp8e4m3(load_w<DT>(w, base + k) / s));
  }
}

template <int DT>
__global__ __launch_bounds__(256) void quantize_fp8_rows16_kernel(const uint16_t* __restrict__ a,
                                                                  int64_t rows, int cols,
                                                                  uint8_t* __restrict__ q,
                                                                  float* __restrict__ scales) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;   // the whole wave exits together
  const int lane = threadIdx.x & 63;
  const u32x4* row = reinterpret_cast<const u32x4*>(a + r * cols);
  const int nvec = cols / 8;
  float amax = 0.0f;
#pragma unroll 4
  for (int v = lane; v < nvec; v += 64) {
    const u32x4 w = row[v];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      amax = fmaxf(amax, fabsf(to_float<DT>(w[j] & 0xffffu)));
      amax = fmaxf(amax, fabsf(to_float<DT>(w[j] >> 16)));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  if (lane == 0) scales[r] = s;
  u32x2* out = reinterpret_cast<u32x2*>(q + r * cols);
#pragma unroll 4
  for (int v = lane; v < nvec; v += 64) {
    const u32x4 w = row[v];
    float f[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[2 * j] = to_float<DT>(w[j] & 0xffffu) / s;
      f[2 * j + 1] = to_float<DT>(w[j] >> 16) / s;
    }
    out[v] = u32x2{pk4_fp8e4m3(f[0], f[1], f[2], f[3]), pk4_fp8e4m3(f[4], f[5], f[6], f[7])};
  }
}

}  // namespace

hipError_t launch_quantize_fp8_rows(const void* w, int64_t rows, int cols, int dtype, uint8_t* q,
                                    float* scales, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((rows + 3) / 4));
  const bool vec = dtype != kF32 && cols % 8 == 0 && reinterpret_cast<uintptr_t>(w) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(q) % 8 == 0;
  if (vec && dtype == kBF16) {
    hipLaunchKernelGGL(quantize_fp8_rows16_kernel<kBF16>, grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(w), rows, cols, q, scales);
  } else if (vec) {
    hipLaunchKernelGGL(quantize_fp8_rows16_kernel<kF16>, grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(w), rows, cols, q, scales);
  } else if (dtype == kBF16) {
    hipLaunchKernelGGL(quantize_fp8_rows_kernel<kBF16>, grid, dim3(256), 0, stream, w, rows, cols,
                       q, scales);
  } else if (dtype == kF16) {
    hipLaunchKernelGGL(quantize_fp8_rows_kernel<kF16>, grid, dim3(256), 0, stream, w, rows, cols,
                       q, scales);
  } else {
    hipLaunchKernelGGL(quantize_fp8_rows_kernel<kF32>, grid, dim3(256), 0, stream, w, rows, cols,
                       q, scales);
  }
  return hipGetLastError();
}

}  // namespace moe
