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

// Eight 16-bit values (one 16-byte load): their largest magnitude, and
// their E4M3 codes at scale s (v / s, then the packed hardware encoding).
template <int DT>
__device__ __forceinline__ float amax8(u32x4 w, float amax) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    amax = fmaxf(amax, fabsf(to_float<DT>(w[j] & 0xffffu)));
    amax = fmaxf(amax, fabsf(to_float<DT>(w[j] >> 16)));
  }
  return amax;
}

template <int DT>
__device__ __forceinline__ u32x2 encode8_fp8(u32x4 w, float s) {
  float f[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = to_float<DT>(w[j] & 0xffffu) / s;
    f[2 * j + 1] = to_float<DT>(w[j] >> 16) / s;
  }
  return u32x2{pk4_fp8e4m3(f[0], f[1], f[2], f[3]), pk4_fp8e4m3(f[4], f[5], f[6], f[7])};
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
  for (int v = lane; v < nvec; v += 64) amax = amax8<DT>(row[v], amax);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  if (lane == 0) scales[r] = s;
  u32x2* out = reinterpret_cast<u32x2*>(q + r * cols);
#pragma unroll 4
  for (int v = lane; v < nvec; v += 64) out[v] = encode8_fp8<DT>(row[v], s);
}

// The same for rows of at most 512 NV values, held in registers between the
// amax and the encoding: the row is read from memory once (with many rows
// in flight per CU the second read of the two-pass form mostly misses the
// cache and reads the row from HBM again).
template <int DT, int NV>
__global__ __launch_bounds__(256) void quantize_fp8_rows_reg_kernel(const uint16_t* __restrict__ a,
                                                                    int64_t rows, int cols,
                                                                    uint8_t* __restrict__ q,
                                                                    float* __restrict__ scales) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;   // the whole wave exits together
  const int lane = threadIdx.x & 63;
  const u32x4* row = reinterpret_cast<const u32x4*>(a + r * cols);
  const int nvec = cols / 8;
  u32x4 w[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = lane + 64 * i;
    w[i] = v < nvec ? row[v] : u32x4{0u, 0u, 0u, 0u};   // zeros leave the amax unchanged
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i) amax = amax8<DT>(w[i], amax);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  if (lane == 0) scales[r] = s;
  u32x2* out = reinterpret_cast<u32x2*>(q + r * cols);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = lane + 64 * i;
    if (v < nvec) out[v] = encode8_fp8<DT>(w[i], s);
  }
}

// Launches the register form for 16-bit rows of at most 8192 values, the
// two-pass form for longer ones.
template <int DT>
void launch_fp8_rows16(const uint16_t* a, int64_t rows, int cols, uint8_t* q, float* scales,
                       dim3 grid, hipStream_t stream) {
  const int nvec = cols / 8;   // 16-byte loads per row; the register form up to 16 per lane
  auto reg = [&](auto NV) {
    hipLaunchKernelGGL((quantize_fp8_rows_reg_kernel<DT, decltype(NV)::value>), grid, dim3(256), 0, stream, a, rows,
                       cols, q, scales);
  };
  if (nvec <= 64) {
    reg(int_c<1>{});
  } else if (nvec <= 128) {
    reg(int_c<2>{});
  } else if (nvec <= 256) {
    reg(int_c<4>{});
  } else if (nvec <= 512) {
    reg(int_c<8>{});
  } else if (nvec <= 1024) {
    reg(int_c<16>{});
  } else {
    hipLaunchKernelGGL(quantize_fp8_rows16_kernel<DT>, grid, dim3(256), 0, stream, a, rows, cols, q, scales);
  }
}

}  // namespace

hipError_t launch_quantize_fp8_rows(const void* w, int64_t rows, int cols, int dtype, uint8_t* q,
                                    float* scales, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((rows + 3) / 4));
  const bool vec = dtype != kF32 && cols % 8 == 0 && reinterpret_cast<uintptr_t>(w) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(q) % 8 == 0;
  if (vec && dtype == kBF16) {
    launch_fp8_rows16<kBF16>(static_cast<const uint16_t*>(w), rows, cols, q, scales, grid, stream);
  } else if (vec) {
    launch_fp8_rows16<kF16>(static_cast<const uint16_t*>(w), rows, cols, q, scales, grid, stream);
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
