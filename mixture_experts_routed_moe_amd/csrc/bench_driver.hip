// moe_bench_driver -- drives libmoe_routed through its C ABI from C++, with no
// Python or torch in the process (for hardware-counter profiler passes, and as
// a usage example of the ABI).
//
//   moe_bench_driver routing FILE [STEPS] [FORMAT]
//       Replays a routing dump written by `bench.py --dump-routing FILE`:
//       header {magic, T, K, E, H, D, dtype, block_m} (int32) then topk_ids
//       int32 [T*K] and topk_weights fp32 [T*K]. x and the stacked expert
//       weights are filled on the device with a hashed pattern of the right
//       scale (the data values do not change the memory traffic), then
//       moe_dispatch + the forward run STEPS times; per-step times from HIP
//       events are printed. FORMAT selects the forward: 16bit (default,
//       moe_routed_forward), weighted (moe_routed_forward_weighted), fp8
//       (FP8 weights, moe_routed_forward_w8), w8a8 (FP8 weights and
//       activations, moe_routed_forward_w8a8), w4a8 (moe_routed_forward_w4a8)
//       or mx (moe_routed_forward_mx), the weights quantised once with the
//       library's quantizers before the steps; or fused
//       (moe_routed_forward_fused: tables with block_m <= 32).
//   moe_bench_driver reduce FILE [STEPS] [bf16|fp8]
//       The standalone moe_reduce_fused of a dump written by `bench.py
//       --dump-reduce FILE`: header {magic, T, K, H} then token_topk_to_pos
//       int32 [T*K] and topk_weights fp32 [T*K]; expert_out [T*K, H] is
//       filled with a hashed pattern (bf16, or FP8 E4M3 codes with a scale
//       per row and per token: the quantized form).
//   moe_bench_driver copy BYTES [STEPS]
//       A plain 16-byte-per-lane device copy of BYTES bytes (calibrates the
//       FETCH_SIZE / WRITE_SIZE counters against a known transfer).
//   moe_bench_driver bf16-rounding
//       Checks the library's fp32 -> bf16 conversion (float_to_bf16 of
//       common.hpp: gfx950's conversion instruction) against the integer
//       round-to-nearest-even (add 0x7fff plus the lowest kept bit, keep the
//       high half) on all 2^32 fp32 bit patterns; prints the non-NaN inputs
//       whose bits differ and the NaN inputs whose result is not a NaN, and
//       exits with status 0 only when both counts are 0.
//   moe_bench_driver read [STEPS]
//       The device's read ceiling for the expert-weight stream: 4096
//       workgroups of 256 threads each read 256 rows of 7168 bytes (7.5 GB in
//       all), 16 bytes per thread and load with 32 loads in flight per
//       thread and 96 KB of LDS reserved (one workgroup per CU, as the GEMM
//       kernels run), once in 128-byte pieces of every row per step (the
//       grouped GEMMs' weight pattern) and once in contiguous 4 KB pieces.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "common.hpp"
#include "moe_routed.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int32_t kMagic = 0x4d6f4531;        // "MoE1": routing dump
constexpr int32_t kMagicReduce = 0x4d6f4532;  // "MoE2": standalone-reduce dump

#define CHECK_HIP(x)                                                                  \
  do {                                                                                \
    hipError_t e_ = (x);                                                              \
    if (e_ != hipSuccess) {                                                           \
      std::fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x,                  \
                   hipGetErrorString(e_));                                            \
      std::exit(2);                                                                   \
    }                                                                                 \
  } while (0)

#define CHECK_MOE(x)                                                                  \
  do {                                                                                \
    moe_status s_ = (x);                                                              \
    if (s_ != MOE_OK) {                                                               \
      std::fprintf(stderr, "%s: %s (%s)\n", #x, moe_status_string(s_), moe_last_error()); \
      std::exit(3);                                                                   \
    }                                                                                 \
  } while (0)

// Hashed uniform values in [-scale, scale) as bfloat16 / binary16 bits.
__global__ void fill_kernel(uint16_t* p, size_t n, uint32_t seed, float scale, int dtype) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    uint32_t h = static_cast<uint32_t>(i) * 2654435761u ^ seed;
    h ^= h >> 16;
    h *= 0x7feb352du;
    h ^= h >> 15;
    const float v = (static_cast<float>(h >> 8) * (1.0f / 16777216.0f) * 2.0f - 1.0f) * scale;
    uint16_t bits;
    if (dtype == MOE_BF16) {
      bits = static_cast<uint16_t>(__float_as_uint(v) >> 16);
    } else {
      bits = __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
    }
    p[i] = bits;
  }
}

// Hashed FP8 E4M3 codes of magnitude <= 1.75 (exponent field <= 7), signed.
__global__ void fill_fp8_kernel(uint8_t* p, size_t n, uint32_t seed) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    uint32_t h = static_cast<uint32_t>(i) * 2654435761u ^ seed;
    h ^= h >> 16;
    h *= 0x7feb352du;
    h ^= h >> 15;
    p[i] = static_cast<uint8_t>((h & 0x80u) | ((h >> 8) & 0x3fu));
  }
}

__global__ void fill_f32_kernel(float* p, size_t n, float v) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    p[i] = v;
  }
}

__global__ void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n16) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n16;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    dst[i] = src[i];
  }
}

// Read-only stream over disjoint slabs of 256 rows x RB bytes per workgroup
// (see `read` above); the XOR of everything read is stored so nothing is
// dropped.
constexpr int kReadRowBytes = 7168;
constexpr int kReadInflight = 32;
template <bool LINEAR>
__global__ __launch_bounds__(256) void read_kernel(const uint8_t* __restrict__ w, uint32_t* out) {
  __shared__ uint8_t reserve[96 * 1024];
  constexpr int kLoads = 8;                        // loads per step: 256 rows x 128 B
  constexpr int kUnroll = kReadInflight / kLoads;  // steps per iteration
  constexpr int kSteps = kReadRowBytes / 128;
  static_assert(kSteps % kUnroll == 0, "whole iterations");
  const int t = threadIdx.x;
  const uint8_t* slab = w + static_cast<int64_t>(blockIdx.x) * 256 * kReadRowBytes;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int s0 = 0; s0 < kSteps; s0 += kUnroll) {
    u32x4 v[kUnroll][kLoads];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const int64_t off = LINEAR
            ? (static_cast<int64_t>(s0 + u) * kLoads + i) * 4096 + t * 16
            : static_cast<int64_t>(t / 8 + 32 * i) * kReadRowBytes + (s0 + u) * 128 + (t % 8) * 16;
        v[u][i] = *reinterpret_cast<const u32x4*>(slab + off);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
      for (int i = 0; i < kLoads; ++i) acc ^= v[u][i];
    }
  }
  if (t == 0) reserve[0] = static_cast<uint8_t>(acc.x);
  out[static_cast<int64_t>(blockIdx.x) * 256 + t] = acc.x ^ acc.y ^ acc.z ^ acc.w ^ reserve[0];
}

int run_read(int steps) {
  const int nwg = 4096;
  const size_t bytes = static_cast<size_t>(nwg) * 256 * kReadRowBytes;
  uint8_t* w = nullptr;
  uint32_t* out = nullptr;
  CHECK_HIP(hipMalloc(&w, bytes));
  CHECK_HIP(hipMalloc(&out, static_cast<size_t>(nwg) * 256 * 4));
  CHECK_HIP(hipMemset(w, 1, bytes));
  hipEvent_t e0, e1;
  CHECK_HIP(hipEventCreate(&e0));
  CHECK_HIP(hipEventCreate(&e1));
  for (int linear = 0; linear < 2; ++linear) {
    for (int s = 0; s < steps; ++s) {
      CHECK_HIP(hipEventRecord(e0, nullptr));
      if (linear) {
        hipLaunchKernelGGL(read_kernel<true>, dim3(nwg), dim3(256), 0, nullptr, w, out);
      } else {
        hipLaunchKernelGGL(read_kernel<false>, dim3(nwg), dim3(256), 0, nullptr, w, out);
      }
      CHECK_HIP(hipGetLastError());
      CHECK_HIP(hipEventRecord(e1, nullptr));
      CHECK_HIP(hipEventSynchronize(e1));
      float ms = 0.0f;
      CHECK_HIP(hipEventElapsedTime(&ms, e0, e1));
      std::printf("read %s %zu bytes: %.4f ms (%.1f GB/s)\n", linear ? "linear-4KB" : "rows-128B",
                  bytes, ms, bytes / (ms * 1e6));
    }
  }
  CHECK_HIP(hipFree(w));
  CHECK_HIP(hipFree(out));
  return 0;
}

// Integer round-to-nearest-even fp32 -> bf16 (the reference of the check).
__device__ uint32_t bf16_rne_integer(uint32_t u) { return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16; }

__global__ void bf16_rounding_kernel(unsigned long long* counts, uint32_t* first_bad) {
  unsigned long long bad = 0, bad_nan = 0;
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
  for (uint64_t x = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; x < (1ull << 32);
       x += stride) {
    const uint32_t u = static_cast<uint32_t>(x);
    const uint32_t got = moe::float_to_bf16(__uint_as_float(u));
    if ((u & 0x7fffffffu) > 0x7f800000u) {
      if ((got & 0x7fffu) <= 0x7f80u) ++bad_nan;
    } else if (got != bf16_rne_integer(u)) {
      ++bad;
      atomicMin(first_bad, u);
    }
  }
  atomicAdd(&counts[0], bad);
  atomicAdd(&counts[1], bad_nan);
}

int run_bf16_rounding() {
  unsigned long long* counts = nullptr;
  uint32_t* first_bad = nullptr;
  CHECK_HIP(hipMalloc(&counts, 2 * sizeof(unsigned long long)));
  CHECK_HIP(hipMalloc(&first_bad, sizeof(uint32_t)));
  CHECK_HIP(hipMemset(counts, 0, 2 * sizeof(unsigned long long)));
  CHECK_HIP(hipMemset(first_bad, 0xff, sizeof(uint32_t)));
  hipLaunchKernelGGL(bf16_rounding_kernel, dim3(8192), dim3(256), 0, nullptr, counts, first_bad);
  CHECK_HIP(hipGetLastError());
  unsigned long long h[2];
  uint32_t first = 0;
  CHECK_HIP(hipMemcpy(h, counts, sizeof(h), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(&first, first_bad, sizeof(first), hipMemcpyDeviceToHost));
  std::printf("bf16-rounding: non-NaN mismatches %llu (first input 0x%08x), NaN inputs not NaN %llu\n",
              h[0], first, h[1]);
  CHECK_HIP(hipFree(counts));
  CHECK_HIP(hipFree(first_bad));
  return (h[0] == 0 && h[1] == 0) ? 0 : 3;
}

void fill(uint16_t* p, size_t n, uint32_t seed, float scale, int dtype) {
  hipLaunchKernelGGL(fill_kernel, dim3(8192), dim3(256), 0, nullptr, p, n, seed, scale, dtype);
  CHECK_HIP(hipGetLastError());
}

int run_copy(size_t bytes, int steps) {
  bytes = bytes / 16 * 16;
  void *a = nullptr, *b = nullptr;
  CHECK_HIP(hipMalloc(&a, bytes));
  CHECK_HIP(hipMalloc(&b, bytes));
  CHECK_HIP(hipMemset(a, 1, bytes));
  hipEvent_t e0, e1;
  CHECK_HIP(hipEventCreate(&e0));
  CHECK_HIP(hipEventCreate(&e1));
  for (int s = 0; s < steps; ++s) {
    CHECK_HIP(hipEventRecord(e0, nullptr));
    hipLaunchKernelGGL(copy_kernel, dim3(16384), dim3(256), 0, nullptr,
                       static_cast<const u32x4*>(a), static_cast<u32x4*>(b), bytes / 16);
    CHECK_HIP(hipGetLastError());
    CHECK_HIP(hipEventRecord(e1, nullptr));
    CHECK_HIP(hipEventSynchronize(e1));
    float ms = 0.0f;
    CHECK_HIP(hipEventElapsedTime(&ms, e0, e1));
    std::printf("copy %zu bytes: %.4f ms (%.1f GB/s read+write)\n", bytes, ms,
                2.0 * bytes / (ms * 1e6));
  }
  CHECK_HIP(hipFree(a));
  CHECK_HIP(hipFree(b));
  return 0;
}

enum Format { kFmt16 = 0, kFmtWeighted, kFmtFp8, kFmtW4a8, kFmtMx, kFmtW8a8, kFmtFused };

int parse_format(const char* s) {
  if (!s || std::strcmp(s, "16bit") == 0) return kFmt16;
  if (std::strcmp(s, "weighted") == 0) return kFmtWeighted;
  if (std::strcmp(s, "fp8") == 0) return kFmtFp8;
  if (std::strcmp(s, "w4a8") == 0) return kFmtW4a8;
  if (std::strcmp(s, "mx") == 0) return kFmtMx;
  if (std::strcmp(s, "w8a8") == 0) return kFmtW8a8;
  if (std::strcmp(s, "fused") == 0) return kFmtFused;
  return -1;
}

void* dmalloc(size_t bytes) {
  void* p = nullptr;
  CHECK_HIP(hipMalloc(&p, bytes ? bytes : 1));
  return p;
}

int run_routing(const char* path, int steps, int fmt) {
  FILE* f = std::fopen(path, "rb");
  if (!f) {
    std::fprintf(stderr, "cannot open %s\n", path);
    return 1;
  }
  int32_t hdr[8];
  if (std::fread(hdr, sizeof(int32_t), 8, f) != 8 || hdr[0] != kMagic) {
    std::fprintf(stderr, "%s is not a routing dump\n", path);
    std::fclose(f);
    return 1;
  }
  const int T = hdr[1], K = hdr[2], E = hdr[3], H = hdr[4], D = hdr[5], dtype = hdr[6],
            block_m = hdr[7];
  const size_t P = static_cast<size_t>(T) * K;
  std::vector<int32_t> ids(P);
  std::vector<float> w(P);
  const bool ok = std::fread(ids.data(), sizeof(int32_t), P, f) == P &&
                  std::fread(w.data(), sizeof(float), P, f) == P;
  std::fclose(f);
  if (!ok) {
    std::fprintf(stderr, "%s is truncated\n", path);
    return 1;
  }
  if (fmt != kFmt16 && fmt != kFmtWeighted && fmt != kFmtFused && dtype == MOE_F32) {
    std::fprintf(stderr, "quantised formats need a 16-bit dtype\n");
    return 1;
  }
  std::printf("routing %s: T=%d K=%d E=%d H=%d D=%d dtype=%d block_m=%d format=%d\n", path, T, K,
              E, H, D, dtype, block_m, fmt);

  int32_t* d_ids = static_cast<int32_t*>(dmalloc(P * sizeof(int32_t)));
  float* d_w = static_cast<float*>(dmalloc(P * sizeof(float)));
  CHECK_HIP(hipMemcpy(d_ids, ids.data(), P * sizeof(int32_t), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_w, w.data(), P * sizeof(float), hipMemcpyHostToDevice));

  const size_t nx = static_cast<size_t>(T) * H;
  const size_t nw = static_cast<size_t>(E) * D * H;
  uint16_t* x = static_cast<uint16_t*>(dmalloc(nx * 2));
  uint16_t* y = static_cast<uint16_t*>(dmalloc(nx * 2));
  uint16_t* wt[3];
  for (auto& p : wt) p = static_cast<uint16_t*>(dmalloc(nw * 2));
  fill(x, nx, 1, 1.7f, dtype);
  fill(wt[0], nw, 2, 1.7f / std::sqrt(static_cast<float>(H)), dtype);
  fill(wt[1], nw, 3, 1.7f / std::sqrt(static_cast<float>(H)), dtype);
  fill(wt[2], nw, 4, 1.7f / std::sqrt(static_cast<float>(D)), dtype);

  // Quantised weights: codes and scales from the library's quantizers; the
  // 16-bit copies are freed before the steps.
  void* q[3] = {nullptr, nullptr, nullptr};
  void* s[3] = {nullptr, nullptr, nullptr};
  const int64_t rows[3] = {static_cast<int64_t>(E) * D, static_cast<int64_t>(E) * D,
                           static_cast<int64_t>(E) * H};
  const int cols[3] = {H, H, D};
  if (fmt == kFmtFp8 || fmt == kFmtW8a8 || fmt == kFmtW4a8 || fmt == kFmtMx) {
    for (int i = 0; i < 3; ++i) {
      const size_t n = static_cast<size_t>(rows[i]) * cols[i];
      if (fmt == kFmtFp8 || fmt == kFmtW8a8) {
        q[i] = dmalloc(n);
        s[i] = dmalloc(rows[i] * sizeof(float));
        CHECK_MOE(moe_quantize_fp8_rows(wt[i], rows[i], cols[i], dtype, static_cast<uint8_t*>(q[i]),
                                        static_cast<float*>(s[i]), nullptr));
      } else if (fmt == kFmtW4a8) {
        q[i] = dmalloc(n / 2);
        s[i] = dmalloc(rows[i] * sizeof(float));
        CHECK_MOE(moe_quantize_int4_rows(wt[i], rows[i], cols[i], dtype,
                                         static_cast<uint8_t*>(q[i]), static_cast<float*>(s[i]),
                                         nullptr));
      } else {
        q[i] = dmalloc(n / 2);
        s[i] = dmalloc(n / 32);
        CHECK_MOE(moe_quantize_mx_rows(wt[i], rows[i], cols[i], dtype, MOE_MX_FP4,
                                       static_cast<uint8_t*>(q[i]), static_cast<uint8_t*>(s[i]),
                                       nullptr));
      }
    }
    CHECK_HIP(hipDeviceSynchronize());
    for (auto& p : wt) {
      CHECK_HIP(hipFree(p));
      p = nullptr;
    }
  }

  const size_t tb = moe_tables_bytes(T, K, E, block_m);
  void* tbuf = dmalloc(tb);
  moe_tables tables;
  CHECK_MOE(moe_tables_bind(&tables, tbuf, tb, T, K, E, block_m));
  size_t wsb = moe_forward_workspace_bytes(T, K, H, D, dtype);
  if (fmt == kFmtW4a8) wsb = moe_forward_w4a8_workspace_bytes(T, K, H, D, dtype);
  if (fmt == kFmtMx) wsb = moe_forward_mx_workspace_bytes(T, K, H, D, dtype);
  if (fmt == kFmtW8a8) wsb = moe_forward_w8a8_workspace_bytes(T, K, H, D, dtype);
  if (fmt == kFmtFused) wsb = moe_fused_workspace_bytes(T, K, H, dtype);
  void* ws = dmalloc(wsb);
  CHECK_HIP(hipDeviceSynchronize());

  const uint8_t* const* qb = reinterpret_cast<const uint8_t* const*>(q);
  hipEvent_t ev[3];
  for (auto& e : ev) CHECK_HIP(hipEventCreate(&e));
  for (int st = 0; st < steps; ++st) {
    CHECK_HIP(hipEventRecord(ev[0], nullptr));
    CHECK_MOE(moe_dispatch(d_ids, d_w, &tables, nullptr));
    CHECK_HIP(hipEventRecord(ev[1], nullptr));
    switch (fmt) {
      case kFmt16:
        CHECK_MOE(moe_routed_forward(x, wt[0], wt[1], wt[2], &tables, H, D, dtype, ws, wsb, y,
                                     nullptr));
        break;
      case kFmtFused:
        CHECK_MOE(moe_routed_forward_fused(x, wt[0], wt[1], wt[2], &tables, H, D, dtype, ws, wsb,
                                           y, nullptr));
        break;
      case kFmtWeighted:
        CHECK_MOE(moe_routed_forward_weighted(x, wt[0], wt[1], wt[2], &tables, H, D, dtype, ws,
                                              wsb, y, nullptr));
        break;
      case kFmtFp8:
        CHECK_MOE(moe_routed_forward_w8(x, qb[0], qb[1], qb[2], static_cast<float*>(s[0]),
                                        static_cast<float*>(s[1]), static_cast<float*>(s[2]),
                                        &tables, H, D, dtype, ws, wsb, y, nullptr));
        break;
      case kFmtW8a8:
        CHECK_MOE(moe_routed_forward_w8a8(x, qb[0], qb[1], qb[2], static_cast<float*>(s[0]),
                                          static_cast<float*>(s[1]), static_cast<float*>(s[2]),
                                          &tables, H, D, dtype, ws, wsb, y, nullptr));
        break;
      case kFmtW4a8:
        CHECK_MOE(moe_routed_forward_w4a8(x, qb[0], qb[1], qb[2], static_cast<float*>(s[0]),
                                          static_cast<float*>(s[1]), static_cast<float*>(s[2]),
                                          &tables, H, D, dtype, ws, wsb, y, nullptr));
        break;
      default:
        CHECK_MOE(moe_routed_forward_mx(x, qb[0], qb[1], qb[2], static_cast<uint8_t*>(s[0]),
                                        static_cast<uint8_t*>(s[1]), static_cast<uint8_t*>(s[2]),
                                        &tables, H, D, dtype, ws, wsb, y, nullptr));
        break;
    }
    CHECK_HIP(hipEventRecord(ev[2], nullptr));
    CHECK_HIP(hipEventSynchronize(ev[2]));
    float ms_d = 0.0f, ms_f = 0.0f;
    CHECK_HIP(hipEventElapsedTime(&ms_d, ev[0], ev[1]));
    CHECK_HIP(hipEventElapsedTime(&ms_f, ev[1], ev[2]));
    std::printf("step %d: dispatch %.4f ms, forward %.4f ms\n", st, ms_d, ms_f);
  }
  int32_t status = 0;
  CHECK_HIP(hipMemcpy(&status, tables.status, sizeof(int32_t), hipMemcpyDeviceToHost));
  std::printf("dispatch status %d\n", status);
  for (void* p : {static_cast<void*>(d_ids), static_cast<void*>(d_w), static_cast<void*>(x),
                  static_cast<void*>(y), tbuf, ws, static_cast<void*>(wt[0]),
                  static_cast<void*>(wt[1]), static_cast<void*>(wt[2]), q[0], q[1], q[2], s[0],
                  s[1], s[2]}) {
    if (p) CHECK_HIP(hipFree(p));
  }
  return 0;
}

int run_reduce(const char* path, int steps, bool fp8) {
  FILE* f = std::fopen(path, "rb");
  if (!f) {
    std::fprintf(stderr, "cannot open %s\n", path);
    return 1;
  }
  int32_t hdr[4];
  if (std::fread(hdr, sizeof(int32_t), 4, f) != 4 || hdr[0] != kMagicReduce) {
    std::fprintf(stderr, "%s is not a reduce dump\n", path);
    std::fclose(f);
    return 1;
  }
  const int T = hdr[1], K = hdr[2], H = hdr[3];
  const size_t P = static_cast<size_t>(T) * K;
  std::vector<int32_t> pos(P);
  std::vector<float> w(P);
  const bool ok = std::fread(pos.data(), sizeof(int32_t), P, f) == P &&
                  std::fread(w.data(), sizeof(float), P, f) == P;
  std::fclose(f);
  if (!ok) {
    std::fprintf(stderr, "%s is truncated\n", path);
    return 1;
  }
  for (int32_t p : pos) {
    if (p >= static_cast<int64_t>(P)) {
      std::fprintf(stderr, "%s holds a position out of range\n", path);
      return 1;
    }
  }
  std::printf("reduce %s: T=%d K=%d H=%d %s\n", path, T, K, H, fp8 ? "fp8" : "bf16");
  int32_t* d_pos = static_cast<int32_t*>(dmalloc(P * sizeof(int32_t)));
  float* d_w = static_cast<float*>(dmalloc(P * sizeof(float)));
  CHECK_HIP(hipMemcpy(d_pos, pos.data(), P * sizeof(int32_t), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_w, w.data(), P * sizeof(float), hipMemcpyHostToDevice));
  const size_t n = P * H;
  void* xo = dmalloc(n * (fp8 ? 1 : 2));
  void* y = dmalloc(static_cast<size_t>(T) * H * (fp8 ? 1 : 2));
  float* x_sf = static_cast<float*>(dmalloc(P * sizeof(float)));
  float* sf = static_cast<float*>(dmalloc(T * sizeof(float)));
  if (fp8) {
    hipLaunchKernelGGL(fill_fp8_kernel, dim3(8192), dim3(256), 0, nullptr,
                       static_cast<uint8_t*>(xo), n, 5u);
    hipLaunchKernelGGL(fill_f32_kernel, dim3(256), dim3(256), 0, nullptr, x_sf, P, 0.03f);
    hipLaunchKernelGGL(fill_f32_kernel, dim3(16), dim3(256), 0, nullptr, sf, static_cast<size_t>(T),
                       2.0f);
    CHECK_HIP(hipGetLastError());
  } else {
    fill(static_cast<uint16_t*>(xo), n, 5, 1.7f, MOE_BF16);
  }
  CHECK_HIP(hipDeviceSynchronize());
  hipEvent_t ev[2];
  for (auto& e : ev) CHECK_HIP(hipEventCreate(&e));
  for (int st = 0; st < steps; ++st) {
    CHECK_HIP(hipEventRecord(ev[0], nullptr));
    if (fp8) {
      CHECK_MOE(moe_reduce_fused_scaled(xo, static_cast<int64_t>(P), d_pos, d_w, x_sf, sf, T, K, H,
                                        MOE_FP8_E4M3, MOE_FP8_E4M3, y, nullptr));
    } else {
      CHECK_MOE(moe_reduce_fused(xo, static_cast<int64_t>(P), d_pos, d_w, T, K, H, MOE_BF16,
                                 MOE_BF16, y, nullptr));
    }
    CHECK_HIP(hipEventRecord(ev[1], nullptr));
    CHECK_HIP(hipEventSynchronize(ev[1]));
    float ms = 0.0f;
    CHECK_HIP(hipEventElapsedTime(&ms, ev[0], ev[1]));
    std::printf("step %d: reduce %.4f ms\n", st, ms);
  }
  for (void* p : {static_cast<void*>(d_pos), static_cast<void*>(d_w), xo, y,
                  static_cast<void*>(x_sf), static_cast<void*>(sf)}) {
    CHECK_HIP(hipFree(p));
  }
  return 0;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc >= 3 && std::strcmp(argv[1], "routing") == 0) {
    const int fmt = parse_format(argc >= 5 ? argv[4] : nullptr);
    if (fmt < 0) {
      std::fprintf(stderr, "unknown format %s\n", argv[4]);
      return 1;
    }
    return run_routing(argv[2], argc >= 4 ? std::atoi(argv[3]) : 3, fmt);
  }
  if (argc >= 3 && std::strcmp(argv[1], "reduce") == 0) {
    const bool fp8 = argc >= 5 && std::strcmp(argv[4], "fp8") == 0;
    return run_reduce(argv[2], argc >= 4 ? std::atoi(argv[3]) : 3, fp8);
  }
  if (argc >= 3 && std::strcmp(argv[1], "copy") == 0) {
    return run_copy(std::strtoull(argv[2], nullptr, 10), argc >= 4 ? std::atoi(argv[3]) : 3);
  }
  if (argc >= 2 && std::strcmp(argv[1], "bf16-rounding") == 0) return run_bf16_rounding();
  if (argc >= 2 && std::strcmp(argv[1], "read") == 0) {
    return run_read(argc >= 3 ? std::atoi(argv[2]) : 5);
  }
  std::fprintf(stderr,
               "usage: %s routing FILE [STEPS] [16bit|weighted|fp8|w8a8|w4a8|mx|fused] | reduce FILE [STEPS] "
               "[bf16|fp8] | copy BYTES [STEPS] | read [STEPS] | bf16-rounding\n",
               argv[0]);
  return 1;
}
