// moe_bench_driver -- drives libmoe_routed through its C ABI from C++, with no
// Python or torch in the process (for hardware-counter profiler passes, and as
// a usage example of the ABI).
//
//   moe_bench_driver routing FILE [STEPS]
//       Replays a routing dump written by `bench.py --dump-routing FILE`:
//       header {magic, T, K, E, H, D, dtype, block_m} (int32) then topk_ids
//       int32 [T*K] and topk_weights fp32 [T*K]. x and the stacked expert
//       weights are filled on the device with a hashed pattern of the right
//       scale (the data values do not change the memory traffic), then
//       moe_dispatch + moe_routed_forward run STEPS times; per-step times
//       from HIP events are printed.
//   moe_bench_driver copy BYTES [STEPS]
//       A plain 16-byte-per-lane device copy of BYTES bytes (calibrates the
//       FETCH_SIZE / WRITE_SIZE counters against a known transfer).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "moe_routed.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int32_t kMagic = 0x4d6f4531;   // "MoE1"

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

__global__ void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n16) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n16;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    dst[i] = src[i];
  }
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

int run_routing(const char* path, int steps) {
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
  std::printf("routing %s: T=%d K=%d E=%d H=%d D=%d dtype=%d block_m=%d\n", path, T, K, E, H,
              D, dtype, block_m);

  int32_t* d_ids = nullptr;
  float* d_w = nullptr;
  CHECK_HIP(hipMalloc(&d_ids, P * sizeof(int32_t)));
  CHECK_HIP(hipMalloc(&d_w, P * sizeof(float)));
  CHECK_HIP(hipMemcpy(d_ids, ids.data(), P * sizeof(int32_t), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_w, w.data(), P * sizeof(float), hipMemcpyHostToDevice));

  const size_t nx = static_cast<size_t>(T) * H;
  const size_t nw = static_cast<size_t>(E) * D * H;
  uint16_t *x = nullptr, *wg = nullptr, *wu = nullptr, *wd = nullptr, *y = nullptr;
  CHECK_HIP(hipMalloc(&x, nx * 2));
  CHECK_HIP(hipMalloc(&wg, nw * 2));
  CHECK_HIP(hipMalloc(&wu, nw * 2));
  CHECK_HIP(hipMalloc(&wd, nw * 2));
  CHECK_HIP(hipMalloc(&y, nx * 2));
  fill(x, nx, 1, 1.7f, dtype);
  fill(wg, nw, 2, 1.7f / std::sqrt(static_cast<float>(H)), dtype);
  fill(wu, nw, 3, 1.7f / std::sqrt(static_cast<float>(H)), dtype);
  fill(wd, nw, 4, 1.7f / std::sqrt(static_cast<float>(D)), dtype);

  const size_t tb = moe_tables_bytes(T, K, E, block_m);
  void* tbuf = nullptr;
  CHECK_HIP(hipMalloc(&tbuf, tb));
  moe_tables tables;
  CHECK_MOE(moe_tables_bind(&tables, tbuf, tb, T, K, E, block_m));
  const size_t wsb = moe_forward_workspace_bytes(T, K, H, D, dtype);
  void* ws = nullptr;
  CHECK_HIP(hipMalloc(&ws, wsb));
  CHECK_HIP(hipDeviceSynchronize());

  hipEvent_t ev[3];
  for (auto& e : ev) CHECK_HIP(hipEventCreate(&e));
  for (int s = 0; s < steps; ++s) {
    CHECK_HIP(hipEventRecord(ev[0], nullptr));
    CHECK_MOE(moe_dispatch(d_ids, d_w, &tables, nullptr));
    CHECK_HIP(hipEventRecord(ev[1], nullptr));
    CHECK_MOE(moe_routed_forward(x, wg, wu, wd, &tables, H, D, dtype, ws, wsb, y, nullptr));
    CHECK_HIP(hipEventRecord(ev[2], nullptr));
    CHECK_HIP(hipEventSynchronize(ev[2]));
    float ms_d = 0.0f, ms_f = 0.0f;
    CHECK_HIP(hipEventElapsedTime(&ms_d, ev[0], ev[1]));
    CHECK_HIP(hipEventElapsedTime(&ms_f, ev[1], ev[2]));
    std::printf("step %d: dispatch %.4f ms, forward %.4f ms\n", s, ms_d, ms_f);
  }
  int32_t status = 0;
  CHECK_HIP(hipMemcpy(&status, tables.status, sizeof(int32_t), hipMemcpyDeviceToHost));
  std::printf("dispatch status %d\n", status);
  for (void* p : {static_cast<void*>(d_ids), static_cast<void*>(d_w), static_cast<void*>(x),
                  static_cast<void*>(wg), static_cast<void*>(wu), static_cast<void*>(wd),
                  static_cast<void*>(y), tbuf, ws}) {
    CHECK_HIP(hipFree(p));
  }
  return 0;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc >= 3 && std::strcmp(argv[1], "routing") == 0) {
    return run_routing(argv[2], argc >= 4 ? std::atoi(argv[3]) : 3);
  }
  if (argc >= 3 && std::strcmp(argv[1], "copy") == 0) {
    return run_copy(std::strtoull(argv[2], nullptr, 10), argc >= 4 ? std::atoi(argv[3]) : 3);
  }
  std::fprintf(stderr, "usage: %s routing FILE [STEPS] | copy BYTES [STEPS]\n", argv[0]);
  return 1;
}
