// moe_reduce_fused on gfx950: top-k weighted, fp32-accumulated reduce of the
// expert outputs back to token order.
//
// Semantics (TileOPs-Metax PR #55 "moe_reduce_fused", sections 1-2):
//   y[t, :] = cast( sum over k ascending with pos[t,k] >= 0 of
//                   w[t,k] * X[pos[t,k], :] )
// accumulated in fp32, with one cast at the end; masked slots (pos < 0) are
// neither read nor accumulated; NULL weights mean all ones.
//
// Design: the step is a pure HBM stream (K gathered input rows in, one row
// out per token). A workgroup owns one token and a 16-byte-per-lane slice of
// the hidden dimension (a 1-D grid of T * H/(8*threads) workgroups), so the
// token's K positions and weights are uniform (scalar loads) and every lane
// issues the loads of ALL its K rows before the
// first multiply-add: each lane keeps K independent 16-byte loads in flight,
// which is the look-ahead the PR builds by hand, without a serial pipeline.
// The multiply-adds then run in k order with fmaf, so the fp32 sums are the
// exact sequence of fused multiply-adds of a k-ascending loop.

#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kVec = 8;        // elements per lane per row (16 B at 16-bit)
constexpr int kSlots = 8;      // rows whose loads are issued together

template <int DT>
struct Row8 {                  // 8 consecutive elements of one row
  u32x4 v[DT == kF32 ? 2 : 1];
};

template <int DT>
__device__ __forceinline__ void load_row8(const void* base, int64_t elem, Row8<DT>& r) {
  if constexpr (DT == kF32) {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const float*>(base) + elem);
    r.v[0] = __builtin_nontemporal_load(p);
    r.v[1] = __builtin_nontemporal_load(p + 1);
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + elem);
    r.v[0] = __builtin_nontemporal_load(p);
  }
}

template <int DT>
__device__ __forceinline__ float row8_elem(const Row8<DT>& r, int i) {
  if constexpr (DT == kF32) {
    return __uint_as_float(r.v[i >> 2][i & 3]);
  } else {
    const uint32_t w = r.v[0][i >> 1];
    return to_float<DT>((i & 1) ? (w >> 16) : (w & 0xffffu));
  }
}

template <int IN_DT, int OUT_DT>
__global__ __launch_bounds__(256) void reduce_fused_kernel(
    const void* __restrict__ x, int64_t rows, const int32_t* __restrict__ pos,
    const float* __restrict__ w, int K, int H, int tiles_per_token, void* __restrict__ y) {
  const int t = blockIdx.x / tiles_per_token;
  const int tile = blockIdx.x - t * tiles_per_token;
  const int c = (tile * blockDim.x + threadIdx.x) * kVec;
  if (c >= H) return;
  const int32_t* pt = pos + static_cast<int64_t>(t) * K;
  const float* wt = w ? w + static_cast<int64_t>(t) * K : nullptr;

  float acc[kVec];
#pragma unroll
  for (int i = 0; i < kVec; ++i) acc[i] = 0.0f;

  for (int k0 = 0; k0 < K; k0 += kSlots) {
    Row8<IN_DT> r[kSlots];
    int32_t p[kSlots];
#pragma unroll
    for (int j = 0; j < kSlots; ++j) {
      p[j] = (k0 + j < K) ? pt[k0 + j] : -1;
      if (p[j] >= rows) p[j] = -1;   // out-of-range positions are a precondition
                                     // violation; they are skipped, never read
      if (p[j] >= 0) load_row8<IN_DT>(x, static_cast<int64_t>(p[j]) * H + c, r[j]);
    }
#pragma unroll
    for (int j = 0; j < kSlots; ++j) {
      if (p[j] >= 0) {
        const float wk = wt ? wt[k0 + j] : 1.0f;
#pragma unroll
        for (int i = 0; i < kVec; ++i) acc[i] = __builtin_fmaf(wk, row8_elem<IN_DT>(r[j], i), acc[i]);
      }
    }
  }

  const int64_t o = static_cast<int64_t>(t) * H + c;
  if constexpr (OUT_DT == kF32) {
    float4* yp = reinterpret_cast<float4*>(static_cast<float*>(y) + o);
    yp[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    yp[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  } else {
    u32x4 q;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      q[i] = from_float<OUT_DT>(acc[2 * i]) | (from_float<OUT_DT>(acc[2 * i + 1]) << 16);
    }
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(y) + o) = q;
  }
}

template <int IN_DT, int OUT_DT>
hipError_t launch_typed(const void* x, int64_t rows, const int32_t* pos, const float* w, int T,
                        int K, int H, void* y, hipStream_t stream) {
  const int lanes = H / kVec;   // H % 256 == 0, so lanes % 32 == 0
  int threads = 256;
  while (lanes % threads != 0) threads >>= 1;
  const int tiles = lanes / threads;
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(tiles) * T));
  hipLaunchKernelGGL((reduce_fused_kernel<IN_DT, OUT_DT>), grid, dim3(threads), 0, stream, x,
                     rows, pos, w, K, H, tiles, y);
  return hipGetLastError();
}

template <int IN_DT>
hipError_t launch_out(const void* x, int64_t rows, const int32_t* pos, const float* w, int T,
                      int K, int H, int out_dtype, void* y, hipStream_t stream) {
  switch (out_dtype) {
    case kF16: return launch_typed<IN_DT, kF16>(x, rows, pos, w, T, K, H, y, stream);
    case kBF16: return launch_typed<IN_DT, kBF16>(x, rows, pos, w, T, K, H, y, stream);
    default: return launch_typed<IN_DT, kF32>(x, rows, pos, w, T, K, H, y, stream);
  }
}

}  // namespace

hipError_t launch_reduce(const void* x, int64_t rows, const int32_t* pos, const float* w, int T,
                         int K, int H, int in_dtype, int out_dtype, void* y, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  switch (in_dtype) {
    case kF16: return launch_out<kF16>(x, rows, pos, w, T, K, H, out_dtype, y, stream);
    case kBF16: return launch_out<kBF16>(x, rows, pos, w, T, K, H, out_dtype, y, stream);
    default: return launch_out<kF32>(x, rows, pos, w, T, K, H, out_dtype, y, stream);
  }
}

}  // namespace moe
