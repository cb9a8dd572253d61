// moe_reduce_fused on gfx950: top-k weighted, fp32-accumulated reduce of the
// expert outputs back to token order, with the optional scale factors and
// FP8 storage of the variants.
//
// Semantics (TileOPs-Metax PR #55 "moe_reduce_fused", sections 1-2 and its
// commit notes on the scaled variants):
//   y[t, :] = cast( sf[t] * sum over k ascending with pos[t,k] >= 0 of
//                   (w[t,k] * x_sf[pos[t,k]]) * X[pos[t,k], :] )
// accumulated in fp32, with one cast at the end; masked slots (pos < 0) are
// neither read nor accumulated; NULL weights / x_sf / sf mean ones. x_sf is a
// scale per expanded row of X (one multiply per routed slot), sf a scale per
// token (one multiply per output element). X and y may be FP8 e4m3 (OCP,
// "fn": no infinities, max 448, the cast saturates).
//
// Design: the step is a pure HBM stream (K gathered input rows in, one row
// out per token). A workgroup owns one token and a slice of the hidden
// dimension (a 1-D grid of one-wave workgroups), so the token's K
// positions, weights and scales are uniform (scalar loads), and every lane
// issues the loads of ALL its K rows (16 bytes of each) before the
// first multiply-add: each lane keeps K independent loads in flight, which is
// the look-ahead the PR builds by hand, without a serial pipeline. The
// multiply-adds then run in k order with fmaf, so the fp32 sums are the
// exact sequence of fused multiply-adds of a k-ascending loop. The gathered
// rows are read once and measured faster with non-temporal loads.

#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kSlots = 8;      // rows whose loads are issued together

template <int DT>
constexpr int elem_bytes() {
  return DT == kF32 ? 4 : (DT == kFP8 ? 1 : 2);
}

// V consecutive elements of one row as 32-bit words (16-byte loads where the
// slice holds a multiple of 16 bytes, else 8-byte loads).
template <int DT, int V>
struct RowV {
  static constexpr int kW = V * elem_bytes<DT>() / 4;
  uint32_t w[kW];
};

template <int DT, int V>
__device__ __forceinline__ void load_row(const void* base, int64_t elem, RowV<DT, V>& r) {
  constexpr int kW = RowV<DT, V>::kW;
  const uint8_t* p = static_cast<const uint8_t*>(base) + elem * elem_bytes<DT>();
  if constexpr (kW % 4 == 0) {
#pragma unroll
    for (int i = 0; i < kW / 4; ++i) {
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + i);
      r.w[4 * i] = v[0];
      r.w[4 * i + 1] = v[1];
      r.w[4 * i + 2] = v[2];
      r.w[4 * i + 3] = v[3];
    }
  } else {
    static_assert(kW == 2, "row slices are 8 or 16*n bytes");
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    r.w[0] = v[0];
    r.w[1] = v[1];
  }
}

// acc[i] = fma(wk, row[i], acc[i]) for the V elements of one row.
template <int DT, int V>
__device__ __forceinline__ void fma_row(float wk, const RowV<DT, V>& r, float* acc) {
  if constexpr (DT == kF32) {
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = __builtin_fmaf(wk, __uint_as_float(r.w[i]), acc[i]);
  } else if constexpr (DT == kFP8) {
    // gfx950's FP8 conversions read the OCP E4M3 format; each decodes the two
    // bytes of one 16-bit half of a word, exactly.
#pragma unroll
    for (int q = 0; q < V / 4; ++q) {
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(r.w[q]), false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(r.w[q]), true);
      acc[4 * q] = __builtin_fmaf(wk, lo[0], acc[4 * q]);
      acc[4 * q + 1] = __builtin_fmaf(wk, lo[1], acc[4 * q + 1]);
      acc[4 * q + 2] = __builtin_fmaf(wk, hi[0], acc[4 * q + 2]);
      acc[4 * q + 3] = __builtin_fmaf(wk, hi[1], acc[4 * q + 3]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const uint32_t w = r.w[i >> 1];
      acc[i] = __builtin_fmaf(wk, to_float<DT>((i & 1) ? (w >> 16) : (w & 0xffffu)), acc[i]);
    }
  }
}

template <int DT, int V>
__device__ __forceinline__ void store_row(void* base, int64_t elem, const float* acc) {
  uint8_t* p = static_cast<uint8_t*>(base) + elem * elem_bytes<DT>();
  if constexpr (DT == kF32) {
#pragma unroll
    for (int i = 0; i < V; i += 4) {
      *reinterpret_cast<float4*>(p + i * 4) =
          make_float4(acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
    }
  } else if constexpr (DT == kFP8) {
    uint32_t q[V / 4];
#pragma unroll
    for (int i = 0; i < V; i += 4) {
      q[i / 4] = pk4_fp8e4m3(acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
    }
    if constexpr (V % 16 == 0) {
#pragma unroll
      for (int i = 0; i < V / 16; ++i) {
        u32x4 v;
        v[0] = q[4 * i];
        v[1] = q[4 * i + 1];
        v[2] = q[4 * i + 2];
        v[3] = q[4 * i + 3];
        *reinterpret_cast<u32x4*>(p + 16 * i) = v;
      }
    } else {
      static_assert(V == 8, "FP8 row slices are 8 or 16*n bytes");
      u32x2 v;
      v[0] = q[0];
      v[1] = q[1];
      *reinterpret_cast<u32x2*>(p) = v;
    }
  } else {
#pragma unroll
    for (int i = 0; i < V; i += 8) {
      u32x4 q;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        q[j] = from_float<DT>(acc[i + 2 * j]) | (from_float<DT>(acc[i + 2 * j + 1]) << 16);
      }
      *reinterpret_cast<u32x4*>(p + i * 2) = q;
    }
  }
}

struct ReduceArgs {
  const void* x;
  int64_t rows;
  const int32_t* pos;
  const float* w;
  const float* x_sf;
  const float* sf;
  void* y;
  int K, H, tiles_per_token;
};

template <int IN_DT, int OUT_DT, int V>
__global__ __launch_bounds__(64) void reduce_fused_kernel(ReduceArgs a) {
  const int t = blockIdx.x / a.tiles_per_token;
  const int tile = blockIdx.x - t * a.tiles_per_token;
  const int c = (tile * blockDim.x + threadIdx.x) * V;
  if (c >= a.H) return;
  const int32_t* pt = a.pos + static_cast<int64_t>(t) * a.K;
  const float* wt = a.w ? a.w + static_cast<int64_t>(t) * a.K : nullptr;

  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.0f;

  for (int k0 = 0; k0 < a.K; k0 += kSlots) {
    RowV<IN_DT, V> r[kSlots];
    int32_t p[kSlots];
#pragma unroll
    for (int j = 0; j < kSlots; ++j) {
      p[j] = (k0 + j < a.K) ? pt[k0 + j] : -1;
      if (p[j] >= a.rows) p[j] = -1;   // out-of-range positions are a precondition
                                       // violation; they are skipped, never read
      if (p[j] >= 0) load_row<IN_DT, V>(a.x, static_cast<int64_t>(p[j]) * a.H + c, r[j]);
    }
#pragma unroll
    for (int j = 0; j < kSlots; ++j) {
      if (p[j] >= 0) {
        float wk = wt ? wt[k0 + j] : 1.0f;
        if (a.x_sf) wk = wk * a.x_sf[p[j]];
        fma_row<IN_DT, V>(wk, r[j], acc);
      }
    }
  }
  if (a.sf) {
    const float s = a.sf[t];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = acc[i] * s;
  }
  store_row<OUT_DT, V>(a.y, static_cast<int64_t>(t) * a.H + c, acc);
}

template <int IN_DT, int OUT_DT>
hipError_t launch_typed(ReduceArgs a, int T, hipStream_t stream) {
  // 16 bytes of each row per lane: 8 elements at 16 bits (16 at FP8, 8 as two
  // 16-byte loads at fp32), one-wave workgroups. Measured on the skewed
  // prefill reduce against: 16 elements per lane at 16 bits, 128- and
  // 256-lane workgroups, one wave per (token, tile) in 4-wave workgroups,
  // two or four tokens per workgroup with the next token's loads issued
  // before the current sums, and a persistent grid striding over the items;
  // all were slower.
  constexpr int V = IN_DT == kFP8 ? 16 : 8;
  const int lanes = a.H / V;        // H % 256 == 0: a multiple of 16 lanes
  int threads = 64;
  while (lanes % threads != 0) threads >>= 1;
  a.tiles_per_token = lanes / threads;
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.tiles_per_token) * T));
  hipLaunchKernelGGL((reduce_fused_kernel<IN_DT, OUT_DT, V>), grid, dim3(threads), 0, stream, a);
  return hipGetLastError();
}

template <int IN_DT>
hipError_t launch_out(const ReduceArgs& a, int T, int out_dtype, hipStream_t stream) {
  switch (out_dtype) {
    case kF16: return launch_typed<IN_DT, kF16>(a, T, stream);
    case kBF16: return launch_typed<IN_DT, kBF16>(a, T, stream);
    case kFP8: return launch_typed<IN_DT, kFP8>(a, T, stream);
    default: return launch_typed<IN_DT, kF32>(a, T, stream);
  }
}

}  // namespace

hipError_t launch_reduce(const void* x, int64_t rows, const int32_t* pos, const float* w,
                         const float* x_sf, const float* sf, int T, int K, int H, int in_dtype,
                         int out_dtype, void* y, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  ReduceArgs a{x, rows, pos, w, x_sf, sf, y, K, H, 0};
  switch (in_dtype) {
    case kF16: return launch_out<kF16>(a, T, out_dtype, stream);
    case kBF16: return launch_out<kBF16>(a, T, out_dtype, stream);
    case kFP8: return launch_out<kFP8>(a, T, out_dtype, stream);
    default: return launch_out<kF32>(a, T, out_dtype, stream);
  }
}

}  // namespace moe
