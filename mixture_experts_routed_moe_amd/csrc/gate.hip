// Router gate in front of the routed experts, on gfx950.
//
// What is computed (the routed-MoE workload recipes: router weights Wr [E, H]
// in fp32, fp32 softmax of the logits x . Wr^T, top-k by score with ties to
// the lower expert index, weights = the selected scores, renormalised to sum
// to 1 where the workload says so; the skewed workload adds a per-expert bias
// of 2*log(1/rank) to the logits):
//   logits[t, e] = (sum over h of x[t, h] * Wr[e, h]) + bias[e]
//   ids[t, :]    = the K largest logits, ties to the lower index (the
//                  softmax is strictly increasing, so this ranks by score)
//   w[t, k]      = softmax(logits[t])[ids[t, k]], optionally / sum over k.
//
// Precision contract: every logit is ONE fp32 fused-multiply-add chain over h
// ascending (then one fp32 addition of the bias), so the logits, and the ids
// decided from them, are reproducible bit for bit by any implementation that
// follows the same definition. The softmax sums are reduced in a tree here;
// the weights therefore agree with a sequential sum to rounding.
//
// Two kernels:
//   * gate_logits_kernel: a tile of tokens x experts per workgroup (16 x 32
//     below 1024 tokens: 256 workgroups at T = 512, E = 256; 32 x 64 from
//     1024 tokens). x and Wr are staged through a double-buffered LDS tile
//     in chunks of 64 h (x widened to fp32) with 16-byte loads issued two
//     chunks ahead; each thread keeps the chains of 1 x 2 (or 2 x 4) token x
//     expert pairs, reading 4 consecutive h per LDS access. Plain fp32 vector
//     FMA (not MFMA: the chain order is the contract).
//   * gate_topk_kernel: one wave per token. Each lane holds E/64 logits; K
//     rounds of a wave-wide argmax (butterfly over (value, index)); lane k
//     keeps the k-th selection; the softmax denominator and the
//     renormalisation are wave reductions.

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kGateKC = 64;             // h per LDS chunk
constexpr int kGateRow = kGateKC + 4;   // padded LDS row (16-byte aligned)

// Tile shapes of the logits kernel: TT tokens x TE experts per workgroup of
// 256 threads; thread (i, j) = (tid / 16, tid % 16) keeps the chains of
// tokens i + 16r (r < TT/16) with experts j + 16c (c < TE/16).
//   16 x 32 (1 x 2 chains per thread): small T, enough workgroups to fill
//     the chip (256 at T = 512, E = 256);
//   32 x 64 (2 x 4 chains): large T, half the LDS bytes per FMA.
template <int DT, int TT, int TE>
struct GateTile {
  static constexpr int kRT = TT / 16;
  static constexpr int kRE = TE / 16;
  static constexpr int kXPer = DT == kF32 ? 4 : 8;           // x elements per 16-byte load
  static constexpr int kXVec = TT * kGateKC / kXPer;          // 16-byte x loads per chunk
  static constexpr int kXLoads = (kXVec + 255) / 256;
  static constexpr int kWVec = TE * kGateKC / 4;              // 16-byte router loads per chunk
  static constexpr int kWLoads = kWVec / 256;
  static_assert(kWVec % 256 == 0, "router tile must split evenly over the threads");
  u32x4 xv[kXLoads];
  u32x4 wv[kWLoads];

  // This thread's share of chunk h0 (rows past T or E read as zeros).
  __device__ __forceinline__ void load(const void* x, const float* wr, int t0, int e0, int T,
                                       int E, int H, int h0, int tid) {
#pragma unroll
    for (int v = 0; v < kXLoads; ++v) {
      const int i = tid + 256 * v;
      const int r = i * kXPer / kGateKC, c = i * kXPer % kGateKC;
      const int64_t off = static_cast<int64_t>(t0 + r) * H + h0 + c;
      if (i < kXVec && t0 + r < T) {
        xv[v] = DT == kF32 ? *reinterpret_cast<const u32x4*>(static_cast<const float*>(x) + off)
                           : *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + off);
      } else {
        xv[v] = u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int v = 0; v < kWLoads; ++v) {
      const int i = tid + 256 * v;
      const int r = i * 4 / kGateKC, c = i * 4 % kGateKC;
      wv[v] = e0 + r < E
                  ? *reinterpret_cast<const u32x4*>(wr + static_cast<int64_t>(e0 + r) * H + h0 + c)
                  : u32x4{0, 0, 0, 0};
    }
  }

  // Write the share into an LDS buffer, x widened to fp32.
  __device__ __forceinline__ void store(float (*xs)[kGateRow], float (*ws)[kGateRow],
                                        int tid) const {
#pragma unroll
    for (int v = 0; v < kXLoads; ++v) {
      const int i = tid + 256 * v;
      if (i >= kXVec) continue;
      const int r = i * kXPer / kGateKC, c = i * kXPer % kGateKC;
      if constexpr (DT == kF32) {
        *reinterpret_cast<u32x4*>(&xs[r][c]) = xv[v];
      } else {
        float4 lo, hi;
        lo.x = to_float<DT>(xv[v].x & 0xffffu);
        lo.y = to_float<DT>(xv[v].x >> 16);
        lo.z = to_float<DT>(xv[v].y & 0xffffu);
        lo.w = to_float<DT>(xv[v].y >> 16);
        hi.x = to_float<DT>(xv[v].z & 0xffffu);
        hi.y = to_float<DT>(xv[v].z >> 16);
        hi.z = to_float<DT>(xv[v].w & 0xffffu);
        hi.w = to_float<DT>(xv[v].w >> 16);
        *reinterpret_cast<float4*>(&xs[r][c]) = lo;
        *reinterpret_cast<float4*>(&xs[r][c + 4]) = hi;
      }
    }
#pragma unroll
    for (int v = 0; v < kWLoads; ++v) {
      const int i = tid + 256 * v;
      const int r = i * 4 / kGateKC, c = i * 4 % kGateKC;
      *reinterpret_cast<u32x4*>(&ws[r][c]) = wv[v];
    }
  }
};

// Logits of a TT-token x TE-expert tile. Pipeline: the loads of chunk c+2
// are issued before chunk c is multiplied; chunk c+1 (loaded during step
// c-1) is written to the other LDS buffer after the multiply; one barrier
// per chunk. Every chain runs over h ascending.
template <int DT, int TT, int TE>
__global__ __launch_bounds__(256) void gate_logits_kernel(const void* __restrict__ x,
                                                          const float* __restrict__ wr,
                                                          const float* __restrict__ bias, int T,
                                                          int H, int E,
                                                          float* __restrict__ logits) {
  using Tile = GateTile<DT, TT, TE>;
  constexpr int RT = Tile::kRT, RE = Tile::kRE;
  __shared__ __attribute__((aligned(16))) float xs[2][TT][kGateRow];
  __shared__ __attribute__((aligned(16))) float ws[2][TE][kGateRow];
  const int t0 = blockIdx.y * TT;
  const int e0 = blockIdx.x * TE;
  const int tid = threadIdx.x;
  const int ti = tid >> 4;
  const int ej = tid & 15;
  const int n = H / kGateKC;
  float acc[RT][RE];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
#pragma unroll
    for (int q = 0; q < RE; ++q) acc[r][q] = 0.0f;
  }
  Tile st[2];

  auto slice = [&](int buf, int c) {
    float4 xv[RT], wv[RE];
#pragma unroll
    for (int r = 0; r < RT; ++r) xv[r] = *reinterpret_cast<const float4*>(&xs[buf][ti + 16 * r][c]);
#pragma unroll
    for (int q = 0; q < RE; ++q) wv[q] = *reinterpret_cast<const float4*>(&ws[buf][ej + 16 * q][c]);
    // h ascending within each chain: c, c+1, c+2, c+3.
#pragma unroll
    for (int r = 0; r < RT; ++r) {
#pragma unroll
      for (int q = 0; q < RE; ++q) {
        acc[r][q] = __builtin_fmaf(xv[r].x, wv[q].x, acc[r][q]);
        acc[r][q] = __builtin_fmaf(xv[r].y, wv[q].y, acc[r][q]);
        acc[r][q] = __builtin_fmaf(xv[r].z, wv[q].z, acc[r][q]);
        acc[r][q] = __builtin_fmaf(xv[r].w, wv[q].w, acc[r][q]);
      }
    }
  };
  auto multiply = [&](int buf) {
    if constexpr (RT * RE <= 2) {
#pragma unroll 4
      for (int c = 0; c < kGateKC; c += 4) slice(buf, c);
    } else {
#pragma unroll 2
      for (int c = 0; c < kGateKC; c += 4) slice(buf, c);
    }
  };
  // One step of the pipeline; U = c % 2 (static register slot).
  auto step = [&](int c, auto U) {
    constexpr int u = decltype(U)::value;
    if (c + 2 < n) st[u].load(x, wr, t0, e0, T, E, H, (c + 2) * kGateKC, tid);
    multiply(u);
    if (c + 1 < n) st[u ^ 1].store(xs[u ^ 1], ws[u ^ 1], tid);
    __syncthreads();
  };

  st[0].load(x, wr, t0, e0, T, E, H, 0, tid);
  if (n > 1) st[1].load(x, wr, t0, e0, T, E, H, kGateKC, tid);
  st[0].store(xs[0], ws[0], tid);
  __syncthreads();
  int c = 0;
  for (; c + 1 < n; c += 2) {
    step(c, std::integral_constant<int, 0>{});
    step(c + 1, std::integral_constant<int, 1>{});
  }
  if (c < n) step(c, std::integral_constant<int, 0>{});

#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int t = t0 + ti + 16 * r;
    if (t >= T) continue;
    float* lt = logits + static_cast<int64_t>(t) * E;
#pragma unroll
    for (int q = 0; q < RE; ++q) {
      const int e = e0 + ej + 16 * q;
      if (e < E) lt[e] = bias ? acc[r][q] + bias[e] : acc[r][q];
    }
  }
}

// (value, index) ordering of the selection: larger value first, then lower
// index. Finite logits only (the contract of the call).
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// NPL = logits per lane (E <= 64 * NPL).
template <int NPL>
__global__ __launch_bounds__(256) void gate_topk_kernel(const float* __restrict__ logits, int T,
                                                        int E, int K, int renorm,
                                                        int32_t* __restrict__ ids,
                                                        float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;                  // whole wave exits together
  const float* lt = logits + static_cast<int64_t>(t) * E;
  float v[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < E ? lt[e] : 0.0f;
  }
  uint32_t taken = 0;                  // bit j: v[j] selected (or past E)
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    if (lane + 64 * j >= E) taken |= 1u << j;
  }

  float my_sel = 0.0f;                 // lane k keeps the k-th selected logit
  int my_id = 0;
  float m = 0.0f;
  for (int k = 0; k < K; ++k) {
    float bv = 0.0f;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int e = lane + 64 * j;
      if (!(taken & (1u << j)) && (bi == 0x7fffffff || better(v[j], e, bv, bi))) {
        bv = v[j];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (oi != 0x7fffffff && (bi == 0x7fffffff || better(ov, oi, bv, bi))) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == k) {
      my_sel = bv;
      my_id = bi;
    }
    if (k == 0) m = bv;
  }

  float z = 0.0f;
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    if (lane + 64 * j < E) z += expf(v[j] - m);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off);
  float p = lane < K ? expf(my_sel - m) / z : 0.0f;
  if (renorm) {
    float s = p;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    p = p / s;
  }
  if (lane < K) {
    ids[static_cast<int64_t>(t) * K + lane] = my_id;
    w[static_cast<int64_t>(t) * K + lane] = p;
  }
}

template <int NPL>
void launch_topk(const float* logits, int T, int E, int K, int renorm, int32_t* ids, float* w,
                 hipStream_t stream) {
  hipLaunchKernelGGL(gate_topk_kernel<NPL>, dim3((T + 3) / 4), dim3(256), 0, stream, logits, T,
                     E, K, renorm, ids, w);
}

template <int TT, int TE>
void launch_logits(const void* x, const float* wr, const float* bias, int T, int H, int E,
                   int dtype, float* logits, hipStream_t stream) {
  const dim3 grid((E + TE - 1) / TE, (T + TT - 1) / TT);
  if (dtype == kBF16) {
    hipLaunchKernelGGL((gate_logits_kernel<kBF16, TT, TE>), grid, dim3(256), 0, stream, x, wr,
                       bias, T, H, E, logits);
  } else if (dtype == kF16) {
    hipLaunchKernelGGL((gate_logits_kernel<kF16, TT, TE>), grid, dim3(256), 0, stream, x, wr,
                       bias, T, H, E, logits);
  } else {
    hipLaunchKernelGGL((gate_logits_kernel<kF32, TT, TE>), grid, dim3(256), 0, stream, x, wr,
                       bias, T, H, E, logits);
  }
}

}  // namespace

hipError_t launch_gate(const void* x, const float* wr, const float* bias, int T, int H, int E,
                       int K, int renorm, int dtype, float* logits, int32_t* ids, float* w,
                       hipStream_t stream) {
  if (T >= 1024) {
    launch_logits<32, 64>(x, wr, bias, T, H, E, dtype, logits, stream);
  } else {
    launch_logits<16, 32>(x, wr, bias, T, H, E, dtype, logits, stream);
  }
  const hipError_t e1 = hipGetLastError();
  if (e1 != hipSuccess) return e1;
  if (E <= 64) {
    launch_topk<1>(logits, T, E, K, renorm, ids, w, stream);
  } else if (E <= 128) {
    launch_topk<2>(logits, T, E, K, renorm, ids, w, stream);
  } else if (E <= 256) {
    launch_topk<4>(logits, T, E, K, renorm, ids, w, stream);
  } else if (E <= 512) {
    launch_topk<8>(logits, T, E, K, renorm, ids, w, stream);
  } else {
    launch_topk<16>(logits, T, E, K, renorm, ids, w, stream);
  }
  return hipGetLastError();
}

}  // namespace moe
