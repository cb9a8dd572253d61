// fp32 ("debug build") grouped expert GEMMs of the routed MoE forward.
//
// Same computation as the bf16/fp16 MFMA kernels ("tilelang baseline" MoE
// walkthrough, sections "stage-1 gate+up" and "stage-2 down"), on fp32
// inputs with no intermediate rounding:
//   gate/up: h[i, j]  = SiLU(x_t . Wg[e, j]) * (x_t . Wu[e, j])
//   down:    eo[i, c] = h[i] . Wd[e, c]   (times the row's routing weight
//            when the weighted-epilogue form is asked for)
// A plain vector-ALU kernel, written for checkability rather than speed:
// every output element is one thread's fmaf chain over the reduction in
// ascending order. A workgroup computes a 32-row x 64-column tile of one
// active row block: the A rows (gathered through sorted_token for gate/up)
// and the weight rows of each 32-element chunk are staged in LDS (rows padded
// to 33 floats), thread t owns column t % 64 for 8 rows.

#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kTileRows = 32;
constexpr int kTileCols = 64;
constexpr int kChunk = 32;

struct F32Args {
  const float* a;
  const float* b0;
  const float* b1;
  const float* row_w;   // down: routing weight per output row, or nullptr
  float* c;
  const int32_t* sorted_token;
  const int32_t* group_sizes;
  const int32_t* group_offsets;
  const int32_t* group_padded_offsets;
  const int32_t* block_expert;
  const int32_t* active_blocks;
  const int32_t* active_count;
  int n, kd, block_m, n_tiles;
};


template <bool GATEUP>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(F32Args g) {
  constexpr int NB = GATEUP ? 2 : 1;
  __shared__ float a_s[kTileRows][kChunk + 1];
  __shared__ float b_s[NB][kTileCols][kChunk + 1];

  const int total = g.active_count[0] * g.n_tiles;
  if (static_cast<int>(blockIdx.x) >= total) return;
  const int ab = blockIdx.x / g.n_tiles;
  const int nt = blockIdx.x - ab * g.n_tiles;
  const int bx = g.active_blocks[ab];
  const int e = g.block_expert[bx];
  const int row_in_group = bx * g.block_m - g.group_padded_offsets[e];
  const int rows = min(g.block_m, g.group_sizes[e] - row_in_group);
  if (rows <= 0) return;
  const int m_start = g.group_offsets[e] + row_in_group;

  const int tid = threadIdx.x;
  const int col = tid % kTileCols;
  const int rgrp = tid / kTileCols;            // rows rgrp*8 .. rgrp*8+7 of the tile
  const int col0 = nt * kTileCols;
  const int64_t kd = g.kd;

  for (int r0 = 0; r0 < rows; r0 += kTileRows) {
    const int rows_pass = min(kTileRows, rows - r0);
    float acc[NB][8];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[j][i] = 0.0f;
    }
    for (int k0 = 0; k0 < g.kd; k0 += kChunk) {
      // A tile: 32 rows x 32 floats, 4 per thread.
      {
        const int r = tid / 8;
        const int kk = (tid % 8) * 4;
        float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (r < rows_pass) {
          const int64_t src = GATEUP ? g.sorted_token[m_start + r0 + r] : (m_start + r0 + r);
          v = *reinterpret_cast<const float4*>(g.a + src * kd + k0 + kk);
        }
        a_s[r][kk + 0] = v.x;
        a_s[r][kk + 1] = v.y;
        a_s[r][kk + 2] = v.z;
        a_s[r][kk + 3] = v.w;
      }
      // Weight tiles: 64 rows x 32 floats per matrix, 8 per thread.
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const float* w = j == 0 ? g.b0 : g.b1;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int wr = tid / 4;
          const int kk = (tid % 4) * 8 + h * 4;
          const float4 v = *reinterpret_cast<const float4*>(
              w + (static_cast<int64_t>(e) * g.n + col0 + wr) * kd + k0 + kk);
          b_s[j][wr][kk + 0] = v.x;
          b_s[j][wr][kk + 1] = v.y;
          b_s[j][wr][kk + 2] = v.z;
          b_s[j][wr][kk + 3] = v.w;
        }
      }
      __syncthreads();
      for (int kk = 0; kk < kChunk; ++kk) {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const float b = b_s[j][col][kk];
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[j][i] = __builtin_fmaf(a_s[rgrp * 8 + i][kk], b, acc[j][i]);
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = rgrp * 8 + i;
      if (r < rows_pass) {
        float* out = g.c + static_cast<int64_t>(m_start + r0 + r) * g.n + col0 + col;
        if constexpr (GATEUP) {
          out[0] = silu(acc[0][i]) * acc[1][i];
        } else {
          out[0] = g.row_w ? acc[0][i] * g.row_w[m_start + r0 + r] : acc[0][i];
        }
      }
    }
  }
}

template <bool GATEUP>
hipError_t launch(const GemmProblem& p, const moe_tables& t, hipStream_t stream) {
  F32Args g;
  g.a = static_cast<const float*>(p.a);
  g.b0 = static_cast<const float*>(p.b0);
  g.b1 = static_cast<const float*>(p.b1);
  g.row_w = GATEUP ? nullptr : p.row_w;
  g.c = static_cast<float*>(p.c);
  g.sorted_token = t.sorted_token;
  g.group_sizes = t.group_sizes;
  g.group_offsets = t.group_offsets;
  g.group_padded_offsets = t.group_padded_offsets;
  g.block_expert = t.block_expert;
  g.active_blocks = t.active_blocks;
  g.active_count = t.active_count;
  g.n = p.n;
  g.kd = p.kd;
  g.block_m = t.block_m;
  g.n_tiles = p.n / kTileCols;
  const int64_t grid = static_cast<int64_t>(t.num_blocks) * g.n_tiles;
  hipLaunchKernelGGL((grouped_gemm_f32_kernel<GATEUP>), dim3(static_cast<unsigned>(grid)),
                     dim3(256), 0, stream, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up_f32(const GemmProblem& p, const moe_tables& t, hipStream_t stream) {
  return launch<true>(p, t, stream);
}

hipError_t launch_down_f32(const GemmProblem& p, const moe_tables& t, hipStream_t stream) {
  return launch<false>(p, t, stream);
}

}  // namespace moe
