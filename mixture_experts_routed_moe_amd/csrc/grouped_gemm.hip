// Grouped expert GEMMs of the routed MoE forward on gfx950 (bf16/fp16 MFMA).
//
// What is computed ("tilelang baseline" MoE walkthrough, devpress.csdn.net,
// sections "stage-1 gate+up" and "stage-2 down"; TileLang tutorial ch.18
// skeletons.py, moe_routed_kernel):
//   gate/up: h[i, j]  = R( SiLU(x_t . Wg[e, j]) * (x_t . Wu[e, j]) ),
//            t = sorted_token[i], e = the expert of sorted row i;
//   down:    eo[i, c] = R( h[i] . Wd[e, c] )   (no routing weight here).
// Each workgroup takes one row block of the dispatch tables and one tile of
// output columns, finds its expert and rows from the tables exactly as the
// pages' kernels do (m_start = bx*BM - padded[e] + offset[e], rows =
// min(BM, size[e] - (bx*BM - padded[e]))), and exits at once when the block
// holds no rows, where the pages' kernels load and discard.
//
// Tile design for CDNA4 (not a translation of the pages' 128x128x128 tiles):
//   * 256 threads = 4 waves. Each wave owns 32 output columns of BOTH gate
//     and up (gate/up), or 64 columns (down), and ALL rows of the block, so
//     a weight element is fetched from HBM once per block and feeds every
//     row's MFMA: weights never go through LDS and are not shared between
//     waves. The weight stream goes straight from global memory into the
//     B-operand registers of v_mfma_f32_32x32x16_{bf16,f16}.
//   * The reduction is walked in chunks of 64 elements. Inside a chunk the
//     MFMA k-order is permuted so that lane half h (lane / 32) owns the 32
//     consecutive elements [32h, 32h + 32): every lane then loads 64
//     contiguous bytes of one weight row, two lanes cover a 128-byte row
//     segment, and A uses the same permutation (a sum over k does not care
//     about its order as long as A and B agree).
//   * The A rows of the block (token rows of x gathered through
//     sorted_token for gate/up; contiguous h rows for down) are shared by the
//     4 waves through a double-buffered LDS tile (rows padded to 144 B so the
//     MFMA fragment reads of 32 consecutive rows spread over the banks); one
//     barrier per chunk.
//   * Register double buffering: the loads of chunk c+1 are issued before
//     the MFMAs of chunk c.
//   * Row groups of 32 rows with no valid row skip their MFMAs, so a block
//     with 16 rows of a 32/64/128-row tile costs one row group of MFMA work.
//   * Only blocks that hold rows are scheduled (the dispatch's active-block
//     list), and they are mapped XCD-aware: workgroup L runs on XCD L % 8, so
//     the natural tile order (active block major, column tile minor) is dealt
//     out in equal contiguous ranges per XCD. The column tiles of one row block then share
//     the A rows in that XCD's L2, and the blocks of one expert that spill
//     into a second row block run at the same time on the same XCD, so their
//     second read of the expert's weights is served by L2.

#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kChunkK = 64;
constexpr int kLdsRow = kChunkK + 8;   // elements per LDS row (144 bytes)

struct GemmArgs {
  const uint16_t* a;
  const uint16_t* b0;
  const uint16_t* b1;
  uint16_t* c;
  const int32_t* sorted_token;
  const int32_t* group_sizes;
  const int32_t* group_offsets;
  const int32_t* group_padded_offsets;
  const int32_t* block_expert;
  const int32_t* active_blocks;
  const int32_t* active_count;
  int n, kd, block_m, n_tiles;
};

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

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// RG = row groups of 32 rows held in accumulators (one pass covers 32*RG
// rows); GATEUP selects the gate/up kernel (two weight matrices, gathered A,
// SiLU(gate)*up epilogue) or the down kernel (one matrix, 64 columns per
// wave, contiguous A).
template <int DT, int RG, bool GATEUP>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t lds_a[2][32 * RG][kLdsRow];

  // Only blocks that hold rows are scheduled: the grid is sized for every
  // block, and workgroups past the active work exit at once.
  const int total = g.active_count[0] * g.n_tiles;
  const int per_xcd = (total + 7) >> 3;
  const int natural = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if ((blockIdx.x >> 3) >= per_xcd || natural >= total) return;
  const int ab = natural / g.n_tiles;
  const int nt = natural - ab * g.n_tiles;
  const int bx = g.active_blocks[ab];

  const int e = g.block_expert[bx];
  const int row_in_group = bx * g.block_m - g.group_padded_offsets[e];
  const int rows = min(g.block_m, g.group_sizes[e] - row_in_group);
  if (rows <= 0) return;
  const int m_start = g.group_offsets[e] + row_in_group;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 31;
  const int lh = lane >> 5;

  const int64_t kd = g.kd;
  const int64_t expert_row0 = static_cast<int64_t>(e) * g.n;
  int col0;
  const uint16_t* bptr[2];
  if constexpr (GATEUP) {
    col0 = nt * 128 + wave * 32;
    bptr[0] = g.b0 + (expert_row0 + col0 + lr) * kd + lh * 32;
    bptr[1] = g.b1 + (expert_row0 + col0 + lr) * kd + lh * 32;
  } else {
    col0 = nt * 256 + wave * 64;
    bptr[0] = g.b0 + (expert_row0 + col0 + lr) * kd + lh * 32;
    bptr[1] = g.b0 + (expert_row0 + col0 + 32 + lr) * kd + lh * 32;
  }

  const int nchunks = g.kd / kChunkK;
  const int a_seg = tid & 7;    // 16-byte segment of a 128-byte A row chunk
  const int a_row = tid >> 3;   // 0..31

  for (int r0 = 0; r0 < rows; r0 += 32 * RG) {
    const int rows_pass = min(32 * RG, rows - r0);
    const int active = (rows_pass + 31) >> 5;

    const uint16_t* asrc[RG];
#pragma unroll
    for (int q = 0; q < RG; ++q) {
      const int r = a_row + 32 * q;
      if (r < rows_pass) {
        const int64_t src = GATEUP ? g.sorted_token[m_start + r0 + r] : (m_start + r0 + r);
        asrc[q] = g.a + src * kd + a_seg * 8;
      } else {
        asrc[q] = nullptr;
      }
    }

    f32x16 acc[RG][2];
#pragma unroll
    for (int q = 0; q < RG; ++q) {
      acc[q][0] = f32x16{};
      acc[q][1] = f32x16{};
    }
    u32x4 areg[RG];
    u32x4 bcur[2][4];
    u32x4 bnxt[2][4];

#pragma unroll
    for (int q = 0; q < RG; ++q) {
      if (asrc[q]) areg[q] = load16(asrc[q]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int s = 0; s < 4; ++s) bcur[j][s] = load16(bptr[j] + s * 8);
    }
#pragma unroll
    for (int q = 0; q < RG; ++q) {
      if (asrc[q]) *reinterpret_cast<u32x4*>(&lds_a[0][a_row + 32 * q][a_seg * 8]) = areg[q];
    }
    __syncthreads();

    for (int c = 0; c < nchunks; ++c) {
      const int buf = c & 1;
      const bool more = c + 1 < nchunks;
      if (more) {
        const int64_t off = static_cast<int64_t>(c + 1) * kChunkK;
#pragma unroll
        for (int q = 0; q < RG; ++q) {
          if (asrc[q]) areg[q] = load16(asrc[q] + off);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int s = 0; s < 4; ++s) bnxt[j][s] = load16(bptr[j] + off + s * 8);
        }
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int q = 0; q < RG; ++q) {
          if (q < active) {
            const u32x4 a =
                *reinterpret_cast<const u32x4*>(&lds_a[buf][q * 32 + lr][lh * 32 + s * 8]);
            acc[q][0] = mfma32x32x16<DT>(a, bcur[0][s], acc[q][0]);
            acc[q][1] = mfma32x32x16<DT>(a, bcur[1][s], acc[q][1]);
          }
        }
      }
      if (more) {
#pragma unroll
        for (int q = 0; q < RG; ++q) {
          if (asrc[q]) {
            *reinterpret_cast<u32x4*>(&lds_a[buf ^ 1][a_row + 32 * q][a_seg * 8]) = areg[q];
          }
        }
      }
      __syncthreads();
      if (more) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int s = 0; s < 4; ++s) bcur[j][s] = bnxt[j][s];
        }
      }
    }

    // Epilogue. MFMA 32x32 accumulator layout: lane l holds column l % 32 and,
    // in register i, row 8*(i/4) + 4*(l/32) + i%4 of the 32x32 tile.
#pragma unroll
    for (int q = 0; q < RG; ++q) {
      if (q < active) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = q * 32 + (i >> 2) * 8 + lh * 4 + (i & 3);
          if (row < rows_pass) {
            uint16_t* out = g.c + static_cast<int64_t>(m_start + r0 + row) * g.n + col0 + lr;
            if constexpr (GATEUP) {
              const float v = silu(acc[q][0][i]) * acc[q][1][i];
              out[0] = static_cast<uint16_t>(from_float<DT>(v));
            } else {
              out[0] = static_cast<uint16_t>(from_float<DT>(acc[q][0][i]));
              out[32] = static_cast<uint16_t>(from_float<DT>(acc[q][1][i]));
            }
          }
        }
      }
    }
  }
}

template <int DT, bool GATEUP>
hipError_t launch_typed(const GemmProblem& p, const moe_tables& t, hipStream_t stream) {
  GemmArgs g;
  g.a = static_cast<const uint16_t*>(p.a);
  g.b0 = static_cast<const uint16_t*>(p.b0);
  g.b1 = static_cast<const uint16_t*>(p.b1);
  g.c = static_cast<uint16_t*>(p.c);
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
  g.n_tiles = p.n / (GATEUP ? 128 : 256);
  const int64_t total = static_cast<int64_t>(t.num_blocks) * g.n_tiles;
  const unsigned grid = static_cast<unsigned>((total + 7) / 8 * 8);
  if (t.block_m <= 32) {
    hipLaunchKernelGGL((grouped_gemm_kernel<DT, 1, GATEUP>), dim3(grid), dim3(kThreads), 0,
                       stream, g);
  } else if (t.block_m == 64) {
    hipLaunchKernelGGL((grouped_gemm_kernel<DT, 2, GATEUP>), dim3(grid), dim3(kThreads), 0,
                       stream, g);
  } else {
    hipLaunchKernelGGL((grouped_gemm_kernel<DT, 4, GATEUP>), dim3(grid), dim3(kThreads), 0,
                       stream, g);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up(const GemmProblem& p, const moe_tables& t, hipStream_t stream) {
  if (p.dtype == kBF16) return launch_typed<kBF16, true>(p, t, stream);
  return launch_typed<kF16, true>(p, t, stream);
}

hipError_t launch_down(const GemmProblem& p, const moe_tables& t, hipStream_t stream) {
  if (p.dtype == kBF16) return launch_typed<kBF16, false>(p, t, stream);
  return launch_typed<kF16, false>(p, t, stream);
}

}  // namespace moe
