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

#include <type_traits>
#include <utility>

#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kChunkK = 64;
constexpr int kLdsRow = kChunkK + 8;   // elements per LDS row (144 bytes)
#ifndef MOE_STAGES_RG1
#define MOE_STAGES_RG1 4
#endif
#ifndef MOE_STAGES_RG1_DOWN
#define MOE_STAGES_RG1_DOWN 2
#endif
#ifndef MOE_STAGES_RG2
#define MOE_STAGES_RG2 4
#endif
// Pipeline depths (chunks in flight), measured on MI355X: blocks of <= 32
// rows stream gate/up best at depth 4 and down (half the bytes per column
// tile, more workgroups) at depth 2.
constexpr int kStagesRG1 = MOE_STAGES_RG1;
constexpr int kStagesRG1Down = MOE_STAGES_RG1_DOWN;
constexpr int kStagesRG2 = MOE_STAGES_RG2;   // 64-row blocks
#ifndef MOE_STAGES_ROWSPLIT
#define MOE_STAGES_ROWSPLIT 4
#endif
constexpr int kStagesRowSplit = MOE_STAGES_ROWSPLIT;

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

// Weight loads: read once per block, so they are streamed past the caches.
__device__ __forceinline__ u32x4 load16_stream(const uint16_t* p) {
#ifdef MOE_NT_B
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#else
  return *reinterpret_cast<const u32x4*>(p);
#endif
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

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

// One pass over the reduction for NA active row groups (NA*32 rows) of the
// block, with a software pipeline of depth S: the A share and the B
// fragments of chunk c+S-1 are loaded while chunk c is multiplied. The loads
// of a chunk are issued A first, then B; since vector loads complete in issue
// order, waiting for the A share of chunk c+1 (to stage it in LDS) never
// waits for B fragments of later chunks, so S-1 chunks of weights stay in
// flight across the per-chunk barrier. The loop body is straight-line (no
// branch touches the accumulators, so they stay in place); the last S
// chunks are a peeled copy without prefetches. S divides the chunk count.
template <int DT, int NA, int RG, bool GATEUP, int S>
__device__ __forceinline__ void gemm_pass(const GemmArgs& g, uint16_t (*lds_a)[32 * RG][kLdsRow],
                                          const uint16_t* const* asrc,
                                          const uint16_t* const* bptr, int nchunks, int rot,
                                          int a_row, int a_seg, int lr, int lh,
                                          int64_t out_row0, int rows_pass, int col0) {
  f32x16 acc[NA][2];
#pragma unroll
  for (int q = 0; q < NA; ++q) {
    acc[q][0] = f32x16{};
    acc[q][1] = f32x16{};
  }
  u32x4 aring[S][NA];
  u32x4 bring[S][2][4];

  auto load_chunk = [&](int c, int slot) {
    int cc = c + rot;
    if (cc >= nchunks) cc -= nchunks;
    const int64_t off = static_cast<int64_t>(cc) * kChunkK;
#pragma unroll
    for (int q = 0; q < NA; ++q) {
      if (a_row + 32 * q < rows_pass) aring[slot][q] = load16(asrc[q] + off);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int t = 0; t < 4; ++t) bring[slot][j][t] = load16_stream(bptr[j] + off + t * 8);
    }
  };
  auto stage_a = [&](int slot, int buf) {
#pragma unroll
    for (int q = 0; q < NA; ++q) {
      if (a_row + 32 * q < rows_pass) *reinterpret_cast<u32x4*>(&lds_a[buf][a_row + 32 * q][a_seg * 8]) = aring[slot][q];
    }
  };

#pragma unroll
  for (int st = 0; st < S - 1; ++st) load_chunk(st, st);
  stage_a(0, 0);
  __syncthreads();

  // One chunk: prefetch chunk c+S-1 (only while it exists: the last group of
  // S chunks is peeled, so nothing past the end is ever loaded), multiply
  // chunk c, stage chunk c+1's A share, barrier.
  auto step = [&](int c, auto U, auto PREFETCH, auto STAGE) {
    constexpr int u = decltype(U)::value;
    if constexpr (decltype(PREFETCH)::value) load_chunk(c + S - 1, (u + S - 1) % S);
    constexpr int buf = u & 1;   // S is even, so c & 1 == u & 1
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int q = 0; q < NA; ++q) {
        const u32x4 a =
            *reinterpret_cast<const u32x4*>(&lds_a[buf][q * 32 + lr][lh * 32 + t * 8]);
        acc[q][0] = mfma32x32x16<DT>(a, bring[u][0][t], acc[q][0]);
        acc[q][1] = mfma32x32x16<DT>(a, bring[u][1][t], acc[q][1]);
      }
    }
    if constexpr (decltype(STAGE)::value) stage_a((u + 1) % S, buf ^ 1);
    __syncthreads();
  };
  int c0 = 0;
  for (; c0 + S < nchunks; c0 += S) {
    static_for<S>([&](auto U) { step(c0 + U, U, std::true_type{}, std::true_type{}); });
  }
  static_for<S>([&](auto U) {
    step(c0 + U, U, std::bool_constant<decltype(U)::value == 0>{},
         std::bool_constant<(decltype(U)::value < S - 1)>{});
  });

  // Epilogue. MFMA 32x32 accumulator layout: lane l holds column l % 32 and,
  // in register i, row 8*(i/4) + 4*(l/32) + i%4 of the 32x32 tile.
#pragma unroll
  for (int q = 0; q < NA; ++q) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = q * 32 + (i >> 2) * 8 + lh * 4 + (i & 3);
      if (row < rows_pass) {
        uint16_t* out = g.c + (out_row0 + row) * g.n + col0 + lr;
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

// RG = row groups of 32 rows per pass (a pass covers 32*RG rows of the
// block); GATEUP selects the gate/up kernel (two weight matrices, gathered A,
// SiLU(gate)*up epilogue) or the down kernel (one matrix, 64 columns per
// wave, contiguous A); S = software-pipeline depth in chunks.
template <int DT, int RG, bool GATEUP, int S>
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
#ifdef MOE_KROT
  const int rot = (natural * 5) % nchunks;   // staggered start of the reduction walk
#else
  const int rot = 0;
#endif
  const int a_seg = tid & 7;    // 16-byte segment of a 128-byte A row chunk
  const int a_row = tid >> 3;   // 0..31

  for (int r0 = 0; r0 < rows; r0 += 32 * RG) {
    const int rows_pass = min(32 * RG, rows - r0);
    const int active = (rows_pass + 31) >> 5;

    // A source row of each of this thread's row slots; slots past the
    // block's rows re-read the pass's first row (in bounds, never stored).
    const uint16_t* asrc[RG];
#pragma unroll
    for (int q = 0; q < RG; ++q) {
      int r = a_row + 32 * q;
      if (r >= rows_pass) r = 0;
      const int64_t src = GATEUP ? g.sorted_token[m_start + r0 + r] : (m_start + r0 + r);
      asrc[q] = g.a + src * kd + a_seg * 8;
    }
    const int64_t out_row0 = m_start + r0;
    if (active == RG) {
      gemm_pass<DT, RG, RG, GATEUP, S>(g, lds_a, asrc, bptr, nchunks, rot, a_row, a_seg, lr, lh,
                                       out_row0, rows_pass, col0);
    } else if constexpr (RG >= 2) {
      if (active == 1) {
        gemm_pass<DT, 1, RG, GATEUP, S>(g, lds_a, asrc, bptr, nchunks, rot, a_row, a_seg, lr, lh,
                                        out_row0, rows_pass, col0);
      } else if constexpr (RG >= 4) {
        if (active == 2) {
          gemm_pass<DT, 2, RG, GATEUP, S>(g, lds_a, asrc, bptr, nchunks, rot, a_row, a_seg, lr, lh,
                                          out_row0, rows_pass, col0);
        } else {
          gemm_pass<DT, 3, RG, GATEUP, S>(g, lds_a, asrc, bptr, nchunks, rot, a_row, a_seg, lr,
                                          lh, out_row0, rows_pass, col0);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Row-split variant for large blocks (prefill-sized groups): NW waves, each
// owning 32 rows of the block (a 128-row block uses 4 waves, a 256-row block
// 8), so one workgroup covers a typical expert's rows and its weights stream
// from HBM once. Each wave loads its own A rows straight into MFMA A-operand
// registers; the workgroup's weight tile (128 weight rows: 64 columns of gate
// and 64 of up, or 128 columns of down) is loaded once per chunk,
// cooperatively, into a double-buffered LDS tile that all waves read. A wave
// holds 4 accumulator tiles (64 registers). Same pipeline as above: chunk
// c+S-1's A rows and weight share are loaded while chunk c is multiplied.
template <int DT, bool GATEUP, int S, int NW, bool HAS_ROWS>
__device__ __forceinline__ void rowsplit_pass(const GemmArgs& g,
                                              uint16_t (*lds_b)[128][kLdsRow],
                                              const uint16_t* a_ptr, const uint16_t* b_ptr,
                                              int nchunks, int b_row, int b_seg, int lr, int lh,
                                              int64_t out_row0, int rows_wave, int col_base) {
  // The 16 KB weight tile of a chunk (128 rows x 128 B) is split over the
  // 64*NW threads: kBVec 16-byte loads per thread.
  constexpr int kBVec = 16 / NW;
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x16{};
  u32x4 aring[S][4];
  u32x4 bring[S][kBVec];

  auto load_chunk = [&](int c, int slot) {
    const int64_t off = static_cast<int64_t>(c) * kChunkK;
    if constexpr (HAS_ROWS) {
#pragma unroll
      for (int t = 0; t < 4; ++t) aring[slot][t] = load16(a_ptr + off + t * 8);
    }
#pragma unroll
    for (int t = 0; t < kBVec; ++t) bring[slot][t] = load16(b_ptr + off + t * 8);
  };
  auto stage_b = [&](int slot, int buf) {
#pragma unroll
    for (int t = 0; t < kBVec; ++t) {
      *reinterpret_cast<u32x4*>(&lds_b[buf][b_row][b_seg * kBVec * 8 + t * 8]) = bring[slot][t];
    }
  };

#pragma unroll
  for (int st = 0; st < S - 1; ++st) load_chunk(st, st);
  stage_b(0, 0);
  __syncthreads();

  auto step = [&](int c, auto U, auto PREFETCH, auto STAGE) {
    constexpr int u = decltype(U)::value;
    if constexpr (decltype(PREFETCH)::value) load_chunk(c + S - 1, (u + S - 1) % S);
    constexpr int buf = u & 1;
    if constexpr (HAS_ROWS) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4 b =
              *reinterpret_cast<const u32x4*>(&lds_b[buf][j * 32 + lr][lh * 32 + t * 8]);
          acc[j] = mfma32x32x16<DT>(aring[u][t], b, acc[j]);
        }
      }
    }
    if constexpr (decltype(STAGE)::value) stage_b((u + 1) % S, buf ^ 1);
    __syncthreads();
  };
  int c0 = 0;
  for (; c0 + S < nchunks; c0 += S) {
    static_for<S>([&](auto U) { step(c0 + U, U, std::true_type{}, std::true_type{}); });
  }
  static_for<S>([&](auto U) {
    step(c0 + U, U, std::bool_constant<decltype(U)::value == 0>{},
         std::bool_constant<(decltype(U)::value < S - 1)>{});
  });

  if constexpr (HAS_ROWS) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = (i >> 2) * 8 + lh * 4 + (i & 3);
      if (row < rows_wave) {
        uint16_t* out = g.c + (out_row0 + row) * g.n + col_base + lr;
        if constexpr (GATEUP) {
          out[0] = static_cast<uint16_t>(from_float<DT>(silu(acc[0][i]) * acc[2][i]));
          out[32] = static_cast<uint16_t>(from_float<DT>(silu(acc[1][i]) * acc[3][i]));
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            out[32 * j] = static_cast<uint16_t>(from_float<DT>(acc[j][i]));
          }
        }
      }
    }
  }
}

template <int DT, bool GATEUP, int S, int NW>
__global__ __launch_bounds__(64 * NW) void grouped_gemm_rowsplit_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t lds_b[2][128][kLdsRow];
  constexpr int kSegs = NW / 2;           // threads per 128-byte weight-row chunk
  constexpr int kBVec = 16 / NW;          // 16-byte loads per thread

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
  const int nchunks = g.kd / kChunkK;

  // This thread's share of the weight tile: row b_row of 128, segment b_seg.
  const int b_row = tid / kSegs;
  const int b_seg = tid % kSegs;
  const int col_base = nt * (GATEUP ? 64 : 128);
  const uint16_t* b_ptr;
  if constexpr (GATEUP) {
    const uint16_t* w = b_row < 64 ? g.b0 : g.b1;
    b_ptr = w + (static_cast<int64_t>(e) * g.n + col_base + (b_row & 63)) * kd +
            b_seg * kBVec * 8;
  } else {
    b_ptr = g.b0 + (static_cast<int64_t>(e) * g.n + col_base + b_row) * kd + b_seg * kBVec * 8;
  }

  for (int r0 = 0; r0 < rows; r0 += 32 * NW) {
    const int rows_wave = min(32, rows - r0 - wave * 32);   // may be <= 0
    int r = wave * 32 + lr;
    if (r >= rows - r0) r = 0;                                // in bounds, never stored
    const int64_t src = GATEUP ? g.sorted_token[m_start + r0 + r] : (m_start + r0 + r);
    const uint16_t* a_ptr = g.a + src * kd + lh * 32;
    const int64_t out_row0 = m_start + r0 + wave * 32;
    if (rows_wave > 0) {
      rowsplit_pass<DT, GATEUP, S, NW, true>(g, lds_b, a_ptr, b_ptr, nchunks, b_row, b_seg, lr,
                                             lh, out_row0, rows_wave, col_base);
    } else {
      rowsplit_pass<DT, GATEUP, S, NW, false>(g, lds_b, a_ptr, b_ptr, nchunks, b_row, b_seg, lr,
                                              lh, out_row0, rows_wave, col_base);
    }
  }
}

template <int DT, bool GATEUP, int NW>
void launch_rowsplit(unsigned grid, const GemmArgs& g, hipStream_t stream) {
  if ((g.kd / kChunkK) % kStagesRowSplit == 0) {
    hipLaunchKernelGGL((grouped_gemm_rowsplit_kernel<DT, GATEUP, kStagesRowSplit, NW>),
                       dim3(grid), dim3(64 * NW), 0, stream, g);
  } else {
    hipLaunchKernelGGL((grouped_gemm_rowsplit_kernel<DT, GATEUP, 2, NW>), dim3(grid),
                       dim3(64 * NW), 0, stream, g);
  }
}

template <int DT, int RG, bool GATEUP, int S>
void launch_rg(unsigned grid, const GemmArgs& g, hipStream_t stream) {
  // The pipeline depth must divide the chunk count (kd / 64, even by the
  // shape rules); fall back to depth 2 when it does not.
  if ((g.kd / kChunkK) % S == 0) {
    hipLaunchKernelGGL((grouped_gemm_kernel<DT, RG, GATEUP, S>), dim3(grid), dim3(kThreads), 0,
                       stream, g);
  } else {
    hipLaunchKernelGGL((grouped_gemm_kernel<DT, RG, GATEUP, 2>), dim3(grid), dim3(kThreads), 0,
                       stream, g);
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
  const bool rowsplit = t.block_m >= 128;
  g.n_tiles = p.n / (rowsplit ? (GATEUP ? 64 : 128) : (GATEUP ? 128 : 256));
  const int64_t total = static_cast<int64_t>(t.num_blocks) * g.n_tiles;
  const unsigned grid = static_cast<unsigned>((total + 7) / 8 * 8);
  if (rowsplit) {
    if (t.block_m == 128) {
      launch_rowsplit<DT, GATEUP, 4>(grid, g, stream);
    } else {
      launch_rowsplit<DT, GATEUP, 8>(grid, g, stream);
    }
    return hipGetLastError();
  }
  if (t.block_m <= 32) {
    launch_rg<DT, 1, GATEUP, GATEUP ? kStagesRG1 : kStagesRG1Down>(grid, g, stream);
  } else {
    launch_rg<DT, 2, GATEUP, kStagesRG2>(grid, g, stream);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up(const GemmProblem& p, const moe_tables& t, hipStream_t stream) {
  if (p.dtype == kF32) return launch_gate_up_f32(p, t, stream);
  if (p.dtype == kBF16) return launch_typed<kBF16, true>(p, t, stream);
  return launch_typed<kF16, true>(p, t, stream);
}

hipError_t launch_down(const GemmProblem& p, const moe_tables& t, hipStream_t stream) {
  if (p.dtype == kF32) return launch_down_f32(p, t, stream);
  if (p.dtype == kBF16) return launch_typed<kBF16, false>(p, t, stream);
  return launch_typed<kF16, false>(p, t, stream);
}

}  // namespace moe
