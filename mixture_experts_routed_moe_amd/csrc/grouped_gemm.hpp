// Grouped expert GEMMs of the routed MoE forward on gfx950 (bf16/fp16 MFMA):
// the kernel templates, shared by grouped_gemm.hip (weights in the
// activation dtype) and grouped_gemm_w8.hip (FP8 E4M3 weights).
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
//     4 waves through a double-buffered LDS tile; every A fragment read from
//     LDS feeds two MFMAs. One barrier per chunk.
//   * Software pipeline: the loads of chunk c+S-1 are issued while chunk c
//     is multiplied (S-1 chunks of weights in flight).
//   * Row groups of 32 rows with no valid row skip their MFMAs, so a block
//     with 16 rows of a 32/64-row tile costs one row group of MFMA work.
//   * Only blocks that hold rows are scheduled (the dispatch's active-block
//     list), and they are mapped XCD-aware: workgroup L runs on XCD L % 8, so
//     the natural tile order (active block major, column tile minor) is dealt
//     out in equal contiguous ranges per XCD. The column tiles of one row
//     block then share the A rows in that XCD's L2.
// Two kernels share this design:
//   * grouped_gemm_kernel, blocks of <= 64 rows (decode-sized groups): up to
//     2 row groups of accumulators, A staged through registers and a padded
//     LDS tile; small enough for two workgroups per CU.
//   * grouped_gemm_wide_kernel, blocks of 128 or 256 rows (prefill-sized
//     groups): up to 6 row groups (192 rows) in one pass over the weights,
//     one workgroup per CU using all 512 registers of each wave, A rows in
//     a swizzled LDS layout. A whole prefill-sized expert group then streams
//     its weights once, where smaller blocks would stream them once per
//     block.

#pragma once

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kChunkK = 64;
constexpr int kLdsRow = kChunkK + 8;   // elements per LDS row (144 bytes)
// Pipeline depths (chunks in flight), measured on MI355X at the DeepSeek
// decode shapes: blocks of <= 32 rows stream gate/up best at depth 6 (2.455
// -> 2.443 ms from depth 4) and down at depth 8 (1.309 -> 1.271 ms from
// depth 2; one workgroup per CU, more weight bytes in flight per wave); FP8
// weights keep depth 4 (the FP8 down measured 0.70 -> 0.74 ms at depth 8).
// 64-row blocks run at depth 4. The wide kernel runs at depth 4 (6 row
// groups of accumulators, the weight ring and the A ring fill the 512
// registers of one wave per SIMD), with FP8 weights too.
constexpr int kStagesRG1 = 6;
constexpr int kStagesRG1Down = 8;
constexpr int kStagesRG1W8 = 4;
constexpr int kStagesRG2 = 4;
constexpr int kStagesWide = 4;
constexpr int kStagesWideW8 = 4;
// Row groups of 32 rows the wide kernel keeps in one pass over the weights
// for 256-row blocks (5 at depth 5 measured 3.58 ms, 6 at depth 4 3.44 ms).
constexpr int kWideNaMax = 6;

struct GemmArgs {
  const uint16_t* a;
  const void* b0;      // weights: 16-bit values, or FP8 E4M3 codes (W8)
  const void* b1;
  const float* s0;     // W8: fp32 scale per row of b0 / b1 (one per output channel)
  const float* s1;
  const float* row_w;  // down: routing weight per output row, or nullptr
  const float* sa;     // W8A8: fp32 scale per activation row (x: by token; h: by row)
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

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}



// One chunk of a wave's weights: for each of its two weight rows, the lane's
// CK/2 reduction elements as loaded -- 16-bit values (CK = 64: 4 x 16 bytes)
// or FP8 E4M3 codes (W8: 2 x 16 bytes at CK = 64, 4 x 16 bytes at CK = 128)
// -- and their MFMA B operand for k-slice t (8 16-bit values, elements
// 8t..8t+7 of the lane's CK/2). FP8 codes are decoded
// to the activation dtype, exactly (every E4M3 value is a bf16 and an fp16
// value), two per v_cvt_scalef32_pk instruction with scale 1.
template <int DT, bool W8, int CK = kChunkK>
struct BChunk {
  // 16-byte loads per row: the lane's CK/2 elements of 1 or 2 bytes.
  static constexpr int kVec = (CK / 2) * (W8 ? 1 : 2) / 16;
  u32x4 v[2][kVec];

  // p: the lane's two row pointers (byte addresses); off: reduction offset.
  __device__ __forceinline__ void load(const uint8_t* const* p, int64_t off) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int i = 0; i < kVec; ++i) {
        v[j][i] = *reinterpret_cast<const u32x4*>(p[j] + off * (W8 ? 1 : 2) + i * 16);
      }
    }
  }

  __device__ __forceinline__ u32x4 operand(int j, int t) const {
    if constexpr (!W8) {
      return v[j][t];
    } else {
      const u32x4 raw = v[j][t >> 1];
      const uint32_t d0 = (t & 1) ? raw.z : raw.x;
      const uint32_t d1 = (t & 1) ? raw.w : raw.y;
      return u32x4{dec2(d0, false), dec2(d0, true), dec2(d1, false), dec2(d1, true)};
    }
  }

 private:
  // Two FP8 codes (bytes 0-1, or 2-3 with hi) -> two 16-bit values.
  static __device__ __forceinline__ uint32_t dec2(uint32_t d, bool hi) {
    if constexpr (DT == kBF16) {
      return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d, 1.0f, true))
                : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d, 1.0f, false));
    } else {
      return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d, 1.0f, true))
                : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d, 1.0f, false));
    }
  }
};



// Eight FP8 E4M3 codes (bytes of w, in order) -> eight 16-bit values of
// dtype DT, exactly (every E4M3 value is a bf16 and an fp16 value).
template <int DT>
__device__ __forceinline__ u32x4 fp8x8_to_16bit(u32x2 w) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t d = w[i >> 1];
    const bool hi = i & 1;
    if constexpr (DT == kBF16) {
      r[i] = hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d, 1.0f, true))
                : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d, 1.0f, false));
    } else {
      r[i] = hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d, 1.0f, true))
                : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d, 1.0f, false));
    }
  }
  return r;
}

// The two weight rows a lane streams and their scales: gate/up -- row col0
// + lane%32 of W_gate and of W_up (col0 = 128*nt + 32*wave); down -- rows
// col0 + lane%32 and col0 + 32 + lane%32 of W_down (col0 = 256*nt +
// 64*wave). The lane starts at reduction element (CK/2)*(lane/32) of each
// row (CK: reduction elements per chunk).
template <bool GATEUP, bool W8, int CK = kChunkK>
__device__ __forceinline__ void weight_rows(const GemmArgs& g, int e, int nt, int wave, int lr,
                                            int lh, int& col0, const uint8_t** bptr,
                                            float* scale) {
  const int64_t kd = g.kd;
  const int64_t eb = W8 ? 1 : 2;   // bytes per weight element
  const int64_t expert_row0 = static_cast<int64_t>(e) * g.n;
  int64_t row[2];
  if constexpr (GATEUP) {
    col0 = nt * 128 + wave * 32;
    row[0] = expert_row0 + col0 + lr;
    row[1] = row[0];
  } else {
    col0 = nt * 256 + wave * 64;
    row[0] = expert_row0 + col0 + lr;
    row[1] = row[0] + 32;
  }
  const uint8_t* b0 = static_cast<const uint8_t*>(g.b0);
  const uint8_t* b1 = static_cast<const uint8_t*>(GATEUP ? g.b1 : g.b0);
  bptr[0] = b0 + (row[0] * kd + lh * (CK / 2)) * eb;
  bptr[1] = b1 + (row[1] * kd + lh * (CK / 2)) * eb;
  if constexpr (W8) {
    scale[0] = g.s0[row[0]];
    scale[1] = (GATEUP ? g.s1 : g.s0)[row[1]];
  } else {
    scale[0] = scale[1] = 1.0f;
  }
}

// One pass over the reduction for NA active row groups (NA*32 rows) of the
// block, with a software pipeline of depth S: the A share and the B
// fragments of chunk c+S-1 are loaded while chunk c is multiplied. The loads
// of a chunk are issued A first, then B; since vector loads complete in issue
// order, waiting for the A share of chunk c+1 (to stage it in LDS) never
// waits for B fragments of later chunks, so S-1 chunks of weights stay in
// flight across the per-chunk barrier. The loop body is straight-line (no
// branch touches the accumulators, so they stay in place); the last chunks
// run as a guarded tail without prefetches past the end. HLDS (gate/up):
// the rounded h values go to h_lds[row * ldh + column] in LDS instead of
// g.c (the fused expert kernel keeps a block's h on chip). A8 (with W8):
// the A rows are FP8 E4M3 codes (asrc holds byte addresses; 8 codes per
// thread and segment), decoded exactly to DT when staged into LDS, and each
// dot product is scaled by its activation row's scale g.sa before the
// weight row's: (sum * s_a) * s_w, the products of two E4M3 values being
// exact in fp32 as on the FP8 MFMA.
template <int DT, int NA, int RG, bool GATEUP, int S, bool W8, int CK, bool HLDS = false,
          bool A8 = false>
__device__ __forceinline__ void gemm_pass(const GemmArgs& g, uint16_t (*lds_a)[32 * RG][CK + 8],
                                          const uint16_t* const* asrc,
                                          const uint8_t* const* bptr, const float* scale,
                                          int nchunks, int rot, int a_row, int a_seg, int lr,
                                          int lh, int64_t out_row0, int rows_pass, int col0,
                                          const float* wrow, uint16_t* h_lds = nullptr,
                                          int ldh = 0) {
  f32x16 acc[NA][2];
#pragma unroll
  for (int q = 0; q < NA; ++q) {
    acc[q][0] = f32x16{};
    acc[q][1] = f32x16{};
  }
  // A rows per pass of the 256 threads over a chunk (one 16-byte segment
  // each): 32 at CK = 64, 16 at CK = 128 (then kSub = 2 rows per thread and
  // row group).
  constexpr int kARows = 256 / (CK / 8);
  constexpr int kSub = 32 / kARows;
  using ARaw = std::conditional_t<A8, u32x2, u32x4>;   // one segment as loaded
  ARaw aring[S][NA][kSub];
  BChunk<DT, W8, CK> bring[S];

  auto load_chunk = [&](int c, int slot) __attribute__((always_inline)) {
    int cc = c + rot;
    if (cc >= nchunks) cc -= nchunks;
    const int64_t off = static_cast<int64_t>(cc) * CK;
#pragma unroll
    for (int q = 0; q < NA; ++q) {
#pragma unroll
      for (int sb = 0; sb < kSub; ++sb) {
        if (a_row + kARows * sb + 32 * q < rows_pass) {
          if constexpr (A8) {
            aring[slot][q][sb] = *reinterpret_cast<const u32x2*>(
                reinterpret_cast<const uint8_t*>(asrc[q * kSub + sb]) + off);
          } else {
            aring[slot][q][sb] = load16(asrc[q * kSub + sb] + off);
          }
        }
      }
    }
    bring[slot].load(bptr, off);
  };
  auto stage_a = [&](int slot, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < NA; ++q) {
#pragma unroll
      for (int sb = 0; sb < kSub; ++sb) {
        const int r = a_row + kARows * sb + 32 * q;
        if (r < rows_pass) {
          u32x4 v;
          if constexpr (A8) {
            v = fp8x8_to_16bit<DT>(aring[slot][q][sb]);
          } else {
            v = aring[slot][q][sb];
          }
          *reinterpret_cast<u32x4*>(&lds_a[buf][r][a_seg * 8]) = v;
        }
      }
    }
  };

#pragma unroll
  for (int st = 0; st < S - 1; ++st) load_chunk(st, st);
  stage_a(0, 0);
  __syncthreads();

  // One chunk: prefetch chunk c+S-1 (only while it exists: nothing past the
  // end is ever loaded), multiply chunk c, stage chunk c+1's A share,
  // barrier. U = c % S (the register slot).
  static_assert(S % 2 == 0, "the LDS buffer of chunk c is c % 2 == slot % 2");
  auto step = [&](int c, auto U, bool prefetch, bool stage) __attribute__((always_inline)) {
    constexpr int u = decltype(U)::value;
    if (prefetch) load_chunk(c + S - 1, (u + S - 1) % S);
    constexpr int buf = u & 1;   // S is even, so c & 1 == u & 1
#pragma unroll
    for (int t = 0; t < CK / 16; ++t) {
#pragma unroll
      for (int q = 0; q < NA; ++q) {
        const u32x4 a =
            *reinterpret_cast<const u32x4*>(&lds_a[buf][q * 32 + lr][lh * (CK / 2) + t * 8]);
        acc[q][0] = mfma32x32x16<DT>(a, bring[u].operand(0, t), acc[q][0]);
        acc[q][1] = mfma32x32x16<DT>(a, bring[u].operand(1, t), acc[q][1]);
      }
    }
    if (stage) stage_a((u + 1) % S, buf ^ 1);
    __syncthreads();
  };
  // Full groups of S steps while every step's prefetch exists, then the last
  // S..2S-1 chunks as a guarded tail (S need not divide the chunk count).
  int c0 = 0;
  for (; c0 + 2 * S - 1 <= nchunks - 1; c0 += S) {
    static_for<S>([&](auto U) { step(c0 + U, U, true, true); });
  }
  const int rem = nchunks - c0;
  static_for<2 * S>([&](auto U) {
    constexpr int u = decltype(U)::value;
    if (u < rem) step(c0 + u, int_c<u % S>{}, u + S - 1 < rem, u + 1 < rem);
  });

  // Epilogue. MFMA 32x32 accumulator layout: lane l holds column l % 32 and,
  // in register i, row 8*(i/4) + 4*(l/32) + i%4 of the 32x32 tile.
  // Down with routing weights: the pass's row weights were staged in LDS
  // (wrow) before the main loop, whose barriers made them visible.
  const bool weighted = !GATEUP && g.row_w != nullptr;
#pragma unroll
  for (int q = 0; q < NA; ++q) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = q * 32 + (i >> 2) * 8 + lh * 4 + (i & 3);
      if (row < rows_pass) {
        uint16_t* out = g.c + (out_row0 + row) * g.n + col0 + lr;
        float v0 = acc[q][0][i], v1 = acc[q][1][i];
        if constexpr (A8) {   // the activation row's scale, then the weight rows'
          const float sa = g.sa[GATEUP ? g.sorted_token[out_row0 + row] : out_row0 + row];
          v0 = v0 * sa * scale[0];
          v1 = v1 * sa * scale[1];
        } else if constexpr (W8) {   // the rows' scales, once per dot product
          v0 *= scale[0];
          v1 *= scale[1];
        }
        if constexpr (GATEUP) {
          const uint16_t hv = static_cast<uint16_t>(from_float<DT>(silu(v0) * v1));
          if constexpr (HLDS) {
            h_lds[row * ldh + col0 + lr] = hv;
          } else {
            out[0] = hv;
          }
        } else {
          if (weighted) {   // the row's routing weight, before the rounding
            const float w = wrow[row];
            v0 *= w;
            v1 *= w;
          }
          out[0] = static_cast<uint16_t>(from_float<DT>(v0));
          out[32] = static_cast<uint16_t>(from_float<DT>(v1));
        }
      }
    }
  }
}

// RG = row groups of 32 rows per pass (a pass covers 32*RG rows of the
// block); GATEUP selects the gate/up kernel (two weight matrices, gathered A,
// SiLU(gate)*up epilogue) or the down kernel (one matrix, 64 columns per
// wave, contiguous A); S = software-pipeline depth in chunks.
template <int DT, int RG, bool GATEUP, int S, bool W8, bool A8 = false>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(GemmArgs g) {
  // Reduction elements per chunk: 64; 128 with FP8 weights, so a lane still
  // loads 64 contiguous bytes of each weight row per chunk (two lanes cover
  // a 128-byte segment) and the A rows of a chunk are 256 bytes.
  constexpr int CK = W8 ? 128 : kChunkK;
  __shared__ __attribute__((aligned(16))) uint16_t lds_a[2][32 * RG][CK + 8];

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

  // Down with routing weights: the block's row weights (block_m <= 64 here),
  // staged in LDS for the epilogue.
  __shared__ float wrow_s[GATEUP ? 1 : 64];
  if (!GATEUP && g.row_w != nullptr && tid < rows) wrow_s[tid] = g.row_w[m_start + tid];

  const int64_t kd = g.kd;
  int col0;
  const uint8_t* bptr[2];
  float scale[2];
  weight_rows<GATEUP, W8, CK>(g, e, nt, wave, lr, lh, col0, bptr, scale);

  const int nchunks = g.kd / CK;
  // Start of the reduction walk (a rotation of the chunk order): 16-bit
  // weights start each workgroup at chunk (its tile index) mod nchunks,
  // so the workgroups streaming at one time touch different columns of
  // their weight rows (rows 4 KB apart otherwise load the same columns
  // together); FP8 weights walk from chunk 0.
  const int rot = W8 ? 0 : static_cast<int>(static_cast<int64_t>(natural) % nchunks);
  constexpr int kASeg = CK / 8;             // 16-byte segments of an A row chunk
  constexpr int kARows = 256 / kASeg;       // A rows per pass of the threads
  constexpr int kSub = 32 / kARows;
  const int a_seg = tid % kASeg;
  const int a_row = tid / kASeg;

  for (int r0 = 0; r0 < rows; r0 += 32 * RG) {
    const int rows_pass = min(32 * RG, rows - r0);
    const int active = (rows_pass + 31) >> 5;

    // A source row of each of this thread's row slots; slots past the
    // block's rows re-read the pass's first row (in bounds, never stored).
    const uint16_t* asrc[RG * kSub];
#pragma unroll
    for (int q = 0; q < RG; ++q) {
#pragma unroll
      for (int sb = 0; sb < kSub; ++sb) {
        int r = a_row + kARows * sb + 32 * q;
        if (r >= rows_pass) r = 0;
        const int64_t src = GATEUP ? g.sorted_token[m_start + r0 + r] : (m_start + r0 + r);
        if constexpr (A8) {   // byte addresses of FP8 codes
          asrc[q * kSub + sb] = reinterpret_cast<const uint16_t*>(
              reinterpret_cast<const uint8_t*>(g.a) + src * kd + a_seg * 8);
        } else {
          asrc[q * kSub + sb] = g.a + src * kd + a_seg * 8;
        }
      }
    }
    const int64_t out_row0 = m_start + r0;
    if (active == RG) {
      gemm_pass<DT, RG, RG, GATEUP, S, W8, CK, false, A8>(g, lds_a, asrc, bptr, scale, nchunks,
                                                          rot, a_row, a_seg, lr, lh, out_row0,
                                                          rows_pass, col0, wrow_s + r0);
    } else if constexpr (RG == 2) {
      gemm_pass<DT, 1, RG, GATEUP, S, W8, CK, false, A8>(g, lds_a, asrc, bptr, scale, nchunks,
                                                         rot, a_row, a_seg, lr, lh, out_row0,
                                                         rows_pass, col0, wrow_s + r0);
    }
  }
}

// ---------------------------------------------------------------------------
// Wide-block kernel for blocks of 128 or 256 rows (prefill-sized groups): the
// layout of grouped_gemm_kernel (4 waves, each owning 32 columns of gate and
// of up, or 64 of down, for ALL rows of the block; weights streamed from HBM
// straight into B-operand registers, so a block reads its expert's weights
// once) with up to NAMAX = 6 row groups of accumulators (192 rows: a whole
// prefill-sized expert group in one pass). Every A fragment read from LDS
// feeds two MFMAs.
//
// A stage holds the pass's rows as 8-row groups of 1 KB (the 16 bytes of
// thread L of a wave: row L/8 of the group, slot L%8). Slot s of row r holds
// segment s ^ f(r), f(r) = (r % 8) ^ ((r / 8) % 2), so the fragment reads of
// 16 consecutive rows at one segment touch 16 different (row parity, slot)
// pairs: distinct banks whether the LDS serves 8 lanes x 16 B or 16 lanes x
// 16 B per clock. Row group q of a chunk (32 rows = 4 groups of 8) is written
// by the 4 waves, one group each.
//
// Pipeline: the loads of chunk c+S-1 (A share and weights, into registers)
// are issued while chunk c is multiplied, so S-1 chunks of weights are in
// flight. Each step waits (vmcnt) for this wave's weights of chunk c, then
// meets the other waves at a plain s_barrier (chunk c's A tile is complete
// in LDS), issues chunk c+S-1 into the register slot that chunk c-1 used,
// multiplies chunk c, and writes chunk c+1's A share into the other LDS
// buffer (which every wave finished reading before the barrier). S need not
// divide the chunk count: full groups of S steps run while every step's
// prefetch exists, and the last S..2S-1 chunks run as a guarded tail.
constexpr int kAGroupElems = 8 * kChunkK;   // one 8-row group of a stage: 1 KB

// Wait until at most `after` chunks of `ops` loads each are outstanding
// (s_waitcnt takes an immediate: one case per possible count).
template <int OPS, int MAXAFTER>
__device__ __forceinline__ void wait_chunks_after(int after) {
  static_for<MAXAFTER + 1>([&](auto I) {
    constexpr int k = decltype(I)::value;
    if (after == k) wait_vmcnt<(k * OPS < 63 ? k * OPS : 63)>();
  });
}

// One pass of the wide kernel over the reduction for NA row groups: the A
// share of chunk c+S-1 is loaded into registers together with its weights (A
// first), and written to a double-buffered LDS tile at the end of step
// c+S-2, one step before it is multiplied. Since vector loads complete in
// issue order, waiting for an A share never waits for the weights issued
// after it, so S-1 chunks of weights stay in flight.
template <int DT, int NA, bool GATEUP, int S, int NAMAX, bool W8>
__device__ __forceinline__ void wide_pass(const GemmArgs& g, uint16_t* lds_ring,
                                          const uint16_t* const* a_src,
                                          const uint8_t* const* bptr, const float* scale,
                                          int nchunks, int rot, int wave, int lane, int lr,
                                          int lh, int64_t out_row0, int rows, int col0,
                                          const float* wrow) {
  constexpr int kStage = NAMAX * 4 * kAGroupElems;
  constexpr int kB = 2 * BChunk<DT, W8>::kVec;   // weight loads per chunk per wave
  constexpr int kOps = NA + kB;                   // vector memory ops per chunk per wave
  f32x16 acc[NA][2];
#pragma unroll
  for (int q = 0; q < NA; ++q) {
    acc[q][0] = f32x16{};
    acc[q][1] = f32x16{};
  }
  BChunk<DT, W8> bring[S];
  u32x4 aring[S][NA];

  auto load_chunk = [&](int c, int slot) __attribute__((always_inline)) {
    int cc = c + rot;
    if (cc >= nchunks) cc -= nchunks;
    const int64_t off = static_cast<int64_t>(cc) * kChunkK;
#pragma unroll
    for (int q = 0; q < NA; ++q) aring[slot][q] = load16(a_src[q] + off);
    bring[slot].load(bptr, off);
  };
  // Write chunk c's A share (ring slot `slot`) into LDS buffer c % 2.
  auto stage_a = [&](int c, int slot) __attribute__((always_inline)) {
    uint16_t* stage = lds_ring + (c & 1) * kStage + wave * kAGroupElems + lane * 8;
#pragma unroll
    for (int q = 0; q < NA; ++q) {
      *reinterpret_cast<u32x4*>(stage + q * 4 * kAGroupElems) = aring[slot][q];
    }
  };

  const int f_row = (lr & 7) ^ ((lr >> 3) & 1);
  const int row_off = (lr >> 3) * kAGroupElems + (lr & 7) * kChunkK;
  // Multiply chunk c: A fragments are read one k-slice ahead, so slice
  // t+1's LDS reads are in flight during slice t's MFMAs.
  auto multiply = [&](int c, auto U) __attribute__((always_inline)) {
    constexpr int u = decltype(U)::value % S;
    const uint16_t* stage = lds_ring + (c & 1) * kStage + row_off;
    u32x4 af[2][NA];
    auto read_a = [&](int t, int b) __attribute__((always_inline)) {
      const int slot = (lh * 4 + t) ^ f_row;
#pragma unroll
      for (int q = 0; q < NA; ++q) {
        af[b][q] = *reinterpret_cast<const u32x4*>(stage + q * 4 * kAGroupElems + slot * 8);
      }
    };
    read_a(0, 0);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t < 3) read_a(t + 1, (t + 1) & 1);
#pragma unroll
      for (int q = 0; q < NA; ++q) {
        acc[q][0] = mfma32x32x16<DT>(af[t & 1][q], bring[u].operand(0, t), acc[q][0]);
        acc[q][1] = mfma32x32x16<DT>(af[t & 1][q], bring[u].operand(1, t), acc[q][1]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Prologue: chunks 0..S-2 in flight; stage chunk 0's A share. The loads
  // keep the loop's order (chunk by chunk, A before B): the compiler's own
  // load counting at the loop head merges this path with the back edge, and
  // a different order here would make it wait for far more than needed.
#pragma unroll
  for (int st = 0; st < S - 1; ++st) {
    load_chunk(st, st);
    __builtin_amdgcn_sched_barrier(0);
  }
  wait_vmcnt<(kB + (S - 2) * kOps < 63 ? kB + (S - 2) * kOps : 63)>();
  stage_a(0, 0);

  // Step c: wait for chunk c's weights, barrier (chunk c's A share is in
  // LDS; every wave is done with buffer (c+1) % 2), prefetch chunk c+S-1,
  // multiply chunk c, then wait for chunk c+1's A share and stage it.
  int c0 = 0;
  for (; c0 + 2 * S - 1 <= nchunks - 1; c0 += S) {
    static_for<S>([&](auto U) {
      constexpr int u = decltype(U)::value;
      wait_vmcnt<(S - 2) * kOps>();
      barrier_no_wait();
      load_chunk(c0 + u + S - 1, (u + S - 1) % S);
      multiply(c0 + u, U);
      wait_vmcnt<(kB + (S - 2) * kOps < 63 ? kB + (S - 2) * kOps : 63)>();
      stage_a(c0 + u + 1, (u + 1) % S);
    });
  }
  // Tail: the last R chunks, S <= R < 2S.
  const int rem = nchunks - c0;
  static_for<2 * S>([&](auto U) {
    constexpr int u = decltype(U)::value;
    if (u < rem) {
      wait_chunks_after<kOps, S - 2>(min(S - 2, rem - 1 - u));
      barrier_no_wait();
      if (u + S - 1 < rem) load_chunk(c0 + u + S - 1, (u + S - 1) % S);
      multiply(c0 + u, U);
      if (u + 1 < rem) {
        // Chunks issued after chunk c+1: up to min(c+S-1, n-1).
        const int after = min(S - 2, rem - 2 - u);
        static_for<S - 1>([&](auto I) {
          constexpr int k = decltype(I)::value;
          if (after == k) wait_vmcnt<(kB + k * kOps < 63 ? kB + k * kOps : 63)>();
        });
        stage_a(c0 + u + 1, (u + 1) % S);
      }
    }
  });

  // Down with routing weights: the pass's row weights were staged in LDS
  // (wrow) before the main loop, whose barriers made them visible.
  const bool weighted = !GATEUP && g.row_w != nullptr;
#pragma unroll
  for (int q = 0; q < NA; ++q) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = q * 32 + (i >> 2) * 8 + lh * 4 + (i & 3);
      if (row < rows) {
        uint16_t* out = g.c + (out_row0 + row) * g.n + col0 + lr;
        float v0 = acc[q][0][i], v1 = acc[q][1][i];
        if constexpr (W8) {   // the rows' scales, once per dot product
          v0 *= scale[0];
          v1 *= scale[1];
        }
        if constexpr (GATEUP) {
          out[0] = static_cast<uint16_t>(from_float<DT>(silu(v0) * v1));
        } else {
          if (weighted) {   // the row's routing weight, before the rounding
            const float w = wrow[row];
            v0 *= w;
            v1 *= w;
          }
          out[0] = static_cast<uint16_t>(from_float<DT>(v0));
          out[32] = static_cast<uint16_t>(from_float<DT>(v1));
        }
      }
    }
  }
}

// One (row block, column tile) of the wide design: the block's rows
// m_start .. m_start + rows - 1 of expert e, column tile nt. lds_ring: the
// double-buffered A stage (2 * NAMAX * 4 * kAGroupElems elements); wrow:
// the block's row weights staged in LDS (down with routing weights; visible
// after the pass's first barrier), or unused.
template <int DT, bool GATEUP, int S, int NAMAX, bool W8>
__device__ __forceinline__ void wide_block(const GemmArgs& g, uint16_t* lds_ring, const float* wrow,
                                           int e, int nt, int m_start, int rows) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const int64_t kd = g.kd;
  const int nchunks = g.kd / kChunkK;
  // Start of the reduction walk, as in grouped_gemm_kernel but by column
  // tile: the row blocks of one expert that share a weight tile still walk
  // it together (and share it in L2), different tiles start apart.
  const int rot = W8 ? 0 : nt % nchunks;

  int col0;
  const uint8_t* bptr[2];
  float scale[2];
  weight_rows<GATEUP, W8>(g, e, nt, wave, lr, lh, col0, bptr, scale);

  // One pass over the weights covers up to NAMAX row groups; a block with
  // more rows (at most 8 groups) takes two balanced passes of up to 4 groups
  // (written out rather than as a loop, so the register allocation of the
  // large pass is not burdened by the loop). Every lambda here is forced
  // inline: an outlined pass (the compiler's choice when the same pass is
  // called three times) goes through a call with its arguments in scratch.
  auto run_pass = [&](int r0, auto NAP) __attribute__((always_inline)) {
    constexpr int kMaxNa = decltype(NAP)::value;
    const int rows_pass = min(32 * kMaxNa, rows - r0);
    // This lane's A source for row group q: row 32q + 8*wave + lane/8 of
    // the pass (row 0 of the pass past its rows: in bounds, never stored),
    // segment (lane % 8) ^ f(row) with f(row) = (lane / 8) ^ (wave % 2).
    const uint16_t* a_src[kMaxNa];
    const int seg = (lane & 7) ^ (lane >> 3) ^ (wave & 1);
#pragma unroll
    for (int q = 0; q < kMaxNa; ++q) {
      int r = 32 * q + 8 * wave + (lane >> 3);
      if (r >= rows_pass) r = 0;
      const int64_t src = GATEUP ? g.sorted_token[m_start + r0 + r] : (m_start + r0 + r);
      a_src[q] = g.a + src * kd + seg * 8;
    }
    const int active = (rows_pass + 31) >> 5;
    static_for<kMaxNa>([&](auto I) {
      constexpr int na = decltype(I)::value + 1;
      if (active == na) {
        wide_pass<DT, na, GATEUP, S, NAMAX, W8>(g, lds_ring, a_src, bptr, scale, nchunks, rot, wave,
                                                lane, lr, lh, m_start + r0, rows_pass, col0,
                                                wrow + r0);
      }
    });
  };
  if (rows <= 32 * NAMAX) {
    run_pass(0, int_c<NAMAX>{});
  } else {
    run_pass(0, int_c<4>{});
    barrier_no_wait();   // every wave is done with the LDS tile
    run_pass(128, int_c<4>{});
  }
}

template <int DT, bool GATEUP, int S, int NAMAX, bool W8>
__global__ __launch_bounds__(kThreads) void grouped_gemm_wide_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) uint16_t lds_ring[2 * NAMAX * 4 * kAGroupElems];

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
  // Down with routing weights: the block's row weights (<= 256 rows),
  // staged in LDS for the epilogue.
  __shared__ float wrow_s[GATEUP ? 1 : kThreads];
  if (!GATEUP && g.row_w != nullptr && static_cast<int>(threadIdx.x) < rows) {
    wrow_s[threadIdx.x] = g.row_w[m_start + threadIdx.x];
  }
  wide_block<DT, GATEUP, S, NAMAX, W8>(g, lds_ring, wrow_s, e, nt, m_start, rows);
}

template <int DT, bool GATEUP, int NAMAX, bool W8>
void launch_wide(unsigned grid, const GemmArgs& g, hipStream_t stream) {
  // Depth S needs at least S chunks; a 128-long reduction (the shortest the
  // shape rules allow: 2 chunks) runs at depth 2.
  constexpr int S = W8 ? kStagesWideW8 : kStagesWide;
  if (g.kd / kChunkK >= S) {
    hipLaunchKernelGGL((grouped_gemm_wide_kernel<DT, GATEUP, S, NAMAX, W8>), dim3(grid),
                       dim3(kThreads), 0, stream, g);
  } else {
    hipLaunchKernelGGL((grouped_gemm_wide_kernel<DT, GATEUP, 2, NAMAX, W8>), dim3(grid),
                       dim3(kThreads), 0, stream, g);
  }
}

template <int DT, int RG, bool GATEUP, int S, bool W8, bool A8 = false>
void launch_rg(unsigned grid, const GemmArgs& g, hipStream_t stream) {
  // Depth S needs at least S chunks (kd / 64, or kd / 128 with FP8 weights;
  // >= 1 by the shape rules); fall back to depth 2 below that (a single
  // chunk runs the tail alone).
  if (g.kd / (W8 ? 128 : kChunkK) >= S) {
    hipLaunchKernelGGL((grouped_gemm_kernel<DT, RG, GATEUP, S, W8, A8>), dim3(grid),
                       dim3(kThreads), 0, stream, g);
  } else {
    hipLaunchKernelGGL((grouped_gemm_kernel<DT, RG, GATEUP, 2, W8, A8>), dim3(grid),
                       dim3(kThreads), 0, stream, g);
  }
}

// Both grouped GEMMs for activation dtype DT (bf16 / fp16) and weights of
// the same dtype or, with W8, FP8 E4M3 codes with per-row scales.
template <int DT, bool GATEUP, bool W8>
hipError_t launch_typed(const GemmProblem& p, const moe_tables& t, hipStream_t stream) {
  GemmArgs g;
  g.a = static_cast<const uint16_t*>(p.a);
  g.b0 = p.b0;
  g.b1 = p.b1;
  g.s0 = p.s0;
  g.s1 = p.s1;
  g.row_w = GATEUP ? nullptr : p.row_w;
  g.sa = nullptr;
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
  // Blocks of <= 64 rows: grouped_gemm_kernel (128 h columns or 256 output
  // columns per workgroup); 128- and 256-row blocks: the wide kernel (same
  // column tiles).
  g.n_tiles = p.n / (GATEUP ? 128 : 256);
  const int64_t total = static_cast<int64_t>(t.num_blocks) * g.n_tiles;
  const unsigned grid = static_cast<unsigned>((total + 7) / 8 * 8);
  if (t.block_m <= 32) {
    // FP8 weights: 128-element chunks of the same bytes per row as the
    // 16-bit chunks, depth 4 for both GEMMs.
    constexpr int S = W8 ? kStagesRG1W8 : (GATEUP ? kStagesRG1 : kStagesRG1Down);
    launch_rg<DT, 1, GATEUP, S, W8>(grid, g, stream);
  } else if (t.block_m == 64) {
    launch_rg<DT, 2, GATEUP, kStagesRG2, W8>(grid, g, stream);
  } else if (t.block_m == 128) {
    launch_wide<DT, GATEUP, 4, W8>(grid, g, stream);
  } else {
    launch_wide<DT, GATEUP, kWideNaMax, W8>(grid, g, stream);
  }
  return hipGetLastError();
}
}  // namespace
}  // namespace moe
