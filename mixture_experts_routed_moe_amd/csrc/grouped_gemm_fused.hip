// Fused expert kernel for decode-sized row blocks (block_m <= 32): gate/up
// and down of one row block in one workgroup, with the block's h kept in LDS
// instead of a round trip through memory ("tilelang baseline" MoE
// walkthrough, devpress.csdn.net, section "stage-2 down", which notes that the
// two stages can be fused so that h is never stored; TileLang tutorial ch.18
// skeletons.py, moe_routed_kernel, for what each stage computes).
//
//   expert_out[i, c] = R( h[i] . Wd[e, c] ),
//   h[i, j]          = R( SiLU(x_t . Wg[e, j]) * (x_t . Wu[e, j]) ),
//   t = sorted_token[i], e the expert of row i, fp32 sums, R = rounding to
//   the 16-bit dtype.
//
// Design (gfx950, 4 waves of 64, one workgroup per active row block):
//   * Phase 1 computes h column tile by column tile (128 h columns: the
//     block's gathered x rows staged through a double-buffered LDS tile,
//     gate and up weights streamed into a register ring, as in
//     grouped_gemm_kernel) with the epilogue writing the rounded h into an
//     LDS matrix of 32 rows x d_expert (rows padded by 16 bytes, so the 32
//     rows of a fragment read fall in different banks).
//   * Phase 2 computes expert_out by column tiles of 256 output columns:
//     each wave streams its 64 W_down rows into the register ring and reads
//     its A fragments straight from the resident h (no staging, no barrier
//     per chunk).
//   * Each phase is one stream of chunks over all its column tiles, the
//     ring running across tile boundaries (see stream_phase); shapes whose
//     chunk count the ring depth does not divide run one pass per tile.
//   * Every dot product is summed in the order of the two-kernel path (the
//     same chunk rotation per (block, column tile), the same MFMA sequence),
//     so expert_out is bit-identical to moe_expert_down(moe_expert_gate_up(x)).
//   A decode layer has one row block per active expert; each workgroup
//   streams its expert's three weight matrices once (88 MB at the DeepSeek
//   shapes), so the work per CU is even when every expert is active.

#include "grouped_gemm.hpp"

namespace moe {
namespace {

constexpr int kFusedMaxD = 2048;               // d_expert the LDS h holds
constexpr int kFusedLdh = kFusedMaxD + 8;      // elements per LDS h row
constexpr int kFusedStages = 8;                // weight-ring depth of both phases

// One pass of the down GEMM for the rows of a block over the resident h:
// S-deep register ring of W_down chunks (the structure of gemm_pass without
// the A staging), then the epilogue into expert_out.
template <int DT, int S>
__device__ __forceinline__ void resident_down_pass(const GemmArgs& g, const uint16_t* h_lds,
                                                   const uint8_t* const* bptr, int nchunks,
                                                   int rot, int lr, int lh, int64_t out_row0,
                                                   int rows, int col0) {
  f32x16 acc[2] = {f32x16{}, f32x16{}};
  BChunk<DT, false> bring[S];
  auto chunk_of = [&](int c) __attribute__((always_inline)) {
    int cc = c + rot;
    if (cc >= nchunks) cc -= nchunks;
    return cc;
  };
  auto load_chunk = [&](int c, int slot) __attribute__((always_inline)) {
    bring[slot].load(bptr, static_cast<int64_t>(chunk_of(c)) * kChunkK);
  };
  // Lane (lr, lh) reads row lr, elements 32 lh + 8 t .. + 7 of each chunk:
  // the A operand that pairs with the weights BChunk holds for the lane.
  const uint16_t* arow = h_lds + lr * kFusedLdh + lh * (kChunkK / 2);
  auto step = [&](int c, auto U, bool prefetch) __attribute__((always_inline)) {
    constexpr int u = decltype(U)::value;
    if (prefetch) load_chunk(c + S - 1, (u + S - 1) % S);
    const uint16_t* a = arow + chunk_of(c) * kChunkK;
#pragma unroll
    for (int t = 0; t < kChunkK / 16; ++t) {
      const u32x4 av = *reinterpret_cast<const u32x4*>(a + t * 8);
      acc[0] = mfma32x32x16<DT>(av, bring[u].operand(0, t), acc[0]);
      acc[1] = mfma32x32x16<DT>(av, bring[u].operand(1, t), acc[1]);
    }
  };
#pragma unroll
  for (int st = 0; st < S - 1; ++st) load_chunk(st, st);
  int c0 = 0;
  for (; c0 + 2 * S - 1 <= nchunks - 1; c0 += S) {
    static_for<S>([&](auto U) { step(c0 + U, U, true); });
  }
  const int rem = nchunks - c0;
  static_for<2 * S>([&](auto U) {
    constexpr int u = decltype(U)::value;
    if (u < rem) step(c0 + u, int_c<u % S>{}, u + S - 1 < rem);
  });

  // Accumulator lane l holds column l % 32 and, in register i, row
  // 8 (i / 4) + 4 (l / 32) + i % 4 of its 32 x 32 tile.
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = (i >> 2) * 8 + lh * 4 + (i & 3);
    if (row < rows) {
      uint16_t* out = g.c + (out_row0 + row) * g.n + col0 + lr;
      out[0] = static_cast<uint16_t>(from_float<DT>(acc[0][i]));
      out[32] = static_cast<uint16_t>(from_float<DT>(acc[1][i]));
    }
  }
}

// The chunk-stream form of a phase: chunk q of the stream is chunk q % nch
// (rotated per tile as in the two-kernel path) of column tile q / nch, and
// the register ring runs across tile boundaries, so the first chunks of
// tile nt+1 are in flight while the last chunks of tile nt are multiplied
// (the per-tile passes restart the pipeline once per tile: one memory
// latency each). nch % S == 0 keeps every ring slot static within a tile;
// past the end the last chunk is loaded again (in bounds, never multiplied),
// so every step issues the same loads.
//
// Loads of the stream in issue order: (tile, chunk) pairs advanced one per
// call, with the tile's rotation and weight-row pointers.
struct StreamCursor {
  int nt, c, rot, count;
};

template <int DT, int S, bool GATEUP>
__device__ __forceinline__ void stream_phase(const GemmArgs& g, uint16_t (*lds_a)[32][kChunkK + 8],
                                             uint16_t* h_lds, int e, int ab, int wave, int lr,
                                             int lh, int m_start, int rows) {
  const int tid = threadIdx.x;
  const int nch = g.kd / kChunkK;
  const int total = g.n_tiles * nch;
  auto rot_of = [&](int nt) __attribute__((always_inline)) {
    return static_cast<int>((static_cast<int64_t>(ab) * g.n_tiles + nt) % nch);
  };
  // Tile 0's weight-row pointers; tile nt's rows lie tile_rows * nt rows on.
  int col00;
  const uint8_t* bptr0[2];
  float scale[2];
  weight_rows<GATEUP, false>(g, e, 0, wave, lr, lh, col00, bptr0, scale);
  const int64_t tile_bytes = static_cast<int64_t>(GATEUP ? 128 : 256) * g.kd * 2;
  // Phase 1's A: this thread stages segment tid % 8 of row tid / 8 of the
  // block's gathered x rows (row 0 past the block's rows: never stored).
  const int a_seg = tid % (kChunkK / 8);
  const int a_row = tid / (kChunkK / 8);
  const uint16_t* asrc = nullptr;
  if constexpr (GATEUP) {
    const int r = a_row < rows ? a_row : 0;
    asrc = g.a + static_cast<int64_t>(g.sorted_token[m_start + r]) * g.kd + a_seg * 8;
  }

  BChunk<DT, false> bring[S];
  u32x4 aring[S];
  StreamCursor ld{0, 0, rot_of(0), 0};
  auto load_next = [&](int slot) __attribute__((always_inline)) {
    int cc = ld.c + ld.rot;
    if (cc >= nch) cc -= nch;
    const int64_t off = static_cast<int64_t>(cc) * kChunkK;
    if constexpr (GATEUP) aring[slot] = load16(asrc + off);
    const uint8_t* p[2] = {bptr0[0] + ld.nt * tile_bytes, bptr0[1] + ld.nt * tile_bytes};
    bring[slot].load(p, off);
    if (++ld.count < total) {
      if (++ld.c == nch) {
        ld.c = 0;
        ++ld.nt;
        ld.rot = rot_of(ld.nt);
      }
    }
  };
  auto stage_a = [&](int slot, int buf) __attribute__((always_inline)) {
    if (a_row < rows) *reinterpret_cast<u32x4*>(&lds_a[buf][a_row][a_seg * 8]) = aring[slot];
  };

#pragma unroll
  for (int st = 0; st < S - 1; ++st) load_next(st);
  if constexpr (GATEUP) {
    stage_a(0, 0);
    __syncthreads();
  }
  const uint16_t* hrow = h_lds + lr * kFusedLdh + lh * (kChunkK / 2);
  for (int nt = 0; nt < g.n_tiles; ++nt) {
    const int rot = rot_of(nt);
    f32x16 acc[2] = {f32x16{}, f32x16{}};
    for (int c0 = 0; c0 < nch; c0 += S) {
      static_for<S>([&](auto U) {
        constexpr int u = decltype(U)::value;
        const int c = c0 + u;
        load_next((u + S - 1) % S);
        int cc = c + rot;
        if (cc >= nch) cc -= nch;
#pragma unroll
        for (int t = 0; t < kChunkK / 16; ++t) {
          u32x4 av;
          if constexpr (GATEUP) {
            av = *reinterpret_cast<const u32x4*>(&lds_a[c & 1][lr][lh * (kChunkK / 2) + t * 8]);
          } else {
            av = *reinterpret_cast<const u32x4*>(hrow + cc * kChunkK + t * 8);
          }
          acc[0] = mfma32x32x16<DT>(av, bring[u].operand(0, t), acc[0]);
          acc[1] = mfma32x32x16<DT>(av, bring[u].operand(1, t), acc[1]);
        }
        if constexpr (GATEUP) {
          // the next chunk of the stream (this tile's or the next tile's
          // first) into the other buffer; every wave has finished reading
          // it (the barrier of the previous step)
          stage_a((u + 1) % S, (c + 1) & 1);
          __syncthreads();
        }
      });
    }
    // Epilogue of tile nt. Accumulator lane l holds column l % 32 and, in
    // register i, row 8 (i / 4) + 4 (l / 32) + i % 4 of its 32 x 32 tile.
    const int col0 = col00 + nt * (GATEUP ? 128 : 256);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = (i >> 2) * 8 + lh * 4 + (i & 3);
      if (row < rows) {
        if constexpr (GATEUP) {
          h_lds[row * kFusedLdh + col0 + lr] =
              static_cast<uint16_t>(from_float<DT>(silu(acc[0][i]) * acc[1][i]));
        } else {
          uint16_t* out = g.c + static_cast<int64_t>(m_start + row) * g.n + col0 + lr;
          out[0] = static_cast<uint16_t>(from_float<DT>(acc[0][i]));
          out[32] = static_cast<uint16_t>(from_float<DT>(acc[1][i]));
        }
      }
    }
  }
}

template <int DT, int S1, int S2>
__global__ __launch_bounds__(kThreads) void fused_expert_kernel(GemmArgs gu, GemmArgs dn) {
  __shared__ __attribute__((aligned(16))) uint16_t lds_a[2][32][kChunkK + 8];
  __shared__ __attribute__((aligned(16))) uint16_t h_lds[32 * kFusedLdh];

  // One workgroup per active row block (XCD-aware: workgroup L runs on XCD
  // L % 8, which takes a contiguous range of the active blocks).
  const int total = gu.active_count[0];
  const int per_xcd = (total + 7) >> 3;
  const int ab = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if ((blockIdx.x >> 3) >= per_xcd || ab >= total) return;
  const int bx = gu.active_blocks[ab];
  const int e = gu.block_expert[bx];
  const int row_in_group = bx * gu.block_m - gu.group_padded_offsets[e];
  const int rows = min(gu.block_m, gu.group_sizes[e] - row_in_group);
  if (rows <= 0) return;
  const int m_start = gu.group_offsets[e] + row_in_group;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 31;
  const int lh = lane >> 5;

  // Phase 1: h of the block into LDS (128 h columns per column tile).
  const int nch1 = gu.kd / kChunkK;
  if (nch1 % S1 == 0) {
    stream_phase<DT, S1, true>(gu, lds_a, h_lds, e, ab, wave, lr, lh, m_start, rows);
  } else {
    // one pass per column tile; this thread stages segment tid % 8 of row
    // tid / 8 (row 0 of the block past its rows: in bounds, never stored)
    const int a_seg = tid % (kChunkK / 8);
    const int a_row = tid / (kChunkK / 8);
    const int r = a_row < rows ? a_row : 0;
    const uint16_t* asrc[1] = {gu.a + static_cast<int64_t>(gu.sorted_token[m_start + r]) * gu.kd +
                               a_seg * 8};
    for (int nt = 0; nt < gu.n_tiles; ++nt) {
      int col0;
      const uint8_t* bptr[2];
      float scale[2];
      weight_rows<true, false>(gu, e, nt, wave, lr, lh, col0, bptr, scale);
      const int rot = static_cast<int>((static_cast<int64_t>(ab) * gu.n_tiles + nt) % nch1);
      gemm_pass<DT, 1, 1, true, S1, false, kChunkK, true>(gu, lds_a, asrc, bptr, scale, nch1, rot,
                                                         a_row, a_seg, lr, lh, 0, rows, col0,
                                                         nullptr, h_lds, kFusedLdh);
    }
  }
  __syncthreads();   // the block's h is complete in LDS

  // Phase 2: expert_out of the block (256 output columns per column tile).
  const int nch2 = dn.kd / kChunkK;
  if (nch2 % S2 == 0) {
    stream_phase<DT, S2, false>(dn, lds_a, h_lds, e, ab, wave, lr, lh, m_start, rows);
  } else {
    for (int nt = 0; nt < dn.n_tiles; ++nt) {
      int col0;
      const uint8_t* bptr[2];
      float scale[2];
      weight_rows<false, false>(dn, e, nt, wave, lr, lh, col0, bptr, scale);
      const int rot = static_cast<int>((static_cast<int64_t>(ab) * dn.n_tiles + nt) % nch2);
      resident_down_pass<DT, S2>(dn, h_lds, bptr, nch2, rot, lr, lh, m_start, rows, col0);
    }
  }
}

GemmArgs fused_args(const GemmProblem& p, const moe_tables& t, int tile_cols) {
  GemmArgs g;
  g.a = static_cast<const uint16_t*>(p.a);
  g.b0 = p.b0;
  g.b1 = p.b1;
  g.s0 = nullptr;
  g.s1 = nullptr;
  g.row_w = nullptr;
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
  g.n_tiles = p.n / tile_cols;
  return g;
}

template <int DT>
hipError_t launch_fused_typed(const GemmProblem& up, const GemmProblem& down, const moe_tables& t,
                              hipStream_t stream) {
  const GemmArgs gu = fused_args(up, t, 128);
  const GemmArgs dn = fused_args(down, t, 256);
  const unsigned grid = static_cast<unsigned>((static_cast<int64_t>(t.num_blocks) + 7) / 8 * 8);
  // Depth 8 in both phases (the LDS h leaves room for one workgroup per CU,
  // so each wave keeps the deeper ring of the two-kernel down GEMM);
  // reductions shorter than that run at depth 2.
  if (gu.kd / kChunkK >= kFusedStages && dn.kd / kChunkK >= kFusedStages) {
    hipLaunchKernelGGL((fused_expert_kernel<DT, kFusedStages, kFusedStages>), dim3(grid),
                       dim3(kThreads), 0, stream, gu, dn);
  } else {
    hipLaunchKernelGGL((fused_expert_kernel<DT, 2, 2>), dim3(grid), dim3(kThreads), 0, stream,
                       gu, dn);
  }
  return hipGetLastError();
}

}  // namespace

int fused_max_d_expert() { return kFusedMaxD; }

hipError_t launch_fused_expert(const GemmProblem& up, const GemmProblem& down,
                               const moe_tables& t, hipStream_t stream) {
  if (up.dtype == kBF16) return launch_fused_typed<kBF16>(up, down, t, stream);
  return launch_fused_typed<kF16>(up, down, t, stream);
}

}  // namespace moe
