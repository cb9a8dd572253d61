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
//   * Phase 1 runs the gate/up passes of grouped_gemm_kernel (one per column
//     tile of 128 h columns: the block's gathered x rows staged through a
//     double-buffered LDS tile, gate and up weights streamed into a register
//     ring) with the epilogue writing the rounded h into an LDS matrix of
//     32 rows x d_expert (rows padded by 16 bytes, so the 32 rows of a
//     fragment read fall in different banks).
//   * Phase 2 runs one pass per column tile of 256 output columns: each wave
//     streams its 64 W_down rows into the register ring and reads its A
//     fragments straight from the resident h (no staging, no barrier per
//     chunk).
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

  // Phase 1: h of the block into LDS, one gate/up pass per 128 h columns.
  // This thread stages segment tid % 8 of row tid / 8 (row 0 of the block
  // past its rows: in bounds, never stored).
  const int a_seg = tid % (kChunkK / 8);
  const int a_row = tid / (kChunkK / 8);
  const int r = a_row < rows ? a_row : 0;
  const uint16_t* asrc[1] = {gu.a + static_cast<int64_t>(gu.sorted_token[m_start + r]) * gu.kd +
                             a_seg * 8};
  const int nch1 = gu.kd / kChunkK;
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
  __syncthreads();   // the block's h is complete in LDS

  // Phase 2: expert_out of the block, one pass per 256 output columns.
  const int nch2 = dn.kd / kChunkK;
  for (int nt = 0; nt < dn.n_tiles; ++nt) {
    int col0;
    const uint8_t* bptr[2];
    float scale[2];
    weight_rows<false, false>(dn, e, nt, wave, lr, lh, col0, bptr, scale);
    const int rot = static_cast<int>((static_cast<int64_t>(ab) * dn.n_tiles + nt) % nch2);
    resident_down_pass<DT, S2>(dn, h_lds, bptr, nch2, rot, lr, lh, m_start, rows, col0);
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
  // The pipeline depths of the two-kernel decode path; reductions shorter
  // than a depth run at depth 2.
  if (gu.kd / kChunkK >= kStagesRG1 && dn.kd / kChunkK >= kStagesRG1Down) {
    hipLaunchKernelGGL((fused_expert_kernel<DT, kStagesRG1, kStagesRG1Down>), dim3(grid),
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
