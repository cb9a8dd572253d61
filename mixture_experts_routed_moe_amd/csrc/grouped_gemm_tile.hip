// Grouped expert GEMMs for prefill-sized row blocks (block_m = 128 or 256),
// bf16 / fp16 weights. One workgroup computes one row block x one column
// tile (gate/up: 128 h columns of gate and the same 128 of up; down: 256
// output columns). A block of at most 128 rows -- a typical prefill-sized
// expert group, HBM-bound -- runs the register-streaming design of
// grouped_gemm.hpp (wide_block with up to 4 row groups: weights straight
// into B-operand registers, read once per block). A larger block (the
// upper end of prefill-sized groups, and the hot experts of skewed routing,
// compute-bound) runs the 256 x 256 tile below, with BOTH operands staged
// through LDS so that every fragment read from LDS feeds 4 MFMAs and the
// whole block takes one pass over the weights (the register design would
// take two beyond 192 rows).
//
// What is computed ("tilelang baseline" MoE walkthrough, devpress.csdn.net,
// sections "stage-1 gate+up" and "stage-2 down"; TileLang tutorial ch.18
// skeletons.py, moe_routed_kernel): gate/up h[i, j] = R(SiLU(x_t . Wg[e, j])
// * (x_t . Wu[e, j])), t = sorted_token[i]; down eo[i, c] = R(h[i] . Wd[e, c])
// (times the row's routing weight before the rounding in the weighted form).
// The block's expert and rows come from the dispatch tables as in every
// grouped kernel of this library (m_start = offset[e] + bx*BM - padded[e]).
//
// Design of the tile (gfx950, 4 waves of 64, one workgroup per CU):
//   * The reduction runs in chunks of 32 elements. A chunk of the tile is
//     256 activation rows and 256 weight rows of 64 bytes each (32 KB); every
//     thread loads 16 bytes of 4 + 4 rows per chunk (four threads per 64-byte
//     row piece) into a register ring R chunks deep, and writes them into one
//     of 3 LDS buffers two chunks ahead of the multiply.
//   * LDS rows are 64 bytes (4 segments of 16) with segment s of row r stored
//     in slot s ^ ((r / 4) % 4). Measured on MI355X with a pattern probe
//     (SQ_LDS_BANK_CONFLICT): the fragment reads (lanes 0-31 rows r..r+31 at
//     one segment, lanes 32-63 the next) and the 16-byte writes of a wave
//     (1 KB contiguous) are conflict-free in this layout; unswizzled rows
//     cost 12 conflict cycles per read, and the swizzle ((r / 2) ^ (r / 8)) % 4
//     costs 4.
//   * Fragments: v_mfma_f32_32x32x16; one A fragment = 32 activation rows x
//     16 reduction elements, one B fragment = 32 weight rows. 2 x 2 wave
//     layout: wave (rh, ch) owns activation rows 128 rh .. +127 and 128
//     weight rows (gate/up: gate and up columns 64 ch .. +63 of the tile;
//     down: output columns 128 ch .. +127), i.e. 4 A and 4 B fragments per
//     16 reduction elements feeding 16 MFMAs (256 accumulator registers).
//   * One step per chunk c: wait for the loads of chunk c+2, then the two
//     k-slices of chunk c from LDS buffer c % 3 (slice 1's fragments read
//     while slice 0 multiplies, and slice 0 of chunk c+1 -- already in buffer
//     (c+1) % 3 -- while slice 1 multiplies), with the LDS writes of chunk c+2
//     into buffer (c+2) % 3 and the loads of chunk c+2+R into the ring slot
//     those writes free placed one by one between the MFMAs, so their issue
//     hides in the matrix pipe's work; one barrier per chunk, after which the
//     next chunk's first fragments are already in registers.
//   * Scheduling: only row blocks holding rows run. Within an expert the
//     (block, column tile) pairs are ordered tile-major, so the row blocks of
//     a hot expert that share a weight tile are adjacent, run together on one
//     XCD and read that tile through its L2 once; granules of positions are
//     dealt out to the XCDs in turn and run alternately from both ends of
//     the expert order (tile_order_position), which spreads a hot expert's
//     tiles over every XCD and mixes them with small experts' tiles.

#include "grouped_gemm_tile.hpp"

namespace moe {
namespace {

template <int DT, bool GATEUP>
__global__ __launch_bounds__(kThreads) void grouped_gemm_tile_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kNBuf * kBufBytes];
  __shared__ float wrow_s[GATEUP ? 1 : kTileRows];

  const int total = g.active_count[0] * g.n_tiles;
  const int natural = tile_order_position(blockIdx.x, total, g.n_tiles);
  if (natural >= total) return;
  // Expert-local tile-major order: the expert of position `natural` in the
  // block-major order owns the same range in both orders.
  const int ab0 = natural / g.n_tiles;
  const int bx0 = g.active_blocks[ab0];
  const int e = g.block_expert[bx0];
  const int first_bx = g.group_padded_offsets[e] / g.block_m;
  const int first_ab = ab0 - (bx0 - first_bx);
  const int nblk = (g.group_sizes[e] + g.block_m - 1) / g.block_m;
  const int local = natural - first_ab * g.n_tiles;
  const int nt = local / nblk;
  const int bx = first_bx + (local - nt * nblk);

  const int row_in_group = bx * g.block_m - g.group_padded_offsets[e];
  const int rows = min(g.block_m, g.group_sizes[e] - row_in_group);
  if (rows <= 0) return;
  const int m_start = g.group_offsets[e] + row_in_group;
  if (!GATEUP && g.row_w != nullptr && static_cast<int>(threadIdx.x) < rows) {
    wrow_s[threadIdx.x] = g.row_w[m_start + threadIdx.x];
  }
  const float* wrow = GATEUP ? nullptr : (g.row_w != nullptr ? wrow_s : nullptr);
  if (rows < kTileMinRows) {
    wide_block<DT, GATEUP, kStagesWide, kStreamNa, false>(g, reinterpret_cast<uint16_t*>(lds),
                                                          wrow_s, e, nt, m_start, rows);
  } else {
    const int nchunks = g.kd * 2 / kRowB;
    const int rot = nt % nchunks;   // column tiles start apart; a tile's row blocks walk it together
    tile_pass<DT, GATEUP, kRing>(g, lds, e, nt, m_start, rows, nchunks, rot, wrow);
  }
}

template <int DT, bool GATEUP>
hipError_t launch_tile_typed(const GemmProblem& p, const moe_tables& t, hipStream_t stream) {
  GemmArgs g;
  g.a = static_cast<const uint16_t*>(p.a);
  g.b0 = p.b0;
  g.b1 = p.b1;
  g.s0 = nullptr;
  g.s1 = nullptr;
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
  g.n_tiles = p.n / (GATEUP ? 128 : 256);
  const int64_t total = static_cast<int64_t>(t.num_blocks) * g.n_tiles;
  if (g.kd / kChunkK < kStagesWide) {
    // reductions shorter than the register design's pipeline: that design alone
    const unsigned grid = static_cast<unsigned>((total + 7) / 8 * 8);
    launch_wide<DT, GATEUP, kWideNaMax, false>(grid, g, stream);
  } else {
    const unsigned grid = static_cast<unsigned>(tile_order_grid(total, g.n_tiles));
    hipLaunchKernelGGL((grouped_gemm_tile_kernel<DT, GATEUP>), dim3(grid), dim3(kThreads), 0,
                       stream, g);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up_tile(const GemmProblem& p, const moe_tables& t, hipStream_t stream) {
  if (p.dtype == kBF16) return launch_tile_typed<kBF16, true>(p, t, stream);
  return launch_tile_typed<kF16, true>(p, t, stream);
}

hipError_t launch_down_tile(const GemmProblem& p, const moe_tables& t, hipStream_t stream) {
  if (p.dtype == kBF16) return launch_tile_typed<kBF16, false>(p, t, stream);
  return launch_tile_typed<kF16, false>(p, t, stream);
}

}  // namespace moe
