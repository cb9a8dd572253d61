// Grouped expert GEMMs with FP8 E4M3 activations against FP8 E4M3 weights
// (W8A8: the weight + activation mode of the TileLang tutorial ch.18
// skeletons.py module docstring, both GEMM operands quantised; the scheme,
// E4M3 with one fp32 scale per row of each operand, is this library's
// reading of an open choice):
//   gate/up: g = (xq_t . Wg8[e, j]) * s_x[t] * s_g[e, j],  u likewise,
//            h[i, j] = R(SiLU(g) * u),  t = sorted_token[i];
//   down:    eo[i, c] = R((hq_i . Wd8[e, c]) * s_h[i] * s_d[e, c]),
// each dot product accumulated in fp32 over the exact products of the E4M3
// codes by the FP8 MFMA, R = rounding to the 16-bit output dtype.
//
// Blocks of 128 or 256 rows run the LDS-tiled pass of grouped_gemm_tile.hpp
// with one-byte operands, its tile cut to the 64-row multiple that covers
// the block's rows: 64 reduction elements per chunk (64 bytes per row, the
// 16-bit tile's layout), one v_mfma_scale_f32_32x32x64_f8f6f4 per fragment
// pair, twice the MFMA throughput of the 16-bit path per byte of
// weights (the prefill layer and the hot experts of skewed routing are
// compute-bound at 16 bits). Scheduling as in grouped_gemm_tile.hip: active
// row blocks only, expert-local tile-major order dealt out to the XCDs in
// granules.
// Blocks of at most 64 rows (decode), bound by the weight stream, run the
// FP8-weight register-streaming kernels of grouped_gemm.hpp in their A8
// form: the activation codes are decoded exactly to the 16-bit dtype as they
// are staged, so each product of two E4M3 values is exact in fp32 as on the
// FP8 MFMA (the sums may differ in order only).

#include "grouped_gemm_tile.hpp"

namespace moe {
namespace {

template <int DT, bool GATEUP, int NQMAX = 4>
__global__ __launch_bounds__(kThreads, NQMAX <= 2 ? 2 : 1) void grouped_gemm_w8a8_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kNBuf * tile_buf_bytes<NQMAX>()];
  __shared__ float scale_s[512];   // the tile's activation-row and weight-row scales

  const int total = g.active_count[0] * g.n_tiles;
  const int natural = tile_order_position(blockIdx.x, total, g.n_tiles);
  if (natural >= total) return;
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
  const int nchunks = g.kd / kRowB;      // one-byte elements: 64 per chunk
  const int rot = nt % nchunks;
  // A tile of 64 rows per row group of each wave, as few as the block needs
  // (a 90-row block of a 256-row table computes 128 rows, not 256).
  const int nq = (rows + 63) >> 6;
  static_for<NQMAX>([&](auto I) {
    constexpr int q = decltype(I)::value + 1;
    // (a deeper ring for the smaller tiles, 6 chunks at 64 and 128 rows and
    // 4 at 192, measured no faster: 3.61 against 3.56 ms at T = 4096)
    if (nq == q) {
      tile_pass<DT, GATEUP, NQMAX <= 2 ? 2 : kRing, true, q>(g, lds, e, nt, m_start, rows, nchunks,
                                                             rot, nullptr, scale_s);
    }
  });
}

template <int DT, bool GATEUP>
hipError_t launch_w8a8_typed(const GemmProblem& p, const moe_tables& t, hipStream_t stream) {
  GemmArgs g;
  g.a = static_cast<const uint16_t*>(p.a);   // FP8 codes, addressed in bytes by the pass
  g.b0 = p.b0;
  g.b1 = p.b1;
  g.s0 = p.s0;
  g.s1 = p.s1;
  g.row_w = nullptr;
  g.sa = p.sa;
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
  if (t.block_m <= 64) {
    // Decode-sized blocks are bound by the weight stream: the register-
    // streaming kernels of the FP8-weight path, with the activation codes
    // decoded exactly to DT in the A staging (the same sums of exact
    // products, on the 16-bit MFMA) and both row scales in the epilogue.
    if (t.block_m <= 32) {
      launch_rg<DT, 1, GATEUP, kStagesRG1W8, true, true>(grid, g, stream);
    } else {
      launch_rg<DT, 2, GATEUP, kStagesRG2, true, true>(grid, g, stream);
    }
  } else if (t.block_m == 128) {
    // blocks of <= 128 rows: the tile's instance for NQ <= 2 (72 KB of LDS,
    // a 2-deep ring, 256 registers), two workgroups per CU
    const unsigned tgrid = static_cast<unsigned>(tile_order_grid(total, g.n_tiles));
    hipLaunchKernelGGL((grouped_gemm_w8a8_kernel<DT, GATEUP, 2>), dim3(tgrid), dim3(kThreads), 0,
                       stream, g);
  } else {
    const unsigned tgrid = static_cast<unsigned>(tile_order_grid(total, g.n_tiles));
    hipLaunchKernelGGL((grouped_gemm_w8a8_kernel<DT, GATEUP>), dim3(tgrid), dim3(kThreads), 0,
                       stream, g);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up_w8a8(const GemmProblem& p, const moe_tables& t, hipStream_t stream) {
  if (p.dtype == kBF16) return launch_w8a8_typed<kBF16, true>(p, t, stream);
  return launch_w8a8_typed<kF16, true>(p, t, stream);
}

hipError_t launch_down_w8a8(const GemmProblem& p, const moe_tables& t, hipStream_t stream) {
  if (p.dtype == kBF16) return launch_w8a8_typed<kBF16, false>(p, t, stream);
  return launch_w8a8_typed<kF16, false>(p, t, stream);
}

}  // namespace moe
