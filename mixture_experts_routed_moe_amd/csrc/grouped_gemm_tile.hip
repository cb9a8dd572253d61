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
//     XCD (workgroup L runs on XCD L % 8, and each XCD takes a contiguous
//     range of the order) and read that tile through its L2 once.

#include "grouped_gemm.hpp"

namespace moe {
namespace {

constexpr int kKC = 32;                         // reduction elements per chunk
constexpr int kRowB = kKC * 2;                  // bytes of one row per chunk
constexpr int kTileRows = 256;                  // activation rows per tile
constexpr int kABytes = kTileRows * kRowB;      // A part of one LDS buffer: 16 KB
constexpr int kBufBytes = kABytes + 256 * kRowB;   // + 256 weight rows: 32 KB
constexpr int kNBuf = 3;
// Register-ring depth (chunks of loads in flight per thread, 8 loads each).
constexpr int kRing = 3;
// Row groups of the register-streaming path inside this kernel (the wide
// kernel's 6: a block of up to 192 rows in one pass over the weights);
// blocks with more rows, which that design would stream twice, take the
// LDS-tiled pass.
constexpr int kStreamNa = kWideNaMax;
constexpr int kTileMinRows = 32 * kStreamNa + 1;

// A thread's loads of one chunk: NAL activation rows and 4 weight rows.
template <int NAL>
struct Slot {
  u32x4 a[NAL];
  u32x4 b[4];
};

constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }

// Wait until at most `after` chunks of `per` loads each are outstanding
// (s_waitcnt takes an immediate: one case per possible count).
template <int PER, int MAXAFTER>
__device__ __forceinline__ void wait_chunks(int after) {
  static_for<MAXAFTER + 1>([&](auto I) {
    constexpr int k = decltype(I)::value;
    if (after == k) wait_vmcnt<(k * PER < 63 ? k * PER : 63)>();
  });
}

__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// One pass over the reduction for a block of at most 256 rows. R =
// register-ring depth.
template <int DT, bool GATEUP, int R>
__device__ __forceinline__ void tile_pass(const GemmArgs& g, uint8_t* lds, int e, int nt,
                                          int m_start, int rows, int nchunks, int rot,
                                          const float* wrow) {
  constexpr int NAL = 4;                   // activation rows each thread loads per chunk
  constexpr int NQ = 4;                    // A fragments per wave per k-slice
  constexpr int NB = 4;                    // B fragments per wave per k-slice
  constexpr int L = NAL + 4;               // loads per thread per chunk
  constexpr int NMF = NQ * NB;             // MFMAs per wave per k-slice
  constexpr int U = kNBuf * R / gcd_c(kNBuf, R);   // unroll: buffer and slot indices static
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t kd = g.kd;

  // ---- load sources: thread t loads segment t % 4 of rows t / 4 + 64 i.
  // Activation rows: a 32-bit byte offset per row from the uniform base
  // (gathered token rows of x, or rows of h); weight rows: the tile's rows
  // are equally spaced, so a uniform base per i and one per-lane offset.
  const int seg = tid & 3;
  const int lrow = tid >> 2;
  const char* a_base = reinterpret_cast<const char*>(g.a);
  uint32_t a_off[NAL];
#pragma unroll
  for (int i = 0; i < NAL; ++i) {
    int r = lrow + 64 * i;
    if (r >= rows) r = 0;                  // rows past the block: row 0 (never stored)
    const int64_t src = GATEUP ? g.sorted_token[m_start + r] : static_cast<int64_t>(m_start + r);
    a_off[i] = static_cast<uint32_t>(src * kd * 2 + seg * 16);
  }
  const int64_t row_bytes = kd * 2;
  const char* b_base0;                     // tile weight rows 0..127
  const char* b_base1;                     // tile weight rows 128..255 (gate/up: up)
  if constexpr (GATEUP) {
    const int64_t first = static_cast<int64_t>(e) * g.n + nt * 128;
    b_base0 = reinterpret_cast<const char*>(g.b0) + first * row_bytes;
    b_base1 = reinterpret_cast<const char*>(g.b1) + first * row_bytes;
  } else {
    const int64_t first = static_cast<int64_t>(e) * g.n + nt * 256;
    b_base0 = reinterpret_cast<const char*>(g.b0) + first * row_bytes;
    b_base1 = b_base0 + 128 * row_bytes;
  }
  const uint32_t b_off = static_cast<uint32_t>(lrow * row_bytes + seg * 16);
  // LDS write address of this thread's rows (row t/4 + 64 i at + 4096 i);
  // f of those rows depends on row % 32 = t/4 % 32 only.
  const int w_off = lrow * kRowB + 16 * (seg ^ ((lrow >> 2) & 3));
  // Fragment read offset of this lane for k-slice s (0, 1) of a chunk: row
  // lane % 32 of a 32-row fragment (f depends on it alone), segment
  // 2 s + lane / 32.
  const int fr = lane & 31;
  const int f_sw = (fr >> 2) & 3;
  const int fr_off0 = fr * kRowB + 16 * ((0 + (lane >> 5)) ^ f_sw);
  const int fr_off1 = fr * kRowB + 16 * ((2 + (lane >> 5)) ^ f_sw);
  // Fragment rows of this wave (tile rows, A and B).
  const int rh = wave >> 1, ch = wave & 1;
  const int a_row0 = 128 * rh;
  int b_rows[NB];
  if constexpr (GATEUP) {
    b_rows[0] = 64 * ch;
    b_rows[1] = 64 * ch + 32;
    b_rows[2] = 128 + 64 * ch;
    b_rows[3] = 128 + 64 * ch + 32;
  } else {
#pragma unroll
    for (int j = 0; j < NB; ++j) b_rows[j] = 128 * ch + 32 * j;
  }

  f32x16 acc[NQ][NB];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[q][j] = f32x16{};
  }
  Slot<NAL> ring[R];
  u32x4 fa[2][NQ], fb[2][NB];   // fragments of k-slice 0 / 1

  // Load i (0 .. L-1: the NAL activation rows, then the 4 weight rows) of
  // the chunk at byte offset `off` into ring slot SLOT. Chunks past the end
  // load the last chunk again (in bounds, never multiplied): every step
  // issues the same loads, so the count of outstanding loads is the same on
  // every path and one wait immediate serves every step.
  auto chunk_off = [&](int c) __attribute__((always_inline)) {
    int cc = (c < nchunks ? c : nchunks - 1) + rot;
    if (cc >= nchunks) cc -= nchunks;
    return static_cast<int64_t>(cc) * (kKC * 2);   // bytes
  };
  auto load_one = [&](int64_t off, auto SLOT, auto I) __attribute__((always_inline)) {
    constexpr int s = decltype(SLOT)::value;
    constexpr int i = decltype(I)::value;
    if constexpr (i < NAL) {
      ring[s].a[i] = *reinterpret_cast<const u32x4*>(a_base + off + a_off[i]);
    } else {
      constexpr int ib = i - NAL;          // weight row lrow + 64 ib of the tile
      const char* base = (ib < 2 ? b_base0 : b_base1) + off + (ib & 1) * 64 * row_bytes;
      ring[s].b[ib] = *reinterpret_cast<const u32x4*>(base + b_off);
    }
  };
  auto write_one = [&](auto SLOT, auto BUF, auto I) __attribute__((always_inline)) {
    constexpr int s = decltype(SLOT)::value;
    constexpr int i = decltype(I)::value;
    uint8_t* w = lds + decltype(BUF)::value * kBufBytes + w_off;
    if constexpr (i < NAL) {
      *reinterpret_cast<u32x4*>(w + i * 4096) = ring[s].a[i];
    } else {
      *reinterpret_cast<u32x4*>(w + kABytes + (i - NAL) * 4096) = ring[s].b[i - NAL];
    }
  };
  auto read_frags = [&](auto BUF, auto SL) __attribute__((always_inline)) {
    constexpr int sl = decltype(SL)::value;
    const uint8_t* base = lds + decltype(BUF)::value * kBufBytes + (sl ? fr_off1 : fr_off0);
    // A0 and B0 first: the first MFMA of the slice needs them.
    fa[sl][0] = *reinterpret_cast<const u32x4*>(base + a_row0 * kRowB);
    fb[sl][0] = *reinterpret_cast<const u32x4*>(base + kABytes + b_rows[0] * kRowB);
#pragma unroll
    for (int j = 1; j < NB; ++j) {
      fb[sl][j] = *reinterpret_cast<const u32x4*>(base + kABytes + b_rows[j] * kRowB);
    }
#pragma unroll
    for (int q = 1; q < NQ; ++q) {
      fa[sl][q] = *reinterpret_cast<const u32x4*>(base + (a_row0 + 32 * q) * kRowB);
    }
  };
  constexpr int kWait = (R - 1) * L < 63 ? (R - 1) * L : 63;   // loads of R-1 chunks

  // Prologue: chunks 0 .. R-1 in flight (each pinned in order by a scheduling
  // barrier: the loop's order); chunks 0 and 1 into buffers 0 and 1, each
  // followed by the load that reuses its slot; slice 0 of chunk 0.
  static_for<R>([&](auto S) {
    const int64_t off = chunk_off(decltype(S)::value);
    static_for<L>([&](auto I) { load_one(off, S, I); });
    __builtin_amdgcn_sched_barrier(0);
  });
  static_for<2>([&](auto C) {
    constexpr int c = decltype(C)::value;
    wait_vmcnt<kWait>();
    static_for<L>([&](auto I) { write_one(int_c<c % R>{}, int_c<c>{}, I); });
    __builtin_amdgcn_sched_barrier(0);
    const int64_t off = chunk_off(R + c);
    static_for<L>([&](auto I) { load_one(off, int_c<c % R>{}, I); });
    __builtin_amdgcn_sched_barrier(0);
  });
  wait_lds();
  barrier_no_wait();
  read_frags(int_c<0>{}, int_c<0>{});

  // Step c (u = c % U): slice 0 of chunk c with the writes of chunk c+2
  // (ring slot (c+2) % R) into buffer (c+2) % 3 between its MFMAs, then
  // slice 1 with the loads of chunk c+2+R into that slot. Past the end these
  // move data nobody multiplies into a buffer nobody reads before the kernel
  // ends.
  auto step = [&](int c, auto UU) __attribute__((always_inline)) {
    constexpr int u = decltype(UU)::value;
    constexpr int buf = u % kNBuf;
    constexpr int buf1 = (u + 1) % kNBuf;
    constexpr int buf2 = (u + 2) % kNBuf;
    constexpr int slot2 = (u + 2) % R;
    wait_vmcnt<kWait>();                   // chunk c+2 has arrived
    const int64_t off_next = chunk_off(c + 2 + R);
    read_frags(int_c<buf>{}, int_c<1>{});
    __builtin_amdgcn_sched_barrier(0);
    static_for<NMF>([&](auto M) {
      constexpr int m = decltype(M)::value;
      acc[m / NB][m % NB] = mfma32x32x16<DT>(fa[0][m / NB], fb[0][m % NB], acc[m / NB][m % NB]);
      if constexpr (m < L) write_one(int_c<slot2>{}, int_c<buf2>{}, int_c<m>{});
      __builtin_amdgcn_sched_barrier(0);
    });
    read_frags(int_c<buf1>{}, int_c<0>{});
    __builtin_amdgcn_sched_barrier(0);
    static_for<NMF>([&](auto M) {
      constexpr int m = decltype(M)::value;
      acc[m / NB][m % NB] = mfma32x32x16<DT>(fa[1][m / NB], fb[1][m % NB], acc[m / NB][m % NB]);
      if constexpr (m < L) load_one(off_next, int_c<slot2>{}, int_c<m>{});
      __builtin_amdgcn_sched_barrier(0);
    });
    wait_lds();
    barrier_no_wait();
  };
  int c0 = 0;
  for (; c0 + U <= nchunks; c0 += U) {
    static_for<U>([&](auto UU) { step(c0 + decltype(UU)::value, UU); });
  }
  static_for<U>([&](auto UU) {
    if (c0 + decltype(UU)::value < nchunks) step(c0 + decltype(UU)::value, UU);
  });
  wait_vmcnt<0>();   // the prefetches past the end, before the registers are reused

  // Epilogue. Accumulator lane l holds column l % 32 of its 32 weight rows
  // and, in register i, row 8 (i / 4) + 4 (l / 32) + i % 4 of its 32 rows.
  const int lc = lane & 31;
  const int lh = lane >> 5;
  const bool weighted = !GATEUP && wrow != nullptr;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = a_row0 + 32 * q + 8 * (i >> 2) + 4 * lh + (i & 3);
      if (row >= rows) continue;
      uint16_t* out = g.c + static_cast<int64_t>(m_start + row) * g.n;
      if constexpr (GATEUP) {
        // gate fragment j pairs with up fragment j + NB / 2 (same h columns)
#pragma unroll
        for (int j = 0; j < NB / 2; ++j) {
          const int col = nt * 128 + (b_rows[j] & 127) + lc;
          out[col] = static_cast<uint16_t>(from_float<DT>(silu(acc[q][j][i]) * acc[q][j + NB / 2][i]));
        }
      } else {
        const float w = weighted ? wrow[row] : 1.0f;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int col = nt * 256 + b_rows[j] + lc;
          float v = acc[q][j][i];
          if (weighted) v *= w;
          out[col] = static_cast<uint16_t>(from_float<DT>(v));
        }
      }
    }
  }
}

template <int DT, bool GATEUP>
__global__ __launch_bounds__(kThreads) void grouped_gemm_tile_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kNBuf * kBufBytes];
  __shared__ float wrow_s[GATEUP ? 1 : kTileRows];

  const int total = g.active_count[0] * g.n_tiles;
  const int per_xcd = (total + 7) >> 3;
  const int natural = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if ((blockIdx.x >> 3) >= per_xcd || natural >= total) return;
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
    const int nchunks = g.kd / kKC;
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
  if (g.kd / kChunkK < kStagesWide) {
    // reductions shorter than the register design's pipeline: that design alone
    launch_wide<DT, GATEUP, kWideNaMax, false>(grid, g, stream);
  } else {
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
