// The LDS tile pass of the grouped expert GEMMs: 64 NQ activation rows
// (NQ = 1..4 row groups per wave; 256 rows at NQ = 4) x 256 weight rows
// (shared by grouped_gemm_tile.hip, 16-bit operands at NQ = 4, and
// grouped_gemm_w8a8.hip, FP8 E4M3 operands with NQ cut to the block's rows).
// The design notes are in grouped_gemm_tile.hip; with FP8 operands a chunk
// is 64 reduction elements
// (the same 64 bytes per row), and the two 16-byte fragments a lane reads
// per chunk are together the 32-byte operand of one
// v_mfma_scale_f32_32x32x64_f8f6f4 (lane half h supplies elements
// 16h..16h+15 and 32+16h..32+16h+15 of the 64; unit scales), so a chunk is
// 16 FP8 MFMAs per wave at twice the FLOPs of a 16-bit chunk. The row
// scales of both operands are applied once per dot product in the epilogue:
// (float) sum * s_a * s_w.

#pragma once

#include "grouped_gemm.hpp"

namespace moe {
namespace {

constexpr int kRowB = 64;                       // bytes of one row per chunk
constexpr int kTileRows = 256;                  // activation rows of the largest tile (NQ = 4)
constexpr int kABytes = kTileRows * kRowB;      // A part of its LDS buffer: 16 KB
constexpr int kBufBytes = kABytes + 256 * kRowB;   // + 256 weight rows: 32 KB (LDS sizing)
constexpr int kNBuf = 3;
// Register-ring depth (chunks of loads in flight per thread, 8 loads each).
constexpr int kRing = 3;
// Row groups of the register-streaming path inside this kernel (the wide
// kernel's 6: a block of up to 192 rows in one pass over the weights);
// blocks with more rows, which that design would stream twice, take the
// LDS-tiled pass.
constexpr int kStreamNa = kWideNaMax;
constexpr int kTileMinRows = 32 * kStreamNa + 1;

// Placement of the (row block, column tile) positions on the XCDs:
// workgroup L runs on XCD L % 8; the positions are cut into granules of G
// (the column-tile count, so a one-block expert's column tiles are one
// granule and share the block's activation rows in one L2), granule i
// belongs to XCD i % 8, and each XCD runs its granules alternately from the
// front and the back of the expert order (first, last, second, second-last,
// ...). In the expert-local tile-major order a hot expert's positions --
// column tile by column tile, each tile's row blocks together -- are thus
// dealt out over every XCD (contiguous per-XCD ranges put a 16-block
// expert's 256 compute-bound tiles on one or two XCDs), and on each XCD its
// compute-bound granules run beside the memory-bound ones of small experts.
// Returns `total` for workgroups past the XCD's granules.
__device__ __forceinline__ int tile_order_position(int L, int total, int G) {
  const int x = L & 7;
  const int j = L >> 3;
  const int k = j / G;
  const int r = j - k * G;
  const int ng = (total + G - 1) / G;
  const int ngx = (ng - x + 7) >> 3;          // granules x, x + 8, ... below ng
  if (k >= ngx) return total;
  const int idx = (k & 1) ? ngx - 1 - (k >> 1) : (k >> 1);
  return (x + 8 * idx) * G + r;
}

// Workgroups that reach every position of any launch with at most
// `positions` positions.
inline int64_t tile_order_grid(int64_t positions, int G) {
  const int64_t granules = (positions + G - 1) / G;
  return (granules + 7) / 8 * 8 * G;
}

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


// FP8 E4M3 operands x FP8 E4M3 operands, fp32 accumulation: the scaled
// MFMA with unit (E8M0 127 = 2^0) scales on both sides.
__device__ __forceinline__ f32x16 mfma_fp8(u32x4 a_lo, u32x4 a_hi, u32x4 b_lo, u32x4 b_hi,
                                           f32x16 c) {
  typedef int i32x8 __attribute__((ext_vector_type(8)));
  const i32x8 a = __builtin_bit_cast(i32x8, (uint32_t __attribute__((ext_vector_type(8)))){
      a_lo.x, a_lo.y, a_lo.z, a_lo.w, a_hi.x, a_hi.y, a_hi.z, a_hi.w});
  const i32x8 b = __builtin_bit_cast(i32x8, (uint32_t __attribute__((ext_vector_type(8)))){
      b_lo.x, b_lo.y, b_lo.z, b_lo.w, b_hi.x, b_hi.y, b_hi.z, b_hi.w});
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// LDS bytes of one buffer of the tile with NQ row groups per wave: 64 NQ
// activation rows and 256 weight rows of 64 bytes.
template <int NQ>
constexpr int tile_buf_bytes() { return (64 * NQ + 256) * kRowB; }

// One pass over the reduction for a block of at most 64 NQ rows (NQ = A
// fragments per wave per k-slice: the 2 x 2 wave layout gives each wave
// 32 NQ activation rows; a smaller NQ skips the MFMAs of row groups a block
// does not have). R = register-ring depth. FP8: operands of one byte
// (activations with a scale per row in g.sa, weights with a scale per row
// in g.s0 / g.s1).
// FP8: scale_s is an LDS array of 512 floats for the tile's row scales.
template <int DT, bool GATEUP, int R, bool FP8 = false, int NQ = 4>
__device__ __forceinline__ void tile_pass(const GemmArgs& g, uint8_t* lds, int e, int nt,
                                          int m_start, int rows, int nchunks, int rot,
                                          const float* wrow, float* scale_s = nullptr) {
  static_assert(NQ >= 1 && NQ <= 4, "row groups per wave");
  constexpr int EB = FP8 ? 1 : 2;          // bytes per operand element
  constexpr int NAL = NQ;                  // activation rows each thread loads per chunk
  constexpr int ABytes = 64 * NQ * kRowB;  // A part of one LDS buffer
  constexpr int BufBytes = tile_buf_bytes<NQ>();
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
    a_off[i] = static_cast<uint32_t>(src * kd * EB + seg * 16);
  }
  const int64_t row_bytes = kd * EB;
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
  const int a_row0 = 32 * NQ * rh;
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
    return static_cast<int64_t>(cc) * kRowB;   // bytes
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
    uint8_t* w = lds + decltype(BUF)::value * BufBytes + w_off;
    if constexpr (i < NAL) {
      *reinterpret_cast<u32x4*>(w + i * 4096) = ring[s].a[i];
    } else {
      *reinterpret_cast<u32x4*>(w + ABytes + (i - NAL) * 4096) = ring[s].b[i - NAL];
    }
  };
  auto read_frags = [&](auto BUF, auto SL) __attribute__((always_inline)) {
    constexpr int sl = decltype(SL)::value;
    const uint8_t* base = lds + decltype(BUF)::value * BufBytes + (sl ? fr_off1 : fr_off0);
    // A0 and B0 first: the first MFMA of the slice needs them.
    fa[sl][0] = *reinterpret_cast<const u32x4*>(base + a_row0 * kRowB);
    fb[sl][0] = *reinterpret_cast<const u32x4*>(base + ABytes + b_rows[0] * kRowB);
#pragma unroll
    for (int j = 1; j < NB; ++j) {
      fb[sl][j] = *reinterpret_cast<const u32x4*>(base + ABytes + b_rows[j] * kRowB);
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
  // FP8: this thread's share of the tile's row scales -- activation row tid
  // (< 64 NQ) and weight row tid -- loaded beside the first chunks and kept
  // in registers until the epilogue (gate/up: the scale of row tid's token,
  // its sorted_token read first, the dependent load after the chunk loads).
  float sa_v = 0.0f, sw_v = 0.0f;
  int tok = 0;
  if constexpr (FP8) {
    if constexpr (GATEUP) {
      if (tid < 64 * NQ && tid < rows) tok = g.sorted_token[m_start + tid];
      const float* sw = (tid < 128 ? g.s0 : g.s1) + static_cast<int64_t>(e) * g.n + nt * 128;
      sw_v = sw[tid & 127];
    } else {
      if (tid < 64 * NQ && tid < rows) sa_v = g.sa[m_start + tid];
      sw_v = g.s0[static_cast<int64_t>(e) * g.n + nt * 256 + tid];
    }
  }
  static_for<R>([&](auto S) {
    const int64_t off = chunk_off(decltype(S)::value);
    static_for<L>([&](auto I) { load_one(off, S, I); });
    __builtin_amdgcn_sched_barrier(0);
  });
  if constexpr (FP8 && GATEUP) {
    if (tid < 64 * NQ && tid < rows) sa_v = g.sa[tok];
  }
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
    if constexpr (FP8) {
      // one 32x32x64 MFMA per (q, j) over both fragment halves; the writes
      // of chunk c+2 after the first L, the loads after the next L
      static_for<NMF>([&](auto M) {
        constexpr int m = decltype(M)::value;
        constexpr int q = m / NB, j = m % NB;
        acc[q][j] = mfma_fp8(fa[0][q], fa[1][q], fb[0][j], fb[1][j], acc[q][j]);
        if constexpr (m < L) write_one(int_c<slot2>{}, int_c<buf2>{}, int_c<m>{});
        if constexpr (m >= L && m < 2 * L) load_one(off_next, int_c<slot2>{}, int_c<m - L>{});
        __builtin_amdgcn_sched_barrier(0);
      });
      static_for<(2 * L > NMF ? 2 * L - NMF : 0)>([&](auto M) {
        constexpr int op = NMF + decltype(M)::value;
        if constexpr (op < L) write_one(int_c<slot2>{}, int_c<buf2>{}, int_c<op>{});
        else load_one(off_next, int_c<slot2>{}, int_c<op - L>{});
      });
      __builtin_amdgcn_sched_barrier(0);
      read_frags(int_c<buf1>{}, int_c<0>{});
    } else {
      static_for<NMF>([&](auto M) {
        constexpr int m = decltype(M)::value;
        acc[m / NB][m % NB] = mfma32x32x16<DT>(fa[0][m / NB], fb[0][m % NB], acc[m / NB][m % NB]);
        if constexpr (m < L) write_one(int_c<slot2>{}, int_c<buf2>{}, int_c<m>{});
        __builtin_amdgcn_sched_barrier(0);
      });
      static_for<(L > NMF ? L - NMF : 0)>([&](auto M) {   // writes beyond the slice's MFMAs
        write_one(int_c<slot2>{}, int_c<buf2>{}, int_c<NMF + decltype(M)::value>{});
      });
      read_frags(int_c<buf1>{}, int_c<0>{});
      __builtin_amdgcn_sched_barrier(0);
      static_for<NMF>([&](auto M) {
        constexpr int m = decltype(M)::value;
        acc[m / NB][m % NB] = mfma32x32x16<DT>(fa[1][m / NB], fb[1][m % NB], acc[m / NB][m % NB]);
        if constexpr (m < L) load_one(off_next, int_c<slot2>{}, int_c<m>{});
        __builtin_amdgcn_sched_barrier(0);
      });
      static_for<(L > NMF ? L - NMF : 0)>([&](auto M) {   // loads beyond the slice's MFMAs
        load_one(off_next, int_c<slot2>{}, int_c<NMF + decltype(M)::value>{});
      });
    }
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
  if constexpr (FP8) {
    // Stored from the accumulators, that is one 2-byte store per value (64
    // or 128 per row group and lane), each after a scale load; measured: a
    // third of the T = 4096 down GEMM's time. Instead the tile's row scales
    // go to LDS, and each wave rounds its sub-tile (32 NQ rows x kCols
    // contiguous output columns) into a private LDS region, up to 2 row
    // groups at a time, and stores whole 16-byte row pieces (16 lanes per
    // 256 bytes of a row). The tile buffers are free: every wave passed the
    // main loop's last barrier after its last fragment read. Each dot
    // product times its activation row's scale, then its weight row's, left
    // to right in fp32.
    constexpr int kCols = GATEUP ? 64 : 128;     // output columns of a wave
    constexpr int kStride = kCols + 8;           // rows 4 apart fall 16 banks apart
    constexpr int kPassQ = NQ < 2 ? NQ : 2;      // row groups per pass
    constexpr int kPieces = kPassQ * 32 * (kCols / 8) / 64;   // 16-byte pieces per lane and pass
    // (callers allocate at least kNBuf buffers of this tile size)
    static_assert(4 * kPassQ * 32 * kStride * 2 <= kNBuf * BufBytes, "epilogue regions fit the LDS");
    const int col_base = GATEUP ? nt * 128 + 64 * ch : nt * 256 + 128 * ch;
    if (tid < 64 * NQ) scale_s[tid] = sa_v;
    scale_s[256 + tid] = sw_v;
    wait_lds();
    barrier_no_wait();   // every thread's scales are visible
    float s_w[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) s_w[j] = scale_s[256 + b_rows[j] + lc];
    uint16_t* region = reinterpret_cast<uint16_t*>(lds) + wave * (kPassQ * 32 * kStride);
    const bool c16 = (reinterpret_cast<uintptr_t>(g.c) & 15) == 0;
    static_for<(NQ + kPassQ - 1) / kPassQ>([&](auto PP) {
      constexpr int q0 = decltype(PP)::value * kPassQ;
      constexpr int nq = NQ - q0 < kPassQ ? NQ - q0 : kPassQ;
#pragma unroll
      for (int qq = 0; qq < nq; ++qq) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int rl = 32 * qq + 8 * (i >> 2) + 4 * lh + (i & 3);
          const int row = a_row0 + 32 * q0 + rl;
          if (row >= rows) continue;
          const float s_a = scale_s[row];
          uint16_t* dst = region + rl * kStride + lc;
          if constexpr (GATEUP) {
            // gate fragment jj pairs with up fragment jj + NB / 2 (same h columns)
#pragma unroll
            for (int jj = 0; jj < NB / 2; ++jj) {
              const float gv = acc[q0 + qq][jj][i] * s_a * s_w[jj];
              const float uv = acc[q0 + qq][jj + NB / 2][i] * s_a * s_w[jj + NB / 2];
              dst[32 * jj] = static_cast<uint16_t>(from_float<DT>(silu(gv) * uv));
            }
          } else {
#pragma unroll
            for (int jj = 0; jj < NB; ++jj) {
              dst[32 * jj] =
                  static_cast<uint16_t>(from_float<DT>(acc[q0 + qq][jj][i] * s_a * s_w[jj]));
            }
          }
        }
      }
      wait_lds();   // this wave's values are in its region
#pragma unroll
      for (int p = 0; p < kPieces; ++p) {
        const int idx = p * 64 + lane;
        const int rl = idx / (kCols / 8);
        const int cc = idx - rl * (kCols / 8);
        const int row = a_row0 + 32 * q0 + rl;
        if (rl < 32 * nq && row < rows) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(region + rl * kStride + cc * 8);
          uint16_t* out = g.c + static_cast<int64_t>(m_start + row) * g.n + col_base + cc * 8;
          if (c16) {
            *reinterpret_cast<u32x4*>(out) = v;
          } else {   // output not 16-byte aligned: the same values, 2 bytes at a time
#pragma unroll
            for (int k = 0; k < 8; ++k) out[k] = static_cast<uint16_t>(v[k >> 1] >> (16 * (k & 1)));
          }
        }
      }
      wait_lds();   // the reads are done before the next pass rewrites the region
    });
  } else {
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
}

}  // namespace
}  // namespace moe
