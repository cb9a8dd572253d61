// Block-scaled (MX) experts: MXFP4 weights against MXFP8 activations on
// v_mfma_scale_f32_32x32x64_f8f6f4 (TileLang tutorial ch.18, module
// docstring: the block-scaled mode, gemm_blockscaled with per-block scale
// factors for both operands; the formats as the OCP Microscaling
// specification v1.0 defines them).
//
// Formats. Along a row every block of 32 values shares one E8M0 scale
// X = 2^(e - 127); elements are FP8 E4M3 (activations) or FP4 E2M1 (weights,
// packed two per byte, element 2i in bits 0..3). Quantisation of a block:
// e = floor(log2 amax) - emax_elem + 127 (emax_elem 8 for E4M3, 2 for E2M1;
// clamped to [0, 254]; 127 for an all-zero block), element = the grid value
// nearest to v / X (ties to the even code, saturating).
//
// GEMM. v_mfma_scale_f32_32x32x64_f8f6f4 takes 32 rows x 64 reduction
// elements per operand and one E8M0 scale per lane; the two lane halves
// hold the scales of the instruction's two 32-element reduction blocks, so
// the scales apply inside the instruction and nothing is decoded. Operand
// layouts (measured: exact-arithmetic inputs with random per-block scales
// on both sides reproduce the exact sums only with this arrangement): an
// FP4 operand's lane half h holds elements 32h..32h+31 (16 bytes); an FP8
// operand's lane half h holds elements 16h..16h+15 in its first 16 bytes
// and 32+16h..32+16h+15 in its last 16 bytes. The reduction runs in
// 256-element chunks in which lane half h of a weight lane owns elements
// 128h..128h+127 of its rows (64 contiguous bytes of packed FP4 per row, as
// in the W4A8 kernel); k-slice t (0..3) pairs weight blocks t and 4 + t of
// the chunk, whose scales are byte t of each lane half's 4-byte scale word,
// with the activation bytes 32t + 16h and 128 + 32t + 16h (16 each) of the
// LDS row. Activations (FP8, 256 bytes per row per chunk) go through a
// double-buffered LDS tile; their scales and the weights come straight from
// memory into a register ring.

#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kCK = 256;                 // reduction elements per chunk
constexpr int kLdsRow = kCK + 16;        // bytes per LDS row of FP8 activations
constexpr int kBlk = 32;                 // MX block
// Weight chunks in the register ring (depth 4 measured slower at decode,
// two workgroups per CU) and row groups per pass for 128/256-row blocks.
constexpr int kStages = 2;
constexpr int kWideNa = 2;

// A = FP8 E4M3 (format code 0), B = FP4 E2M1 (format code 4); byte T of each
// scale word is the E8M0 scale of the lane half's reduction block. The FP4
// operand uses the first 4 dwords of its 8-dword register tuple.
template <int T>
__device__ __forceinline__ f32x16 mfma_mx(const u32x4& a_lo, const u32x4& a_hi, const u32x4& b,
                                          uint32_t sa, uint32_t sb, f32x16 c) {
  const i32x8 a = __builtin_bit_cast(i32x8, (uint32_t __attribute__((ext_vector_type(8)))){
      a_lo.x, a_lo.y, a_lo.z, a_lo.w, a_hi.x, a_hi.y, a_hi.z, a_hi.w});
  const i32x8 bb = __builtin_bit_cast(i32x8, (uint32_t __attribute__((ext_vector_type(8)))){
      b.x, b.y, b.z, b.w, 0u, 0u, 0u, 0u});
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bb, c, 0, 4, T, static_cast<int>(sa), T,
                                                          static_cast<int>(sb));
}



// A lane's share of one chunk: its two weight rows (64 bytes of FP4 each)
// with their 4-byte scale words, and for each of its NA activation rows the
// activation scale word (the activation codes go through LDS).
template <int NA>
struct MxChunk {
  u32x4 w[2][4];
  uint32_t sw[2];
  uint32_t sa[NA];
};

// Scale words of two consecutive chunks, loaded together (PAIR form): for
// each weight row and activation row the 16 bytes [h0, h1] of chunk c and
// [h0, h1] of chunk c + 1.
template <int NA>
struct MxScalePair {
  u32x4 sw[2];
  u32x4 sa[NA];
};

struct MxGroupedArgs {
  const uint8_t* a;         // gate/up: xq [T, kd] E4M3; down: hq [P, kd]
  const uint8_t* as;        // their E8M0 scales [rows, kd/32]
  const uint8_t* b0;        // packed E2M1 weights [E, n, kd/2]
  const uint8_t* b1;        // gate/up: W_up; down: unused
  const uint8_t* s0;        // E8M0 scales of b0 [E, n, kd/32]
  const uint8_t* s1;
  uint16_t* c;              // gate/up: h [P, n]; down: expert_out [P, n]
  const int32_t* sorted_token;
  const int32_t* group_sizes;
  const int32_t* group_offsets;
  const int32_t* group_padded_offsets;
  const int32_t* block_expert;
  const int32_t* active_blocks;
  const int32_t* active_count;
  int n, kd, block_m, n_tiles;
};


// One pass over the reduction for NA groups of 32 activation rows (LDS tile
// of 32 * NAS rows). asrc[2q + sb]: this thread's staging row of group q
// (row 32q + a_row + 16 sb); ascale[q]: the lane's activation row 32q + lr,
// at its lane-half's scale bytes; bptr / bscale: the lane's two weight rows.
//
// PAIR (reduction length a multiple of 512 and no rotation of the chunk
// walk): the scale words are loaded once per two chunks, 16 bytes per row
// at every even chunk (scale rows are then 16-byte aligned and hold an even
// number of chunks); the even chunk reads its lane half's word h, the odd
// chunk the word 2 + h, copied to its ring slot before the next even load
// overwrites the pair.
template <int NA, int NAS, bool PAIR = false>
__device__ __forceinline__ void mx_pass(const uint8_t* const* asrc, const uint8_t* const* ascale,
                                        int a_row, int a_seg, const uint8_t* const* bptr,
                                        const uint8_t* const* bscale, int nch, int rot, int rows_pass,
                                        int lr, int lh, uint8_t (*lds)[32 * NAS][kLdsRow],
                                        f32x16* acc) {
  constexpr int S = kStages;
  static_assert(!PAIR || S == 2, "paired scale loads assume a 2-deep ring (even chunks in slot 0)");
#pragma unroll
  for (int q = 0; q < 2 * NA; ++q) acc[q] = f32x16{};
  u32x4 aring[S][2 * NA];
  MxChunk<NA> ring[S];
  MxScalePair<NA> pair;

  auto load_chunk = [&](int ci, int slot) __attribute__((always_inline)) {
    int c = ci + rot;                       // chunks are walked from `rot` on
    if (c >= nch) c -= nch;
    // Unconditional: the staging rows past the pass's rows read row 0 (in
    // bounds) and fill LDS rows whose results are never stored; a branch
    // here would split the step and let the compiler move the MFMAs.
#pragma unroll
    for (int q = 0; q < 2 * NA; ++q) {
      aring[slot][q] = *reinterpret_cast<const u32x4*>(asrc[q] + static_cast<int64_t>(c) * kCK);
    }
    if constexpr (PAIR) {
      if ((c & 1) == 0) {   // this chunk's and the next one's scale words
#pragma unroll
        for (int q = 0; q < NA; ++q) {
          pair.sa[q] = *reinterpret_cast<const u32x4*>(ascale[q] - lh * 4 + c * (kCK / kBlk));
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < NA; ++q) {
        ring[slot].sa[q] = *reinterpret_cast<const uint32_t*>(ascale[q] + c * (kCK / kBlk));
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ring[slot].w[j][i] = *reinterpret_cast<const u32x4*>(bptr[j] + static_cast<int64_t>(c) * (kCK / 2) + i * 16);
      }
      if constexpr (PAIR) {
        if ((c & 1) == 0) {
          pair.sw[j] = *reinterpret_cast<const u32x4*>(bscale[j] - lh * 4 + c * (kCK / kBlk));
        }
      } else {
        ring[slot].sw[j] = *reinterpret_cast<const uint32_t*>(bscale[j] + c * (kCK / kBlk));
      }
    }
  };
  // PAIR: the even chunk (slot 0) takes word h of the pair and hands word
  // 2 + h to the odd chunk's slot.
  auto take_pair = [&](auto U) __attribute__((always_inline)) {
    if constexpr (PAIR && decltype(U)::value == 0) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        ring[0].sw[j] = lh ? pair.sw[j].y : pair.sw[j].x;
        ring[1].sw[j] = lh ? pair.sw[j].w : pair.sw[j].z;
      }
#pragma unroll
      for (int q = 0; q < NA; ++q) {
        ring[0].sa[q] = lh ? pair.sa[q].y : pair.sa[q].x;
        ring[1].sa[q] = lh ? pair.sa[q].w : pair.sa[q].z;
      }
    }
  };
  auto stage_a = [&](int slot, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 2 * NA; ++q) {
      *reinterpret_cast<u32x4*>(&lds[buf][a_row + 16 * q][a_seg * 16]) = aring[slot][q];
    }
  };

#pragma unroll
  for (int st = 0; st < S - 1; ++st) {
    if (st < nch) load_chunk(st, st);
    __builtin_amdgcn_sched_barrier(0);
  }
  stage_a(0, 0);
  __syncthreads();

  static_assert(S % 2 == 0, "the LDS buffer of chunk i is i % 2 == slot % 2");
  auto step = [&](int c, auto U, bool prefetch, bool stage) __attribute__((always_inline)) {
    constexpr int u = decltype(U)::value;
    take_pair(U);   // before this step's prefetch of the next pair (S = 2: chunk c + 1 is odd)
    if (prefetch) load_chunk(c + S - 1, (u + S - 1) % S);
    constexpr int buf = u & 1;
    static_for<4>([&](auto TT) {
      constexpr int t = decltype(TT)::value;
#pragma unroll
      for (int q = 0; q < NA; ++q) {
        // FP8 operand: lane half h holds elements 16h..16h+15 and
        // 32+16h..32+16h+15 of the instruction's 64 (see mfma_mx)
        const uint8_t* arow = &lds[buf][32 * q + lr][t * 32 + lh * 16];
        const u32x4 a_lo = *reinterpret_cast<const u32x4*>(arow);
        const u32x4 a_hi = *reinterpret_cast<const u32x4*>(arow + 128);
        acc[2 * q] = mfma_mx<t>(a_lo, a_hi, ring[u].w[0][t], ring[u].sa[q], ring[u].sw[0], acc[2 * q]);
        acc[2 * q + 1] = mfma_mx<t>(a_lo, a_hi, ring[u].w[1][t], ring[u].sa[q], ring[u].sw[1],
                                    acc[2 * q + 1]);
      }
      // Keep each k-slice's reads and MFMAs together: left free, the
      // compiler sinks the MFMAs past the next step's loads and has to
      // rotate the register ring with copies that wait for every load.
      __builtin_amdgcn_sched_barrier(0);
    });
    if (stage) stage_a((u + 1) % S, buf ^ 1);
    __syncthreads();
  };
  int c0 = 0;
  for (; c0 + 2 * S - 1 <= nch - 1; c0 += S) {
    static_for<S>([&](auto U) { step(c0 + U, U, true, true); });
  }
  const int rem = nch - c0;
  static_for<2 * S>([&](auto U) {
    constexpr int u = decltype(U)::value;
    if (u < rem) step(c0 + u, int_c<u % S>{}, u + S - 1 < rem, u + 1 < rem);
  });
}

// Grouped MX GEMM: the schedule and column tiles of the 16-bit and W4A8
// grouped kernels (gate/up: wave w owns columns 128 nt + 32 w + l%32 of
// W_gate and W_up, writes h = R(SiLU(g) * u); down: columns 256 nt + 64 w +
// l%32 and + 32 of W_down, writes expert_out), rows in passes of up to
// 32 * NAMAX.
template <int DT, bool GATEUP, int NAMAX, bool PAIR = false>
__global__ __launch_bounds__(kThreads) void mx_grouped_kernel(MxGroupedArgs g) {
  static_assert(!PAIR || NAMAX == 1, "paired scale loads need the unrotated walk of single-group passes");
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][32 * NAMAX][kLdsRow];

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
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const int64_t kd = g.kd;
  const int64_t kb = kd / kBlk;   // scale bytes per row

  int col0;
  int64_t wrow[2];
  if constexpr (GATEUP) {
    col0 = nt * 128 + wave * 32;
    wrow[0] = static_cast<int64_t>(e) * g.n + col0 + lr;
    wrow[1] = wrow[0];
  } else {
    col0 = nt * 256 + wave * 64;
    wrow[0] = static_cast<int64_t>(e) * g.n + col0 + lr;
    wrow[1] = wrow[0] + 32;
  }
  const uint8_t* wb1 = GATEUP ? g.b1 : g.b0;
  const uint8_t* ws1 = GATEUP ? g.s1 : g.s0;
  const uint8_t* bptr[2] = {g.b0 + wrow[0] * (kd / 2) + lh * 64, wb1 + wrow[1] * (kd / 2) + lh * 64};
  const uint8_t* bscale[2] = {g.s0 + wrow[0] * kb + lh * 4, ws1 + wrow[1] * kb + lh * 4};

  const int a_seg = tid & 15;
  const int a_row = tid >> 4;
  const int nch = g.kd / kCK;
  // start of the reduction walk, rotated for prefill-sized blocks only
  const int rot = NAMAX > 1 ? natural % nch : 0;
  for (int r0 = 0; r0 < rows; r0 += 32 * NAMAX) {
    if (r0 > 0) __syncthreads();
    const int rows_pass = min(32 * NAMAX, rows - r0);
    const uint8_t* asrc[2 * NAMAX];
#pragma unroll
    for (int q = 0; q < 2 * NAMAX; ++q) {
      int r = a_row + 16 * q;
      if (r >= rows_pass) r = 0;  // in bounds, never staged
      const int64_t src = GATEUP ? g.sorted_token[m_start + r0 + r] : (m_start + r0 + r);
      asrc[q] = g.a + src * kd + a_seg * 16;
    }
    const uint8_t* ascale[NAMAX];
#pragma unroll
    for (int q = 0; q < NAMAX; ++q) {
      int r = 32 * q + lr;
      if (r >= rows_pass) r = 0;  // in bounds; its results are never stored
      const int64_t src = GATEUP ? g.sorted_token[m_start + r0 + r] : (m_start + r0 + r);
      ascale[q] = g.as + src * kb + lh * 4;
    }
    f32x16 acc[2 * NAMAX];
    auto run = [&](auto NAC) __attribute__((always_inline)) {
      constexpr int na = decltype(NAC)::value;
      mx_pass<na, NAMAX, PAIR>(asrc, ascale, a_row, a_seg, bptr, bscale, nch, rot, rows_pass, lr, lh, lds,
                         acc);
#pragma unroll
      for (int q = 0; q < na; ++q) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = 32 * q + (i >> 2) * 8 + lh * 4 + (i & 3);
          if (row < rows_pass) {
            uint16_t* out = g.c + (m_start + r0 + row) * g.n + col0 + lr;
            const float v0 = acc[2 * q][i], v1 = acc[2 * q + 1][i];
            if constexpr (GATEUP) {
              out[0] = static_cast<uint16_t>(from_float<DT>(silu(v0) * v1));
            } else {
              out[0] = static_cast<uint16_t>(from_float<DT>(v0));
              out[32] = static_cast<uint16_t>(from_float<DT>(v1));
            }
          }
        }
      }
    };
    const int active = (rows_pass + 31) >> 5;
    static_for<NAMAX>([&](auto I) {
      constexpr int na = decltype(I)::value + 1;
      if (active == na) run(int_c<na>{});
    });
  }
}

// ------------------------------------------------------------ quantizer --

template <int DT>
__device__ __forceinline__ float load_v(const void* v, int64_t i) {
  if constexpr (DT == kF32) {
    return static_cast<const float*>(v)[i];
  } else {
    return to_float<DT>(static_cast<const uint16_t*>(v)[i]);
  }
}

__device__ __forceinline__ int mx_scale_exp(float amax, int emax_elem) {
  if (!(amax > 0.0f)) return 127;
  int e2;
  frexpf(amax, &e2);                        // amax = f * 2^e2, f in [0.5, 1)
  const int e = (e2 - 1) - emax_elem + 127;
  return e < 0 ? 0 : (e > 254 ? 254 : e);
}

// Nearest E2M1 code (ties to the even code, saturating at 6; NaN -> 0).
__device__ __forceinline__ uint32_t float_to_fp4e2m1(float v) {
  const float a = fabsf(v);
  uint32_t c;
  if (!(a == a)) return 0u;
  if (a <= 0.25f) c = 0u;
  else if (a < 0.75f) c = 1u;
  else if (a <= 1.25f) c = 2u;
  else if (a < 1.75f) c = 3u;
  else if (a <= 2.5f) c = 4u;
  else if (a < 3.5f) c = 5u;
  else if (a <= 5.0f) c = 6u;
  else c = 7u;
  return (v < 0.0f && c != 0u) ? (c | 8u) : c;
}

// One wave per row; lane L quantises blocks L, L + 64, ... of the row.
template <int DT, int FMT>
__global__ __launch_bounds__(256) void quantize_mx_rows_kernel(const void* __restrict__ v,
                                                               int64_t rows, int cols,
                                                               uint8_t* __restrict__ codes,
                                                               uint8_t* __restrict__ scales) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;   // the whole wave exits together
  const int lane = threadIdx.x & 63;
  const int nb = cols / kBlk;
  const int64_t base = r * cols;
  for (int b = lane; b < nb; b += 64) {
    float x[kBlk];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kBlk; ++i) {
      x[i] = load_v<DT>(v, base + b * kBlk + i);
      amax = fmaxf(amax, fabsf(x[i]));
    }
    const int e = mx_scale_exp(amax, FMT == 4 ? 2 : 8);
    scales[r * nb + b] = static_cast<uint8_t>(e);
    const float X = ldexpf(1.0f, e - 127);
    if constexpr (FMT == 4) {
      uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < kBlk; ++i) w[i >> 3] |= float_to_fp4e2m1(x[i] / X) << (4 * (i & 7));
      *reinterpret_cast<u32x4*>(codes + r * (cols / 2) + b * (kBlk / 2)) = u32x4{w[0], w[1], w[2], w[3]};
    } else {
      uint32_t w[8];
#pragma unroll
      for (int i = 0; i < kBlk; i += 4) {
        w[i >> 2] = pk4_fp8e4m3(x[i] / X, x[i + 1] / X, x[i + 2] / X, x[i + 3] / X);
      }
      u32x4* dst = reinterpret_cast<u32x4*>(codes + base + b * kBlk);
      dst[0] = u32x4{w[0], w[1], w[2], w[3]};
      dst[1] = u32x4{w[4], w[5], w[6], w[7]};
    }
  }
}

template <int FMT>
hipError_t launch_quant(const void* v, int64_t rows, int cols, int dtype, uint8_t* codes,
                        uint8_t* scales, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((rows + 3) / 4));
  if (dtype == kBF16) {
    hipLaunchKernelGGL((quantize_mx_rows_kernel<kBF16, FMT>), grid, dim3(256), 0, stream, v, rows,
                       cols, codes, scales);
  } else if (dtype == kF16) {
    hipLaunchKernelGGL((quantize_mx_rows_kernel<kF16, FMT>), grid, dim3(256), 0, stream, v, rows,
                       cols, codes, scales);
  } else {
    hipLaunchKernelGGL((quantize_mx_rows_kernel<kF32, FMT>), grid, dim3(256), 0, stream, v, rows,
                       cols, codes, scales);
  }
  return hipGetLastError();
}

template <int DT, bool GATEUP>
hipError_t launch_grouped(const MxGemmProblem& p, const moe_tables& t, hipStream_t stream) {
  MxGroupedArgs g;
  g.a = p.a;
  g.as = p.as;
  g.b0 = p.b0;
  g.b1 = p.b1;
  g.s0 = p.s0;
  g.s1 = p.s1;
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
  // Paired scale loads: 16-byte loads of two chunks' scale words, which
  // need scale rows of a multiple of 16 bytes (kd a multiple of 512, so an
  // even chunk count) and 16-byte aligned scale arrays.
  const auto al16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; };
  const bool pair = p.kd % (2 * kCK) == 0 && al16(p.as) && al16(p.s0) && (!GATEUP || al16(p.s1));
  if (t.block_m <= 32 && pair) {
    hipLaunchKernelGGL((mx_grouped_kernel<DT, GATEUP, 1, true>), dim3(grid), dim3(kThreads), 0,
                       stream, g);
  } else if (t.block_m <= 32) {
    hipLaunchKernelGGL((mx_grouped_kernel<DT, GATEUP, 1>), dim3(grid), dim3(kThreads), 0, stream, g);
  } else if (t.block_m == 64) {
    hipLaunchKernelGGL((mx_grouped_kernel<DT, GATEUP, 2>), dim3(grid), dim3(kThreads), 0, stream, g);
  } else {
    hipLaunchKernelGGL((mx_grouped_kernel<DT, GATEUP, kWideNa>), dim3(grid), dim3(kThreads),
                       0, stream, g);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_mx_rows(const void* v, int64_t rows, int cols, int dtype, int fmt,
                                   uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  if (fmt == 4) return launch_quant<4>(v, rows, cols, dtype, codes, scales, stream);
  return launch_quant<0>(v, rows, cols, dtype, codes, scales, stream);
}

hipError_t launch_gate_up_mx(const MxGemmProblem& p, const moe_tables& t, hipStream_t stream) {
  if (p.dtype == kBF16) return launch_grouped<kBF16, true>(p, t, stream);
  return launch_grouped<kF16, true>(p, t, stream);
}

hipError_t launch_down_mx(const MxGemmProblem& p, const moe_tables& t, hipStream_t stream) {
  if (p.dtype == kBF16) return launch_grouped<kBF16, false>(p, t, stream);
  return launch_grouped<kF16, false>(p, t, stream);
}

}  // namespace moe
