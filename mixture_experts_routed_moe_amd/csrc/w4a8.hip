// W4A8: int4 weights (packed two per byte) with int8 activations and int32
// accumulation, on v_mfma_i32_32x32x32_i8 (TileLang tutorial ch.18,
// w4a8_dequant_gemm: the packed weights are unpacked in registers and fed to
// the integer GEMM; module docstring: the weight + activation quantised mode).
//
// Formats. A packed row holds field 2i in bits 0..3 of byte i and field 2i+1
// in bits 4..7; a field is a 4-bit two's complement number in [-8, 7].
// Quantisation is symmetric per row (the scheme is left open by the pages):
// int8 activations s = amax / 127, int4 weights s = amax / 7 (1 for a zero
// row), code = the nearest integer to v / s (fp32 division, ties to even),
// clamped to [-127, 127] / [-8, 7].
//
// Unpacking. A packed word holds 8 fields; (w << 4) & 0xF0F0F0F0 puts fields
// 0, 2, 4, 6 and w & 0xF0F0F0F0 fields 1, 3, 5, 7 at the top of a byte each,
// which as an int8 is 16 x the field (sign included), and one byte permute
// per 4 fields restores field order. The MFMA then accumulates 16 x the dot
// product; an arithmetic shift by 4 returns it exactly as long as 16 x the
// sum fits in int32 (|a| <= 128, |16 q| <= 128: K <= 131072).
//
// Tiling (both kernels): 256 threads = 4 waves; the reduction runs in
// chunks of 256 elements, in which lane half h of a lane owns elements
// 128h..128h+127 of its weight rows: 64 contiguous bytes per row and chunk
// (two lanes per 128-byte segment), four 16-byte loads. k-slice t (0..7) of
// the chunk is elements 128h + 16t .. +15 on both operands. The activation
// rows of a chunk (32 rows x 256 bytes) are staged through a double-buffered
// LDS tile; the weights stream straight from HBM into registers with a
// 4-deep ring, as in the 16-bit grouped GEMM.

#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kCK = 256;                 // reduction elements per chunk
constexpr int kLdsRow = kCK + 16;        // bytes per LDS A row (16 bytes of padding)
// Weight chunks in the register ring of the grouped kernels (depth 4
// measured slower at decode, two workgroups per CU) and of the plain GEMM;
// workgroups the plain GEMM aims for (split-K); row groups per pass for
// 128/256-row blocks.
constexpr int kStages = 2;
constexpr int kGemmStages = 4;
constexpr int kGemmWorkgroups = 256;
constexpr int kWideNa = 4;

__device__ __forceinline__ i32x16 mfma_i8(u32x4 a, u32x4 b, i32x16 c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a),
                                               __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
}

// 8 packed int4 fields -> 8 int8 bytes holding 16 x each field, in order.
__device__ __forceinline__ u32x2 unpack8(uint32_t w) {
  const uint32_t lo = (w << 4) & 0xF0F0F0F0u;   // fields 0, 2, 4, 6
  const uint32_t hi = w & 0xF0F0F0F0u;          // fields 1, 3, 5, 7
  // v_perm_b32: selector bytes 0..3 pick bytes of the second operand, 4..7
  // bytes of the first.
  return u32x2{__builtin_amdgcn_perm(hi, lo, 0x05010400u),
               __builtin_amdgcn_perm(hi, lo, 0x07030602u)};
}

// A lane's weights of one chunk: two rows x 64 bytes (128 fields each).
struct W4Chunk {
  u32x4 v[2][4];

  __device__ __forceinline__ void load(const uint8_t* const* p, int64_t byte_off) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[j][i] = *reinterpret_cast<const u32x4*>(p[j] + byte_off + i * 16);
    }
  }

  // MFMA operand of row j for k-slice t: fields 16t..16t+15 (words 2t, 2t+1).
  __device__ __forceinline__ u32x4 operand(int j, int t) const {
    const u32x4 r = v[j][t >> 1];
    const u32x2 a = unpack8((t & 1) ? r.z : r.x);
    const u32x2 b = unpack8((t & 1) ? r.w : r.y);
    return u32x4{a.x, a.y, b.x, b.y};
  }
};



// One pass over chunks [c_begin, c_begin + nch) for NA groups of 32
// activation rows (the LDS tile holds 32 * NAS rows, NAS >= NA).
//   asrc[2q + sb]: this thread's staging row of group q (row 32q + a_row +
//            16 sb of the pass), pointing at element 16 * a_seg of the row;
//   bptr[2]: the lane's two weight rows (packed bytes, lane-half offset
//            included); each unpacked weight operand feeds the NA groups;
//   SWAP:    false -- MFMA A = activations, B = weights: accumulator lane l
//            holds weight row l % 32 (output column), activation rows
//            8(i/4) + 4(l/32) + i%4 of the group; true -- the operands
//            swapped: lane l holds activation row l % 32 and weight rows
//            8(i/4) + 4(l/32) + i%4.
// acc[2q + j]: group q against weight row j (16 x the dot products).
template <bool SWAP, int NA, int NAS, int S>
__device__ __forceinline__ void w4a8_pass(const int8_t* const* asrc, int a_row, int a_seg,
                                          const uint8_t* const* bptr, int c_begin, int nch,
                                          int rot, int rows_pass, int lr, int lh,
                                          uint8_t (*lds)[32 * NAS][kLdsRow], i32x16* acc) {
#pragma unroll
  for (int q = 0; q < 2 * NA; ++q) acc[q] = i32x16{};
  u32x4 aring[S][2 * NA];
  W4Chunk bring[S];

  auto load_chunk = [&](int i, int slot) __attribute__((always_inline)) {
    int ii = i + rot;                       // chunks are walked from `rot` on
    if (ii >= nch) ii -= nch;
    const int64_t c = c_begin + ii;
#pragma unroll
    for (int q = 0; q < 2 * NA; ++q) {
      if (a_row + 16 * q < rows_pass) {
        aring[slot][q] = *reinterpret_cast<const u32x4*>(asrc[q] + c * kCK);
      }
    }
    bring[slot].load(bptr, c * (kCK / 2));
  };
  auto stage_a = [&](int slot, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 2 * NA; ++q) {
      const int r = a_row + 16 * q;
      if (r < rows_pass) *reinterpret_cast<u32x4*>(&lds[buf][r][a_seg * 16]) = aring[slot][q];
    }
  };

#pragma unroll
  for (int st = 0; st < S - 1; ++st) {
    if (st < nch) load_chunk(st, st);
    __builtin_amdgcn_sched_barrier(0);
  }
  stage_a(0, 0);
  __syncthreads();

  // Step i: prefetch chunk i+S-1 (only while it exists), multiply chunk i,
  // stage chunk i+1's activations in the other buffer, barrier.
  static_assert(S % 2 == 0, "the LDS buffer of chunk i is i % 2 == slot % 2");
  auto step = [&](int i, auto U, bool prefetch, bool stage) __attribute__((always_inline)) {
    constexpr int u = decltype(U)::value;
    if (prefetch) load_chunk(i + S - 1, (u + S - 1) % S);
    constexpr int buf = u & 1;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const u32x4 b0 = bring[u].operand(0, t);
      const u32x4 b1 = bring[u].operand(1, t);
#pragma unroll
      for (int q = 0; q < NA; ++q) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(&lds[buf][32 * q + lr][lh * 128 + t * 16]);
        if constexpr (SWAP) {
          acc[2 * q] = mfma_i8(b0, a, acc[2 * q]);
          acc[2 * q + 1] = mfma_i8(b1, a, acc[2 * q + 1]);
        } else {
          acc[2 * q] = mfma_i8(a, b0, acc[2 * q]);
          acc[2 * q + 1] = mfma_i8(a, b1, acc[2 * q + 1]);
        }
      }
    }
    if (stage) stage_a((u + 1) % S, buf ^ 1);
    __syncthreads();
  };
  int i0 = 0;
  for (; i0 + 2 * S - 1 <= nch - 1; i0 += S) {
    static_for<S>([&](auto U) { step(i0 + U, U, true, true); });
  }
  const int rem = nch - i0;
  static_for<2 * S>([&](auto U) {
    constexpr int u = decltype(U)::value;
    if (u < rem) step(i0 + u, int_c<u % S>{}, u + S - 1 < rem, u + 1 < rem);
  });
}


// (float) acc * s_a * s_w, left to right in fp32 (acc: the exact int32 sum).
__device__ __forceinline__ float dequant(int acc, float sa, float sw) {
  return __fmul_rn(__fmul_rn(static_cast<float>(acc), sa), sw);
}

struct W4GroupedArgs {
  const int8_t* a;          // gate/up: xq [T, kd]; down: hq [P, kd]
  const float* sa;          // gate/up: sx [T]; down: sh [P]
  const uint8_t* b0;        // packed weights [E, n, kd/2]
  const uint8_t* b1;        // gate/up: W_up; down: unused
  const float* s0;          // row scales of b0 [E * n]
  const float* s1;
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

// Grouped W4A8 GEMM over the active row blocks: workgroup = (row block,
// column tile), dealt out to XCDs in contiguous ranges; a block's rows run
// in passes of up to 32 * NAMAX rows (the weights stream once per pass).
// Gate/up: wave w owns columns 128 nt + 32 w + l%32 of W_gate and W_up (one
// row of each per lane) and writes h = R(SiLU(g) * u); down: wave w owns
// columns 256 nt + 64 w + l%32 and + 32 of W_down and writes expert_out.
template <int DT, bool GATEUP, int NAMAX>
__global__ __launch_bounds__(kThreads) void w4a8_grouped_kernel(W4GroupedArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][32 * NAMAX][kLdsRow];
  __shared__ float sa_s[32 * NAMAX];   // the pass's activation-row scales

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
  const uint8_t* bptr[2] = {g.b0 + wrow[0] * (kd / 2) + lh * 64,
                            (GATEUP ? g.b1 : g.b0) + wrow[1] * (kd / 2) + lh * 64};
  const float sw0 = g.s0[wrow[0]];
  const float sw1 = (GATEUP ? g.s1 : g.s0)[wrow[1]];

  const int a_seg = tid & 15;     // 16-byte segment of a 256-byte row chunk
  const int a_row = tid >> 4;     // 0..15 (+ 16 sb + 32 q)
  const int nch = g.kd / kCK;
  // Start of the reduction walk: with prefill-sized blocks, workgroups
  // streaming at one time begin at different chunks, so rows a power of two
  // apart do not load the same columns together (measured: faster there,
  // slower for decode-sized blocks).
  const int rot = NAMAX > 1 ? natural % nch : 0;   // prefill-sized blocks only
  for (int r0 = 0; r0 < rows; r0 += 32 * NAMAX) {
    if (r0 > 0) __syncthreads();  // every wave is done with the LDS tile
    const int rows_pass = min(32 * NAMAX, rows - r0);
    const int8_t* asrc[2 * NAMAX];
#pragma unroll
    for (int q = 0; q < 2 * NAMAX; ++q) {
      int r = a_row + 16 * q;
      if (r >= rows_pass) r = 0;  // in bounds, never staged
      const int64_t src = GATEUP ? g.sorted_token[m_start + r0 + r] : (m_start + r0 + r);
      asrc[q] = g.a + src * kd + a_seg * 16;
    }
    // Row tid's activation scale, loaded now and used after the pass (a
    // load per row in the epilogue -- through sorted_token for gate/up --
    // put one or two memory latencies at the end of every pass).
    float sa_mine = 0.0f;
    if (tid < rows_pass) {
      const int64_t row = m_start + r0 + tid;
      sa_mine = g.sa[GATEUP ? g.sorted_token[row] : row];
    }
    i32x16 acc[2 * NAMAX];
    auto epilogue = [&](auto NAC) __attribute__((always_inline)) {
      constexpr int na = decltype(NAC)::value;
      w4a8_pass<false, na, NAMAX, kStages>(asrc, a_row, a_seg, bptr, 0, nch, rot, rows_pass, lr, lh,
                                            lds, acc);
      if (tid < rows_pass) sa_s[tid] = sa_mine;
      __syncthreads();   // every row's scale is visible
#pragma unroll
      for (int q = 0; q < na; ++q) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = 32 * q + (i >> 2) * 8 + lh * 4 + (i & 3);
          if (row < rows_pass) {
            const int64_t out_row = m_start + r0 + row;
            const float sa = sa_s[row];
            uint16_t* out = g.c + out_row * g.n + col0 + lr;
            const float v0 = dequant(acc[2 * q][i] >> 4, sa, sw0);
            const float v1 = dequant(acc[2 * q + 1][i] >> 4, sa, sw1);
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
      if (active == na) epilogue(int_c<na>{});
    });
  }
}

// The tutorial's plain W4A8 GEMM: Ct[n, m] = sum_k A[m, k] * B4[n, k], int32,
// written transposed ([N, M]). Workgroup = (256 columns, chunk range): wave w
// owns weight rows 256 bx + 64 w + l%32 and + 32; the reduction is split into
// `splits` ranges of chunks when the column tiles alone cannot fill the GPU,
// and the partial sums of a split are added with int32 atomics (exact, so
// the result does not depend on their order). The operands are swapped in
// the MFMA so that lanes hold consecutive m of one output row.
__global__ __launch_bounds__(kThreads) void w4a8_gemm_kernel(const int8_t* __restrict__ A,
                                                            const uint8_t* __restrict__ B,
                                                            int32_t* __restrict__ Ct, int M, int N,
                                                            int K, int chunks_per_split,
                                                            int atomic) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][32][kLdsRow];
  const int col_tile = blockIdx.x;
  const int split = blockIdx.y;
  const int nch_total = K / kCK;
  const int c_begin = split * chunks_per_split;
  const int nch = min(chunks_per_split, nch_total - c_begin);
  if (nch <= 0) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const int n0 = col_tile * 256 + wave * 64;
  const uint8_t* bptr[2] = {B + static_cast<int64_t>(n0 + lr) * (K / 2) + lh * 64,
                            B + static_cast<int64_t>(n0 + 32 + lr) * (K / 2) + lh * 64};
  const int a_seg = tid & 15;
  const int a_row = tid >> 4;
  for (int r0 = 0; r0 < M; r0 += 32) {
    if (r0 > 0) __syncthreads();
    const int rows_pass = min(32, M - r0);
    const int8_t* asrc[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      int r = a_row + 16 * sb;
      if (r >= rows_pass) r = 0;
      asrc[sb] = A + static_cast<int64_t>(r0 + r) * K + a_seg * 16;
    }
    i32x16 acc[2];
    w4a8_pass<true, 1, 1, kGemmStages>(asrc, a_row, a_seg, bptr, c_begin, nch, 0, rows_pass, lr, lh,
                                       lds, acc);
    // lane l: activation row m = r0 + l % 32; weight rows n0 + 32 j + 8(i/4) + 4(l/32) + i%4
    const int m = r0 + lr;
    if (m < M) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int n = n0 + 32 * j + (i >> 2) * 8 + lh * 4 + (i & 3);
          const int v = acc[j][i] >> 4;
          int32_t* dst = Ct + static_cast<int64_t>(n) * M + m;
          if (atomic) {
            atomicAdd(dst, v);
          } else {
            *dst = v;
          }
        }
      }
    }
  }
}

__global__ void fill_zero_i32(int32_t* __restrict__ p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// ------------------------------------------------------------ quantizers --

template <int DT>
__device__ __forceinline__ float load_v(const void* v, int64_t i) {
  if constexpr (DT == kF32) {
    return static_cast<const float*>(v)[i];
  } else {
    return to_float<DT>(static_cast<const uint16_t*>(v)[i]);
  }
}

template <int DT>
__device__ __forceinline__ float row_scale(const void* v, int64_t base, int cols, int lane,
                                           float qmax) {
  float amax = 0.0f;
  for (int k = lane; k < cols; k += 64) amax = fmaxf(amax, fabsf(load_v<DT>(v, base + k)));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  return amax > 0.0f ? amax / qmax : 1.0f;
}

__device__ __forceinline__ int quant_code(float v, float s, float qmin, float qmax) {
  return static_cast<int>(fminf(fmaxf(rintf(v / s), qmin), qmax));
}

// One wave per row.
template <int DT>
__global__ __launch_bounds__(256) void quantize_int8_rows_kernel(const void* __restrict__ a,
                                                                 int64_t rows, int cols,
                                                                 int8_t* __restrict__ q,
                                                                 float* __restrict__ scales) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;   // the whole wave exits together
  const int lane = threadIdx.x & 63;
  const int64_t base = r * cols;
  const float s = row_scale<DT>(a, base, cols, lane, 127.0f);
  if (lane == 0) scales[r] = s;
  for (int k = lane; k < cols; k += 64) {
    q[base + k] = static_cast<int8_t>(quant_code(load_v<DT>(a, base + k), s, -127.0f, 127.0f));
  }
}

// Eight 16-bit values (one 16-byte load): their largest magnitude, and
// their int8 codes at scale s, packed in order.
template <int DT>
__device__ __forceinline__ float amax8_int(u32x4 w, float amax) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    amax = fmaxf(amax, fabsf(to_float<DT>(w[j] & 0xffffu)));
    amax = fmaxf(amax, fabsf(to_float<DT>(w[j] >> 16)));
  }
  return amax;
}

template <int DT>
__device__ __forceinline__ u32x2 encode8_int8(u32x4 w, float s) {
  uint32_t packed[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t c0 = static_cast<uint32_t>(quant_code(to_float<DT>(w[j] & 0xffffu), s, -127.0f, 127.0f)) & 0xffu;
    const uint32_t c1 = static_cast<uint32_t>(quant_code(to_float<DT>(w[j] >> 16), s, -127.0f, 127.0f)) & 0xffu;
    const uint32_t pair = c0 | (c1 << 8);
    if (j & 1) packed[j >> 1] |= pair << 16;
    else packed[j >> 1] = pair;
  }
  return u32x2{packed[0], packed[1]};
}

// The same for 16-bit rows of a multiple of 8 values on a 16-byte aligned
// base (the activations of the forward): each lane reads 8 values per
// 16-byte load, the row's loads all in flight at once, and writes 8 codes
// per 8-byte store; the second pass reads the row again from the cache.
template <int DT>
__global__ __launch_bounds__(256) void quantize_int8_rows16_kernel(const uint16_t* __restrict__ a,
                                                                   int64_t rows, int cols,
                                                                   int8_t* __restrict__ q,
                                                                   float* __restrict__ scales) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;   // the whole wave exits together
  const int lane = threadIdx.x & 63;
  const u32x4* row = reinterpret_cast<const u32x4*>(a + r * cols);
  const int nvec = cols / 8;
  float amax = 0.0f;
#pragma unroll 4
  for (int v = lane; v < nvec; v += 64) amax = amax8_int<DT>(row[v], amax);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float s = amax > 0.0f ? amax / 127.0f : 1.0f;
  if (lane == 0) scales[r] = s;
  u32x2* out = reinterpret_cast<u32x2*>(q + r * cols);
#pragma unroll 4
  for (int v = lane; v < nvec; v += 64) out[v] = encode8_int8<DT>(row[v], s);
}

// Rows of at most 512 NV values held in registers between the amax and the
// encoding, so the row is read from memory once (with many rows in flight
// per CU the two-pass form's second read mostly misses the cache).
template <int DT, int NV>
__global__ __launch_bounds__(256) void quantize_int8_rows_reg_kernel(const uint16_t* __restrict__ a,
                                                                     int64_t rows, int cols,
                                                                     int8_t* __restrict__ q,
                                                                     float* __restrict__ scales) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;   // the whole wave exits together
  const int lane = threadIdx.x & 63;
  const u32x4* row = reinterpret_cast<const u32x4*>(a + r * cols);
  const int nvec = cols / 8;
  u32x4 w[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = lane + 64 * i;
    w[i] = v < nvec ? row[v] : u32x4{0u, 0u, 0u, 0u};   // zeros leave the amax unchanged
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i) amax = amax8_int<DT>(w[i], amax);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float s = amax > 0.0f ? amax / 127.0f : 1.0f;
  if (lane == 0) scales[r] = s;
  u32x2* out = reinterpret_cast<u32x2*>(q + r * cols);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = lane + 64 * i;
    if (v < nvec) out[v] = encode8_int8<DT>(w[i], s);
  }
}

template <int DT>
void launch_int8_rows16(const uint16_t* a, int64_t rows, int cols, int8_t* q, float* scales,
                        dim3 grid, hipStream_t stream) {
  const int nvec = cols / 8;   // 16-byte loads per row; the register form up to 16 per lane
  auto reg = [&](auto NV) {
    hipLaunchKernelGGL((quantize_int8_rows_reg_kernel<DT, decltype(NV)::value>), grid, dim3(256), 0, stream, a, rows,
                       cols, q, scales);
  };
  if (nvec <= 64) {
    reg(int_c<1>{});
  } else if (nvec <= 128) {
    reg(int_c<2>{});
  } else if (nvec <= 256) {
    reg(int_c<4>{});
  } else if (nvec <= 512) {
    reg(int_c<8>{});
  } else if (nvec <= 1024) {
    reg(int_c<16>{});
  } else {
    hipLaunchKernelGGL(quantize_int8_rows16_kernel<DT>, grid, dim3(256), 0, stream, a, rows, cols, q, scales);
  }
}

template <int DT>
__global__ __launch_bounds__(256) void quantize_int4_rows_kernel(const void* __restrict__ w,
                                                                 int64_t rows, int cols,
                                                                 uint8_t* __restrict__ packed,
                                                                 float* __restrict__ scales) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int lane = threadIdx.x & 63;
  const int64_t base = r * cols;
  const float s = row_scale<DT>(w, base, cols, lane, 7.0f);
  if (lane == 0) scales[r] = s;
  const int half = cols / 2;
  for (int b = lane; b < half; b += 64) {
    const int q0 = quant_code(load_v<DT>(w, base + 2 * b), s, -8.0f, 7.0f);
    const int q1 = quant_code(load_v<DT>(w, base + 2 * b + 1), s, -8.0f, 7.0f);
    packed[r * half + b] = static_cast<uint8_t>((q0 & 0xF) | ((q1 & 0xF) << 4));
  }
}

}  // namespace

hipError_t launch_quantize_int8_rows(const void* a, int64_t rows, int cols, int dtype, int8_t* q,
                                     float* scales, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((rows + 3) / 4));
  const bool vec = dtype != kF32 && cols % 8 == 0 && reinterpret_cast<uintptr_t>(a) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(q) % 8 == 0;
  if (vec && dtype == kBF16) {
    launch_int8_rows16<kBF16>(static_cast<const uint16_t*>(a), rows, cols, q, scales, grid, stream);
  } else if (vec) {
    launch_int8_rows16<kF16>(static_cast<const uint16_t*>(a), rows, cols, q, scales, grid, stream);
  } else if (dtype == kBF16) {
    hipLaunchKernelGGL(quantize_int8_rows_kernel<kBF16>, grid, dim3(256), 0, stream, a, rows, cols,
                       q, scales);
  } else if (dtype == kF16) {
    hipLaunchKernelGGL(quantize_int8_rows_kernel<kF16>, grid, dim3(256), 0, stream, a, rows, cols,
                       q, scales);
  } else {
    hipLaunchKernelGGL(quantize_int8_rows_kernel<kF32>, grid, dim3(256), 0, stream, a, rows, cols,
                       q, scales);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_int4_rows(const void* w, int64_t rows, int cols, int dtype,
                                     uint8_t* packed, float* scales, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((rows + 3) / 4));
  if (dtype == kBF16) {
    hipLaunchKernelGGL(quantize_int4_rows_kernel<kBF16>, grid, dim3(256), 0, stream, w, rows, cols,
                       packed, scales);
  } else if (dtype == kF16) {
    hipLaunchKernelGGL(quantize_int4_rows_kernel<kF16>, grid, dim3(256), 0, stream, w, rows, cols,
                       packed, scales);
  } else {
    hipLaunchKernelGGL(quantize_int4_rows_kernel<kF32>, grid, dim3(256), 0, stream, w, rows, cols,
                       packed, scales);
  }
  return hipGetLastError();
}

hipError_t launch_w4a8_gemm(const int8_t* A, const uint8_t* B, int M, int N, int K, int32_t* Ct,
                            hipStream_t stream) {
  // Split the reduction while the column tiles give fewer than
  // kGemmWorkgroups workgroups, keeping at least 2 chunks per split.
  const int col_tiles = N / 256;
  const int nch = K / kCK;
  int per = static_cast<int>((static_cast<int64_t>(col_tiles) * nch + kGemmWorkgroups - 1) /
                             kGemmWorkgroups);
  per = max(2, per);
  if (per > nch) per = nch;
  const int splits = (nch + per - 1) / per;
  const int atomic = splits > 1 ? 1 : 0;
  if (atomic) {
    const int64_t n = static_cast<int64_t>(N) * M;
    hipLaunchKernelGGL(fill_zero_i32, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                       stream, Ct, n);
  }
  hipLaunchKernelGGL(w4a8_gemm_kernel, dim3(col_tiles, splits), dim3(kThreads), 0, stream, A, B,
                     Ct, M, N, K, per, atomic);
  return hipGetLastError();
}

template <int DT, bool GATEUP>
static hipError_t launch_grouped(const W4GemmProblem& p, const moe_tables& t, hipStream_t stream) {
  W4GroupedArgs g;
  g.a = p.a;
  g.sa = p.sa;
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
  // Row groups per pass: 1 for decode-sized blocks (two workgroups per CU),
  // 2 for 64-row blocks, 4 (two passes of 128 rows) for 128- and 256-row
  // blocks.
  if (t.block_m <= 32) {
    hipLaunchKernelGGL((w4a8_grouped_kernel<DT, GATEUP, 1>), dim3(grid), dim3(kThreads), 0, stream, g);
  } else if (t.block_m == 64) {
    hipLaunchKernelGGL((w4a8_grouped_kernel<DT, GATEUP, 2>), dim3(grid), dim3(kThreads), 0, stream, g);
  } else {
    hipLaunchKernelGGL((w4a8_grouped_kernel<DT, GATEUP, kWideNa>), dim3(grid), dim3(kThreads),
                       0, stream, g);
  }
  return hipGetLastError();
}

hipError_t launch_gate_up_w4a8(const W4GemmProblem& p, const moe_tables& t, hipStream_t stream) {
  if (p.dtype == kBF16) return launch_grouped<kBF16, true>(p, t, stream);
  return launch_grouped<kF16, true>(p, t, stream);
}

hipError_t launch_down_w4a8(const W4GemmProblem& p, const moe_tables& t, hipStream_t stream) {
  if (p.dtype == kBF16) return launch_grouped<kBF16, false>(p, t, stream);
  return launch_grouped<kF16, false>(p, t, stream);
}

}  // namespace moe
