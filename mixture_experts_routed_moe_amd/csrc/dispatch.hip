// moe_dispatch on gfx950: a stable counting sort of the (token, slot) pairs
// by expert, plus the group / padded-offset / block->expert tables.
//
// What is computed follows the "tilelang baseline" MoE walkthrough
// (devpress.csdn.net), section "forward": argsort of the flat expert ids,
// per-expert counts and their prefix sums, padded offsets that give every
// expert ceil((count + 1) / block_m) blocks, and the table that gives every
// block its expert. The walkthrough does all of it on the host after copying
// the counts off the device; here it stays on the GPU in three kernels with
// no host round trip:
//
//   count  one 1024-thread workgroup per chunk of 1024 pairs. Each wave
//          matches lanes holding the same expert with one ballot per id bit,
//          so a lane's rank among equal experts in its wave is a popcount of
//          the lower lanes of its match mask. Per-wave counts go to LDS and
//          give the rank inside the chunk; per-chunk counts go to global.
//   scan   one workgroup: an exclusive scan of every expert's column of
//          chunk counts (the chunk prefix), then workgroup-wide scans over
//          the experts for group_offsets and group_padded_offsets, then each
//          expert writes its own range of block_expert and its entries of the
//          compact list of blocks that hold rows (active_blocks), which the
//          GEMMs use to spread only real work over the chip.
//   place  pos = group_offsets[e] + chunk_prefix[chunk][e] + rank, and the
//          sorted_* arrays and token_topk_to_pos are written.
// The order is stable in the flat slot index p = t*K + k by construction;
// no atomic decides a position, so the tables are bit-reproducible.

#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kChunk = 1024;   // pairs per count/place workgroup (16 waves)
constexpr int kWaves = kChunk / 64;
constexpr int kMaxE = 1024;

__global__ __launch_bounds__(kChunk) void dispatch_count_kernel(
    const int32_t* __restrict__ ids, int64_t P, int E, int nbits,
    int32_t* __restrict__ chunk_counts, int32_t* __restrict__ pair_rank,
    int32_t* __restrict__ chunk_flags) {
  __shared__ uint16_t wave_cnt[kWaves][kMaxE];
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int i = tid; i < kWaves * E; i += kChunk) wave_cnt[i / E][i % E] = 0;
  if (tid == 0) s_bad = 0;
  __syncthreads();

  const int64_t p = static_cast<int64_t>(blockIdx.x) * kChunk + tid;
  int e = (p < P) ? ids[p] : -1;
  if (e >= E) {        // precondition violation: flag it, treat as masked
    s_bad = 1;
    e = -1;
  }
  const bool valid = e >= 0;
  const uint64_t valid_mask = __ballot(valid);
  uint64_t match = valid ? valid_mask : 0ull;
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t m = __ballot(bit);
    match &= bit ? m : ~m;
  }
  const uint64_t lower = (1ull << lane) - 1ull;
  const int rank_in_wave = __popcll(match & lower);
  const int count_in_wave = __popcll(match);
  if (valid && rank_in_wave == count_in_wave - 1) {
    wave_cnt[wave][e] = static_cast<uint16_t>(count_in_wave);
  }
  __syncthreads();
  if (valid) {
    int r = rank_in_wave;
    for (int w = 0; w < wave; ++w) r += wave_cnt[w][e];
    pair_rank[p] = r;
  }
  for (int x = tid; x < E; x += kChunk) {
    int s = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s += wave_cnt[w][x];
    chunk_counts[static_cast<int64_t>(blockIdx.x) * E + x] = s;
  }
  if (tid == 0) chunk_flags[blockIdx.x] = s_bad;
}

// Inclusive scan of one int per thread over a 1024-thread workgroup.
__device__ int block_inclusive_scan(int v, int* s_wave) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  if (lane == 63) s_wave[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < kWaves; ++w) {
      const int c = s_wave[w];
      s_wave[w] = run;
      run += c;
    }
  }
  __syncthreads();
  v += s_wave[wave];
  __syncthreads();
  return v;
}

// The expert scan, one expert per thread (E <= 1024): from this expert's
// row count, the group size / offset / padded offset, its range of
// block_expert and its entries of the active-block list. Returns the
// group offset (threads e >= E pass cnt = 0 and get 0).
__device__ int scan_experts(int cnt, int E, int BM, int num_blocks, int* s_wave,
                            int32_t* __restrict__ group_sizes, int32_t* __restrict__ group_offsets,
                            int32_t* __restrict__ group_padded_offsets,
                            int32_t* __restrict__ block_expert,
                            int32_t* __restrict__ active_blocks,
                            int32_t* __restrict__ active_count) {
  const int e = threadIdx.x;
  const int padded_size = (e < E) ? ((cnt + 1 + BM - 1) / BM) * BM : 0;
  const int n_active = (e < E) ? (cnt + BM - 1) / BM : 0;
  const int incl_off = block_inclusive_scan(e < E ? cnt : 0, s_wave);
  const int incl_pad = block_inclusive_scan(padded_size, s_wave);
  const int incl_act = block_inclusive_scan(n_active, s_wave);
  if (e < E) {
    const int pad_start = incl_pad - padded_size;
    group_sizes[e] = cnt;
    group_offsets[e] = incl_off - cnt;
    group_padded_offsets[e] = pad_start;
    const int b0 = pad_start / BM;
    const int b1 = (e + 1 < E) ? incl_pad / BM : num_blocks;
    for (int b = b0; b < b1; ++b) block_expert[b] = e;
    const int a0 = incl_act - n_active;
    for (int j = 0; j < n_active; ++j) active_blocks[a0 + j] = b0 + j;
    if (e == E - 1) active_count[0] = incl_act;
  }
  return e < E ? incl_off - cnt : 0;
}

__global__ __launch_bounds__(1024) void dispatch_scan_kernel(
    int32_t* __restrict__ chunk_counts, const int32_t* __restrict__ chunk_flags, int C, int E,
    int BM, int num_blocks, int32_t* __restrict__ group_sizes,
    int32_t* __restrict__ group_offsets, int32_t* __restrict__ group_padded_offsets,
    int32_t* __restrict__ block_expert, int32_t* __restrict__ status,
    int32_t* __restrict__ active_blocks, int32_t* __restrict__ active_count) {
  __shared__ int s_wave[kWaves];
  const int e = threadIdx.x;   // E <= 1024: one expert per thread
  int bad = 0;
  for (int c = threadIdx.x; c < C; c += 1024) bad |= chunk_flags[c];
  bad = __syncthreads_or(bad);
  if (threadIdx.x == 0) status[0] = bad ? 1 : 0;
  int cnt = 0;
  if (e < E) {
    // Exclusive prefix of this expert's column, in batches so the loads of a
    // batch are all in flight before the dependent stores.
    for (int c0 = 0; c0 < C; c0 += 16) {
      int v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        v[j] = (c0 + j < C) ? chunk_counts[static_cast<int64_t>(c0 + j) * E + e] : 0;
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (c0 + j < C) chunk_counts[static_cast<int64_t>(c0 + j) * E + e] = cnt;
        cnt += v[j];
      }
    }
  }
  scan_experts(cnt, E, BM, num_blocks, s_wave, group_sizes, group_offsets, group_padded_offsets,
               block_expert, active_blocks, active_count);
}

__global__ __launch_bounds__(kChunk) void dispatch_place_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ w, int64_t P, int K, int E,
    const int32_t* __restrict__ chunk_prefix, const int32_t* __restrict__ group_offsets,
    const int32_t* __restrict__ pair_rank, int32_t* __restrict__ sorted_pair,
    int32_t* __restrict__ sorted_token, float* __restrict__ sorted_weight,
    int32_t* __restrict__ pos_out, float* __restrict__ w_copy) {
  const int64_t p = static_cast<int64_t>(blockIdx.x) * kChunk + threadIdx.x;
  if (p >= P) return;
  const int e = ids[p];
  const float wv = w ? w[p] : 1.0f;
  w_copy[p] = wv;
  if (e < 0 || e >= E) {
    pos_out[p] = -1;
    return;
  }
  const int i = group_offsets[e] + chunk_prefix[static_cast<int64_t>(blockIdx.x) * E + e] +
                pair_rank[p];
  sorted_pair[i] = static_cast<int32_t>(p);
  sorted_token[i] = static_cast<int32_t>(p / K);
  sorted_weight[i] = wv;
  pos_out[p] = i;
}

// Small dispatches (at most kSmallChunks chunks) in one 1024-thread
// workgroup: the count of each chunk in turn (the same ballot ranks and
// per-wave counts as dispatch_count_kernel), the chunk counts kept in LDS
// and each thread's ranks in registers, then the expert scan
// (scan_experts) and the placement (as dispatch_place_kernel). Same tables
// as the three kernels, in one launch; the tables' internal chunk arrays
// are not used. Used for one chunk (T*K <= 1024): measured on MI355X, the
// tiny workload (128 pairs) dispatches in 8.1 us against 13.7 us for the
// three kernels, while four chunks in turn (the decode workload's 4096
// pairs) took 30.4 us against 18.5.
constexpr int kSmallChunks = 4;
constexpr int kSmallUpTo = 1;

__global__ __launch_bounds__(kChunk) void dispatch_small_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ w, int64_t P, int K, int E,
    int nbits, int C, int BM, int num_blocks, int32_t* __restrict__ group_sizes,
    int32_t* __restrict__ group_offsets, int32_t* __restrict__ group_padded_offsets,
    int32_t* __restrict__ block_expert, int32_t* __restrict__ status,
    int32_t* __restrict__ active_blocks, int32_t* __restrict__ active_count,
    int32_t* __restrict__ sorted_pair, int32_t* __restrict__ sorted_token,
    float* __restrict__ sorted_weight, int32_t* __restrict__ pos_out,
    float* __restrict__ w_copy) {
  __shared__ uint16_t wave_cnt[kWaves][kMaxE];
  __shared__ int s_cnt[kSmallChunks][kMaxE];   // chunk counts, then exclusive prefixes
  __shared__ int s_off[kMaxE];                 // group offsets
  __shared__ int s_wave[kWaves];
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  if (tid == 0) s_bad = 0;
  int ec[kSmallChunks];
  int rank[kSmallChunks];
#pragma unroll
  for (int c = 0; c < kSmallChunks; ++c) {
    const int64_t p = static_cast<int64_t>(c) * kChunk + tid;
    ec[c] = (c < C && p < P) ? ids[p] : -1;
    rank[c] = 0;
  }
#pragma unroll
  for (int c = 0; c < kSmallChunks; ++c) {
    if (c >= C) break;
    for (int i = tid; i < kWaves * E; i += kChunk) wave_cnt[i / E][i % E] = 0;
    __syncthreads();
    int e = ec[c];
    if (e >= E) {      // precondition violation: flag it, treat as masked
      s_bad = 1;
      e = -1;
      ec[c] = -1;
    }
    const bool valid = e >= 0;
    const uint64_t valid_mask = __ballot(valid);
    uint64_t match = valid ? valid_mask : 0ull;
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      match &= bit ? m : ~m;
    }
    const uint64_t lower = (1ull << lane) - 1ull;
    const int rank_in_wave = __popcll(match & lower);
    const int count_in_wave = __popcll(match);
    if (valid && rank_in_wave == count_in_wave - 1) {
      wave_cnt[wave][e] = static_cast<uint16_t>(count_in_wave);
    }
    __syncthreads();
    if (valid) {
      int r = rank_in_wave;
      for (int w2 = 0; w2 < wave; ++w2) r += wave_cnt[w2][e];
      rank[c] = r;
    }
    for (int x = tid; x < E; x += kChunk) {
      int sum = 0;
#pragma unroll
      for (int w2 = 0; w2 < kWaves; ++w2) sum += wave_cnt[w2][x];
      s_cnt[c][x] = sum;
    }
    __syncthreads();   // wave_cnt is cleared for the next chunk
  }
  if (tid == 0) status[0] = s_bad;
  int cnt = 0;
  if (tid < E) {
    for (int c = 0; c < C; ++c) {
      const int v = s_cnt[c][tid];
      s_cnt[c][tid] = cnt;
      cnt += v;
    }
  }
  const int off = scan_experts(cnt, E, BM, num_blocks, s_wave, group_sizes, group_offsets,
                               group_padded_offsets, block_expert, active_blocks, active_count);
  if (tid < E) s_off[tid] = off;
  __syncthreads();
#pragma unroll
  for (int c = 0; c < kSmallChunks; ++c) {
    if (c >= C) break;
    const int64_t p = static_cast<int64_t>(c) * kChunk + tid;
    if (p >= P) break;
    const float wv = w ? w[p] : 1.0f;
    w_copy[p] = wv;
    const int e = ec[c];
    if (e < 0) {
      pos_out[p] = -1;
      continue;
    }
    const int i = s_off[e] + s_cnt[c][e] + rank[c];
    sorted_pair[i] = static_cast<int32_t>(p);
    sorted_token[i] = static_cast<int32_t>(p / K);
    sorted_weight[i] = wv;
    pos_out[p] = i;
  }
}

}  // namespace

hipError_t launch_dispatch(const int32_t* topk_ids, const float* topk_weights,
                           const moe_tables& t, hipStream_t stream) {
  const int64_t P = static_cast<int64_t>(t.T) * t.K;
  int nbits = 0;
  while ((1 << nbits) < t.E) ++nbits;
  if (t.num_chunks <= kSmallUpTo) {
    hipLaunchKernelGGL(dispatch_small_kernel, dim3(1), dim3(kChunk), 0, stream, topk_ids,
                       topk_weights, P, t.K, t.E, nbits, t.num_chunks, t.block_m, t.num_blocks,
                       t.group_sizes, t.group_offsets, t.group_padded_offsets, t.block_expert,
                       t.status, t.active_blocks, t.active_count, t.sorted_pair, t.sorted_token,
                       t.sorted_weight, t.token_topk_to_pos, t.topk_weights);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(dispatch_count_kernel, dim3(t.num_chunks), dim3(kChunk), 0, stream,
                     topk_ids, P, t.E, nbits, t.chunk_counts, t.pair_rank, t.chunk_flags);
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(1024), 0, stream, t.chunk_counts,
                     t.chunk_flags, t.num_chunks, t.E, t.block_m, t.num_blocks, t.group_sizes,
                     t.group_offsets, t.group_padded_offsets, t.block_expert, t.status,
                     t.active_blocks, t.active_count);
  hipLaunchKernelGGL(dispatch_place_kernel, dim3(t.num_chunks), dim3(kChunk), 0, stream,
                     topk_ids, topk_weights, P, t.K, t.E, t.chunk_counts, t.group_offsets,
                     t.pair_rank, t.sorted_pair, t.sorted_token, t.sorted_weight,
                     t.token_topk_to_pos, t.topk_weights);
  return hipGetLastError();
}

}  // namespace moe
