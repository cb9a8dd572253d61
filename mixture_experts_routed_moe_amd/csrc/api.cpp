// C-ABI layer of libmoe_routed: argument validation, table/workspace layout
// and launches. Every check runs on the host before anything is launched.

#include <hip/hip_runtime_api.h>

#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <string>

#include "launch.hpp"
#include "moe_routed.h"

namespace {

thread_local std::string g_last_error;

constexpr size_t kAlign = 256;
constexpr int kDispatchChunk = 1024;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

moe_status fail(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

moe_status ok() {
  g_last_error.clear();
  return MOE_OK;
}

}  // namespace

namespace moe {

moe_status set_error(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

}  // namespace moe

namespace {

bool block_m_ok(int bm) { return bm == 16 || bm == 32 || bm == 64 || bm == 128 || bm == 256; }

bool is_16bit(int dt) { return dt == MOE_F16 || dt == MOE_BF16; }

bool is_float(int dt) { return is_16bit(dt) || dt == MOE_F32; }

size_t dtype_bytes(int dt) { return dt == MOE_F32 ? 4 : (dt == MOE_FP8_E4M3 ? 1 : 2); }

moe_status check_table_sizes(int T, int K, int E, int block_m) {
  if (T < 1) return fail(MOE_ERR_SHAPE, "T must be >= 1 (got %d)", T);
  if (K < 1 || K > 64) return fail(MOE_ERR_SHAPE, "K must be in [1, 64] (got %d)", K);
  if (E < 1 || E > 1024) return fail(MOE_ERR_SHAPE, "E must be in [1, 1024] (got %d)", E);
  if (!block_m_ok(block_m)) {
    return fail(MOE_ERR_UNSUPPORTED, "block_m must be one of 16, 32, 64, 128, 256 (got %d)",
                block_m);
  }
  const int64_t P = static_cast<int64_t>(T) * K;
  const int64_t nb = (P + block_m - 1) / block_m + E;
  if (P >= (int64_t{1} << 31) || nb * block_m >= (int64_t{1} << 31)) {
    return fail(MOE_ERR_SHAPE, "T*K too large (%lld pairs)", static_cast<long long>(P));
  }
  return MOE_OK;
}

struct TableLayout {
  size_t group_sizes, group_offsets, group_padded_offsets, block_expert, sorted_pair,
      sorted_token, sorted_weight, token_topk_to_pos, topk_weights, status, active_blocks,
      active_count, chunk_counts, chunk_flags, pair_rank, total;
  int num_blocks, num_chunks;
};

TableLayout table_layout(int T, int K, int E, int block_m) {
  TableLayout L{};
  const size_t P = static_cast<size_t>(T) * K;
  L.num_blocks = static_cast<int>((P + block_m - 1) / block_m + E);
  L.num_chunks = static_cast<int>((P + kDispatchChunk - 1) / kDispatchChunk);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L.group_sizes = take(4 * static_cast<size_t>(E));
  L.group_offsets = take(4 * static_cast<size_t>(E));
  L.group_padded_offsets = take(4 * static_cast<size_t>(E));
  L.block_expert = take(4 * static_cast<size_t>(L.num_blocks));
  L.sorted_pair = take(4 * P);
  L.sorted_token = take(4 * P);
  L.sorted_weight = take(4 * P);
  L.token_topk_to_pos = take(4 * P);
  L.topk_weights = take(4 * P);
  L.status = take(4);
  L.active_blocks = take(4 * static_cast<size_t>(L.num_blocks));
  L.active_count = take(4);
  L.chunk_counts = take(4 * static_cast<size_t>(L.num_chunks) * E);
  L.chunk_flags = take(4 * static_cast<size_t>(L.num_chunks));
  L.pair_rank = take(4 * P);
  L.total = off;
  return L;
}

bool tables_bound(const moe_tables* t) {
  return t && t->group_sizes && t->group_offsets && t->group_padded_offsets &&
         t->block_expert && t->sorted_pair && t->sorted_token && t->sorted_weight &&
         t->token_topk_to_pos && t->topk_weights && t->status && t->active_blocks &&
         t->active_count && t->chunk_counts &&
         t->chunk_flags && t->pair_rank;
}

moe_status hip_status(hipError_t err, const char* what) {
  if (err != hipSuccess) {
    return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
  }
  return ok();
}

moe_status check_expert_shapes(const moe_tables* t, int H, int D, int dtype) {
  if (!tables_bound(t)) return fail(MOE_ERR_NULL, "tables are NULL or not bound");
  if (!is_float(dtype)) {
    return fail(MOE_ERR_DTYPE, "expert GEMMs take MOE_F16, MOE_BF16 or MOE_F32 (got dtype %d)",
                dtype);
  }
  if (H <= 0 || H % 256 != 0) return fail(MOE_ERR_SHAPE, "H must be a positive multiple of 256 (got %d)", H);
  if (D <= 0 || D % 128 != 0) return fail(MOE_ERR_SHAPE, "D must be a positive multiple of 128 (got %d)", D);
  return MOE_OK;
}

// W4A8 reductions: 16 x the dot product must fit in int32 (|a| <= 128,
// |16 q| <= 128 per term).
constexpr int kW4MaxK = 131072;

moe_status check_w4a8_shapes(const moe_tables* t, int H, int D, int dtype) {
  moe_status s = check_expert_shapes(t, H, D, dtype);
  if (s != MOE_OK) return s;
  if (!is_16bit(dtype)) return fail(MOE_ERR_DTYPE, "W4A8 experts take MOE_F16 or MOE_BF16 activations");
  if (D % 256 != 0) return fail(MOE_ERR_SHAPE, "W4A8 experts need D a multiple of 256 (got %d)", D);
  if (H > kW4MaxK || D > kW4MaxK) return fail(MOE_ERR_SHAPE, "W4A8 reductions are limited to %d", kW4MaxK);
  return MOE_OK;
}

// Workspace of the W4A8 forward: the 16-bit forward's h and expert_out, then
// xq [T, H] int8, sx [T], hq [P, D] int8, sh [P] (fp32), each 256-aligned.
struct W4Layout {
  size_t xq, sx, hq, sh, total;
};

W4Layout w4_layout(int T, int K, int H, int D, size_t base) {
  const size_t P = static_cast<size_t>(T) * K;
  W4Layout L;
  L.xq = base;
  L.sx = L.xq + align_up(static_cast<size_t>(T) * H);
  L.hq = L.sx + align_up(static_cast<size_t>(T) * 4);
  L.sh = L.hq + align_up(P * D);
  L.total = L.sh + align_up(P * 4);
  return L;
}

moe_status check_mx_shapes(const moe_tables* t, int H, int D, int dtype) {
  moe_status s = check_expert_shapes(t, H, D, dtype);
  if (s != MOE_OK) return s;
  if (!is_16bit(dtype)) return fail(MOE_ERR_DTYPE, "MX experts take MOE_F16 or MOE_BF16 activations");
  if (D % 256 != 0) return fail(MOE_ERR_SHAPE, "MX experts need D a multiple of 256 (got %d)", D);
  return MOE_OK;
}

// Workspace of the MX forward: the 16-bit forward's h and expert_out, then
// xq [T, H] E4M3, xs [T, H/32] E8M0, hq [P, D], hs [P, D/32], each 256-aligned.
struct MxLayout {
  size_t xq, xs, hq, hs, total;
};

MxLayout mx_layout(int T, int K, int H, int D, size_t base) {
  const size_t P = static_cast<size_t>(T) * K;
  MxLayout L;
  L.xq = base;
  L.xs = L.xq + align_up(static_cast<size_t>(T) * H);
  L.hq = L.xs + align_up(static_cast<size_t>(T) * (H / 32));
  L.hs = L.hq + align_up(P * D);
  L.total = L.hs + align_up(P * (D / 32));
  return L;
}

size_t ws_h_bytes(int T, int K, int D, int dtype) {
  return static_cast<size_t>(T) * K * D * dtype_bytes(dtype);
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_NULL: return "MOE_ERR_NULL";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE";
    case MOE_ERR_DTYPE: return "MOE_ERR_DTYPE";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

size_t moe_tables_bytes(int T, int K, int E, int block_m) {
  if (check_table_sizes(T, K, E, block_m) != MOE_OK) return 0;
  return table_layout(T, K, E, block_m).total;
}

moe_status moe_tables_bind(moe_tables* tables, void* buffer, size_t bytes, int T, int K, int E,
                           int block_m) {
  if (!tables || !buffer) return fail(MOE_ERR_NULL, "tables and buffer must not be NULL");
  const moe_status s = check_table_sizes(T, K, E, block_m);
  if (s != MOE_OK) return s;
  if (reinterpret_cast<uintptr_t>(buffer) % kAlign != 0) {
    return fail(MOE_ERR_WORKSPACE, "table buffer must be 256-byte aligned");
  }
  const TableLayout L = table_layout(T, K, E, block_m);
  if (bytes < L.total) {
    return fail(MOE_ERR_WORKSPACE, "table buffer has %zu bytes, needs %zu", bytes, L.total);
  }
  char* b = static_cast<char*>(buffer);
  tables->T = T;
  tables->K = K;
  tables->E = E;
  tables->block_m = block_m;
  tables->num_blocks = L.num_blocks;
  tables->num_chunks = L.num_chunks;
  tables->group_sizes = reinterpret_cast<int32_t*>(b + L.group_sizes);
  tables->group_offsets = reinterpret_cast<int32_t*>(b + L.group_offsets);
  tables->group_padded_offsets = reinterpret_cast<int32_t*>(b + L.group_padded_offsets);
  tables->block_expert = reinterpret_cast<int32_t*>(b + L.block_expert);
  tables->sorted_pair = reinterpret_cast<int32_t*>(b + L.sorted_pair);
  tables->sorted_token = reinterpret_cast<int32_t*>(b + L.sorted_token);
  tables->sorted_weight = reinterpret_cast<float*>(b + L.sorted_weight);
  tables->token_topk_to_pos = reinterpret_cast<int32_t*>(b + L.token_topk_to_pos);
  tables->topk_weights = reinterpret_cast<float*>(b + L.topk_weights);
  tables->status = reinterpret_cast<int32_t*>(b + L.status);
  tables->active_blocks = reinterpret_cast<int32_t*>(b + L.active_blocks);
  tables->active_count = reinterpret_cast<int32_t*>(b + L.active_count);
  tables->chunk_counts = reinterpret_cast<int32_t*>(b + L.chunk_counts);
  tables->chunk_flags = reinterpret_cast<int32_t*>(b + L.chunk_flags);
  tables->pair_rank = reinterpret_cast<int32_t*>(b + L.pair_rank);
  return ok();
}

moe_status moe_gate(const void* x, const float* w_router, const float* bias, int T, int H, int E,
                    int K, int renorm, int dtype, float* logits, int32_t* topk_ids,
                    float* topk_weights, void* stream) {
  if (!x || !w_router || !logits || !topk_ids || !topk_weights) {
    return fail(MOE_ERR_NULL, "x, w_router, logits, topk_ids and topk_weights must not be NULL");
  }
  if (T < 0) return fail(MOE_ERR_SHAPE, "T must be >= 0 (got %d)", T);
  if (H <= 0 || H % 64 != 0) {
    return fail(MOE_ERR_SHAPE, "H must be a positive multiple of 64 (got %d)", H);
  }
  if (E < 1 || E > 1024) return fail(MOE_ERR_SHAPE, "E must be in [1, 1024] (got %d)", E);
  if (K < 1 || K > 64 || K > E) {
    return fail(MOE_ERR_SHAPE, "K must be in [1, min(E, 64)] (got K=%d, E=%d)", K, E);
  }
  if (!is_float(dtype)) return fail(MOE_ERR_DTYPE, "dtype must be MOE_F16, MOE_BF16 or MOE_F32");
  if (T == 0) return ok();
  return hip_status(moe::launch_gate(x, w_router, bias, T, H, E, K, renorm, dtype, logits,
                                     topk_ids, topk_weights, static_cast<hipStream_t>(stream)),
                    "moe_gate launch");
}

moe_status moe_dispatch(const int32_t* topk_ids, const float* topk_weights, moe_tables* tables,
                        void* stream) {
  if (!topk_ids) return fail(MOE_ERR_NULL, "topk_ids must not be NULL");
  if (!tables_bound(tables)) return fail(MOE_ERR_NULL, "tables are NULL or not bound");
  const moe_status s = check_table_sizes(tables->T, tables->K, tables->E, tables->block_m);
  if (s != MOE_OK) return s;
  return hip_status(moe::launch_dispatch(topk_ids, topk_weights, *tables,
                                         static_cast<hipStream_t>(stream)),
                    "moe_dispatch launch");
}

moe_status moe_expert_gate_up(const void* x, const void* w_gate, const void* w_up,
                              const moe_tables* tables, int H, int D, int dtype, void* h,
                              void* stream) {
  if (!x || !w_gate || !w_up || !h) return fail(MOE_ERR_NULL, "x, w_gate, w_up and h must not be NULL");
  moe_status s = check_expert_shapes(tables, H, D, dtype);
  if (s != MOE_OK) return s;
  moe::GemmProblem p{x, w_gate, w_up, h, D, H, dtype};
  return hip_status(moe::launch_gate_up(p, *tables, static_cast<hipStream_t>(stream)),
                    "moe_expert_gate_up launch");
}

moe_status moe_expert_down(const void* h, const void* w_down, const moe_tables* tables, int H,
                           int D, int dtype, void* expert_out, void* stream) {
  if (!h || !w_down || !expert_out) return fail(MOE_ERR_NULL, "h, w_down and expert_out must not be NULL");
  moe_status s = check_expert_shapes(tables, H, D, dtype);
  if (s != MOE_OK) return s;
  moe::GemmProblem p{h, w_down, nullptr, expert_out, H, D, dtype};
  return hip_status(moe::launch_down(p, *tables, static_cast<hipStream_t>(stream)),
                    "moe_expert_down launch");
}

moe_status moe_expert_down_weighted(const void* h, const void* w_down, const moe_tables* tables,
                                    int H, int D, int dtype, void* expert_out, void* stream) {
  if (!h || !w_down || !expert_out) return fail(MOE_ERR_NULL, "h, w_down and expert_out must not be NULL");
  moe_status s = check_expert_shapes(tables, H, D, dtype);
  if (s != MOE_OK) return s;
  moe::GemmProblem p{h, w_down, nullptr, expert_out, H, D, dtype};
  p.row_w = tables->sorted_weight;
  return hip_status(moe::launch_down(p, *tables, static_cast<hipStream_t>(stream)),
                    "moe_expert_down_weighted launch");
}

size_t moe_forward_workspace_expert_out_offset(int T, int K, int H, int D, int dtype) {
  if (T < 1 || K < 1 || H <= 0 || D <= 0 || !is_float(dtype)) return 0;
  return align_up(ws_h_bytes(T, K, D, dtype));
}

size_t moe_forward_workspace_bytes(int T, int K, int H, int D, int dtype) {
  const size_t off = moe_forward_workspace_expert_out_offset(T, K, H, D, dtype);
  if (off == 0) return 0;
  return off + align_up(static_cast<size_t>(T) * K * H * dtype_bytes(dtype));
}

// The 16-bit / fp32 forward; weighted_down selects where the routing weight
// is applied (the down epilogue, then an unweighted sum, or the reduce).
static moe_status routed_forward(const void* x, const void* w_gate, const void* w_up,
                                 const void* w_down, const moe_tables* tables, int H, int D,
                                 int dtype, void* workspace, size_t workspace_bytes, void* y,
                                 void* stream, bool weighted_down) {
  if (!x || !w_gate || !w_up || !w_down || !workspace || !y) {
    return fail(MOE_ERR_NULL, "x, w_gate, w_up, w_down, workspace and y must not be NULL");
  }
  moe_status s = check_expert_shapes(tables, H, D, dtype);
  if (s != MOE_OK) return s;
  const size_t need = moe_forward_workspace_bytes(tables->T, tables->K, H, D, dtype);
  if (workspace_bytes < need) {
    return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  }
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) {
    return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  char* ws = static_cast<char*>(workspace);
  void* hbuf = ws;
  void* eo = ws + moe_forward_workspace_expert_out_offset(tables->T, tables->K, H, D, dtype);
  hipStream_t st = static_cast<hipStream_t>(stream);
  moe::GemmProblem up{x, w_gate, w_up, hbuf, D, H, dtype};
  hipError_t err = moe::launch_gate_up(up, *tables, st);
  if (err != hipSuccess) return hip_status(err, "moe_routed_forward gate/up launch");
  moe::GemmProblem down{hbuf, w_down, nullptr, eo, H, D, dtype};
  if (weighted_down) down.row_w = tables->sorted_weight;
  err = moe::launch_down(down, *tables, st);
  if (err != hipSuccess) return hip_status(err, "moe_routed_forward down launch");
  const int64_t P = static_cast<int64_t>(tables->T) * tables->K;
  err = moe::launch_reduce(eo, P, tables->token_topk_to_pos,
                           weighted_down ? nullptr : tables->topk_weights, nullptr, nullptr,
                           tables->T, tables->K, H, dtype, dtype, y, st);
  return hip_status(err, "moe_routed_forward reduce launch");
}

moe_status moe_routed_forward(const void* x, const void* w_gate, const void* w_up,
                              const void* w_down, const moe_tables* tables, int H, int D,
                              int dtype, void* workspace, size_t workspace_bytes, void* y,
                              void* stream) {
  return routed_forward(x, w_gate, w_up, w_down, tables, H, D, dtype, workspace,
                        workspace_bytes, y, stream, false);
}

moe_status moe_routed_forward_weighted(const void* x, const void* w_gate, const void* w_up,
                                       const void* w_down, const moe_tables* tables, int H,
                                       int D, int dtype, void* workspace,
                                       size_t workspace_bytes, void* y, void* stream) {
  return routed_forward(x, w_gate, w_up, w_down, tables, H, D, dtype, workspace,
                        workspace_bytes, y, stream, true);
}

static moe_status check_fused(const moe_tables* tables, int H, int D, int dtype) {
  moe_status s = check_expert_shapes(tables, H, D, dtype);
  if (s != MOE_OK) return s;
  if (!is_16bit(dtype)) return fail(MOE_ERR_DTYPE, "the fused expert kernel takes MOE_F16 or MOE_BF16");
  if (tables->block_m > 32) {
    return fail(MOE_ERR_UNSUPPORTED, "the fused expert kernel needs tables with block_m <= 32 (got %d)",
                tables->block_m);
  }
  if (D > moe::fused_max_d_expert()) {
    return fail(MOE_ERR_UNSUPPORTED, "the fused expert kernel holds h in LDS: D <= %d (got %d)",
                moe::fused_max_d_expert(), D);
  }
  return MOE_OK;
}

moe_status moe_expert_fused(const void* x, const void* w_gate, const void* w_up,
                            const void* w_down, const moe_tables* tables, int H, int D,
                            int dtype, void* expert_out, void* stream) {
  if (!x || !w_gate || !w_up || !w_down || !expert_out) {
    return fail(MOE_ERR_NULL, "x, w_gate, w_up, w_down and expert_out must not be NULL");
  }
  moe_status s = check_fused(tables, H, D, dtype);
  if (s != MOE_OK) return s;
  moe::GemmProblem up{x, w_gate, w_up, nullptr, D, H, dtype};
  moe::GemmProblem down{nullptr, w_down, nullptr, expert_out, H, D, dtype};
  return hip_status(moe::launch_fused_expert(up, down, *tables, static_cast<hipStream_t>(stream)),
                    "moe_expert_fused launch");
}

size_t moe_fused_workspace_bytes(int T, int K, int H, int dtype) {
  if (T < 1 || K < 1 || H <= 0 || !is_float(dtype)) return 0;
  return align_up(static_cast<size_t>(T) * K * H * dtype_bytes(dtype));
}

moe_status moe_routed_forward_fused(const void* x, const void* w_gate, const void* w_up,
                                    const void* w_down, const moe_tables* tables, int H, int D,
                                    int dtype, void* workspace, size_t workspace_bytes, void* y,
                                    void* stream) {
  if (!x || !w_gate || !w_up || !w_down || !workspace || !y) {
    return fail(MOE_ERR_NULL, "x, w_gate, w_up, w_down, workspace and y must not be NULL");
  }
  moe_status s = check_fused(tables, H, D, dtype);
  if (s != MOE_OK) return s;
  const size_t need = moe_fused_workspace_bytes(tables->T, tables->K, H, dtype);
  if (workspace_bytes < need) {
    return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  }
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) {
    return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  moe::GemmProblem up{x, w_gate, w_up, nullptr, D, H, dtype};
  moe::GemmProblem down{nullptr, w_down, nullptr, workspace, H, D, dtype};
  hipError_t err = moe::launch_fused_expert(up, down, *tables, st);
  if (err != hipSuccess) return hip_status(err, "moe_routed_forward_fused expert launch");
  const int64_t P = static_cast<int64_t>(tables->T) * tables->K;
  err = moe::launch_reduce(workspace, P, tables->token_topk_to_pos, tables->topk_weights, nullptr,
                           nullptr, tables->T, tables->K, H, dtype, dtype, y, st);
  return hip_status(err, "moe_routed_forward_fused reduce launch");
}

moe_status moe_quantize_fp8_rows(const void* w, int64_t rows, int cols, int dtype, uint8_t* q,
                                 float* scales, void* stream) {
  if (!w || !q || !scales) return fail(MOE_ERR_NULL, "w, q and scales must not be NULL");
  if (rows < 0 || cols <= 0) return fail(MOE_ERR_SHAPE, "rows must be >= 0 and cols > 0");
  if (rows > (int64_t{1} << 33)) return fail(MOE_ERR_SHAPE, "too many rows for one launch");
  if (!is_float(dtype)) return fail(MOE_ERR_DTYPE, "dtype must be MOE_F16, MOE_BF16 or MOE_F32");
  if (rows == 0) return ok();
  return hip_status(moe::launch_quantize_fp8_rows(w, rows, cols, dtype, q, scales,
                                                  static_cast<hipStream_t>(stream)),
                    "moe_quantize_fp8_rows launch");
}

moe_status moe_expert_gate_up_w8(const void* x, const uint8_t* w_gate, const uint8_t* w_up,
                                 const float* s_gate, const float* s_up, const moe_tables* tables,
                                 int H, int D, int dtype, void* h, void* stream) {
  if (!x || !w_gate || !w_up || !s_gate || !s_up || !h) {
    return fail(MOE_ERR_NULL, "x, w_gate, w_up, s_gate, s_up and h must not be NULL");
  }
  moe_status s = check_expert_shapes(tables, H, D, dtype);
  if (s != MOE_OK) return s;
  if (!is_16bit(dtype)) return fail(MOE_ERR_DTYPE, "FP8 weights take MOE_F16 or MOE_BF16 activations");
  moe::GemmProblem p{x, w_gate, w_up, h, D, H, dtype, s_gate, s_up};
  return hip_status(moe::launch_gate_up_w8(p, *tables, static_cast<hipStream_t>(stream)),
                    "moe_expert_gate_up_w8 launch");
}

moe_status moe_expert_down_w8(const void* h, const uint8_t* w_down, const float* s_down,
                              const moe_tables* tables, int H, int D, int dtype, void* expert_out,
                              void* stream) {
  if (!h || !w_down || !s_down || !expert_out) {
    return fail(MOE_ERR_NULL, "h, w_down, s_down and expert_out must not be NULL");
  }
  moe_status s = check_expert_shapes(tables, H, D, dtype);
  if (s != MOE_OK) return s;
  if (!is_16bit(dtype)) return fail(MOE_ERR_DTYPE, "FP8 weights take MOE_F16 or MOE_BF16 activations");
  moe::GemmProblem p{h, w_down, nullptr, expert_out, H, D, dtype, s_down, nullptr};
  return hip_status(moe::launch_down_w8(p, *tables, static_cast<hipStream_t>(stream)),
                    "moe_expert_down_w8 launch");
}

moe_status moe_routed_forward_w8(const void* x, const uint8_t* w_gate, const uint8_t* w_up,
                                 const uint8_t* w_down, const float* s_gate, const float* s_up,
                                 const float* s_down, const moe_tables* tables, int H, int D,
                                 int dtype, void* workspace, size_t workspace_bytes, void* y,
                                 void* stream) {
  if (!x || !w_gate || !w_up || !w_down || !s_gate || !s_up || !s_down || !workspace || !y) {
    return fail(MOE_ERR_NULL,
                "x, the weights, their scales, workspace and y must not be NULL");
  }
  moe_status s = check_expert_shapes(tables, H, D, dtype);
  if (s != MOE_OK) return s;
  if (!is_16bit(dtype)) return fail(MOE_ERR_DTYPE, "FP8 weights take MOE_F16 or MOE_BF16 activations");
  const size_t need = moe_forward_workspace_bytes(tables->T, tables->K, H, D, dtype);
  if (workspace_bytes < need) {
    return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  }
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) {
    return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  char* ws = static_cast<char*>(workspace);
  void* hbuf = ws;
  void* eo = ws + moe_forward_workspace_expert_out_offset(tables->T, tables->K, H, D, dtype);
  hipStream_t st = static_cast<hipStream_t>(stream);
  moe::GemmProblem up{x, w_gate, w_up, hbuf, D, H, dtype, s_gate, s_up};
  hipError_t err = moe::launch_gate_up_w8(up, *tables, st);
  if (err != hipSuccess) return hip_status(err, "moe_routed_forward_w8 gate/up launch");
  moe::GemmProblem down{hbuf, w_down, nullptr, eo, H, D, dtype, s_down, nullptr};
  err = moe::launch_down_w8(down, *tables, st);
  if (err != hipSuccess) return hip_status(err, "moe_routed_forward_w8 down launch");
  const int64_t P = static_cast<int64_t>(tables->T) * tables->K;
  err = moe::launch_reduce(eo, P, tables->token_topk_to_pos, tables->topk_weights, nullptr,
                           nullptr, tables->T, tables->K, H, dtype, dtype, y, st);
  return hip_status(err, "moe_routed_forward_w8 reduce launch");
}

moe_status moe_quantize_int8_rows(const void* a, int64_t rows, int cols, int dtype, int8_t* q,
                                  float* scales, void* stream) {
  if (!a || !q || !scales) return fail(MOE_ERR_NULL, "a, q and scales must not be NULL");
  if (rows < 0 || cols <= 0) return fail(MOE_ERR_SHAPE, "rows must be >= 0 and cols > 0");
  if (rows > (int64_t{1} << 33)) return fail(MOE_ERR_SHAPE, "too many rows for one launch");
  if (!is_float(dtype)) return fail(MOE_ERR_DTYPE, "dtype must be MOE_F16, MOE_BF16 or MOE_F32");
  if (rows == 0) return ok();
  return hip_status(moe::launch_quantize_int8_rows(a, rows, cols, dtype, q, scales,
                                                   static_cast<hipStream_t>(stream)),
                    "moe_quantize_int8_rows launch");
}

moe_status moe_quantize_int4_rows(const void* w, int64_t rows, int cols, int dtype,
                                  uint8_t* packed, float* scales, void* stream) {
  if (!w || !packed || !scales) return fail(MOE_ERR_NULL, "w, packed and scales must not be NULL");
  if (rows < 0 || cols <= 0 || cols % 2 != 0) {
    return fail(MOE_ERR_SHAPE, "rows must be >= 0 and cols a positive even number");
  }
  if (rows > (int64_t{1} << 33)) return fail(MOE_ERR_SHAPE, "too many rows for one launch");
  if (!is_float(dtype)) return fail(MOE_ERR_DTYPE, "dtype must be MOE_F16, MOE_BF16 or MOE_F32");
  if (rows == 0) return ok();
  return hip_status(moe::launch_quantize_int4_rows(w, rows, cols, dtype, packed, scales,
                                                   static_cast<hipStream_t>(stream)),
                    "moe_quantize_int4_rows launch");
}

moe_status moe_w4a8_gemm(const int8_t* A, const uint8_t* B, int M, int N, int K, int32_t* Ct,
                         void* stream) {
  if (!A || !B || !Ct) return fail(MOE_ERR_NULL, "A, B and Ct must not be NULL");
  if (M < 1) return fail(MOE_ERR_SHAPE, "M must be >= 1 (got %d)", M);
  if (N <= 0 || N % 256 != 0) return fail(MOE_ERR_SHAPE, "N must be a positive multiple of 256 (got %d)", N);
  if (K <= 0 || K % 256 != 0 || K > kW4MaxK) {
    return fail(MOE_ERR_SHAPE, "K must be a positive multiple of 256, at most %d (got %d)", kW4MaxK, K);
  }
  if (static_cast<int64_t>(N) * M >= (int64_t{1} << 31)) return fail(MOE_ERR_SHAPE, "N * M too large");
  return hip_status(moe::launch_w4a8_gemm(A, B, M, N, K, Ct, static_cast<hipStream_t>(stream)),
                    "moe_w4a8_gemm launch");
}

moe_status moe_expert_gate_up_w4a8(const int8_t* xq, const float* sx, const uint8_t* w_gate,
                                   const uint8_t* w_up, const float* s_gate, const float* s_up,
                                   const moe_tables* tables, int H, int D, int dtype, void* h,
                                   void* stream) {
  if (!xq || !sx || !w_gate || !w_up || !s_gate || !s_up || !h) {
    return fail(MOE_ERR_NULL, "xq, sx, w_gate, w_up, s_gate, s_up and h must not be NULL");
  }
  moe_status s = check_w4a8_shapes(tables, H, D, dtype);
  if (s != MOE_OK) return s;
  moe::W4GemmProblem p{xq, sx, w_gate, w_up, s_gate, s_up, h, D, H, dtype};
  return hip_status(moe::launch_gate_up_w4a8(p, *tables, static_cast<hipStream_t>(stream)),
                    "moe_expert_gate_up_w4a8 launch");
}

moe_status moe_expert_down_w4a8(const int8_t* hq, const float* sh, const uint8_t* w_down,
                                const float* s_down, const moe_tables* tables, int H, int D,
                                int dtype, void* expert_out, void* stream) {
  if (!hq || !sh || !w_down || !s_down || !expert_out) {
    return fail(MOE_ERR_NULL, "hq, sh, w_down, s_down and expert_out must not be NULL");
  }
  moe_status s = check_w4a8_shapes(tables, H, D, dtype);
  if (s != MOE_OK) return s;
  moe::W4GemmProblem p{hq, sh, w_down, nullptr, s_down, nullptr, expert_out, H, D, dtype};
  return hip_status(moe::launch_down_w4a8(p, *tables, static_cast<hipStream_t>(stream)),
                    "moe_expert_down_w4a8 launch");
}

size_t moe_forward_w4a8_workspace_bytes(int T, int K, int H, int D, int dtype) {
  const size_t base = moe_forward_workspace_bytes(T, K, H, D, dtype);
  if (base == 0) return 0;
  const W4Layout L = w4_layout(T, K, H, D, base);
  return L.total;
}

moe_status moe_routed_forward_w4a8(const void* x, const uint8_t* w_gate, const uint8_t* w_up,
                                   const uint8_t* w_down, const float* s_gate, const float* s_up,
                                   const float* s_down, const moe_tables* tables, int H, int D,
                                   int dtype, void* workspace, size_t workspace_bytes, void* y,
                                   void* stream) {
  if (!x || !w_gate || !w_up || !w_down || !s_gate || !s_up || !s_down || !workspace || !y) {
    return fail(MOE_ERR_NULL,
                "x, the weights, their scales, workspace and y must not be NULL");
  }
  moe_status s = check_w4a8_shapes(tables, H, D, dtype);
  if (s != MOE_OK) return s;
  const size_t need = moe_forward_w4a8_workspace_bytes(tables->T, tables->K, H, D, dtype);
  if (workspace_bytes < need) {
    return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  }
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) {
    return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  const int T = tables->T, K = tables->K;
  const int64_t P = static_cast<int64_t>(T) * K;
  char* ws = static_cast<char*>(workspace);
  const W4Layout L = w4_layout(T, K, H, D, moe_forward_workspace_bytes(T, K, H, D, dtype));
  void* hbuf = ws;
  void* eo = ws + moe_forward_workspace_expert_out_offset(T, K, H, D, dtype);
  int8_t* xq = reinterpret_cast<int8_t*>(ws + L.xq);
  float* sx = reinterpret_cast<float*>(ws + L.sx);
  int8_t* hq = reinterpret_cast<int8_t*>(ws + L.hq);
  float* sh = reinterpret_cast<float*>(ws + L.sh);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t err = moe::launch_quantize_int8_rows(x, T, H, dtype, xq, sx, st);
  if (err != hipSuccess) return hip_status(err, "moe_routed_forward_w4a8 x quantisation launch");
  moe::W4GemmProblem up{xq, sx, w_gate, w_up, s_gate, s_up, hbuf, D, H, dtype};
  err = moe::launch_gate_up_w4a8(up, *tables, st);
  if (err != hipSuccess) return hip_status(err, "moe_routed_forward_w4a8 gate/up launch");
  err = moe::launch_quantize_int8_rows(hbuf, P, D, dtype, hq, sh, st);
  if (err != hipSuccess) return hip_status(err, "moe_routed_forward_w4a8 h quantisation launch");
  moe::W4GemmProblem down{hq, sh, w_down, nullptr, s_down, nullptr, eo, H, D, dtype};
  err = moe::launch_down_w4a8(down, *tables, st);
  if (err != hipSuccess) return hip_status(err, "moe_routed_forward_w4a8 down launch");
  err = moe::launch_reduce(eo, P, tables->token_topk_to_pos, tables->topk_weights, nullptr,
                           nullptr, T, K, H, dtype, dtype, y, st);
  return hip_status(err, "moe_routed_forward_w4a8 reduce launch");
}

moe_status check_w8a8_shapes(const moe_tables* t, int H, int D, int dtype) {
  moe_status s = check_expert_shapes(t, H, D, dtype);
  if (s != MOE_OK) return s;
  if (!is_16bit(dtype)) return fail(MOE_ERR_DTYPE, "W8A8 experts take MOE_F16 or MOE_BF16 outputs");
  return MOE_OK;
}

moe_status moe_expert_gate_up_w8a8(const uint8_t* xq, const float* sx, const uint8_t* w_gate,
                                   const uint8_t* w_up, const float* s_gate, const float* s_up,
                                   const moe_tables* tables, int H, int D, int dtype, void* h,
                                   void* stream) {
  if (!xq || !sx || !w_gate || !w_up || !s_gate || !s_up || !h) {
    return fail(MOE_ERR_NULL, "xq, sx, w_gate, w_up, s_gate, s_up and h must not be NULL");
  }
  moe_status s = check_w8a8_shapes(tables, H, D, dtype);
  if (s != MOE_OK) return s;
  if (reinterpret_cast<uintptr_t>(xq) % 16 != 0) return fail(MOE_ERR_SHAPE, "xq must be 16-byte aligned");
  moe::GemmProblem p{xq, w_gate, w_up, h, D, H, dtype, s_gate, s_up};
  p.sa = sx;
  return hip_status(moe::launch_gate_up_w8a8(p, *tables, static_cast<hipStream_t>(stream)),
                    "moe_expert_gate_up_w8a8 launch");
}

moe_status moe_expert_down_w8a8(const uint8_t* hq, const float* sh, const uint8_t* w_down,
                                const float* s_down, const moe_tables* tables, int H, int D,
                                int dtype, void* expert_out, void* stream) {
  if (!hq || !sh || !w_down || !s_down || !expert_out) {
    return fail(MOE_ERR_NULL, "hq, sh, w_down, s_down and expert_out must not be NULL");
  }
  moe_status s = check_w8a8_shapes(tables, H, D, dtype);
  if (s != MOE_OK) return s;
  if (reinterpret_cast<uintptr_t>(hq) % 16 != 0) return fail(MOE_ERR_SHAPE, "hq must be 16-byte aligned");
  moe::GemmProblem p{hq, w_down, nullptr, expert_out, H, D, dtype, s_down, nullptr};
  p.sa = sh;
  return hip_status(moe::launch_down_w8a8(p, *tables, static_cast<hipStream_t>(stream)),
                    "moe_expert_down_w8a8 launch");
}

size_t moe_forward_w8a8_workspace_bytes(int T, int K, int H, int D, int dtype) {
  const size_t base = moe_forward_workspace_bytes(T, K, H, D, dtype);
  if (base == 0) return 0;
  return w4_layout(T, K, H, D, base).total;   // one-byte codes + fp32 row scales
}

moe_status moe_routed_forward_w8a8(const void* x, const uint8_t* w_gate, const uint8_t* w_up,
                                   const uint8_t* w_down, const float* s_gate, const float* s_up,
                                   const float* s_down, const moe_tables* tables, int H, int D,
                                   int dtype, void* workspace, size_t workspace_bytes, void* y,
                                   void* stream) {
  if (!x || !w_gate || !w_up || !w_down || !s_gate || !s_up || !s_down || !workspace || !y) {
    return fail(MOE_ERR_NULL,
                "x, the weights, their scales, workspace and y must not be NULL");
  }
  moe_status s = check_w8a8_shapes(tables, H, D, dtype);
  if (s != MOE_OK) return s;
  const size_t need = moe_forward_w8a8_workspace_bytes(tables->T, tables->K, H, D, dtype);
  if (workspace_bytes < need) {
    return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  }
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) {
    return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  const int T = tables->T, K = tables->K;
  const int64_t P = static_cast<int64_t>(T) * K;
  char* ws = static_cast<char*>(workspace);
  const W4Layout L = w4_layout(T, K, H, D, moe_forward_workspace_bytes(T, K, H, D, dtype));
  void* hbuf = ws;
  void* eo = ws + moe_forward_workspace_expert_out_offset(T, K, H, D, dtype);
  uint8_t* xq = reinterpret_cast<uint8_t*>(ws + L.xq);
  float* sx = reinterpret_cast<float*>(ws + L.sx);
  uint8_t* hq = reinterpret_cast<uint8_t*>(ws + L.hq);
  float* sh = reinterpret_cast<float*>(ws + L.sh);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t err = moe::launch_quantize_fp8_rows(x, T, H, dtype, xq, sx, st);
  if (err != hipSuccess) return hip_status(err, "moe_routed_forward_w8a8 x quantisation launch");
  moe::GemmProblem up{xq, w_gate, w_up, hbuf, D, H, dtype, s_gate, s_up};
  up.sa = sx;
  err = moe::launch_gate_up_w8a8(up, *tables, st);
  if (err != hipSuccess) return hip_status(err, "moe_routed_forward_w8a8 gate/up launch");
  err = moe::launch_quantize_fp8_rows(hbuf, P, D, dtype, hq, sh, st);
  if (err != hipSuccess) return hip_status(err, "moe_routed_forward_w8a8 h quantisation launch");
  moe::GemmProblem down{hq, w_down, nullptr, eo, H, D, dtype, s_down, nullptr};
  down.sa = sh;
  err = moe::launch_down_w8a8(down, *tables, st);
  if (err != hipSuccess) return hip_status(err, "moe_routed_forward_w8a8 down launch");
  err = moe::launch_reduce(eo, P, tables->token_topk_to_pos, tables->topk_weights, nullptr,
                           nullptr, T, K, H, dtype, dtype, y, st);
  return hip_status(err, "moe_routed_forward_w8a8 reduce launch");
}

moe_status moe_quantize_mx_rows(const void* v, int64_t rows, int cols, int dtype, int fmt,
                                uint8_t* codes, uint8_t* scales, void* stream) {
  if (!v || !codes || !scales) return fail(MOE_ERR_NULL, "v, codes and scales must not be NULL");
  if (rows < 0 || cols <= 0 || cols % 32 != 0) {
    return fail(MOE_ERR_SHAPE, "rows must be >= 0 and cols a positive multiple of 32");
  }
  if (rows > (int64_t{1} << 33)) return fail(MOE_ERR_SHAPE, "too many rows for one launch");
  if (!is_float(dtype)) return fail(MOE_ERR_DTYPE, "dtype must be MOE_F16, MOE_BF16 or MOE_F32");
  if (fmt != MOE_MX_FP8 && fmt != MOE_MX_FP4) {
    return fail(MOE_ERR_DTYPE, "fmt must be MOE_MX_FP8 or MOE_MX_FP4 (got %d)", fmt);
  }
  if (reinterpret_cast<uintptr_t>(codes) % 16 != 0) {
    return fail(MOE_ERR_SHAPE, "codes must be 16-byte aligned");
  }
  if (rows == 0) return ok();
  return hip_status(moe::launch_quantize_mx_rows(v, rows, cols, dtype, fmt, codes, scales,
                                                 static_cast<hipStream_t>(stream)),
                    "moe_quantize_mx_rows launch");
}

moe_status moe_expert_gate_up_mx(const uint8_t* xq, const uint8_t* xs, const uint8_t* w_gate,
                                 const uint8_t* w_up, const uint8_t* s_gate, const uint8_t* s_up,
                                 const moe_tables* tables, int H, int D, int dtype, void* h,
                                 void* stream) {
  if (!xq || !xs || !w_gate || !w_up || !s_gate || !s_up || !h) {
    return fail(MOE_ERR_NULL, "xq, xs, w_gate, w_up, s_gate, s_up and h must not be NULL");
  }
  moe_status s = check_mx_shapes(tables, H, D, dtype);
  if (s != MOE_OK) return s;
  moe::MxGemmProblem p{xq, xs, w_gate, w_up, s_gate, s_up, h, D, H, dtype};
  return hip_status(moe::launch_gate_up_mx(p, *tables, static_cast<hipStream_t>(stream)),
                    "moe_expert_gate_up_mx launch");
}

moe_status moe_expert_down_mx(const uint8_t* hq, const uint8_t* hs, const uint8_t* w_down,
                              const uint8_t* s_down, const moe_tables* tables, int H, int D,
                              int dtype, void* expert_out, void* stream) {
  if (!hq || !hs || !w_down || !s_down || !expert_out) {
    return fail(MOE_ERR_NULL, "hq, hs, w_down, s_down and expert_out must not be NULL");
  }
  moe_status s = check_mx_shapes(tables, H, D, dtype);
  if (s != MOE_OK) return s;
  moe::MxGemmProblem p{hq, hs, w_down, nullptr, s_down, nullptr, expert_out, H, D, dtype};
  return hip_status(moe::launch_down_mx(p, *tables, static_cast<hipStream_t>(stream)),
                    "moe_expert_down_mx launch");
}

size_t moe_forward_mx_workspace_bytes(int T, int K, int H, int D, int dtype) {
  const size_t base = moe_forward_workspace_bytes(T, K, H, D, dtype);
  if (base == 0) return 0;
  return mx_layout(T, K, H, D, base).total;
}

moe_status moe_routed_forward_mx(const void* x, const uint8_t* w_gate, const uint8_t* w_up,
                                 const uint8_t* w_down, const uint8_t* s_gate, const uint8_t* s_up,
                                 const uint8_t* s_down, const moe_tables* tables, int H, int D,
                                 int dtype, void* workspace, size_t workspace_bytes, void* y,
                                 void* stream) {
  if (!x || !w_gate || !w_up || !w_down || !s_gate || !s_up || !s_down || !workspace || !y) {
    return fail(MOE_ERR_NULL,
                "x, the weights, their scales, workspace and y must not be NULL");
  }
  moe_status s = check_mx_shapes(tables, H, D, dtype);
  if (s != MOE_OK) return s;
  const size_t need = moe_forward_mx_workspace_bytes(tables->T, tables->K, H, D, dtype);
  if (workspace_bytes < need) {
    return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  }
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) {
    return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  const int T = tables->T, K = tables->K;
  const int64_t P = static_cast<int64_t>(T) * K;
  char* ws = static_cast<char*>(workspace);
  const MxLayout L = mx_layout(T, K, H, D, moe_forward_workspace_bytes(T, K, H, D, dtype));
  void* hbuf = ws;
  void* eo = ws + moe_forward_workspace_expert_out_offset(T, K, H, D, dtype);
  uint8_t* xq = reinterpret_cast<uint8_t*>(ws + L.xq);
  uint8_t* xs = reinterpret_cast<uint8_t*>(ws + L.xs);
  uint8_t* hq = reinterpret_cast<uint8_t*>(ws + L.hq);
  uint8_t* hs = reinterpret_cast<uint8_t*>(ws + L.hs);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t err = moe::launch_quantize_mx_rows(x, T, H, dtype, MOE_MX_FP8, xq, xs, st);
  if (err != hipSuccess) return hip_status(err, "moe_routed_forward_mx x quantisation launch");
  moe::MxGemmProblem up{xq, xs, w_gate, w_up, s_gate, s_up, hbuf, D, H, dtype};
  err = moe::launch_gate_up_mx(up, *tables, st);
  if (err != hipSuccess) return hip_status(err, "moe_routed_forward_mx gate/up launch");
  err = moe::launch_quantize_mx_rows(hbuf, P, D, dtype, MOE_MX_FP8, hq, hs, st);
  if (err != hipSuccess) return hip_status(err, "moe_routed_forward_mx h quantisation launch");
  moe::MxGemmProblem down{hq, hs, w_down, nullptr, s_down, nullptr, eo, H, D, dtype};
  err = moe::launch_down_mx(down, *tables, st);
  if (err != hipSuccess) return hip_status(err, "moe_routed_forward_mx down launch");
  err = moe::launch_reduce(eo, P, tables->token_topk_to_pos, tables->topk_weights, nullptr,
                           nullptr, T, K, H, dtype, dtype, y, st);
  return hip_status(err, "moe_routed_forward_mx reduce launch");
}

moe_status moe_reduce_fused_scaled(const void* expert_out, int64_t rows,
                                   const int32_t* token_topk_to_pos, const float* topk_weights,
                                   const float* x_sf, const float* sf, int T, int K, int H,
                                   int in_dtype, int out_dtype, void* y, void* stream) {
  if (!expert_out || !token_topk_to_pos || !y) {
    return fail(MOE_ERR_NULL, "expert_out, token_topk_to_pos and y must not be NULL");
  }
  if (rows < 0) return fail(MOE_ERR_SHAPE, "rows must be >= 0");
  if (T < 0) return fail(MOE_ERR_SHAPE, "T must be >= 0 (got %d)", T);
  if (K < 1 || K > 64) return fail(MOE_ERR_SHAPE, "K must be in [1, 64] (got %d)", K);
  if (H <= 0 || H % 256 != 0) {
    return fail(MOE_ERR_SHAPE, "H must be a positive multiple of 256 (got %d)", H);
  }
  if (in_dtype < MOE_F16 || in_dtype > MOE_FP8_E4M3 || out_dtype < MOE_F16 ||
      out_dtype > MOE_FP8_E4M3) {
    return fail(MOE_ERR_DTYPE,
                "dtype codes must be MOE_F16, MOE_BF16, MOE_F32 or MOE_FP8_E4M3");
  }
  if (static_cast<int64_t>(T) * (H / 8) > 0xffffffffLL) {   // work-items of one launch
    return fail(MOE_ERR_SHAPE, "T * H too large for one launch");
  }
  return hip_status(moe::launch_reduce(expert_out, rows, token_topk_to_pos, topk_weights, x_sf,
                                       sf, T, K, H, in_dtype, out_dtype, y,
                                       static_cast<hipStream_t>(stream)),
                    "moe_reduce_fused launch");
}

moe_status moe_reduce_fused(const void* expert_out, int64_t rows,
                            const int32_t* token_topk_to_pos, const float* topk_weights, int T,
                            int K, int H, int in_dtype, int out_dtype, void* y, void* stream) {
  return moe_reduce_fused_scaled(expert_out, rows, token_topk_to_pos, topk_weights, nullptr,
                                 nullptr, T, K, H, in_dtype, out_dtype, y, stream);
}

}  // extern "C"
