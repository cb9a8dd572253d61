// Host-side launchers of the HIP kernels (internal to libmoe_routed).
// Arguments have been validated by the C-ABI layer before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_routed.h"

namespace moe {

// Sets the calling thread's last-error message (printf-style) and returns s.
moe_status set_error(moe_status s, const char* fmt, ...);

hipError_t launch_dispatch(const int32_t* topk_ids, const float* topk_weights,
                           const moe_tables& t, hipStream_t stream);

struct GemmProblem {
  const void* a;         // gate/up: x [T, Kd]; down: h [P, Kd]
  const void* b0;        // gate/up: W_gate [E, N, Kd]; down: W_down [E, N, Kd]
  const void* b1;        // gate/up: W_up; down: unused
  void* c;               // gate/up: h [P, N]; down: expert_out [P, N]
  int n;                 // output columns (D for gate/up, H for down)
  int kd;                // reduction length (H for gate/up, D for down)
  int dtype;             // kF16 / kBF16 / kF32
  const float* s0 = nullptr;   // FP8 weights: fp32 scale per row of b0
  const float* s1 = nullptr;   // FP8 weights: fp32 scale per row of b1
  // down only: fp32 routing weight per output row (the tables'
  // sorted_weight), multiplied into each dot product before the rounding to
  // dtype; nullptr = unweighted rows.
  const float* row_w = nullptr;
  // W8A8 (FP8 activations a with FP8 weights): fp32 scale per activation
  // row -- x by token (gate/up), h by sorted row (down).
  const float* sa = nullptr;
};

hipError_t launch_gate_up(const GemmProblem& p, const moe_tables& t, hipStream_t stream);
// 16-bit weights, blocks of 128 or 256 rows: one kernel that streams blocks
// of <= 192 rows through registers and larger ones through an LDS tile.
hipError_t launch_gate_up_tile(const GemmProblem& p, const moe_tables& t, hipStream_t stream);
hipError_t launch_down_tile(const GemmProblem& p, const moe_tables& t, hipStream_t stream);
// W8A8: FP8 E4M3 activations (a, scales sa) against FP8 E4M3 weights (b0 /
// b1, scales s0 / s1); output c in dtype (kF16 / kBF16).
hipError_t launch_gate_up_w8a8(const GemmProblem& p, const moe_tables& t, hipStream_t stream);
hipError_t launch_down_w8a8(const GemmProblem& p, const moe_tables& t, hipStream_t stream);
hipError_t launch_down(const GemmProblem& p, const moe_tables& t, hipStream_t stream);
// Gate/up and down of each row block in one workgroup (block_m <= 32,
// d_expert <= fused_max_d_expert()), h kept in LDS; up.c is unused.
hipError_t launch_fused_expert(const GemmProblem& up, const GemmProblem& down,
                               const moe_tables& t, hipStream_t stream);
int fused_max_d_expert();
// FP8 E4M3 weights (b0 / b1 hold codes; s0 / s1 the per-row scales).
hipError_t launch_gate_up_w8(const GemmProblem& p, const moe_tables& t, hipStream_t stream);
hipError_t launch_down_w8(const GemmProblem& p, const moe_tables& t, hipStream_t stream);
hipError_t launch_quantize_fp8_rows(const void* w, int64_t rows, int cols, int dtype, uint8_t* q,
                                    float* scales, hipStream_t stream);
// W4A8: int8 activations (per-row scales sa) against packed int4 weights
// (b0 / b1, per-row scales s0 / s1); output c in dtype (kF16 / kBF16).
struct W4GemmProblem {
  const int8_t* a;       // gate/up: xq [T, kd]; down: hq [P, kd]
  const float* sa;       // gate/up: sx [T] (by token); down: sh [P] (by row)
  const uint8_t* b0;     // gate/up: W_gate [E, n, kd/2]; down: W_down
  const uint8_t* b1;     // gate/up: W_up; down: unused
  const float* s0;
  const float* s1;
  void* c;               // gate/up: h [P, n]; down: expert_out [P, n]
  int n;
  int kd;
  int dtype;
};
hipError_t launch_gate_up_w4a8(const W4GemmProblem& p, const moe_tables& t, hipStream_t stream);
hipError_t launch_down_w4a8(const W4GemmProblem& p, const moe_tables& t, hipStream_t stream);
hipError_t launch_w4a8_gemm(const int8_t* A, const uint8_t* B, int M, int N, int K, int32_t* Ct,
                            hipStream_t stream);
hipError_t launch_quantize_int8_rows(const void* a, int64_t rows, int cols, int dtype, int8_t* q,
                                     float* scales, hipStream_t stream);
hipError_t launch_quantize_int4_rows(const void* w, int64_t rows, int cols, int dtype,
                                     uint8_t* packed, float* scales, hipStream_t stream);
// MX: MXFP8 activations (E4M3 codes a, E8M0 block scales as) against MXFP4
// weights (packed E2M1 b0 / b1, E8M0 block scales s0 / s1); output c in
// dtype (kF16 / kBF16).
struct MxGemmProblem {
  const uint8_t* a;      // gate/up: xq [T, kd]; down: hq [P, kd]
  const uint8_t* as;     // [rows, kd/32]
  const uint8_t* b0;     // [E, n, kd/2]
  const uint8_t* b1;
  const uint8_t* s0;     // [E, n, kd/32]
  const uint8_t* s1;
  void* c;
  int n;
  int kd;
  int dtype;
};
hipError_t launch_gate_up_mx(const MxGemmProblem& p, const moe_tables& t, hipStream_t stream);
hipError_t launch_down_mx(const MxGemmProblem& p, const moe_tables& t, hipStream_t stream);
hipError_t launch_quantize_mx_rows(const void* v, int64_t rows, int cols, int dtype, int fmt,
                                   uint8_t* codes, uint8_t* scales, hipStream_t stream);
hipError_t launch_gate_up_f32(const GemmProblem& p, const moe_tables& t, hipStream_t stream);
hipError_t launch_down_f32(const GemmProblem& p, const moe_tables& t, hipStream_t stream);

hipError_t launch_gate(const void* x, const float* wr, const float* bias, int T, int H, int E,
                       int K, int renorm, int dtype, float* logits, int32_t* ids, float* w,
                       hipStream_t stream);

hipError_t launch_reduce(const void* x, int64_t rows, const int32_t* pos, const float* w,
                         const float* x_sf, const float* sf, int T, int K, int H, int in_dtype,
                         int out_dtype, void* y, hipStream_t stream);

}  // namespace moe
