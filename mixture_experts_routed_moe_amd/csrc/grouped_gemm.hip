// Grouped expert GEMMs with weights in the activation dtype (bf16 / fp16;
// fp32 goes to the vector-ALU debug path). Blocks of <= 64 rows run the
// register-streaming kernels of grouped_gemm.hpp; blocks of 128 or 256 rows
// the LDS-tiled kernels of grouped_gemm_tile.hip.

#include "grouped_gemm.hpp"

namespace moe {

hipError_t launch_gate_up(const GemmProblem& p, const moe_tables& t, hipStream_t stream) {
  if (p.dtype == kF32) return launch_gate_up_f32(p, t, stream);
  if (t.block_m >= 128) return launch_gate_up_tile(p, t, stream);
  if (p.dtype == kBF16) return launch_typed<kBF16, true, false>(p, t, stream);
  return launch_typed<kF16, true, false>(p, t, stream);
}

hipError_t launch_down(const GemmProblem& p, const moe_tables& t, hipStream_t stream) {
  if (p.dtype == kF32) return launch_down_f32(p, t, stream);
  if (t.block_m >= 128) return launch_down_tile(p, t, stream);
  if (p.dtype == kBF16) return launch_typed<kBF16, false, false>(p, t, stream);
  return launch_typed<kF16, false, false>(p, t, stream);
}

}  // namespace moe
