// Grouped expert GEMMs with FP8 E4M3 expert weights and one fp32 scale per
// weight row (per output channel); activations, h and expert_out stay in
// bf16 / fp16. The weight stream (the decode layer's bytes) halves; the
// codes are decoded to the activation dtype exactly in registers and the
// scale is applied once per dot product in the epilogue. Kernels:
// grouped_gemm.hpp.

#include "grouped_gemm.hpp"

namespace moe {

hipError_t launch_gate_up_w8(const GemmProblem& p, const moe_tables& t, hipStream_t stream) {
  if (p.dtype == kBF16) return launch_typed<kBF16, true, true>(p, t, stream);
  return launch_typed<kF16, true, true>(p, t, stream);
}

hipError_t launch_down_w8(const GemmProblem& p, const moe_tables& t, hipStream_t stream) {
  if (p.dtype == kBF16) return launch_typed<kBF16, false, true>(p, t, stream);
  return launch_typed<kF16, false, true>(p, t, stream);
}

}  // namespace moe
