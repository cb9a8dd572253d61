// moe_routed_forward_noalloc: the routed forward for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc). The forward's workspace (h [P, D], then
// expert_out [P, H] at the next 256-byte boundary) lives in a file-scope
// device array of MOE_NOALLOC_SCRATCH_BYTES instead of a caller buffer.
//
// Each GPU the library runs on holds its own copy of the array until the
// process ends. Its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and kept; host code never
// passes the array's name to a kernel (in host code that name is only a
// stand-in, not a device address). Nothing in the workspace has to start at
// zero: every h and expert_out row the kernels read was written earlier in
// the same call. Calls that overlap on one GPU (two streams, two threads)
// share the array and race.

#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"
#include "moe_routed.h"

namespace {

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (looked up on the
// first call per device). Returns MOE_OK or MOE_ERR_HIP.
moe_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return moe::set_error(MOE_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(err));
  if (dev < 0 || dev >= kMaxDevices) {
    return moe::set_error(MOE_ERR_HIP, "device %d is beyond the %d devices this library tracks", dev,
                          kMaxDevices);
  }
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess || !p) {
      return moe::set_error(MOE_ERR_HIP, "hipGetSymbolAddress of the static scratch failed: %s",
                            hipGetErrorString(err));
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_routed_forward_noalloc(const void* x, const void* w_gate,
                                                 const void* w_up, const void* w_down,
                                                 const moe_tables* tables, int H, int D,
                                                 int dtype, void* y, void* stream) {
  if (!tables) return moe::set_error(MOE_ERR_NULL, "tables must not be NULL");
  const size_t need = moe_forward_workspace_bytes(tables->T, tables->K, H, D, dtype);
  if (need == 0) {
    return moe::set_error(MOE_ERR_SHAPE, "invalid sizes (T=%d K=%d H=%d D=%d dtype=%d)", tables->T,
                          tables->K, H, D, dtype);
  }
  if (need > static_cast<size_t>(MOE_NOALLOC_SCRATCH_BYTES)) {
    return moe::set_error(MOE_ERR_WORKSPACE,
                          "moe_routed_forward_noalloc needs %zu bytes of workspace (h and "
                          "expert_out); its static scratch holds %zu",
                          need, static_cast<size_t>(MOE_NOALLOC_SCRATCH_BYTES));
  }
  void* ws = nullptr;
  const moe_status s = scratch_for_current_device(&ws);
  if (s != MOE_OK) return s;
  return moe_routed_forward(x, w_gate, w_up, w_down, tables, H, D, dtype, ws,
                            static_cast<size_t>(MOE_NOALLOC_SCRATCH_BYTES), y, stream);
}
