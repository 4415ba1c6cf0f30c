// The prefill entry point that allocates nothing: axon_ssm_prefill with the time-chunked scan's
// workspace taken from a scratch array of the library's own, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses that forbid it).
//
// The array is a file-scope device variable: every GPU the library runs on holds its own copy
// for the life of the process. Host code never uses its name as an address (on the host it only
// stands for the symbol): the device address is looked up once per device, with that device
// current, by hipGetSymbolAddress, and kept per device. Calls on one GPU share that GPU's array,
// so calls that overlap in time on one GPU race; nothing in the array needs to start at zero
// (the carry pass writes every carry before the combine and the final pass read it).
#include <hip/hip_runtime.h>

#include <cstddef>
#include <mutex>

#include "axon_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // 64 MiB per device
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch` per device (null: not yet)

// The device address of this device's copy of the scratch array.
axon_status scratch_of_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return AXON_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return AXON_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return AXON_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return AXON_OK;
}

}  // namespace

extern "C" axon_status axon_ssm_prefill_noalloc(const axon_ssm_shape* shape,
                                                const axon_ssm_params* params, const void* x,
                                                const void* z, const void* dt_raw, const void* B,
                                                const void* C, const float* conv_cache_in,
                                                const float* ssm_state_in, void* y,
                                                float* conv_cache_out, float* ssm_state_out,
                                                void* stream) {
  // Every argument check first (no device call), with the plan limited to the scratch size.
  axon::PrefillLaunch a;
  axon::PrefillPlan plan;
  axon_status st = axon::prepare_prefill(shape, params, x, z, dt_raw, B, C, conv_cache_in,
                                         ssm_state_in, y, conv_cache_out, ssm_state_out, nullptr,
                                         kScratchBytes, true, kScratchBytes, &a, &plan);
  if (st != AXON_OK) return st;
  if (plan.workspace_bytes > kScratchBytes) return AXON_ERR_WORKSPACE_TOO_SMALL;
  if (a.seqlen > 0 && plan.workspace_bytes > 0) {
    void* ws = nullptr;
    st = scratch_of_current_device(&ws);
    if (st != AXON_OK) return st;
    a.workspace = ws;
  }
  return axon::launch_prefill(a, plan, stream) == 0 ? AXON_OK : AXON_ERR_HIP;
}
