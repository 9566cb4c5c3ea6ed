// moe_forward_static: moe_forward with its workspace in a scratch array that the
// library owns on each device, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  The call allocates nothing: it resolves the device address of
// the array once per device and hands it to moe_forward as the workspace.
#include <mutex>

#include <hip/hip_runtime.h>

#include "moe_ffn.h"

namespace {

constexpr size_t kStaticScratchBytes = (size_t)MOE_STATIC_SCRATCH_BYTES;
static_assert(kStaticScratchBytes % 256 == 0, "whole 256-byte workspace blocks");

// One copy per device, held until the process ends.  In host code `scratch` is
// a host-side stand-in, never a device address: only the address that
// hipGetSymbolAddress returns for the current device is passed on.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device, resolved once

moe_status scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOE_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_forward_static(const moe_handle* h, int32_t num_tokens, const void* x, const void* x_sf,
                                         void* topk_idx, float* topk_weights, const float* routing_logits,
                                         const moe_weights* w, void* out, hipStream_t stream) {
  if (h == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  const size_t need = moe_workspace_size(h, num_tokens);
  if (need == 0) return MOE_ERR_INVALID_ARGUMENT;  // num_tokens outside [0, max_num_tokens]
  if (need > kStaticScratchBytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  const moe_status st = scratch_on_current_device(&ws);
  if (st != MOE_OK) return st;
  return moe_forward(h, num_tokens, x, x_sf, topk_idx, topk_weights, routing_logits, w, out, ws,
                     kStaticScratchBytes, stream);
}
