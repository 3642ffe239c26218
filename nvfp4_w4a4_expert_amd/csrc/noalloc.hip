// Allocation-free variant of the MoE forward, for callers that cannot call
// hipMalloc (code under HIP graph capture, tight serving loops, harnesses
// that forbid allocation).  The workspace is a static device buffer that the
// library holds on every device it runs on, until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory, so
// it is never passed to a kernel or a copy: on each device's first call the
// buffer's device address is looked up (hipGetSymbolAddress, with that device
// current) and kept per device, and only that address is used afterwards.
#include <atomic>
#include <mutex>

#include <hip/hip_runtime.h>

#define NVFP4_BUILDING_LIBRARY 1
#include "../../include/nvfp4_moe.h"

namespace {

constexpr size_t kScratchBytes = NVFP4_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte units");

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device, looked up once per
// device and kept.
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (err != hipSuccess) return err;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" {

NVFP4_API nvfp4_status_t nvfp4_moe_forward_noalloc(const nvfp4_moe_weights_t* w,
                                                   const void* x_bf16,
                                                   const float* router_logits,
                                                   int32_t num_tokens, int32_t k,
                                                   const void* residual_bf16, void* out_bf16,
                                                   const nvfp4_moe_debug_t* debug,
                                                   nvfp4_stream_t stream) {
  size_t need = 0;
  nvfp4_status_t st = nvfp4_moe_workspace_size(num_tokens, k, w, &need);
  if (st != NVFP4_OK) return st;
  if (need > kScratchBytes) return NVFP4_ERR_TOO_LARGE;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return NVFP4_ERR_DEVICE;
  // The forward writes every workspace byte it reads (routing, permutation,
  // quantised activations, GEMM outputs) before reading it, so the previous
  // call's contents need no clearing.
  return nvfp4_moe_forward(w, x_bf16, router_logits, num_tokens, k, residual_bf16, out_bf16, ws,
                           kScratchBytes, debug, stream);
}

}  // extern "C"
