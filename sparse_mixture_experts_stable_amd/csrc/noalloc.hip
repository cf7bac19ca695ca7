// moe_forward_noalloc: the whole forward pass with its workspace in a device array the
// library owns, for callers that cannot allocate device memory (code under HIP graph
// capture, serving loops, harnesses that forbid allocation).
//
// The array is a file-scope __device__ variable: each GPU the library is loaded on holds
// its own copy, at its own address, for the life of the process. Its address is taken
// once per device with hipGetSymbolAddress (with that device current) and kept; the
// array's name is never passed to a kernel or a copy from host code. Every call on one
// GPU uses the same array, so calls that overlap on one GPU (different streams, no
// ordering between them) race; calls in stream order do not. No state carries over
// from one call to the next: every value the forward reads from its workspace is
// written earlier in the same call (the routing partials, the chunk sums, the error
// word, the shared expert's hidden activation).

#include <mutex>

#include "internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;

__device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The device address of this GPU's array, looked up on the first call on the device.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" {

moe_status_t moe_forward_noalloc(const moe_forward_args_t* a, void* stream) {
  if (!a) return MOE_ERR_INVALID_ARG;
  // every buffer moe_forward could otherwise take from its workspace is an output here
  const bool hidden = a->experts.kind != MOE_EXPERT_LINEAR && a->capacity > 0;
  if ((hidden && !a->hidden_cache) || (a->shared.w_in && !a->shared_out))
    return MOE_ERR_INVALID_ARG;
  const size_t need = moe_forward_workspace_size(a);
  if (need == 0) return MOE_ERR_INVALID_ARG;
  if (need > kScratchBytes) return MOE_ERR_WORKSPACE;
  void* ws = scratch_on_current_device();
  if (!ws) return MOE_ERR_HIP;
  return moe_forward(a, ws, kScratchBytes, stream);
}

}  // extern "C"
