// moe_layer_forward_noalloc: the layer forward with its workspace in a fixed
// device array of this library, for callers that cannot allocate.
//
// `scratch` below is a file-scope device array.  In host code its name is a
// host-side stand-in, not a device address, so host code never passes it to
// a kernel or a copy: the device address comes from hipGetSymbolAddress,
// taken once per device with that device current, and is kept per device
// (each GPU holds its own copy of the array at its own address).
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "host_device.h"
#include "moe.h"

namespace {

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

std::atomic<void*> g_scratch[moe::kMaxDevices];  // zero-initialised: not looked up yet
std::mutex g_lookup;

// Device address of `scratch` on the current device (nullptr on failure).
void* scratch_on_current_device() {
  const int dev = moe::current_device();
  if (dev >= moe::kMaxDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_lookup);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
    g_scratch[dev].store(q, std::memory_order_release);
    p = q;
  }
  return p;
}

}  // namespace

extern "C" moe_status_t moe_layer_forward_noalloc(const moe_config_t* cfg, const moe_weights_t* w,
                                                  const void* x, const moe_layer_out_t* out,
                                                  const moe_trace_t* trace, void* stream) {
  size_t need = 0;
  const moe_status_t st = moe_workspace_size(cfg, &need);
  if (st != MOE_OK) return st;
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  if (cfg->T == 0) return moe_layer_forward(cfg, w, x, out, nullptr, 0, trace, stream);
  void* ws = scratch_on_current_device();
  if (!ws) return MOE_ERR_HIP;
  // every workspace value the forward reads it writes first in the same
  // call (no buffer there has to start at zero), so the previous call's
  // contents do no harm
  return moe_layer_forward(cfg, w, x, out, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES, trace, stream);
}
