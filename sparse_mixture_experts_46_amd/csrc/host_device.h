// Host-side, per-device caches of the launch code.
//
// The library's only process-wide state: write-once facts about each device
// (its compute-unit count, whether a kernel's dynamic-LDS limit has been
// raised there).  Each lives in an atomic per device, and a racing first use
// stores the same value, so any host thread may launch on any device.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

namespace moe {

constexpr int kMaxDevices = 64;

inline int current_device() {
  int d = 0;
  if (hipGetDevice(&d) != hipSuccess || d < 0) d = 0;
  return d;
}

// Compute units of the current device (256 if the runtime cannot tell).
inline int device_cus() {
  static std::atomic<int> cache[kMaxDevices];  // zero-initialised: not yet known
  const int dev = current_device();
  if (dev < kMaxDevices) {
    const int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
  }
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    v = 256;
  if (dev < kMaxDevices) cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

// Raise the dynamic-LDS limit of `kern` to `bytes` on the current device,
// once per device (`done` is the kernel's own bit mask of devices).
inline hipError_t set_dynamic_lds_once(const void* kern, int bytes, std::atomic<uint64_t>& done) {
  const int dev = current_device();
  const uint64_t bit = dev < kMaxDevices ? (uint64_t(1) << dev) : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

}  // namespace moe
