// noalloc.hip -- the fixed device scratch of xattn_bwd_noalloc, the backward
// entry point for callers that cannot allocate (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// The backward's only scratch is its per-row workspace: -D and LSE*log2e, two
// floats per query row, written by the dq kernel before the dk/dv kernel reads
// them (so nothing in it has to start at zero).  Here it lives in a file-scope
// device array: every GPU the library runs on holds its own copy, from the
// first use until the process ends, and every call on that GPU shares it, so
// calls that overlap on one GPU (e.g. on two streams) race on it.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "launch.hpp"

namespace xattn {

static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
// Device address of `scratch` per device.  In host code the array's name is
// only a host-side stand-in: kernels and copies must be given this address.
std::atomic<float*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

float* noalloc_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  float* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (!p) {
    // once per device, with that device current (hipGetDevice above)
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return nullptr;
    p = static_cast<float*>(addr);
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace xattn
