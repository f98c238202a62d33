// attn_jvp_noalloc.hip -- the fixed device buffer behind attn_jvp_fwd_noalloc,
// the entry point for callers that cannot allocate (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// `scratch` holds the tile images (and their headers) that the pack kernels
// write and the fused kernel reads, in place of a workspace the caller or a
// pool would provide.  Each GPU that runs the library holds one copy, at its
// own address, until the process ends.  In host code the array's name stands
// for a host-side handle, not a device address: the address of this device's
// copy is looked up once per device with hipGetSymbolAddress and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "attn_jvp.h"
#include "launch.hpp"

namespace {

constexpr size_t kScratchBytes = size_t(128) << 20;  // 128 MiB per device
static_assert(kScratchBytes == ATTN_JVP_NOALLOC_BYTES, "the size the header states");

static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

namespace ajvp {

size_t scratch_bytes() { return kScratchBytes; }

hipError_t scratch_buffer(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace ajvp
