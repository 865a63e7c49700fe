// The workspace of mha_forward_noalloc (defined with the other entry points in
// mha_api.cpp): mha_forward for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation).
//
// mha_forward keeps its Q, K, V and concatenated-head intermediates in a
// workspace. Here that workspace is a file-scope device array, `scratch`, of
// kScratchBytes: the code object holds it, so each GPU the library runs on
// has its own copy, allocated when the library's code is loaded on that
// device and kept until the process ends. Nothing in this file allocates.
//
// In host code the array's name stands for a host-side shadow, not a device
// address. Its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and kept; kernels only ever
// receive that looked-up pointer.
//
// Every call on one GPU shares that GPU's array: calls that overlap on one
// GPU (on different streams, or from different threads) race on it. The
// array needs no clearing: each region is written by one launch before the
// next reads it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace {

constexpr size_t kScratchBytes = MHA_NOALLOC_MAX_WORKSPACE;  // the largest workspace served
constexpr int kMaxDevices = 64;

__device__ __attribute__((aligned(256))) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch`, per device

// The current device's copy of `scratch`, looked up on first use.
mha_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return mha::report_error(MHA_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return mha::report_error(MHA_ERR_UNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return mha::report_error(MHA_ERR_HIP, "hipGetSymbolAddress of the scratch array failed");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MHA_OK;
}

}  // namespace

namespace mha {

// The current device's copy of `scratch` and its size (for
// mha_forward_noalloc in mha_api.cpp).
mha_status noalloc_scratch(void** ptr, size_t* bytes) {
  mha_status s = scratch_of_current_device(ptr);
  *bytes = kScratchBytes;
  return s;
}

}  // namespace mha
