// Device scratch of the write-back that allocates nothing (hc_write_back_all_layers_noalloc).
//
// The ordinary write-back uploads its per-burst plan (a device copy of the host token
// list, and the shard pages whose pad it clears) into plan buffers the pool grows on
// demand with hipHostMalloc / hipMalloc.  A caller that may not allocate (a tight
// serving loop, a harness that forbids it) gets a variant whose plan is one fixed-size
// array in the code object instead: the copy of the host token list, HC_NOALLOC_MAX_TOKENS
// int64 entries (2 MiB), held by every GPU the library runs on until the process ends.
// Every call on a GPU shares that GPU's copy of the array, so calls that overlap on one
// GPU (pools on different streams) race on it; calls on one stream run in order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "hc_internal.h"

namespace {

static __device__ __align__(256) int64_t scratch[HC_NOALLOC_MAX_TOKENS];

// Per-device address of `scratch`.  In host code the name `scratch` is a host-side stand-in,
// not a device address, so every host use goes through the address looked up here.
constexpr int kMaxDevices = 64;
std::mutex g_mu;
int64_t* g_ptr[kMaxDevices] = {};

}  // namespace

namespace hc {

int noalloc_scratch(int device, int64_t** out) {
  *out = nullptr;
  if (device < 0 || device >= kMaxDevices)
    return set_error(HC_ERR_UNSUPPORTED, "device %d: the no-allocation scratch serves devices 0..%d", device,
                     kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[device]) {
    // looked up once per device, with that device current (the caller made it current)
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess || cur != device)
      return set_error(HC_ERR_HIP, "the no-allocation scratch lookup needs device %d current", device);
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return set_error(HC_ERR_HIP, "hipGetSymbolAddress of the no-allocation scratch failed: %s",
                       hipGetErrorString(e));
    }
    g_ptr[device] = static_cast<int64_t*>(ptr);
  }
  *out = g_ptr[device];
  return HC_OK;
}

}  // namespace hc
