// dsa_forward_noalloc: the whole path (dsa_forward) with its workspace in a
// static device array instead of a caller buffer, for callers that cannot
// allocate device memory (code under HIP graph capture, serving loops or
// harnesses that forbid hipMalloc).  It calls no allocating routine.
//
// The array holds what dsa_forward keeps in its workspace: the score rows or
// the fused kernel's candidate lists, the selected positions, top-k's
// candidate lists for long rows and the attention's split partials.  None of
// the kernels reads a byte of it that the same call has not written first,
// so nothing in it needs clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "libdsa.h"

namespace dsa {
// status and message helper of libdsa.cpp
dsa_status_t report(dsa_status_t st, const char *fmt, ...);
}  // namespace dsa

namespace {
constexpr size_t kScratchBytes = DSA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
}  // namespace

// One copy per GPU, at its own device address, held from the first use of
// the library on that GPU to the end of the process.  In host code this
// name is only a stand-in for the symbol, not a device address: host code
// uses the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_mu;
void *g_scratch[kMaxDevices];  // device address of each GPU's copy, once queried

// Device address of `dev`'s copy of the array, queried once per device with
// that device current.
dsa_status_t scratch_of(int dev, void **out) {
  if (dev < 0 || dev >= kMaxDevices)
    return dsa::report(DSA_ERR_UNSUPPORTED, "dsa_forward_noalloc: device %d is beyond the %d it supports", dev,
                       kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return dsa::report(DSA_ERR_HIP, "dsa_forward_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
      return dsa::report(DSA_ERR_HIP, "dsa_forward_noalloc: hipSetDevice: %s", hipGetErrorString(e));
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess && e2 != hipSuccess) e = e2;
    }
    if (e != hipSuccess || !p)
      return dsa::report(DSA_ERR_HIP, "dsa_forward_noalloc: hipGetSymbolAddress: %s",
                         e != hipSuccess ? hipGetErrorString(e) : "null address");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return DSA_OK;
}

}  // namespace

extern "C" dsa_status_t dsa_forward_noalloc(const dsa_forward_args_t *args, hipStream_t stream) {
  if (!args) return dsa::report(DSA_ERR_INVALID_ARGUMENT, "args is NULL");
  size_t need = 0;
  dsa_status_t st = dsa_forward_workspace_size(args, &need);
  if (st != DSA_OK) return st;
  if (need > kScratchBytes)
    return dsa::report(DSA_ERR_WORKSPACE_TOO_SMALL,
                       "dsa_forward_noalloc: this call needs %zu workspace bytes but the static scratch holds %zu; "
                       "pass scores and indices buffers, or call dsa_forward with a workspace",
                       need, kScratchBytes);
  if (need == 0) return dsa_forward(args, nullptr, 0, stream);
  int dev = -1;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess)
    return dsa::report(DSA_ERR_HIP, "dsa_forward_noalloc: hipStreamGetDevice: %s", hipGetErrorString(e));
  void *ws = nullptr;
  st = scratch_of(dev, &ws);
  if (st != DSA_OK) return st;
  return dsa_forward(args, ws, need, stream);
}
