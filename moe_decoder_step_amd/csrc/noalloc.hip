// lmhead_argmax_noalloc: lmhead_argmax with its workspace in a static device
// array of the library instead of caller memory, for callers that cannot
// allocate (code under graph capture, tight serving loops).
//
// The array `scratch` is a file-scope __device__ variable: every GPU the
// library runs on holds its own copy, at its own address, until the process
// ends.  Host code never passes the array's name to a kernel (on the host it
// is only a stand-in for the symbol); it looks up the device address once per
// device with hipGetSymbolAddress, with that device current, and passes that
// pointer.  Every call on a GPU shares that GPU's copy: calls that overlap on
// one GPU (two streams, or two host threads) race on it.  The LM head writes
// every partial key it later reads, so nothing needs clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/moestep.h"
#include "kernels.hpp"
#include "validate.hpp"

namespace {

constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this device's `scratch`: looked up on the first call
// on the device (with the device current), then cached.  The device is the
// stream's (the current one for the NULL stream).
int scratch_address(hipStream_t stream, void** out) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return MOE_ERR_HIP;
  int dev = cur;
  if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return MOE_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return MOE_ERR_HIP;
    if (e != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" int lmhead_argmax_noalloc(const void* h, const void* w_lm, int T, int H, int V, int dtype,
                                     int32_t* argmax_ids, float* max_logit, void* stream) {
  // argument checks as lmhead_argmax, with the static array as the workspace
  // (its address is 256-byte aligned; a stand-in of that alignment passes
  // the pointer checks before the real address is known)
  const size_t need = moe::lmhead_ws_bytes(T, V, dtype);
  int st = moe::check_lmhead(h, w_lm, T, H, V, dtype, argmax_ids, reinterpret_cast<const void*>(256),
                             need > kScratchBytes ? 0 : kScratchBytes);
  if (st != MOE_OK || T == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  st = scratch_address(s, &ws);
  if (st != MOE_OK) return st;
  return moe::launch_lmhead(h, w_lm, T, H, V, dtype, argmax_ids, max_logit, ws, s) == hipSuccess ? MOE_OK
                                                                                                  : MOE_ERR_HIP;
}
