// Device-side data errors: the kernels never address memory with an index
// argument they have not clamped into range; where the argument itself was
// out of range they also record its kind (MOE_DATA_ERR_*) in one 32-bit word
// per GPU, which moe_data_errors reads back and clears on a stream.
//
// The word is a file-scope __device__ variable: each GPU holds its own copy at
// its own address until the process ends.  Host code never passes the
// variable's name to a kernel (on the host it only stands for the symbol); it
// looks up the device address once per device with hipGetSymbolAddress, with
// that device current, and passes that pointer.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/moestep.h"
#include "kernels.hpp"

namespace {

constexpr int kMaxDevices = 64;

__device__ __align__(256) uint32_t data_errors[64];   // word 0 used; one 256-byte line of its own

std::mutex g_mu;
std::atomic<uint32_t*> g_word[kMaxDevices];

// this word's device and the current device -> address (cached per device)
uint32_t* word_for(int dev, int cur) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  uint32_t* p = g_word[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_mu);
  p = g_word[dev].load(std::memory_order_relaxed);
  if (p) return p;
  if (dev != cur && hipSetDevice(dev) != hipSuccess) return nullptr;
  void* a = nullptr;
  const hipError_t e = hipGetSymbolAddress(&a, HIP_SYMBOL(data_errors));
  if (dev != cur && hipSetDevice(cur) != hipSuccess) return nullptr;
  if (e != hipSuccess || !a) return nullptr;
  p = static_cast<uint32_t*>(a);
  g_word[dev].store(p, std::memory_order_release);
  return p;
}

// one thread: out = word; word = 0 if asked (a kernel, not a copy or memset,
// so that the call can sit in a captured graph)
__global__ void read_errors_kernel(uint32_t* word, uint32_t* out, int clear) {
  const uint32_t v = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  *out = v;
  if (clear) __hip_atomic_fetch_and(word, ~v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

namespace moe {

uint32_t* data_error_word(hipStream_t s) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  int dev = cur;
  if (s && hipStreamGetDevice(s, &dev) != hipSuccess) return nullptr;
  return word_for(dev, cur);
}

}  // namespace moe

extern "C" int moe_data_errors(uint32_t* flags_out, int clear, void* stream) {
  if (!flags_out) return MOE_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(flags_out) % 4) return MOE_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t* w = moe::data_error_word(s);
  if (!w) return MOE_ERR_HIP;
  hipLaunchKernelGGL(read_errors_kernel, dim3(1), dim3(1), 0, s, w, flags_out, clear ? 1 : 0);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
