// spec_verify: greedy longest-prefix acceptance with the bonus token, and the
// harness-side draft planting.  One thread per sequence (K <= 15 drafts).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

__global__ __launch_bounds__(64) void verify_kernel(const int32_t* __restrict__ d, const int32_t* __restrict__ g,
                                                    int B, int K, int32_t* __restrict__ accepted,
                                                    int32_t* __restrict__ committed,
                                                    int32_t* __restrict__ n_commit) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int32_t* db = d + (size_t)b * K;
  const int32_t* gb = g + (size_t)b * (K + 1);
  int n = 0;
  while (n < K && db[n] == gb[n]) ++n;
  int32_t* cb = committed + (size_t)b * (K + 1);
  for (int i = 0; i <= K; ++i) cb[i] = i < n ? db[i] : (i == n ? gb[n] : -1);
  accepted[b] = n;
  n_commit[b] = n + 1;
}

__global__ __launch_bounds__(256) void plant_kernel(const int32_t* __restrict__ g, const uint8_t* __restrict__ keep,
                                                    const int32_t* __restrict__ repl, int B, int K,
                                                    int32_t* __restrict__ drafts) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= B * K) return;
  const int b = idx / K, i = idx % K;
  const int32_t gi = g[(size_t)b * (K + 1) + i];
  const int32_t u = repl[idx];
  drafts[idx] = keep[idx] ? gi : u + (u >= gi ? 1 : 0);
}

}  // namespace

hipError_t launch_verify(const int32_t* drafts, const int32_t* argmax_ids, int B, int K,
                         int32_t* accepted, int32_t* committed, int32_t* n_commit, hipStream_t s) {
  hipLaunchKernelGGL(verify_kernel, dim3((B + 63) / 64), dim3(64), 0, s, drafts, argmax_ids, B, K, accepted,
                     committed, n_commit);
  return hipGetLastError();
}

hipError_t launch_plant(const int32_t* argmax_ids, const uint8_t* keep, const int32_t* repl, int B,
                        int K, int V, int32_t* drafts, hipStream_t s) {
  (void)V;
  const int n = B * K;
  hipLaunchKernelGGL(plant_kernel, dim3((n + 255) / 256), dim3(256), 0, s, argmax_ids, keep, repl, B, K, drafts);
  return hipGetLastError();
}

}  // namespace moe
