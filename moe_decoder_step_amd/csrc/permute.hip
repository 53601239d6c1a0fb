// moe_permute: stable counting sort of the T*k (token, slot) pairs by expert.
//
// Slots are cut into chunks of 4096.  Within a chunk, wavefront w owns the
// experts e = w, w+16, ...; it walks the chunk 64 slots at a time and ranks the
// slots of its expert with a ballot and a popcount, which keeps ascending
// slot (= token) order without atomics, so the result is deterministic.
// One chunk (T*k <= 4096, every decode batch) is a single block; larger
// inputs take a histogram pass, a one-block scan over (chunk, expert) and a
// scatter pass.
#include "common.hpp"
#include "kernels.hpp"
#include "validate.hpp"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;

// Rank and scatter the slots of one chunk.  sid: the chunk's expert ids (LDS),
// base[e]: first row of expert e for this chunk.
__device__ void scatter_chunk(const int* sid, int n, int slot0, int k, int E, const int* base,
                              int32_t* __restrict__ gather, int32_t* __restrict__ inv) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int e = wave; e < E; e += kWaves) {
    int run = base[e];
    for (int p = 0; p < n; p += kWave) {
      const int s = p + lane;
      const bool mine = s < n && sid[s] == e;
      const unsigned long long mask = __ballot(mine);
      if (mine) {
        const int pos = run + __popcll(mask & below);
        const int slot = slot0 + s;
        gather[pos] = slot / k;
        inv[slot] = pos;
      }
      run += __popcll(mask);
    }
  }
}

__device__ void fill_shared_rows(int T, int k, int S, int32_t* __restrict__ gather, int start, int stride) {
  const long long n = (long long)S * T, base = (long long)T * k;
  for (long long i = start; i < n; i += stride) gather[base + i] = (int32_t)(i % T);
}

__global__ __launch_bounds__(kThreads) void permute_one_block(const int32_t* __restrict__ ids, int T, int k,
                                                              int E, int S, int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ gather,
                                                              int32_t* __restrict__ inv) {
  __shared__ int sid[kPermuteChunk];
  __shared__ int cnt[kMaxExperts];
  __shared__ int base[kMaxExperts];
  const int n = T * k;
  if (threadIdx.x < kMaxExperts) cnt[threadIdx.x] = 0;
  for (int i = threadIdx.x; i < n; i += kThreads) sid[i] = clampi(ids[i], 0, E - 1);
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += kThreads) atomicAdd(&cnt[sid[i]], 1);
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int e = 0; e < E; ++e) {
      base[e] = acc;
      offsets[e] = acc;
      acc += cnt[e];
    }
    offsets[E] = acc;
    for (int s = 0; s < S; ++s) offsets[E + 1 + s] = acc + (s + 1) * T;
  }
  __syncthreads();
  scatter_chunk(sid, n, 0, k, E, base, gather, inv);
  fill_shared_rows(T, k, S, gather, threadIdx.x, kThreads);
}

__global__ __launch_bounds__(kThreads) void permute_hist(const int32_t* __restrict__ ids, int n_slots, int E,
                                                         int32_t* __restrict__ counts) {
  __shared__ int cnt[kMaxExperts];
  if (threadIdx.x < kMaxExperts) cnt[threadIdx.x] = 0;
  __syncthreads();
  const int s0 = blockIdx.x * kPermuteChunk;
  const int n = min(kPermuteChunk, n_slots - s0);
  for (int i = threadIdx.x; i < n; i += kThreads) atomicAdd(&cnt[clampi(ids[s0 + i], 0, E - 1)], 1);
  __syncthreads();
  if (threadIdx.x < E) counts[blockIdx.x * E + threadIdx.x] = cnt[threadIdx.x];
}

// One block of 64 threads: thread e walks the chunks in order.
__global__ __launch_bounds__(64) void permute_scan(const int32_t* __restrict__ counts, int n_chunks, int E,
                                                   int S, int T, int32_t* __restrict__ bases,
                                                   int32_t* __restrict__ offsets) {
  __shared__ int total[kMaxExperts];
  __shared__ int first[kMaxExperts];
  const int e = threadIdx.x;
  if (e < E) {
    int run = 0;
    for (int c = 0; c < n_chunks; ++c) {
      bases[c * E + e] = run;
      run += counts[c * E + e];
    }
    total[e] = run;
  }
  __syncthreads();
  if (e == 0) {
    int acc = 0;
    for (int i = 0; i < E; ++i) {
      first[i] = acc;
      offsets[i] = acc;
      acc += total[i];
    }
    offsets[E] = acc;
    for (int s = 0; s < S; ++s) offsets[E + 1 + s] = acc + (s + 1) * T;
  }
  __syncthreads();
  if (e < E)
    for (int c = 0; c < n_chunks; ++c) bases[c * E + e] += first[e];
}

__global__ __launch_bounds__(kThreads) void permute_scatter(const int32_t* __restrict__ ids, int T, int k,
                                                            int E, int S, const int32_t* __restrict__ bases,
                                                            int32_t* __restrict__ gather,
                                                            int32_t* __restrict__ inv) {
  __shared__ int sid[kPermuteChunk];
  __shared__ int base[kMaxExperts];
  const int n_slots = T * k;
  const int s0 = blockIdx.x * kPermuteChunk;
  const int n = min(kPermuteChunk, n_slots - s0);
  for (int i = threadIdx.x; i < n; i += kThreads) sid[i] = clampi(ids[s0 + i], 0, E - 1);
  if (threadIdx.x < E) base[threadIdx.x] = bases[blockIdx.x * E + threadIdx.x];
  __syncthreads();
  scatter_chunk(sid, n, s0, k, E, base, gather, inv);
  fill_shared_rows(T, k, S, gather, blockIdx.x * kThreads + threadIdx.x, gridDim.x * kThreads);
}

}  // namespace

hipError_t launch_permute(const int32_t* ids, int T, int k, int E, int S, int32_t* offsets,
                          int32_t* gather, int32_t* inv, void* ws, hipStream_t s) {
  const int n_slots = T * k;
  const int n_chunks = (n_slots + kPermuteChunk - 1) / kPermuteChunk;
  if (n_chunks <= 1) {
    hipLaunchKernelGGL(permute_one_block, dim3(1), dim3(kThreads), 0, s, ids, T, k, E, S, offsets, gather, inv);
    return hipGetLastError();
  }
  int32_t* counts = static_cast<int32_t*>(ws);
  int32_t* bases = counts + (size_t)n_chunks * E;
  hipLaunchKernelGGL(permute_hist, dim3(n_chunks), dim3(kThreads), 0, s, ids, n_slots, E, counts);
  hipLaunchKernelGGL(permute_scan, dim3(1), dim3(64), 0, s, counts, n_chunks, E, S, T, bases, offsets);
  hipLaunchKernelGGL(permute_scatter, dim3(n_chunks), dim3(kThreads), 0, s, ids, T, k, E, S, bases, gather, inv);
  return hipGetLastError();
}

}  // namespace moe
