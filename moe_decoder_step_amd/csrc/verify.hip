// spec_verify: greedy longest-prefix acceptance with the bonus token, the
// harness-side draft planting (one thread per sequence, K <= 15 drafts), and
// the bookkeeping of a decode loop over a shrinking batch (spec_advance,
// spec_gather_rows).
#include "common.hpp"
#include "kernels.hpp"
#include "validate.hpp"

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
  // every draft and target token loaded at once, then compared in registers
  // (a compare-as-you-load loop waits out one round trip per position)
  int32_t dv[kMaxDrafts], gv[kMaxDrafts + 1];
#pragma unroll
  for (int i = 0; i < kMaxDrafts; ++i) dv[i] = i < K ? db[i] : 0;
#pragma unroll
  for (int i = 0; i <= kMaxDrafts; ++i) gv[i] = i <= K ? gb[i] : -1;
  int n = K;
#pragma unroll
  for (int i = kMaxDrafts - 1; i >= 0; --i)
    if (i < K && dv[i] != gv[i]) n = i;       // the first mismatch
  int32_t* cb = committed + (size_t)b * (K + 1);
#pragma unroll
  for (int i = 0; i <= kMaxDrafts; ++i)
    if (i <= K) cb[i] = i < n ? dv[i] : (i == n ? gv[i] : -1);
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

// One block: slot i of the active batch (sequence seq_ids[i]) appends up to
// target - total of its committed tokens to that sequence's stream; the
// sequences still short of target are compacted in slot order.
__global__ __launch_bounds__(1024) void advance_kernel(const int32_t* __restrict__ n_commit,
                                                       const int32_t* __restrict__ committed,
                                                       const int32_t* __restrict__ seq_ids, int B, int K, int S,
                                                       int target, int32_t* __restrict__ total,
                                                       int32_t* __restrict__ steps, int32_t* __restrict__ tokens,
                                                       int32_t* __restrict__ seq_out, int32_t* __restrict__ n_active,
                                                       uint32_t* err) {
  __shared__ int wave_count[kAdvanceMaxB / 64];
  const int i = threadIdx.x, wave = i >> 6, lane = i & 63;
  bool alive = false;
  int seq = 0;
  if (i < B && seq_ids[i] >= 0) {   // a negative id is an empty slot
    seq = clamp_report(seq_ids[i], 0, S - 1, err, kDataErrSequence);
    const int before = clampi(total[seq], 0, target);
    const int take = min(clamp_report(n_commit[i], 0, K + 1, err, kDataErrSequence), target - before);
    for (int j = 0; j < take; ++j) tokens[(size_t)seq * target + before + j] = committed[(size_t)i * (K + 1) + j];
    total[seq] = before + take;
    steps[seq] += 1;
    alive = before + take < target;
  }
  const unsigned long long mask = __ballot(alive);
  if (lane == 0) wave_count[wave] = __popcll(mask);
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wave_count[w];
  const int rank = __popcll(mask & ((1ull << lane) - 1ull));
  if (alive) seq_out[base + rank] = seq;
  int n = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) n += wave_count[w];
  // slots n .. B-1 of the new list are empty: a pass launched before n is
  // known (with the previous batch size) skips them
  if (i >= n && i < B) seq_out[i] = -1;
  if (i == blockDim.x - 1) n_active[0] = n;
}

// out row i*R + r = pool row (seq_ids[i] * J + min(steps[seq], J - 1)) * R + r,
// row_bytes bytes each (4-byte words when aligned, else bytes)
__global__ __launch_bounds__(256) void gather_rows_kernel(const char* __restrict__ pool, const int32_t* __restrict__ seq_ids,
                                                          const int32_t* __restrict__ steps, int B, int R, int J, int S,
                                                          int row_bytes, bool words, char* __restrict__ out,
                                                          uint32_t* err) {
  const int o = blockIdx.x;  // output row
  const int i = o / R, r = o % R;
  const int sid = seq_ids[i];   // < 0: an empty slot (reads sequence 0), >= S: reported
  report_error(threadIdx.x == 0 ? err : nullptr, sid >= S, kDataErrSequence);
  const int seq = clampi(sid, 0, S - 1);
  const int st = clampi(steps[seq], 0, J - 1);
  const char* src = pool + (((size_t)seq * J + st) * R + r) * row_bytes;
  char* dst = out + (size_t)o * row_bytes;
  if (words) {
    for (int c = threadIdx.x; c < row_bytes / 4; c += blockDim.x)
      reinterpret_cast<int32_t*>(dst)[c] = reinterpret_cast<const int32_t*>(src)[c];
  } else {
    for (int c = threadIdx.x; c < row_bytes; c += blockDim.x) dst[c] = src[c];
  }
}

}  // namespace

hipError_t launch_advance(const int32_t* n_commit, const int32_t* committed, const int32_t* seq_ids, int B, int K,
                          int S, int target, int32_t* total, int32_t* steps, int32_t* tokens, int32_t* seq_out,
                          int32_t* n_active, hipStream_t s) {
  const int threads = ((B + 63) / 64) * 64;
  hipLaunchKernelGGL(advance_kernel, dim3(1), dim3(threads < 64 ? 64 : threads), 0, s, n_commit, committed, seq_ids,
                     B, K, S, target, total, steps, tokens, seq_out, n_active, data_error_word(s));
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* pool, const int32_t* seq_ids, const int32_t* steps, int B, int R, int J,
                              int S, int row_bytes, void* out, hipStream_t s) {
  const bool words = row_bytes % 4 == 0 && (reinterpret_cast<uintptr_t>(pool) & 3) == 0 &&
                     (reinterpret_cast<uintptr_t>(out) & 3) == 0;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(B * R), dim3(256), 0, s, static_cast<const char*>(pool), seq_ids,
                     steps, B, R, J, S, row_bytes, words, static_cast<char*>(out), data_error_word(s));
  return hipGetLastError();
}

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
