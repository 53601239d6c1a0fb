// moe_permute: stable counting sort of the T*k (token, slot) pairs by expert.
//
// Slots are cut into chunks of 4096 = 64 pieces of 64 slots, one piece per
// wavefront pass.  For a piece, the wavefront takes one ballot per expert:
// the popcount of the lanes below a slot in its expert's ballot is the slot's
// rank inside the piece, and the ballot's popcount is the expert's count in
// the piece.  A scan of the counts over pieces (per expert) and over experts
// turns ranks into rows.  Ranks follow slot order, so the sort is stable
// (ascending token inside an expert) and deterministic, with no atomics.
// One chunk (every decode batch) is a single block; larger inputs take a
// count pass, a one-block scan over (chunk, expert) and a scatter pass that
// re-ranks its chunk, with chunks of 1024 slots there (one piece per
// wavefront: 217 blocks at 36,992 x 6 slots, where 4096-slot chunks gave 55).
#include "common.hpp"
#include "kernels.hpp"
#include "validate.hpp"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;                // 16
constexpr int kPieces = kPermuteChunk / kWave;          // 64 pieces per chunk
constexpr int kPiecesPerWave = kPieces / kWaves;        // 4
static_assert(kPermuteChunkM == kWaves * kWave, "multi-block chunks: one piece per wavefront");

// Rank the slots of one chunk.  Fills pcount[p][e] (count of expert e in
// piece p; lanes >= E write nothing) and, per pass pi, the lane's expert and
// rank inside its piece.  Ids outside [0, E) count as the nearest expert and,
// with err set, are reported.
template <int PPW>
__device__ __forceinline__ void rank_chunk(const int32_t* __restrict__ ids, int s0, int n, int E,
                                           int (*pcount)[kMaxExperts], int* my_e, int* my_rank,
                                           uint32_t* err) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int pi = 0; pi < PPW; ++pi) {
    const int p = wave + kWaves * pi;
    const int s = p * kWave + lane;
    const int e = s < n ? clamp_report(ids[s0 + s], 0, E - 1, err, kDataErrExpertId) : -1;
    int rank = 0, cnt = 0;
    if (p * kWave < n) {
      for (int ee = 0; ee < E; ++ee) {
        const unsigned long long b = __ballot(e == ee);
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0));
        if (e == ee) rank = below;
        if (lane == ee) cnt = __popcll(b);
      }
      if (lane < E) pcount[p][lane] = cnt;
    }
    my_e[pi] = e;
    my_rank[pi] = rank;
  }
}

// Exclusive scan of pcount[.][e] over the pieces of a chunk, in place; returns
// the chunk total of expert e (threads e < E only).
__device__ __forceinline__ int scan_pieces(int (*pcount)[kMaxExperts], int n_pieces, int e) {
  int run = 0;
  for (int p = 0; p < n_pieces; ++p) {
    const int c = pcount[p][e];
    pcount[p][e] = run;
    run += c;
  }
  return run;
}

template <int PPW>
__device__ __forceinline__ void scatter_chunk(int s0, int n, int k, const int* base,
                                              int (*pcount)[kMaxExperts], const int* my_e, const int* my_rank,
                                              int32_t* __restrict__ gather, int32_t* __restrict__ inv) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int pi = 0; pi < PPW; ++pi) {
    const int p = wave + kWaves * pi;
    const int s = p * kWave + lane;
    if (s < n) {
      const int e = my_e[pi];
      const int pos = base[e] + pcount[p][e] + my_rank[pi];
      gather[pos] = (s0 + s) / k;
      inv[s0 + s] = pos;
    }
  }
}

__device__ void fill_shared_rows(int T, int k, int S, int32_t* __restrict__ gather, int start, int stride) {
  const long long n = (long long)S * T, base = (long long)T * k;
  for (long long i = start; i < n; i += stride) gather[base + i] = (int32_t)(i % T);
}

// exclusive scan over experts by one wavefront: base[e], offsets[0..E], shared offsets
__device__ __forceinline__ void scan_experts(const int* tot, int E, int S, int T, int* base,
                                             int32_t* __restrict__ offsets) {
  const int e = threadIdx.x;
  const int c = e < E ? tot[e] : 0;
  int incl = c;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int v = __shfl_up(incl, o, kWave);
    if (e >= o) incl += v;
  }
  const int total = __shfl(incl, kWave - 1, kWave);
  if (e < E) {
    base[e] = incl - c;
    offsets[e] = incl - c;
  }
  if (e == 0) offsets[E] = total;
  if (e < S) offsets[E + 1 + e] = total + (e + 1) * T;
}

__global__ __launch_bounds__(kThreads) void permute_one_block(const int32_t* __restrict__ ids, int T, int k,
                                                              int E, int S, int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ gather,
                                                              int32_t* __restrict__ inv, uint32_t* err) {
  __shared__ int pcount[kPieces][kMaxExperts];
  __shared__ int tot[kMaxExperts];
  __shared__ int base[kMaxExperts];
  const int n = T * k;
  const int n_pieces = (n + kWave - 1) / kWave;
  int my_e[kPiecesPerWave], my_rank[kPiecesPerWave];
  rank_chunk<kPiecesPerWave>(ids, 0, n, E, pcount, my_e, my_rank, err);
  __syncthreads();
  if (threadIdx.x < E) tot[threadIdx.x] = scan_pieces(pcount, n_pieces, threadIdx.x);
  __syncthreads();
  if (threadIdx.x < kWave) scan_experts(tot, E, S, T, base, offsets);
  __syncthreads();
  scatter_chunk<kPiecesPerWave>(0, n, k, base, pcount, my_e, my_rank, gather, inv);
  fill_shared_rows(T, k, S, gather, threadIdx.x, kThreads);
}

// count pass: per-chunk expert totals
__global__ __launch_bounds__(kThreads) void permute_count(const int32_t* __restrict__ ids, int n_slots, int E,
                                                          int32_t* __restrict__ counts, uint32_t* err) {
  __shared__ int pcount[kWaves][kMaxExperts];
  const int s0 = blockIdx.x * kPermuteChunkM;
  const int n = min(kPermuteChunkM, n_slots - s0);
  const int n_pieces = (n + kWave - 1) / kWave;
  int my_e[1], my_rank[1];
  rank_chunk<1>(ids, s0, n, E, pcount, my_e, my_rank, err);
  __syncthreads();
  if (threadIdx.x < E) counts[blockIdx.x * E + threadIdx.x] = scan_pieces(pcount, n_pieces, threadIdx.x);
}

// One block: wavefront j owns the chunks [j per, (j+1) per), lane e the
// expert.  Pass 1 sums the lane's counts over the wavefront's chunks, the
// wavefronts' sums (through LDS) give each run's start, and the experts'
// totals are scanned into their first rows; pass 2 writes each chunk's base
// (first row + the counts of the expert's earlier chunks).  Integer sums:
// the same bases as a sequential walk over the chunks.
__global__ __launch_bounds__(kThreads) void permute_scan(const int32_t* __restrict__ counts, int n_chunks, int E,
                                                         int S, int T, int32_t* __restrict__ bases,
                                                         int32_t* __restrict__ offsets) {
  __shared__ int part[kWaves][kMaxExperts];   // per wavefront's chunk range and expert: its pairs
  __shared__ int tot[kMaxExperts];
  __shared__ int first[kMaxExperts];
  static_assert(kThreads == kWaves * kMaxExperts && kMaxExperts == kWave, "a wavefront covers every expert");
  // lane = expert, wavefront j = chunks [j per, (j + 1) per): every load and
  // store of a wavefront is one row of 64 experts, 256 contiguous bytes
  const int e = threadIdx.x & (kWave - 1), j = threadIdx.x >> 6;
  const int per = (n_chunks + kWaves - 1) / kWaves, c0 = min(j * per, n_chunks), c1 = min(c0 + per, n_chunks);
  const bool act = e < E;
  // up to kRegChunks chunks per wavefront (every layer of up to 16 x 16 x
  // 1024 slots): all counts loaded at once and kept in registers for the
  // second pass, so the kernel waits for one memory round trip instead of
  // four
  constexpr int kRegChunks = 16;
  const bool in_regs = per <= kRegChunks;
  int vr[kRegChunks];
  int sum = 0;
  if (in_regs) {
#pragma unroll
    for (int u = 0; u < kRegChunks; ++u) vr[u] = act && c0 + u < c1 ? counts[(size_t)(c0 + u) * E + e] : 0;
#pragma unroll
    for (int u = 0; u < kRegChunks; ++u) sum += vr[u];
  } else {
    for (int c = c0; c < c1; c += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = act && c + u < c1 ? counts[(size_t)(c + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) sum += v[u];
    }
  }
  part[j][e] = sum;
  __syncthreads();
  int before = 0;   // pairs of expert e in the chunks of wavefronts 0 .. j-1
  for (int jj = 0; jj < j; ++jj) before += part[jj][e];
  if (j == kWaves - 1) tot[e] = act ? before + sum : 0;
  __syncthreads();
  if (threadIdx.x < kWave) scan_experts(tot, E, S, T, first, offsets);
  __syncthreads();
  if (!act) return;
  int run = first[e] + before;
  if (in_regs) {
#pragma unroll
    for (int u = 0; u < kRegChunks; ++u)
      if (c0 + u < c1) {
        bases[(size_t)(c0 + u) * E + e] = run;
        run += vr[u];
      }
    return;
  }
  for (int c = c0; c < c1; c += 8) {
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = c + u < c1 ? counts[(size_t)(c + u) * E + e] : 0;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (c + u < c1) {
        bases[(size_t)(c + u) * E + e] = run;
        run += v[u];
      }
  }
}

__global__ __launch_bounds__(kThreads) void permute_scatter(const int32_t* __restrict__ ids, int T, int k,
                                                            int E, int S, const int32_t* __restrict__ bases,
                                                            int32_t* __restrict__ gather,
                                                            int32_t* __restrict__ inv) {
  __shared__ int pcount[kWaves][kMaxExperts];
  __shared__ int base[kMaxExperts];
  const int n_slots = T * k;
  const int s0 = blockIdx.x * kPermuteChunkM;
  const int n = min(kPermuteChunkM, n_slots - s0);
  const int n_pieces = (n + kWave - 1) / kWave;
  int my_e[1], my_rank[1];
  rank_chunk<1>(ids, s0, n, E, pcount, my_e, my_rank, nullptr);   // the count pass reported
  if (threadIdx.x < E) base[threadIdx.x] = bases[blockIdx.x * E + threadIdx.x];
  __syncthreads();
  if (threadIdx.x < E) scan_pieces(pcount, n_pieces, threadIdx.x);
  __syncthreads();
  scatter_chunk<1>(s0, n, k, base, pcount, my_e, my_rank, gather, inv);
  fill_shared_rows(T, k, S, gather, blockIdx.x * kThreads + threadIdx.x, gridDim.x * kThreads);
}

}  // namespace

hipError_t launch_permute(const int32_t* ids, int T, int k, int E, int S, int32_t* offsets,
                          int32_t* gather, int32_t* inv, void* ws, hipStream_t s) {
  const int n_slots = T * k;
  uint32_t* err = data_error_word(s);
  if (n_slots <= kPermuteChunk) {
    hipLaunchKernelGGL(permute_one_block, dim3(1), dim3(kThreads), 0, s, ids, T, k, E, S, offsets, gather, inv,
                       err);
    return hipGetLastError();
  }
  const int n_chunks = (n_slots + kPermuteChunkM - 1) / kPermuteChunkM;
  int32_t* counts = static_cast<int32_t*>(ws);
  int32_t* bases = counts + (size_t)n_chunks * E;
  hipLaunchKernelGGL(permute_count, dim3(n_chunks), dim3(kThreads), 0, s, ids, n_slots, E, counts, err);
  hipLaunchKernelGGL(permute_scan, dim3(1), dim3(kThreads), 0, s, counts, n_chunks, E, S, T, bases, offsets);
  hipLaunchKernelGGL(permute_scatter, dim3(n_chunks), dim3(kThreads), 0, s, ids, T, k, E, S, bases, gather, inv);
  return hipGetLastError();
}

}  // namespace moe
