// moe_grouped_swiglu: per expert group, a = silu(W_g x) * (W_u x); y = W_d a.
//
// bf16 path (decode-sized groups): the expert weights are the bytes that
// matter -- each row of W is read once from HBM and used for every token of
// its group -- so the kernel is a weight stream feeding MFMA:
//   * a block of 8 wavefronts owns a tile of output columns of one group;
//     wavefront w owns 16 of them (for the gated stage, its 16 gate rows and
//     the matching 16 up rows; for the down projection two 16-row blocks) and
//     streams those weight rows straight into registers as the A operand of
//     v_mfma_f32_16x16x32_bf16, three 32-wide k-steps in flight; the weights
//     are packed (moe_pack_weights) so every load is 1 KB of consecutive
//     bytes -- row-major rows would give 64-byte half-line requests and
//     halve the cache's request throughput;
//   * the block's activation rows (up to 16 gathered tokens, the B operand)
//     are staged once into LDS for the whole reduction length: one barrier,
//     then every wavefront streams on its own with no activation traffic;
//     in the gated stage, groups of more than 16 rows (the shared experts
//     see every token) take items of 32 or 64 rows, staged in K-chunks, so
//     each weight fragment is streamed once per 64 rows instead of per 16;
//   * each block finds its (group, column tile, 16-row range) from the group
//     offsets on the device, so untouched experts are never read and the
//     launch holds few empty blocks; the ranges of one group and tile run
//     back to back on one XCD and share its L2 copy of the weights;
// The fp32 reduction order along K is fixed (chunk by chunk, 32 per MFMA)
// and does not depend on how many rows a group has.
//
// fp32 path (the tiny fp32 configuration): one thread per output element,
// plain sequential fp32 dot products.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"
#include "validate.hpp"

namespace moe {
namespace {


// fp32 path (the tiny fp32 configuration, one code path at every size):
// libm's expf and an IEEE division.  The bf16 paths use silu_bf16path.
__device__ __forceinline__ float silu_f32path(float z) { return z / (1.0f + expf(-z)); }

constexpr int kRoutedMaxPairs = kPermuteChunk;   // (token, slot) pairs of one routed launch (host-checked)
constexpr int kWaves = 8;                 // wavefronts per block
constexpr int kBlockThreads = kWaves * 64;
constexpr int kStage1 = 5;                // 16-byte activation segments per thread staged before the weights
constexpr int kRows = 16;                 // activation rows per block (one MFMA block)

__host__ __device__ constexpr int lds_row(int K) { return K + 8; }  // padded LDS row (bf16): conflict-free

// One wavefront's stream: two sets of 16 weight rows (the gate rows and the
// matching up rows, or two neighbouring 16-row output blocks) over the full
// reduction length K, against the block's 16 activation rows in LDS.  Lane
// l supplies weight row l%16 and activation row l%16 at k-offset 8*(l/16) of
// every 32-wide MFMA step.  D steps of weight loads stay in flight in
// rotating registers; the loop body has no conditional load (a conditional
// load makes the compiler drain every outstanding load).
// Weight loads: non-temporal where a tile is read by one block (measured on
// MI355X: 6.5 TB/s streamed against 3.5 for ordinary loads of distinct
// lines).  A gate/up tile of a group with several 16-row ranges is read by
// several blocks at about the same time; there ordinary loads let the later
// reads hit L2 (a non-temporal line is not kept), which measured ~3 us
// faster per layer at 32 x 4 tokens.  The down projection measured the same
// either way and stays non-temporal.
template <bool NT>
__device__ __forceinline__ uint4 wload(const bf16_t* p) { return NT ? ldg16_stream(p) : ldg16(p); }

template <int D, bool NT>
__device__ __forceinline__ void stream_rows(const bf16_t* wa, const bf16_t* wb, const bf16_t* xs, int nK,
                                            uint4* ra, uint4* rb, f32x4_t& acc_a, f32x4_t& acc_b) {
  auto mma = [&](int d, int kk) __attribute__((always_inline)) {
    const bf16x8_t bx = as_bf16x8(*reinterpret_cast<const uint4*>(xs + kk * 32));
    acc_a = mfma16x16x32(as_bf16x8(ra[d]), bx, acc_a);
    acc_b = mfma16x16x32(as_bf16x8(rb[d]), bx, acc_b);
  };
  const int nfull = nK / D;
  // Enter the loop with no load outstanding (the staging before it already
  // waited on younger loads), so the wait at the loop head needs to cover
  // only the slot it consumes.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  for (int g = 0; g < nfull; ++g) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      mma(d, g * D + d);
      const int kk = min((g + 1) * D + d, nK - 1);  // past the end: a repeat of the last step, never used
      ra[d] = wload<NT>(wa + kk * 1024);
      rb[d] = wload<NT>(wb + kk * 1024);
    }
    // keep each step's order -- LDS read, its two MFMAs, then the two loads
    // that refill the same slot -- so loads leave in step order and the wait
    // before a step covers only its own slot, not the whole pipeline
#pragma unroll
    for (int d = 0; d < D; ++d) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);  // VMEM read
    }
  }
  const int rem = nK - nfull * D;
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (d < rem) mma(d, nfull * D + d);
}

// The multi-row form of stream_rows for items of RB 16-row blocks: one
// chunk of k-steps [s0, s0 + cl) against the chunk's activation columns in
// LDS (row stride ldr, the chunk's first k-step at column 0), each weight
// fragment feeding 2*RB MFMAs.  The weight pipeline runs on across chunks:
// chunks start at multiples of D, so slot d always holds a step s with
// s % D == d, and the loads issued by a chunk's last D steps are the next
// chunk's first steps.
template <int D, int RB, bool NT>
__device__ __forceinline__ void stream_chunk(const bf16_t* wa, const bf16_t* wb, const bf16_t* xs, int ldr,
                                             int s0, int cl, int nK, uint4* ra, uint4* rb, f32x4_t* acc_a,
                                             f32x4_t* acc_b) {
  auto mma = [&](int d, int lk) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const bf16x8_t bx = as_bf16x8(*reinterpret_cast<const uint4*>(xs + r * kRows * ldr + lk * 32));
      acc_a[r] = mfma16x16x32(as_bf16x8(ra[d]), bx, acc_a[r]);
      acc_b[r] = mfma16x16x32(as_bf16x8(rb[d]), bx, acc_b[r]);
    }
  };
  const int nfull = cl / D;
  for (int g = 0; g < nfull; ++g) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      mma(d, g * D + d);
      const int kk = min(s0 + (g + 1) * D + d, nK - 1);
      ra[d] = wload<NT>(wa + kk * 1024);
      rb[d] = wload<NT>(wb + kk * 1024);
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
      __builtin_amdgcn_sched_group_barrier(0x100, RB, 0);      // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * RB, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);       // VMEM read
    }
  }
  const int rem = cl - nfull * D;
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (d < rem) mma(d, nfull * D + d);
}

// Items of more than 16 rows (groups with more than 16 rows: a shared
// expert sees every token): an item of RB = 2 or 4 row blocks streams each
// weight fragment once for 32 or 64 rows, where 16-row items would stream
// it once per 16 rows -- the bytes moved to the CUs, not the HBM bytes, are
// what the weight stream pays for.  The rows do not fit LDS for the whole
// reduction, so they pass through it in chunks of chunk_steps(RB) k-steps:
// each thread holds its share of the next chunk in a few registers, loaded
// while the current chunk streams, and writes it to LDS between two
// barriers.  A full chunk is straight-line code (stream_chunk_fixed), so
// the compiler's waits on the weight slots stay exact around the prefetch.
// A row's fp32 sums run over the same k-steps in the same order whatever
// its item, so results do not depend on RB.
constexpr int chunk_steps(int RB) { return RB == 4 ? 6 : 12; }
constexpr int chunk_regs(int RB) { return (RB * kRows * chunk_steps(RB) * 4 + kBlockThreads - 1) / kBlockThreads; }
// LDS bytes of a chunk of RB row blocks (rows padded by 8 elements)
constexpr size_t chunk_lds(int RB) { return (size_t)RB * kRows * (chunk_steps(RB) * 32 + 8) * sizeof(bf16_t); }

// A full chunk of CL k-steps [s0, s0 + CL), unrolled; `prefetch` (the next
// chunk's activation loads) is issued after the first D steps' weight loads.
template <int D, int RB, int CL, int NPF, bool NT, typename F>
__device__ __forceinline__ void stream_chunk_fixed(const bf16_t* wa, const bf16_t* wb, const bf16_t* xs, int ldr,
                                                   int s0, int nK, uint4* ra, uint4* rb, f32x4_t* acc_a,
                                                   f32x4_t* acc_b, F&& prefetch) {
  static_assert(CL % D == 0 && CL >= 2 * D, "a full chunk is at least two pipeline groups");
#pragma unroll
  for (int g = 0; g < CL / D; ++g) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const bf16x8_t bx = as_bf16x8(*reinterpret_cast<const uint4*>(xs + r * kRows * ldr + (g * D + d) * 32));
        acc_a[r] = mfma16x16x32(as_bf16x8(ra[d]), bx, acc_a[r]);
        acc_b[r] = mfma16x16x32(as_bf16x8(rb[d]), bx, acc_b[r]);
      }
      const int kk = min(s0 + (g + 1) * D + d, nK - 1);
      ra[d] = wload<NT>(wa + kk * 1024);
      rb[d] = wload<NT>(wb + kk * 1024);
    }
    if (g == 0) prefetch();
#pragma unroll
    for (int d = 0; d < D; ++d) {
      __builtin_amdgcn_sched_group_barrier(0x100, RB, 0);      // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * RB, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);       // VMEM read
    }
    if (g == 0) __builtin_amdgcn_sched_group_barrier(0x020, NPF, 0);   // the prefetch
  }
}

// GATED: x = token rows [T,K] read through gather, W = [G, 2N, K] packed as
//        gate/up pairs (gate rows 16p.., up rows N+16p..), out = a [n_rows, N]; wavefront w owns output
//        columns 16w..16w+15 of a 128-column block tile (its 16 gate rows and
//        16 up rows are the two streamed row sets).
// plain: x = activation rows [n_rows, K] read directly, W = [G, N, K] packed
//        as row pairs, out = y [n_rows, N]; wavefront w owns output columns 32w..32w+31 of a
//        256-column block tile (two 16-row sets), so that every wavefront
//        streams as many bytes per k-step as in the gated stage.
// A block of 8 wavefronts owns one column tile of one group and one range of
// up to 16 rows, staged once into LDS (one barrier) and shared by its waves.
//
// K split (one-group launches, the dense projections): the block's 8
// wavefronts are CG column groups x KS slices of the reduction (KS = 2^
// ks_log2, CG = 8 / KS); slice ks streams k-steps [ks nK/KS, (ks+1) nK/KS)
// and the KS partial sums of a column group are added in slice order
// through LDS.  A dense layer has one group, so with one column group per
// wavefront it would get as few as N / 256 blocks (5 for N = 1280, each
// streaming 1.8 MB at K = 3584) where an expert launch gets one per touched
// expert and tile; the split multiplies the blocks by KS.  KS depends on
// the weight shape only, never on the number of rows, so a row's result
// does not depend on the batch.
// The 16-row item form keeps 6 k-steps of weights in flight per wavefront
// (the multi-row forms 3).  Bandwidth per block is about its bytes in
// flight over the memory latency: a launch with few items (batch 1: ~20
// touched experts) needs the depth to cover the latency at all, and in a
// launch of many items it shortens the tail where the last blocks stream
// alone.  Measured against a 3-deep ring from 1 to 1,000 tokens it was as
// fast or faster at every size, although the down kernel then holds 2
// blocks per CU instead of 3.  The depth does not change any row's k-order.
template <bool GATED, bool ROUTED>
__global__ __launch_bounds__(kBlockThreads) void skinny_kernel(
    const bf16_t* __restrict__ x, const int32_t* __restrict__ gather,
    const int32_t* __restrict__ offsets, int G, int n_rows, int T,
    const bf16_t* __restrict__ W, int K, int N, int n_ctiles, int ks_log2, int chunk_cfg, bf16_t* out,
    const bf16_t* res, RoutedArgs rt, uint32_t* err) {
  static_assert(!ROUTED || GATED, "only the gate/up stage derives its rows from the expert ids");
  constexpr int D = 3;                    // k-steps of weights in flight per wavefront (64-row items)
  constexpr int DB = 6;                   // the same for 16-row items
  constexpr int WCOLS = GATED ? 16 : 32;  // output columns per wavefront
  extern __shared__ __align__(16) bf16_t xl[];   // [kRows][lds_row(K)]

  // Work items are (group g, column tile ct, 16-row range) for the non-empty
  // ranges.  Pair (g, ct) belongs to XCD (g*n_ctiles + ct) % 8 (block b runs
  // on XCD b % 8); on each XCD the items are ordered by group, tile, range,
  // so the ranges of one large group (a shared expert sees every token) run
  // back to back on one XCD and share its L2 copy of the weights.  The
  // groups go in reverse order: the shared experts, last in group order,
  // have the most rows and the longest items, and their blocks, dispatched
  // first, no longer end the launch (128-token step: 1.153 -> 1.124 ms).
  // Block b takes the (b/8)-th item of XCD b%8; the launch holds an upper
  // bound of items per XCD and the surplus blocks, last in every XCD's list,
  // exit.
  // Wavefront 0 finds the item: lane l handles groups l and l+64 (G <= 128),
  // counts its items on this XCD, and a wavefront prefix sum places them.
  __shared__ int item_g, item_ct, item_r0, item_r1, item_gs, item_rb;
  __shared__ int s_cnt[2 * kWave];   // ROUTED: rows per group
  __shared__ int s_tok[4 * kRows];   // ROUTED: tokens of the block's rows (routed groups)
  __shared__ int s_ids[ROUTED ? kRoutedMaxPairs : 1];   // ROUTED: the (token, slot) expert ids, clamped
  __shared__ __align__(16) int s_chunk[ROUTED ? kRoutedMaxPairs / kWave : 4];   // ROUTED: the group's pairs per 64-pair chunk
  // row blocks per item allowed (chunk_cfg: 0 = 16-row items only)
  const int rb_max = (chunk_cfg >> 16) ? 4 : (chunk_cfg & 0xffff) ? 2 : 1;
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  // Where a CU holds two blocks, the one that starts streaming first takes
  // nearly all of the CU's memory issue and the other's staging loads wait
  // behind its weight stream (measured per block: the second block's staging
  // took 3-4x as long).  The set-up and staging run at raised wave priority
  // so that both blocks reach the stream early; streaming runs at the
  // normal priority.
  __builtin_amdgcn_s_setprio(3);
  if (ROUTED) {
    // rows per group: a histogram of the (token, slot) expert ids; each
    // shared group holds every token.  The ids stay in LDS for the token
    // scan below.  Every thread loads all its ids (at most 8) before using
    // any, so the loads overlap.
    static_assert(kRoutedMaxPairs <= 8 * kBlockThreads, "8 ids per thread");
    for (int g = threadIdx.x; g < G; g += kBlockThreads) s_cnt[g] = g < rt.E ? 0 : T;
    const int np = T * rt.k;
    int idv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) idv[u] = rt.ids[min((int)threadIdx.x + u * kBlockThreads, np - 1)];
    lds_barrier();
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = threadIdx.x + u * kBlockThreads;
      if (p < np) {
        const int e = clamp_report(idv[u], 0, rt.E - 1, err, kDataErrExpertId);
        s_ids[p] = e;
        atomicAdd(&s_cnt[e], 1);
      }
    }
    lds_barrier();
  }
  if (threadIdx.x < kWave) {
    const int l = threadIdx.x;
    int r0[2], r1[2], nr[2], nc[2], rbs[2];
    if (ROUTED) {
      // group row ranges: an exclusive scan of the counts (routed groups in
      // expert order, then the shared groups), as moe_permute lays them out
      int c[2], inc[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int g = l + h * kWave;
        c[h] = g < G ? s_cnt[g] : 0;
        inc[h] = c[h];
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
          const int v = __shfl_up(inc[h], o, kWave);
          if (l >= o) inc[h] += v;
        }
      }
      inc[1] += __shfl(inc[0], kWave - 1, kWave);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        r1[h] = inc[h];
        r0[h] = inc[h] - c[h];
      }
      if (blockIdx.x == 0) {  // the offsets for the down projection and the combine
#pragma unroll
        for (int h = 0; h < 2; ++h)
          if (l + h * kWave <= G) rt.offsets[l + h * kWave] = l + h * kWave < G ? r0[h] : n_rows;
      }
      // the items run in reverse group order (below): lane l, half h takes
      // group G - 1 - (l + 64 h), whose range another lane holds
      int q0[2], q1[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int gg = max(G - 1 - (l + h * kWave), 0), sl = gg & (kWave - 1);
        const int a0 = __shfl(r0[0], sl, kWave), a1 = __shfl(r0[1], sl, kWave);
        const int b0 = __shfl(r1[0], sl, kWave), b1 = __shfl(r1[1], sl, kWave);
        q0[h] = gg >= kWave ? a1 : a0;
        q1[h] = gg >= kWave ? b1 : b0;
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        r0[h] = q0[h];
        r1[h] = q1[h];
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int g = G - 1 - (l + h * kWave);   // groups in reverse order
      if (!ROUTED) {
        // (block 0 reports ranges outside [0, n_rows] or decreasing)
        uint32_t* const eb = blockIdx.x == 0 ? err : nullptr;
        r0[h] = g >= 0 ? clamp_report(offsets[g], 0, n_rows, eb, kDataErrOffsets) : 0;
        r1[h] = g >= 0 ? clamp_report(offsets[g + 1], r0[h], n_rows, eb, kDataErrOffsets) : 0;
      }
      const int rows = r1[h] - r0[h];
      rbs[h] = rows > 2 * kRows && rb_max >= 4 ? 4 : rows > kRows && rb_max >= 2 ? 2 : 1;
      nr[h] = (rows + rbs[h] * kRows - 1) / (rbs[h] * kRows);
      // tiles of group g on this XCD: ct = c0, c0+8, ... < n_ctiles
      const int c0 = ((xcd - g * n_ctiles) % 8 + 8) % 8;
      nc[h] = g >= 0 && g < G && c0 < n_ctiles ? (n_ctiles - c0 + 7) / 8 : 0;
    }
    int cnt[2] = {nr[0] * nc[0], nr[1] * nc[1]};
    int incl[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      incl[h] = cnt[h];
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int v = __shfl_up(incl[h], o, kWave);
        if (l >= o) incl[h] += v;
      }
    }
    incl[1] += __shfl(incl[0], kWave - 1, kWave);
    if (l == 0) item_g = -1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int first = incl[h] - cnt[h];
      if (j >= first && j < incl[h]) {
        const int g = G - 1 - (l + h * kWave);
        const int li = j - first;              // ordered by tile, then range
        const int c0 = ((xcd - g * n_ctiles) % 8 + 8) % 8;
        item_g = g;
        item_ct = c0 + 8 * (li / nr[h]);
        item_r0 = r0[h] + (li % nr[h]) * rbs[h] * kRows;
        item_r1 = r1[h];
        item_gs = r0[h];
        item_rb = rbs[h];
      }
    }
  }
  lds_barrier();
  const int g = item_g;
  if (g < 0) return;
  const int ct = item_ct;
  const int mstart = item_r0;
  const int irb = item_rb;
  const int mr = min(kRows * irb, item_r1 - mstart);
  const int r_begin = ROUTED ? item_gs : clampi(offsets[g], 0, n_rows);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int KS = 1 << ks_log2, CG = kWaves >> ks_log2;
  const int cg = wave & (CG - 1), ks = wave >> (3 - ks_log2);
  const int col0 = ct * (CG * WCOLS) + cg * WCOLS;
  const bool active = col0 < N;
  // packed weights: [group][pair][k-step][set][lane][8]; a pair is this
  // wavefront's two 16-row sets, a (pair, k-step) is 2 KB of consecutive bytes
  const int nK = K / 32;
  const int nKs = nK >> ks_log2, k0 = ks * nKs;   // this wavefront's k-steps
  const int n_pairs = GATED ? N / 16 : (N + 31) / 32;
  const int pair = min(col0 / WCOLS, n_pairs - 1);  // inactive wavefronts load a valid pair, store nothing
  const bf16_t* wa = W + (((size_t)g * n_pairs + pair) * nK + k0) * 1024 + lane * 8;
  const bf16_t* wb = wa + 512;
  const int ldr = lds_row(K);
  const int nseg = K / 8;                 // 16-byte segments per activation row

  // ordinary weight loads where several items read a gate/up tile (see wload)
  const bool shared_tile = GATED && item_r1 - r_begin > kRows * irb;
  const bool pre = ROUTED && g < rt.E;   // a routed group: rows from the token scan
  auto token_scan = [&]() __attribute__((always_inline)) {
    // the tokens of this block's rows: the group's (token, slot) pairs in
    // ascending order, ranks mstart - r_begin .. +mr; the blocks of the first
    // column tile also record each pair's row (inv) for the combine.
    // Wavefront w takes the 64-pair chunks w, w + 8, ...: it counts the
    // group's pairs in each, the counts of the chunks before a chunk give
    // its first rank, and the pairs of the wanted ranks are written.
    const int np = T * rt.k, nch = (np + kWave - 1) / kWave;
    const int want0 = mstart - r_begin, want1 = want0 + mr;
#pragma unroll 1
    for (int c = wave; c < nch; c += kWaves) {
      const int p = c * kWave + lane;
      const unsigned long long m = __ballot(p < np && s_ids[p] == g);
      if (lane == 0) s_chunk[c] = __popcll(m);
    }
    lds_barrier();
    const bool owner = ct == 0;
    const int4* cnt4 = reinterpret_cast<const int4*>(s_chunk);
    int base4 = 0, c4 = 0;   // pairs of the group in chunks [0, c4), c4 a multiple of 4
#pragma unroll 1
    for (int c = wave; c < nch; c += kWaves) {
      for (; c4 + 4 <= c; c4 += 4) {
        const int4 q = cnt4[c4 >> 2];
        base4 += q.x + q.y + q.z + q.w;
      }
      int base = base4;   // pairs of the group in chunks [0, c)
      for (int cc = c4; cc < c; ++cc) base += s_chunk[cc];
      if (base >= want1) break;
      const int p = c * kWave + lane;
      const bool f = p < np && s_ids[p] == g;
      const unsigned long long m = __ballot(f);
      const int rank = base + __popcll(m & ((1ull << lane) - 1ull));
      if (f && rank >= want0 && rank < want1) {
        s_tok[rank - want0] = p / rt.k;
        if (owner) rt.inv[p] = r_begin + rank;
      }
    }
    lds_barrier();
  };

  // lane holds D[col 4*(lane/16)+v][row lane%16]: 4 consecutive output columns of one row
  auto emit = [&](f32x4_t acc_a, f32x4_t acc_b, int row) __attribute__((always_inline)) {
    if (row >= mr) return;
    bf16_t* orow = out + (size_t)(mstart + row) * N + col0 + 4 * (lane >> 4);
    if (GATED) {
      uint2 pk;
      pk.x = pack_bf16x2(silu_bf16path(acc_a[0]) * acc_b[0], silu_bf16path(acc_a[1]) * acc_b[1]);
      pk.y = pack_bf16x2(silu_bf16path(acc_a[2]) * acc_b[2], silu_bf16path(acc_a[3]) * acc_b[3]);
      *reinterpret_cast<uint2*>(orow) = pk;
    } else {
      if (res) {
        // out = residual + y: y rounded to bf16 first, then the fp32 sum
        // rounded once (the same bits as moe_combine adding y as a shared row)
        const bf16_t* rrow = res + (size_t)(mstart + row) * N + col0 + 4 * (lane >> 4);
        auto add = [](float a, uint32_t r16) {
          return __uint_as_float(r16 << 16) + __uint_as_float((uint32_t)f32_to_bf16(a) << 16);
        };
        const uint2 ra2 = *reinterpret_cast<const uint2*>(rrow);
        uint2 rb2 = ra2;
        if (col0 + 16 < N) rb2 = *reinterpret_cast<const uint2*>(rrow + 16);
        acc_a[0] = add(acc_a[0], ra2.x & 0xffffu); acc_a[1] = add(acc_a[1], ra2.x >> 16);
        acc_a[2] = add(acc_a[2], ra2.y & 0xffffu); acc_a[3] = add(acc_a[3], ra2.y >> 16);
        acc_b[0] = add(acc_b[0], rb2.x & 0xffffu); acc_b[1] = add(acc_b[1], rb2.x >> 16);
        acc_b[2] = add(acc_b[2], rb2.y & 0xffffu); acc_b[3] = add(acc_b[3], rb2.y >> 16);
      }
      uint2 pa, pb;
      pa.x = pack_bf16x2(acc_a[0], acc_a[1]);
      pa.y = pack_bf16x2(acc_a[2], acc_a[3]);
      pb.x = pack_bf16x2(acc_b[0], acc_b[1]);
      pb.y = pack_bf16x2(acc_b[2], acc_b[3]);
      *reinterpret_cast<uint2*>(orow) = pa;
      if (col0 + 16 < N) *reinterpret_cast<uint2*>(orow + 16) = pb;
    }
  };
  // the token (or activation row) of item row `row` (rows past the item repeat a valid row)
  auto src_row = [&](int row) __attribute__((always_inline)) {
    const int r = mstart + min(row, mr - 1);
    if (ROUTED) return clampi(g < rt.E ? s_tok[min(row, mr - 1)] : r - r_begin, 0, T - 1);
    if (GATED)
      return gather ? clamp_report(gather[r], 0, T - 1, err, kDataErrRowIndex)
                    : clamp_report(r - r_begin, 0, T - 1, err, kDataErrOffsets);
    return r;
  };

  auto body = [&](auto nt) __attribute__((always_inline)) {
    constexpr bool NT = decltype(nt)::value;
    uint4 ra[DB], rb[DB];
    if constexpr (ROUTED) {
      // The first weight steps depend on the item only: they go out before
      // the token scan that finds a routed group's rows, so their latency
      // overlaps the scan and the staging.
#pragma unroll
      for (int d = 0; d < DB; ++d) {
        const int kk = min(d, nKs - 1);
        ra[d] = wload<NT>(wa + kk * 1024);
        rb[d] = wload<NT>(wb + kk * 1024);
      }
      if (pre) token_scan();
    }
    // Stage the range's activation rows (rows past the group repeat a valid
    // row).  Without a token scan their loads go out first, then the weights
    // of the first DB steps: loads retire in issue order, so the LDS stores
    // below wait for the activation rows only and the weight latency
    // overlaps the staging.
    // The first round covers kStage1 segments per thread (K <= 1280 in one
    // round); longer rows stage the rest after it.
    const int nstg = kRows * nseg;
    uint4 v[kStage1];
    int dst[kStage1];
#pragma unroll
    for (int u = 0; u < kStage1; ++u) {
      const int idx = min((int)threadIdx.x + u * kBlockThreads, nstg - 1);
      const int row = idx / nseg, seg = idx % nseg;
      v[u] = ldg16(x + (size_t)src_row(row) * K + seg * 8);
      dst[u] = row * ldr + seg * 8;
    }
    if constexpr (!ROUTED) {
#pragma unroll
      for (int d = 0; d < DB; ++d) {
        const int kk = min(d, nKs - 1);
        ra[d] = wload<NT>(wa + kk * 1024);
        rb[d] = wload<NT>(wb + kk * 1024);
      }
    }
#pragma unroll
    for (int u = 0; u < kStage1; ++u)
      if ((int)threadIdx.x + u * kBlockThreads < nstg) *reinterpret_cast<uint4*>(xl + dst[u]) = v[u];
    for (int i = threadIdx.x + kStage1 * kBlockThreads; i < nstg; i += kBlockThreads) {
      const int row = i / nseg, seg = i % nseg;
      *reinterpret_cast<uint4*>(xl + row * ldr + seg * 8) = ldg16(x + (size_t)src_row(row) * K + seg * 8);
    }
    lds_barrier();

    __builtin_amdgcn_s_setprio(0);
    f32x4_t acc_a = f32x4_t{0.f, 0.f, 0.f, 0.f}, acc_b = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (active || KS > 1)   // with a K split every wavefront streams (inactive ones a valid pair) to reach the barriers
      stream_rows<DB, NT>(wa, wb, xl + (lane & 15) * ldr + (lane >> 4) * 8 + k0 * 32, nKs, ra, rb, acc_a, acc_b);
    if (KS > 1) {
      // partial sums of the slices, added in slice order; the staged rows are
      // dead, their LDS holds the partials [wavefront][lane][8]
      float* red = reinterpret_cast<float*>(xl);
      lds_barrier();
      if (ks > 0) {
        *reinterpret_cast<f32x4_t*>(red + (wave * kWave + lane) * 8) = acc_a;
        *reinterpret_cast<f32x4_t*>(red + (wave * kWave + lane) * 8 + 4) = acc_b;
      }
      lds_barrier();
      if (ks == 0)
        for (int q = 1; q < KS; ++q) {
          acc_a += *reinterpret_cast<const f32x4_t*>(red + ((cg + q * CG) * kWave + lane) * 8);
          acc_b += *reinterpret_cast<const f32x4_t*>(red + ((cg + q * CG) * kWave + lane) * 8 + 4);
        }
    }
    if (active && ks == 0) emit(acc_a, acc_b, lane & 15);
  };

  // items of RB > 1 row blocks: the activations pass through LDS in chunks
  // (K split off: ks == 0, k0 == 0)
  auto chunked = [&](auto rbc, auto nt) __attribute__((always_inline)) {
    constexpr int RB = decltype(rbc)::value;
    constexpr bool NT = decltype(nt)::value;
    constexpr int RR = RB * kRows;
    // weight k-steps in flight: 32-row items take the 16-row items' 6-deep
    // ring (they had ended the launch at half the 16-row items' stream rate;
    // 6 deep, 118 VGPRs, still two blocks per CU); 64-row items stay at 3
    constexpr int DR = RB == 2 ? DB : D;
    constexpr int CL = chunk_steps(RB);
    constexpr int NSC = CL * 4;          // 16-byte segments of a row in one chunk
    constexpr int NPF = chunk_regs(RB);  // of them, per thread
    constexpr int LDC = CL * 32 + 8;     // LDS row stride of a chunk (padded)
    // every thread holds exactly NPF segments: no conditional store for the
    // compiler to sink a prefetch load into
    static_assert(RR * NSC == NPF * kBlockThreads, "a chunk is a whole number of segments per thread");
    // a routed group's token scan comes first here (issuing the weights
    // before it, as the 16-row form does, took the kernel to 140 VGPRs: one
    // block per CU)
    if (pre) token_scan();
    // this thread's segments u of a chunk: row offsets in x and segment numbers
    int srow[NPF], sseg[NPF];
#pragma unroll
    for (int u = 0; u < NPF; ++u) {
      const int idx = threadIdx.x + u * kBlockThreads;
      srow[u] = src_row(idx / NSC) * K;
      sseg[u] = idx % NSC;
    }
    uint4 pf[NPF];
    // the chunk starting at k-step c0 (segments past the end of K repeat the
    // row's last valid segment, never read)
    auto ld_chunk = [&](int c0) __attribute__((always_inline)) {
      const int last = (nK - c0) * 4 - 1;
#pragma unroll
      for (int u = 0; u < NPF; ++u) pf[u] = ldg16(x + srow[u] + c0 * 32 + min(sseg[u], last) * 8);
    };
    auto st_chunk = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < NPF; ++u) {
        const int idx = threadIdx.x + u * kBlockThreads;
        *reinterpret_cast<uint4*>(xl + (idx / NSC) * LDC + (idx % NSC) * 8) = pf[u];
      }
    };
    // the first chunk's loads go out before the weights of the first D
    // steps, so its LDS stores wait for the activation rows only
    ld_chunk(0);
    uint4 ra[DR], rb[DR];
#pragma unroll
    for (int d = 0; d < DR; ++d) {
      const int kk = min(d, nK - 1);
      ra[d] = wload<NT>(wa + kk * 1024);
      rb[d] = wload<NT>(wb + kk * 1024);
    }
    st_chunk();
    lds_barrier();
    __builtin_amdgcn_s_setprio(0);
    f32x4_t acc_a[RB], acc_b[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) acc_a[r] = acc_b[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const bf16_t* xs = xl + (lane & 15) * LDC + (lane >> 4) * 8;
    int c0 = 0;
    for (; c0 + CL < nK; c0 += CL) {    // full chunks with a successor
      stream_chunk_fixed<DR, RB, CL, NPF, NT>(wa, wb, xs, LDC, c0, nK, ra, rb, acc_a, acc_b,
                                             [&]() __attribute__((always_inline)) { ld_chunk(c0 + CL); });
      lds_barrier();                    // every wavefront is done with this chunk
      st_chunk();
      lds_barrier();
    }
    stream_chunk<DR, RB, NT>(wa, wb, xs, LDC, c0, nK - c0, nK, ra, rb, acc_a, acc_b);   // the last chunk
    if (active)
#pragma unroll
      for (int r = 0; r < RB; ++r) emit(acc_a[r], acc_b[r], r * kRows + (lane & 15));
  };

  if constexpr (GATED) {
    if (irb == 4) {
      if (shared_tile) chunked(std::integral_constant<int, 4>{}, std::false_type{});
      else chunked(std::integral_constant<int, 4>{}, std::true_type{});
      return;
    }
    if (irb == 2) {
      if (shared_tile) chunked(std::integral_constant<int, 2>{}, std::false_type{});
      else chunked(std::integral_constant<int, 2>{}, std::true_type{});
      return;
    }
  }
  if (shared_tile) {
    body(std::false_type{});
  } else {
    body(std::true_type{});
  }
}

template <bool GATED, bool ROUTED = false>
hipError_t launch_skinny(const bf16_t* x, const int32_t* gather, const int32_t* offsets, int G, int n_rows, int T,
                         const bf16_t* W, int K, int N, bf16_t* out, hipStream_t s, RoutedArgs ra = {},
                         const bf16_t* res = nullptr) {
  // K split for one-group launches (by the weight shape only): enough
  // slices for ~64 column tiles, each slice at least 2 k-steps, the staged
  // rows' LDS large enough for the partials (K >= 512)
  const int nK = K / 32;
  const int n_cg = GATED ? N / 16 : (N + 31) / 32;
  int ks_log2 = 0;
  if (G == 1 && !ROUTED && K >= 512)
    while (ks_log2 < 3 && (n_cg << ks_log2) < 64 * kWaves && nK % (2 << ks_log2) == 0 && nK / (2 << ks_log2) >= 2)
      ++ks_log2;
  const int tile = (kWaves >> ks_log2) * (GATED ? 16 : 32);
  const int n_ctiles = (N + tile - 1) / tile;
  // items on one XCD <= ceil(n_ctiles / 8) * sum over groups of ceil(rows / 16)
  //                  <= ceil(n_ctiles / 8) * (n_rows / 16 + G)
  const int per_xcd = (n_ctiles + 7) / 8 * ((n_rows + kRows - 1) / kRows + G);
  const int blocks = 8 * per_xcd;
  // items of 32 / 64 rows for groups of more than 16 rows (not with a K
  // split)
  size_t lds = (size_t)kRows * lds_row(K) * sizeof(bf16_t);
  int chunk_cfg = 0;
  if (GATED && ks_log2 == 0) {
    chunk_cfg = 2 | (4 << 16);
    lds = std::max(lds, std::max(chunk_lds(2), chunk_lds(4)));
  }
  auto kern = &skinny_kernel<GATED, ROUTED>;
  if (lds > 64 * 1024) {  // K > 2040: allow up to the CU's 160 KB of LDS
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(kBlockThreads), lds, s, x, gather, offsets, G, n_rows, T, W, K, N,
                     n_ctiles, ks_log2, chunk_cfg, out, res, ra, data_error_word(s));
  return hipGetLastError();
}

// ---------------------------------------------------------------- fp32 path

__device__ __forceinline__ int find_group(const int32_t* offsets, int G, int n_rows, int r, int* r_begin) {
  for (int g = 0; g < G; ++g) {
    const int a = clampi(offsets[g], 0, n_rows), e = clampi(offsets[g + 1], a, n_rows);
    if (r >= a && r < e) {
      *r_begin = a;
      return g;
    }
  }
  return -1;
}

// block 0 checks the group row ranges once: within [0, n_rows], non-decreasing
__device__ __forceinline__ void check_offsets(const int32_t* offsets, int G, int n_rows, uint32_t* err) {
  if (blockIdx.x != 0 || !err) return;
  for (int g = threadIdx.x; g < G; g += blockDim.x) {
    const int a = offsets[g], b = offsets[g + 1];
    report_error(err, a < 0 || b < a || b > n_rows, kDataErrOffsets);
  }
}

__global__ __launch_bounds__(256) void f32_gate_up_kernel(const float* __restrict__ x,
                                                          const int32_t* __restrict__ gather,
                                                          const int32_t* __restrict__ offsets, int G,
                                                          int n_rows, int T, const float* __restrict__ wgu,
                                                          int H, int I, float* __restrict__ act, uint32_t* err) {
  check_offsets(offsets, G, n_rows, err);
  const int r = blockIdx.x;
  int r_begin = 0;
  const int g = find_group(offsets, G, n_rows, r, &r_begin);
  if (g < 0) return;
  const int t = gather ? clamp_report(gather[r], 0, T - 1, err, kDataErrRowIndex)
                       : clamp_report(r - r_begin, 0, T - 1, err, kDataErrOffsets);
  const float* xr = x + (size_t)t * H;
  for (int c = threadIdx.x; c < I; c += blockDim.x) {
    const float* wg = wgu + ((size_t)g * 2 * I + c) * H;
    const float* wu = wg + (size_t)I * H;
    float a = 0.f, u = 0.f;
    for (int h = 0; h < H; ++h) {
      a = fmaf(wg[h], xr[h], a);
      u = fmaf(wu[h], xr[h], u);
    }
    act[(size_t)r * I + c] = silu_f32path(a) * u;
  }
}

__global__ __launch_bounds__(256) void f32_down_kernel(const float* __restrict__ act,
                                                       const int32_t* __restrict__ offsets, int G, int n_rows,
                                                       const float* __restrict__ wd, int H, int I, float* y,
                                                       const float* res, uint32_t* err) {
  check_offsets(offsets, G, n_rows, err);
  const int r = blockIdx.x;
  int r_begin = 0;
  const int g = find_group(offsets, G, n_rows, r, &r_begin);
  if (g < 0) return;
  const float* ar = act + (size_t)r * I;
  for (int o = threadIdx.x; o < H; o += blockDim.x) {
    const float* w = wd + ((size_t)g * H + o) * I;
    float acc = 0.f;
    for (int c = 0; c < I; ++c) acc = fmaf(w[c], ar[c], acc);
    y[(size_t)r * H + o] = res ? res[(size_t)r * H + o] + acc : acc;
  }
}

}  // namespace

hipError_t launch_gate_up(const void* x, const int32_t* gather, const int32_t* offsets, int G, int n_rows,
                          const void* w_gate_up, int T, int H, int I, int max_rows, int dtype, void* act,
                          hipStream_t s) {
  if (dtype == kF32) {
    hipLaunchKernelGGL(f32_gate_up_kernel, dim3(n_rows), dim3(256), 0, s, static_cast<const float*>(x), gather,
                       offsets, G, n_rows, T, static_cast<const float*>(w_gate_up), H, I,
                       static_cast<float*>(act), data_error_word(s));
    return hipGetLastError();
  }
  if (gemm_path_ok(H, I, max_rows))
    return launch_gemm(true, x, gather, offsets, G, n_rows, T, w_gate_up, H, I, act, s);
  return launch_skinny<true>(static_cast<const bf16_t*>(x), gather, offsets, G, n_rows, T,
                             static_cast<const bf16_t*>(w_gate_up), H, I, static_cast<bf16_t*>(act), s);
}

hipError_t launch_gate_up_routed(const void* x, const int32_t* ids, int T, int k, int E, int S, const void* w_gate_up,
                                 int H, int I, void* act, int32_t* offsets, int32_t* inv, hipStream_t s) {
  const RoutedArgs ra{ids, k, E, S, offsets, inv};
  return launch_skinny<true, true>(static_cast<const bf16_t*>(x), nullptr, nullptr, E + S, T * k + S * T, T,
                                   static_cast<const bf16_t*>(w_gate_up), H, I, static_cast<bf16_t*>(act), s, ra);
}

hipError_t launch_down(const void* act, const int32_t* offsets, int G, int n_rows, const void* w_down, int H,
                       int I, int max_rows, int dtype, void* y, hipStream_t s, const void* residual) {
  if (dtype == kF32) {
    hipLaunchKernelGGL(f32_down_kernel, dim3(n_rows), dim3(256), 0, s, static_cast<const float*>(act), offsets,
                       G, n_rows, static_cast<const float*>(w_down), H, I, static_cast<float*>(y),
                       static_cast<const float*>(residual), data_error_word(s));
    return hipGetLastError();
  }
  // the tiled GEMM has no residual epilogue: with a residual the weight-streaming form serves every size
  if (!residual && gemm_path_ok(I, H, max_rows))
    return launch_gemm(false, act, nullptr, offsets, G, n_rows, n_rows, w_down, I, H, y, s);
  return launch_skinny<false>(static_cast<const bf16_t*>(act), nullptr, offsets, G, n_rows, n_rows,
                              static_cast<const bf16_t*>(w_down), I, H, static_cast<bf16_t*>(y), s, RoutedArgs{},
                              static_cast<const bf16_t*>(residual));
}

}  // namespace moe
