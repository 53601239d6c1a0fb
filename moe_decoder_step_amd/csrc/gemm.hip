// Grouped expert GEMM for prefill-sized groups (hundreds to tens of
// thousands of rows per expert), the MFMA-bound regime of the grouped SwiGLU.
//
// With many rows per group every weight element is used by many tokens, so
// the work is a dense contraction per group.  A block of 8 wavefronts owns a
// tile of 256 rows (tokens of one group) by 8 weight-row pairs:
//   gated stage: 8 (gate 16-row, up 16-row) pairs = 128 activation columns;
//   down stage:  8 pairs of 16 weight rows = 256 output columns.
// The reduction runs in stages of 32.  A stage's activations (16 KB) go
// through LDS, its weights (the pair's two packed 16 x 32 fragments,
// moe_pack_weights) straight into registers.  Wavefront w computes all 256
// rows by pair w, 128 fp32 accumulators per lane, so every weight byte is
// fetched once per block (32 KB per stage from memory in all) and every
// wavefront reads all 16 KB of a stage's activations from LDS.
//
// The multiply:
//   gated: v_mfma_f32_16x16x32_bf16, the fragments as they lie in memory
//          (lane l: row l % 16, k-elements 8 (l / 16) .. +7) as the A
//          operand, 16 token rows as the B operand, 32 MFMAs per stage;
//   down:  v_mfma_f32_32x32x16_bf16, the pair's 32 weight rows as one A
//          operand, 32 token rows as the B operand, 2 MFMAs (k-halves) per
//          row block, 16 per stage.
// On the same data one 16x16x32 MFMA and the two 32x32x16 MFMAs of its
// k-halves give the same bits (an in-bounds probe over 4.2M outputs --
// random, wide-exponent, cancelling and large-accumulator inputs -- found no
// difference), so both stages, and the weight-streaming kernel, sum a row's
// products identically.  The larger shape ran the LDS-fed stage loop alone at
// 0.94 of the MFMA peak against 0.74, and the down GEMM 8% faster; the gate/up
// GEMM measured 5% slower with it (stores, load lane order and LDS read
// schedule ruled out) and keeps the smaller one.
//
// Activations are loaded from global memory straight into LDS
// (global_load_lds_dwordx4: lane l's 16 bytes land at offset 16 l of a 1 KB
// block, one load covering the 64-byte stage segments of 16 token rows),
// rows gathered per lane, into a ring of kGAheadA + 1 stage buffers,
// kGAheadA stages ahead of the multiply; the block layout is per shape
// (act_slot).  The weights go into a register ring, kGAhead stages ahead.
//
// The fp32 accumulation order along K is fixed: 32 elements per 16x16x32
// MFMA (16 per 32x32x16 MFMA, the same sums), in increasing k.
#include <atomic>
#include "common.hpp"
#include "kernels.hpp"
#include "validate.hpp"

namespace moe {
namespace {

constexpr int kGM = 256;                  // rows per tile
constexpr int kGPairs = 8;                // weight-row pairs per tile
constexpr int kGK = 32;                   // reduction elements per stage
constexpr int kGAhead = 4;                // weight stages in flight (register ring)
constexpr int kGAheadA = 4;               // activation stages in flight (LDS ring), a multiple of kGAhead
constexpr int kGRing = kGAheadA + 1;      // activation stage buffers
constexpr int kGWaves = 8;
constexpr int kGThreads = kGWaves * 64;
constexpr int kGStage = 16384;            // activation bytes per stage
constexpr int kGLoads = 4;                // loads per wavefront and stage: 2 activation + 2 weight fragments
constexpr size_t kGLds = (size_t)kGRing * kGStage;

typedef __attribute__((address_space(3))) void lds_void_t;

// 16 bytes per lane from global memory straight into LDS at base + 16 lane
__device__ __forceinline__ void load_lds16(const bf16_t* g, char* base) {
  __builtin_amdgcn_global_load_lds(static_cast<const void*>(g), (lds_void_t*)(base), 16, 0, 0);
}

// wait until at most N of this wavefront's global loads are outstanding (and
// all its LDS accesses are done), then a workgroup barrier; no fence, so the
// loads of later stages stay in flight
template <int N>
__device__ __forceinline__ void wait_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  // vmcnt(N) (bits 3:0 and 15:14) expcnt(7) lgkmcnt(0)
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070);
  asm volatile("s_barrier" ::: "memory");
}

// The epilogue's SiLU is silu_bf16path (hardware exp2 and reciprocal), the
// same function as the weight-streaming kernel's.  The epilogue evaluates 64
// per lane: with libm's expf and an IEEE division it took 8 us of a 48 us
// block.

__device__ __forceinline__ uint4 lds16(const char* p) { return *reinterpret_cast<const uint4*>(p); }

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

__device__ __forceinline__ f32x16_t mfma32x32x16(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// A stage's 16 KB of activations: 16 blocks of 1 KB, block b = token rows
// 16 b .. 16 b + 15 of the tile; the place of row q's chunk c (k-elements
// 8 c .. 8 c + 7) in a block:
//   16x16x32: 16 (16 c + q), lane order of the B operand (lane 16 c + q);
//   32x32x16: 64 q + 16 (c ^ (q / 4 mod 4)): the whole 64-byte row segment
//     comes from one load (4 lanes per row, one request per segment), and
//     the swizzle keeps the operand reads (16 rows, one chunk) free of bank
//     conflicts.  (The 16x16x32 gate/up GEMM measured 2% slower with it.)
template <bool M32>
__device__ __forceinline__ int act_slot(int q, int c) {
  return M32 ? q * 64 + ((c ^ ((q >> 2) & 3)) << 4) : (16 * c + q) * 16;
}

// The accumulators of a wavefront (256 rows by its pair) and the stage
// multiply, by MFMA shape.
template <bool M32>
struct Mma;

// 16x16x32: row block i (16 rows) by fragment h; B operand lane l = row
// l % 16, chunk l / 16.
template <>
struct Mma<false> {
  f32x4_t acc[16][2];
  int boff;
  __device__ __forceinline__ void init(int lane) {
    boff = act_slot<false>(lane & 15, lane >> 4);
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) acc[i][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  // half 0 or 1 of a stage: row blocks 8 half .. 8 half + 7
  __device__ __forceinline__ void half(const char* cur, int hf, const uint4 (&bw)[2]) {
#pragma unroll
    for (int i = 8 * hf; i < 8 * hf + 8; ++i) {
      const bf16x8_t xa = as_bf16x8(lds16(cur + i * 1024 + boff));
#pragma unroll
      for (int h = 0; h < 2; ++h) acc[i][h] = mfma16x16x32(as_bf16x8(bw[h]), xa, acc[i][h]);
    }
  }
};

// 32x32x16: row block i (32 rows) by the pair's 32 weight rows, k-halves
// h = 0, 1; B operand lane l = row l % 32 (block 2 i + (l % 32) / 16), chunk
// 2 h + l / 32.
template <>
struct Mma<true> {
  f32x16_t acc[8];
  int boff[2];
  __device__ __forceinline__ void init(int lane) {
    const int q = lane & 31;
#pragma unroll
    for (int h = 0; h < 2; ++h) boff[h] = (q >> 4) * 1024 + act_slot<true>(q & 15, 2 * h + (lane >> 5));
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;
  }
  // half 0 or 1 of a stage: row blocks 4 half .. 4 half + 3, k-half 0 of
  // all four, then k-half 1
  __device__ __forceinline__ void half(const char* cur, int hf, const uint4 (&bw)[2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 4 * hf; i < 4 * hf + 4; ++i) {
        const bf16x8_t xa = as_bf16x8(lds16(cur + i * 2048 + boff[h]));
        acc[i] = mfma32x32x16(as_bf16x8(bw[h]), xa, acc[i]);
      }
  }
};

// One stage that refills: the first half of the stage in `cur`, the barrier
// (N loads may stay outstanding), this wavefront's activation loads of a later
// stage into `nxt`, the second half.  The two buffers are distinct; saying so
// (restrict) lets the compiler see that the reads of `cur` do not depend on
// the loads into `nxt` still in flight, so it adds no wait for them.
template <int N, bool M32>
__device__ __forceinline__ void gemm_stage(const char* __restrict__ cur, char* __restrict__ nxt,
                                           const bf16_t* const (&src)[2], size_t step, const uint4 (&bw)[2],
                                           Mma<M32>& mma) {
  mma.half(cur, 0, bw);
  wait_barrier<N>();
#pragma unroll
  for (int u = 0; u < 2; ++u) load_lds16(src[u] + step, nxt + u * 1024);
  mma.half(cur, 1, bw);
}

// This wavefront's 2 weight operands of stage s (its pair), lane l's 16 bytes
// each, wsrc being the lane's place in the stage's 2 KB:
//   16x16x32: fragments h = 0, 1 as they lie (wsrc = 8 l elements on);
//   32x32x16: k-halves h = 0, 1 of the 32 x 32 pair, 256 elements apart.
template <bool M32>
__device__ __forceinline__ void load_weights(uint4 (&bw)[2], const bf16_t* wsrc, int s) {
#pragma unroll
  for (int h = 0; h < 2; ++h)
    bw[h] = *reinterpret_cast<const uint4*>(wsrc + (size_t)s * 1024 + h * (M32 ? 256 : 512));
}

// The place of lane l's 16 weight bytes in a stage, in elements.
//   16x16x32: 8 l.
//   32x32x16: A-operand row i = l % 32 stands for row r of fragment f,
//     f = (i / 4) mod 2, r = 4 (i / 8) + i mod 4.  Accumulator v of lane l
//     holds operand row 8 (v / 4) + 4 (l / 32) + v % 4, which this map makes
//     output column 16 (l / 32) + v of the pair: 16 consecutive columns per
//     lane.  Its k-half-0 chunk (k-elements 8 (l / 32) .. +7) is the one lane
//     16 (l / 32) + r of fragment f holds: 512 f + 8 (16 (l / 32) + r).
template <bool M32>
__device__ __forceinline__ int wlane_offset(int lane) {
  if (!M32) return 8 * lane;
  const int i = lane & 31;
  const int f = (i >> 2) & 1, r = 4 * (i >> 3) + (i & 3);
  return 512 * f + 8 * (16 * (lane >> 5) + r);
}

// A tile: an M-tile (rows m0 .. m1-1 of group g, which starts at row rb; up
// to 256) by column tile nt.  g < 0: the tile index is past the last M-tile.
struct GTile {
  int g, m0, m1, rb, nt;
};

// Tile index jt -> tile.  M-tile m runs on XCD m % 8 (tile jt runs on XCD
// jt % 8) and its column tiles are consecutive tile indices of that XCD, so
// they share the XCD's L2 copy of the activation rows, and neighbouring
// M-tiles of one group share the weight tiles.  s_first[g] counts the
// M-tiles of the groups before g (s_first[G]: all of them); s_r0, s_r1 are
// the groups' row ranges.  Every lane returns the same tile.
__device__ __forceinline__ GTile find_tile(int jt, int n_ntiles, int G, const int* s_first, const int* s_r0,
                                           const int* s_r1, int lane) {
  GTile tl;
  const int j = jt >> 3;
  tl.nt = j % n_ntiles;
  const int m = (j / n_ntiles) * 8 + (jt & 7);
  tl.g = -1;
  tl.m0 = tl.m1 = tl.rb = 0;
  if (m >= s_first[G]) return tl;
  int hit = -1;  // the one group with s_first[g] <= m < s_first[g + 1]
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int g = lane + h * kWave;
    if (g < G && m >= s_first[g] && m < s_first[g + 1]) hit = g;
  }
  const unsigned long long bal = __ballot(hit >= 0);
  const int g = __builtin_amdgcn_readlane(hit, __ffsll((long long)bal) - 1);
  tl.g = g;
  tl.rb = s_r0[g];
  tl.m0 = tl.rb + (m - s_first[g]) * kGM;
  tl.m1 = s_r1[g];
  return tl;
}

// Persistent: block b takes tiles b, b + gridDim.x, ... (gridDim.x a
// multiple of 8, so every tile keeps its XCD).  The stages of a block's
// tiles form one stream: the last kGAhead stages of a tile issue the first
// kGAhead stages of the next, so the pipeline never drains between tiles and
// the epilogue of one tile overlaps the loads of the next.
template <bool GATED>
__global__ __launch_bounds__(kGThreads) void gemm_kernel(
    const bf16_t* __restrict__ x, const int32_t* __restrict__ gather, const int32_t* __restrict__ offsets,
    int G, int n_rows, int T, const bf16_t* __restrict__ W, int K, int N, int n_pairs, int n_ntiles,
    bf16_t* __restrict__ out, uint32_t* err) {
  extern __shared__ __align__(16) char lds[];
  __shared__ int s_first[2 * kWave + 1], s_r0[2 * kWave], s_r1[2 * kWave];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (wave == 0) {
    // lane l counts the M-tiles of groups l and l + 64 (G <= 128); a prefix
    // sum over the wavefront numbers them
    int r0[2], r1[2], cnt[2], incl[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int g = lane + h * kWave;
      // (block 0 reports ranges outside [0, n_rows] or decreasing)
      uint32_t* const eb = blockIdx.x == 0 ? err : nullptr;
      r0[h] = g < G ? clamp_report(offsets[g], 0, n_rows, eb, kDataErrOffsets) : 0;
      r1[h] = g < G ? clamp_report(offsets[g + 1], r0[h], n_rows, eb, kDataErrOffsets) : 0;
      cnt[h] = (r1[h] - r0[h] + kGM - 1) / kGM;
      incl[h] = cnt[h];
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int v = __shfl_up(incl[h], o, kWave);
        if (lane >= o) incl[h] += v;
      }
    }
    incl[1] += __shfl(incl[0], kWave - 1, kWave);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int g = lane + h * kWave;
      s_first[g] = incl[h] - cnt[h];
      s_r0[g] = r0[h];
      s_r1[g] = r1[h];
    }
    // groups from G on count no M-tiles: s_first[G .. 128] hold the total
    if (lane == kWave - 1) s_first[2 * kWave] = incl[1];
  }
  __syncthreads();

  int jt = blockIdx.x;
  GTile cur = find_tile(jt, n_ntiles, G, s_first, s_r0, s_r1, lane);
  if (cur.g < 0) return;

  const int nS = K / kGK;  // stages = MFMA k-steps

  constexpr bool M32 = !GATED;  // the MFMA shape: 32x32x16 for down, 16x16x32 for gate/up

  // activation loads: wavefront w fetches blocks 2 w and 2 w + 1 of each
  // stage (token rows 32 w + 16 u .. +15, load u = 0, 1), lane l the (row,
  // chunk) that act_slot places at 16 l: 16x16x32 row l % 16, chunk l / 16;
  // 32x32x16 row l / 4, chunk (l % 4) ^ (l / 16 mod 4) (rows past the group
  // repeat a valid row); weight loads: wavefront w fetches pair w of the tile
  // (clamped pairs: loaded, never stored)
  const int lrow = M32 ? lane >> 2 : lane & 15;
  const int chunk = M32 ? (lane & 3) ^ ((lane >> 4) & 3) : lane >> 4;
  auto act_row = [&](const GTile& tl, int u) { return min(tl.m0 + 32 * wave + 16 * u + lrow, tl.m1 - 1); };
  auto act_src = [&](const GTile& tl, int u, int gv) {
    int t;
    if (GATED)
      t = gather ? clamp_report(gv, 0, T - 1, err, kDataErrRowIndex)
                 : clamp_report(act_row(tl, u) - tl.rb, 0, T - 1, err, kDataErrOffsets);
    else t = act_row(tl, u);
    return x + (size_t)t * K + 8 * chunk;
  };
  const int wlane = wlane_offset<M32>(lane);
  auto w_src = [&](const GTile& tl) {
    const int pair = min(tl.nt * kGPairs + wave, n_pairs - 1);
    return W + ((size_t)tl.g * n_pairs + pair) * nS * 1024 + wlane;
  };
  const bf16_t* src[2];
  const bf16_t* wsrc;
#pragma unroll
  for (int u = 0; u < 2; ++u) src[u] = act_src(cur, u, GATED && gather ? gather[act_row(cur, u)] : 0);
  wsrc = w_src(cur);

  Mma<M32> mma;
  mma.init(lane);

  // Stage s multiplies its first half, waits at a barrier until the next
  // stage of the stream has landed, issues the activation loads kGAhead
  // stages ahead into the buffer of the previous stage (every wavefront is
  // past it), multiplies its second half, and refills its weight slot kGAhead
  // stages ahead.  So no barrier sits between two stages: the LDS reads of
  // the next stage start while the last MFMAs of this one run.  The loads
  // issued in one stage (act, w) form one group, the groups in stream order
  // (the prologue's kept apart by compiler fences; inside a group the
  // compiler may reorder).  Halfway through a stage, waiting until at most
  // kGLoads (kGAhead - 2) of this wavefront's loads are outstanding leaves
  // only the groups of the stages 2 .. kGAhead-1 ahead; other loads in the
  // stream (the gathered row numbers of the next tile) only make that wait
  // stricter.  nS is a multiple of kGAhead, at least 2 kGAhead, so a tile's
  // stages use the weight slots 0 .. kGAhead-1 in turn.
  static_assert(kGAhead >= 2, "the half-stage wait needs the next stage issued");
  char* const mine = lds + wave * 2 * 1024;  // this wavefront's 2 fragments of a stage buffer
  static_assert(kGAheadA >= kGAhead && kGAheadA % kGAhead == 0, "activations run at least as far ahead");
  uint4 bw[kGAhead][2];
#pragma unroll
  for (int t = 0; t < kGAheadA; ++t) {
#pragma unroll
    for (int u = 0; u < 2; ++u) load_lds16(src[u] + t * kGK, mine + t * kGStage + u * 1024);
    if (t < kGAhead) load_weights<M32>(bw[t], wsrc, t);
    asm volatile("" ::: "memory");
  }
  // the first stage: after its weights come kGAhead - 1 groups of both and
  // kGAheadA - kGAhead activation-only groups
  wait_barrier<kGLoads * (kGAhead - 1) + 2 * (kGAheadA - kGAhead)>();
  int gb = 0;                               // stage buffer of the current stage
  for (;;) {
    const GTile nxt = find_tile(jt + (int)gridDim.x, n_ntiles, G, s_first, s_r0, s_r1, lane);
    int gv[2] = {0, 0};  // the next tile's gathered row numbers
    int sa_off = 0, sw_off = 0;
    int s0 = 0;
    do {
      if (s0 == nS - kGAheadA && nxt.g >= 0) {
        // from here the activation loads kGAheadA stages ahead are the next tile's
#pragma unroll
        for (int u = 0; u < 2; ++u) src[u] = act_src(nxt, u, gv[u]);
        sa_off = -nS;
      }
      if (s0 == nS - kGAhead && nxt.g >= 0) {
        // and from here the weight loads kGAhead stages ahead
        wsrc = w_src(nxt);
        sw_off = -nS;
      }
      // Loaded in the tile's first pass of this loop and read at the switch
      // above in a later pass (nS >= kGAheadA + kGAhead): the half-stage waits in
      // between retire them, so the compiler adds no wait at the switch (a
      // wait there for a load issued just before would drain every load in
      // flight).
      if (GATED && gather && s0 == 0 && nxt.g >= 0) {
#pragma unroll
        for (int u = 0; u < 2; ++u) gv[u] = gather[act_row(nxt, u)];
      }
#pragma unroll
      for (int t = 0; t < kGAhead; ++t) {
        // the stages kGAheadA and kGAhead ahead in the stream; after the last
        // tile, stage nS - 1 of this one again (loaded, never read)
        const int sna = min(s0 + t + kGAheadA + sa_off, nS - 1);
        const int snw = min(s0 + t + kGAhead + sw_off, nS - 1);
        const int nb = gb == 0 ? kGRing - 1 : gb - 1;  // the previous stage's buffer
        gemm_stage<kGLoads * (kGAhead - 2), M32>(lds + gb * kGStage, mine + nb * kGStage, src, (size_t)sna * kGK,
                                                 bw[t], mma);
        load_weights<M32>(bw[t], wsrc, snw);
        gb = gb == kGRing - 1 ? 0 : gb + 1;
      }
      s0 += kGAhead;
    } while (s0 < nS);

    const int pair = cur.nt * kGPairs + wave;
    if constexpr (!M32) {
      // lane holds D[4 (lane/16) + v][lane % 16]: weight rows (columns of the
      // pair) 4 (lane/16) .. +3 of its fragments, for row lane % 16 of the
      // row block; SiLU(gate) * up pairs fragment 0 with fragment 1
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = cur.m0 + i * 16 + (lane & 15);
        if (row >= cur.m1 || pair >= n_pairs) continue;
        const f32x4_t a = mma.acc[i][0], b = mma.acc[i][1];
        uint2 pk;
        pk.x = pack_bf16x2(silu_bf16path(a[0]) * b[0], silu_bf16path(a[1]) * b[1]);
        pk.y = pack_bf16x2(silu_bf16path(a[2]) * b[2], silu_bf16path(a[3]) * b[3]);
        *reinterpret_cast<uint2*>(out + (size_t)row * N + pair * 16 + 4 * (lane >> 4)) = pk;
      }
    } else {
      // lane holds output columns pair * 32 + 16 (lane/32) .. +15 of token
      // row 32 i + lane % 32 (wlane_offset)
      const int col = pair * 32 + 16 * (lane >> 5);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = cur.m0 + i * 32 + (lane & 31);
        if (row >= cur.m1 || col >= N) continue;
        const f32x16_t a = mma.acc[i];
        uint4 p0, p1;
        p0.x = pack_bf16x2(a[0], a[1]);
        p0.y = pack_bf16x2(a[2], a[3]);
        p0.z = pack_bf16x2(a[4], a[5]);
        p0.w = pack_bf16x2(a[6], a[7]);
        p1.x = pack_bf16x2(a[8], a[9]);
        p1.y = pack_bf16x2(a[10], a[11]);
        p1.z = pack_bf16x2(a[12], a[13]);
        p1.w = pack_bf16x2(a[14], a[15]);
        uint4* o = reinterpret_cast<uint4*>(out + (size_t)row * N + col);
        o[0] = p0;
        o[1] = p1;
      }
    }
    if (nxt.g < 0) break;
    mma.init(lane);
    cur = nxt;
    jt += gridDim.x;
  }
  // the LDS must not be released with loads into it in flight
  __builtin_amdgcn_s_waitcnt(0);
}

}  // namespace

bool gemm_path_ok(int K, int N, int max_rows) {
  return max_rows >= kGemmMinRows && K >= kGK * (kGAheadA + kGAhead) && K % (kGK * kGAhead) == 0 && N % 16 == 0;
}

// blocks of the persistent grid: one per CU (one 8-wavefront block fills a
// CU's registers), a multiple of 8 so that every tile keeps its XCD.  The CU
// count is cached per device in atomics: threads that race store the same
// value.
static int persistent_blocks() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8) cus = 256;
    n = cus / 8 * 8;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <bool GATED>
hipError_t launch_gemm_t(const bf16_t* x, const int32_t* gather, const int32_t* offsets, int G, int n_rows, int T,
                         const bf16_t* W, int K, int N, bf16_t* out, hipStream_t s) {
  const int n_pairs = GATED ? N / 16 : (N + 31) / 32;
  const int n_ntiles = (n_pairs + kGPairs - 1) / kGPairs;
  // M-tiles <= sum over groups of ceil(rows / 256) <= n_rows / 256 + G
  const int mtiles = n_rows / kGM + G;
  const long long tiles = 8LL * ((mtiles + 7) / 8) * n_ntiles;
  const long long blocks = std::min<long long>(tiles, persistent_blocks());
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_kernel<GATED>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kGLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gemm_kernel<GATED>), dim3((unsigned)blocks), dim3(kGThreads), kGLds, s, x, gather, offsets,
                     G, n_rows, T, W, K, N, n_pairs, n_ntiles, out, data_error_word(s));
  return hipGetLastError();
}

hipError_t launch_gemm(bool gated, const void* x, const int32_t* gather, const int32_t* offsets, int G, int n_rows,
                       int T, const void* W, int K, int N, void* out, hipStream_t s) {
  const bf16_t* xb = static_cast<const bf16_t*>(x);
  const bf16_t* wb = static_cast<const bf16_t*>(W);
  bf16_t* ob = static_cast<bf16_t*>(out);
  return gated ? launch_gemm_t<true>(xb, gather, offsets, G, n_rows, T, wb, K, N, ob, s)
               : launch_gemm_t<false>(xb, gather, offsets, G, n_rows, T, wb, K, N, ob, s);
}

}  // namespace moe
