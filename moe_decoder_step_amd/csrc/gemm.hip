// Grouped expert GEMM for prefill-sized groups (hundreds to tens of
// thousands of rows per expert), the MFMA-bound regime of the grouped SwiGLU.
//
// With many rows per group every weight element is used by many tokens, so
// the work is a dense contraction per group.  A block of 8 wavefronts owns a
// tile of 256 rows (tokens of one group) by 8 weight-row pairs:
//   gated stage: 8 (gate 16-row, up 16-row) pairs = 128 activation columns;
//   down stage:  8 pairs of 16 weight rows = 256 output columns.
// The reduction runs in stages of 32 (one MFMA k-step).  A stage's 16
// activation fragments (16 KB) go through LDS, its 16 weight fragments
// straight into registers.  A 1 KB fragment holds, in lane order, the 16 rows
// x 32 k-elements one wavefront feeds to v_mfma_f32_16x16x32_bf16, so every
// LDS read is 1 KB of consecutive bytes (no bank conflicts).  Activation
// fragments are loaded from global memory straight into LDS
// (global_load_lds_dwordx4: lane l's 16 bytes land at fragment offset 16 l),
// rows gathered per lane, into a ring of kGAheadA + 1 stage buffers, kGAheadA
// stages ahead of the multiply; each wavefront loads the 2 packed weight
// fragments it multiplies (1 KB each, as they lie in memory,
// moe_pack_weights) into a register ring, kGAhead stages ahead.
//
// Wavefront w computes all 256 rows (16 MFMA row blocks) by pair w (2 weight
// fragments): 32 MFMAs per stage, 128 fp32 accumulators per lane.  So every
// weight fragment is fetched once per block (32 KB per stage from memory in
// all), and every wavefront reads all 16 activation fragments of a stage
// from LDS.  The weights are the MFMA A operand and the activations the B
// operand, so a lane ends with 4 consecutive output columns of one row
// (8-byte stores).
//
// The fp32 accumulation order along K is fixed: 32 elements per MFMA, in
// increasing k.
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

// Row blocks i0 .. i0 + 3 of one stage: multiply the stage in `cur` with the
// weight fragments `bw`.
__device__ __forceinline__ void gemm_half(const char* cur, int i0, const uint4 (&bw)[2],
                                          f32x4_t (&acc)[16][2], int lane) {
#pragma unroll
  for (int i = i0; i < i0 + 8; ++i) {
    const bf16x8_t xa = as_bf16x8(lds16(cur + i * 1024 + lane * 16));
#pragma unroll
    for (int h = 0; h < 2; ++h) acc[i][h] = mfma16x16x32(as_bf16x8(bw[h]), xa, acc[i][h]);
  }
}

// One stage that refills: row blocks 0-7 of the stage in `cur`, the barrier
// (N loads may stay outstanding), this wavefront's activation loads of a later
// stage into `nxt`, row blocks 8-15.  The two buffers are distinct; saying so
// (restrict) lets the compiler see that the reads of `cur` do not depend on
// the loads into `nxt` still in flight, so it adds no wait for them.
template <int N>
__device__ __forceinline__ void gemm_stage(const char* __restrict__ cur, char* __restrict__ nxt,
                                           const bf16_t* const (&src)[2], size_t step, const uint4 (&bw)[2],
                                           f32x4_t (&acc)[16][2], int lane) {
  gemm_half(cur, 0, bw, acc, lane);
  wait_barrier<N>();
#pragma unroll
  for (int u = 0; u < 2; ++u) load_lds16(src[u] + step, nxt + u * 1024);
  gemm_half(cur, 8, bw, acc, lane);
}

// this wavefront's 2 weight fragments of stage s (its pair; sets h = 0, 1)
__device__ __forceinline__ void load_weights(uint4 (&bw)[2], const bf16_t* wsrc, int s) {
#pragma unroll
  for (int h = 0; h < 2; ++h) bw[h] = *reinterpret_cast<const uint4*>(wsrc + (size_t)s * 1024 + h * 512);
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
    bf16_t* __restrict__ out) {
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
      r0[h] = g < G ? clampi(offsets[g], 0, n_rows) : 0;
      r1[h] = g < G ? clampi(offsets[g + 1], r0[h], n_rows) : 0;
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

  // activation loads: wavefront w fetches row blocks 2 w and 2 w + 1 of each
  // stage (rows past the group repeat a valid row); weight loads: wavefront
  // w fetches pair w of the tile (clamped pairs: loaded, never stored)
  auto act_row = [&](const GTile& tl, int u) { return min(tl.m0 + 16 * (wave * 2 + u) + (lane & 15), tl.m1 - 1); };
  auto act_src = [&](const GTile& tl, int u, int gv) {
    int t;
    if (GATED) t = gather ? clampi(gv, 0, T - 1) : clampi(act_row(tl, u) - tl.rb, 0, T - 1);
    else t = act_row(tl, u);
    return x + (size_t)t * K + 8 * (lane >> 4);
  };
  auto w_src = [&](const GTile& tl) {
    const int pair = min(tl.nt * kGPairs + wave, n_pairs - 1);
    return W + ((size_t)tl.g * n_pairs + pair) * nS * 1024 + lane * 8;
  };
  const bf16_t* src[2];
  const bf16_t* wsrc;
#pragma unroll
  for (int u = 0; u < 2; ++u) src[u] = act_src(cur, u, GATED && gather ? gather[act_row(cur, u)] : 0);
  wsrc = w_src(cur);

  f32x4_t acc[16][2];
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) acc[i][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Stage s multiplies row blocks 0-7, waits at a barrier until the next
  // stage of the stream has landed, issues the activation loads kGAhead
  // stages ahead into the buffer of the previous stage (every wavefront is
  // past it), multiplies row blocks 8-15, and refills its weight slot kGAhead
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
    if (t < kGAhead) load_weights(bw[t], wsrc, t);
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
        gemm_stage<kGLoads * (kGAhead - 2)>(lds + gb * kGStage, mine + nb * kGStage, src, (size_t)sna * kGK, bw[t],
                                            acc, lane);
        load_weights(bw[t], wsrc, snw);
        gb = gb == kGRing - 1 ? 0 : gb + 1;
      }
      s0 += kGAhead;
    } while (s0 < nS);

    // lane holds D[4 (lane/16) + v][lane % 16]: weight rows (output columns)
    // 4 (lane/16) .. +3 of its fragment, for row lane % 16 of the row block
    const int pair = cur.nt * kGPairs + wave;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = cur.m0 + i * 16 + (lane & 15);
      if (row >= cur.m1) continue;
      if (GATED) {
        if (pair >= n_pairs) continue;
        const f32x4_t a = acc[i][0], b = acc[i][1];
        uint2 pk;
        pk.x = pack_bf16x2(silu_bf16path(a[0]) * b[0], silu_bf16path(a[1]) * b[1]);
        pk.y = pack_bf16x2(silu_bf16path(a[2]) * b[2], silu_bf16path(a[3]) * b[3]);
        *reinterpret_cast<uint2*>(out + (size_t)row * N + pair * 16 + 4 * (lane >> 4)) = pk;
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int col = pair * 32 + h * 16 + 4 * (lane >> 4);
          if (col >= N) continue;
          const f32x4_t a = acc[i][h];
          uint2 pk;
          pk.x = pack_bf16x2(a[0], a[1]);
          pk.y = pack_bf16x2(a[2], a[3]);
          *reinterpret_cast<uint2*>(out + (size_t)row * N + col) = pk;
        }
      }
    }
    if (nxt.g < 0) break;
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) acc[i][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
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
                     G, n_rows, T, W, K, N, n_pairs, n_ntiles, out);
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
