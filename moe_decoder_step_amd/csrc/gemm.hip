// Grouped expert GEMM for prefill-sized groups (hundreds to tens of
// thousands of rows per expert), the MFMA-bound regime of the grouped SwiGLU.
//
// With many rows per group every weight element is used by many tokens, so
// the work is a dense contraction per group.  A block of 8 wavefronts owns a
// tile of 256 rows (tokens of one group) by 8 weight-row pairs:
//   gated stage: 8 (gate 16-row, up 16-row) pairs = 128 activation columns;
//   down stage:  8 pairs of 16 weight rows = 256 output columns.
// The reduction runs in stages of 64 (two 32-wide MFMA k-steps).  Each stage
// stages 32 KB of activation rows and 32 KB of weights in LDS, double
// buffered (128 KB), both in fragment order: a 1 KB fragment holds, in lane
// order, the 16 rows x 32 k-elements one wavefront feeds to
// v_mfma_f32_16x16x32_bf16, so every LDS read is 1 KB of consecutive bytes
// (no bank conflicts) and the packed weights (moe_pack_weights) copy into LDS
// as they lie in memory.  Global loads of the next stage are in flight while
// the current one is multiplied; one barrier per stage.
//
// Wavefront (wm, wn) = (w / 4, w % 4) computes rows 128 wm .. +127 (8 MFMA
// row blocks) by pairs 2 wn, 2 wn + 1 (4 weight fragments): 32 MFMAs per
// k-step, 128 fp32 accumulators per lane.  The weights are the MFMA A operand
// and the activations the B operand, so a lane ends with 4 consecutive output
// columns of one row (8-byte stores).
//
// M-tiles are numbered group by group; M-tile m runs on XCD m % 8 (block b
// runs on XCD b % 8) and its 8 (or 5, 7 ...) column tiles are consecutive
// blocks of that XCD, so they share the XCD's L2 copy of the activation
// rows, and neighbouring M-tiles of one group share the weight tiles.
// The fp32 accumulation order along K is fixed: 32 elements per MFMA, in
// increasing k.
#include "common.hpp"
#include "kernels.hpp"
#include "validate.hpp"

namespace moe {
namespace {

constexpr int kGM = 256;                  // rows per tile
constexpr int kGPairs = 8;                // weight-row pairs per tile
constexpr int kGK = 64;                   // reduction elements per stage
constexpr int kGWaves = 8;
constexpr int kGThreads = kGWaves * 64;
constexpr int kGStage = 2 * 32768;        // bytes per stage: A 32 KB + B 32 KB
constexpr size_t kGLds = 2 * (size_t)kGStage;

__device__ __forceinline__ float silu_g(float z) { return z / (1.0f + expf(-z)); }

__device__ __forceinline__ uint4 lds16(const char* p) { return *reinterpret_cast<const uint4*>(p); }

template <bool GATED>
__global__ __launch_bounds__(kGThreads) void gemm_kernel(
    const bf16_t* __restrict__ x, const int32_t* __restrict__ gather, const int32_t* __restrict__ offsets,
    int G, int n_rows, int T, const bf16_t* __restrict__ W, int K, int N, int n_pairs, int n_ntiles,
    bf16_t* __restrict__ out) {
  extern __shared__ __align__(16) char lds[];
  __shared__ int s_g, s_m0, s_m1, s_rb;

  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int nt = j % n_ntiles;
  const int m = (j / n_ntiles) * 8 + xcd;  // M-tile index, counted group by group
  if (threadIdx.x < kWave) {
    // lane l counts the M-tiles of groups l and l + 64 (G <= 128); a prefix
    // sum over the wavefront finds the group that holds M-tile m
    const int l = threadIdx.x;
    int r0[2], r1[2], cnt[2], incl[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int g = l + h * kWave;
      r0[h] = g < G ? clampi(offsets[g], 0, n_rows) : 0;
      r1[h] = g < G ? clampi(offsets[g + 1], r0[h], n_rows) : 0;
      cnt[h] = (r1[h] - r0[h] + kGM - 1) / kGM;
      incl[h] = cnt[h];
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int v = __shfl_up(incl[h], o, kWave);
        if (l >= o) incl[h] += v;
      }
    }
    incl[1] += __shfl(incl[0], kWave - 1, kWave);
    if (l == 0) s_g = -1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int first = incl[h] - cnt[h];
      if (m >= first && m < incl[h]) {
        s_g = l + h * kWave;
        s_m0 = r0[h] + (m - first) * kGM;
        s_m1 = r1[h];
        s_rb = r0[h];
      }
    }
  }
  __syncthreads();
  const int g = s_g;
  if (g < 0) return;
  const int m0 = s_m0, m1 = s_m1, r_begin = s_rb;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nK = K / 32;
  const int nS = K / kGK;

  // activation loads: round u fills fragment f = 8u + wave (row block f/2,
  // k-step f%2) of the stage; this lane's row and 16-byte segment
  const bf16_t* asrc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int f = u * kGWaves + wave;
    const int r = min(m0 + 16 * (f >> 1) + (lane & 15), m1 - 1);  // rows past the group repeat a valid row
    int src;
    if (GATED) src = gather ? clampi(gather[r], 0, T - 1) : clampi(r - r_begin, 0, T - 1);
    else src = r;
    asrc[u] = x + (size_t)src * K + 8 * (4 * (f & 1) + (lane >> 4));
  }
  // weight loads: 16-byte unit c = 512u + tid of the stage's 8 pairs x 4 KB
  // (pairs past the last are clamped: loaded, never stored)
  const bf16_t* bsrc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int c = u * kGThreads + threadIdx.x;
    const int pair = min(nt * kGPairs + (c >> 8), n_pairs - 1);
    bsrc[u] = W + ((size_t)g * n_pairs + pair) * nK * 1024 + (c & 255) * 8;
  }

  uint4 ra[4], rb[4];
  auto load = [&](int s) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      ra[u] = ldg16(asrc[u] + s * kGK);
      rb[u] = ldg16(bsrc[u] + (size_t)s * 2048);
    }
  };
  auto store = [&](int buf) __attribute__((always_inline)) {
    char* base = lds + buf * kGStage;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      *reinterpret_cast<uint4*>(base + (u * kGWaves + wave) * 1024 + lane * 16) = ra[u];
      *reinterpret_cast<uint4*>(base + 32768 + (u * kGThreads + threadIdx.x) * 16) = rb[u];
    }
  };

  const int wm = wave >> 2, wn = wave & 3;
  f32x4_t acc[8][2][2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int h = 0; h < 2; ++h) acc[i][q][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  load(0);
  store(0);
  __syncthreads();
  for (int s = 0; s < nS; ++s) {
    if (s + 1 < nS) load(s + 1);
    const char* base = lds + (s & 1) * kGStage;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t bw[2][2];
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          bw[q][h] = as_bf16x8(lds16(base + 32768 + (wn * 2 + q) * 4096 + ks * 2048 + h * 1024 + lane * 16));
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bf16x8_t xa = as_bf16x8(lds16(base + ((wm * 8 + i) * 2 + ks) * 1024 + lane * 16));
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int h = 0; h < 2; ++h) acc[i][q][h] = mfma16x16x32(bw[q][h], xa, acc[i][q][h]);
      }
    }
    if (s + 1 < nS) store((s + 1) & 1);
    __syncthreads();
  }

  // lane holds D[4 (lane/16) + v][lane % 16]: weight rows (output columns)
  // 4 (lane/16) .. +3 of its fragment, for row lane % 16 of the row block
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = m0 + (wm * 8 + i) * 16 + (lane & 15);
    if (row >= m1) continue;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int pair = nt * kGPairs + wn * 2 + q;
      if (GATED) {
        if (pair >= n_pairs) continue;
        const f32x4_t a = acc[i][q][0], b = acc[i][q][1];
        uint2 pk;
        pk.x = pack2(f32_to_bf16(silu_g(a[0]) * b[0]), f32_to_bf16(silu_g(a[1]) * b[1]));
        pk.y = pack2(f32_to_bf16(silu_g(a[2]) * b[2]), f32_to_bf16(silu_g(a[3]) * b[3]));
        *reinterpret_cast<uint2*>(out + (size_t)row * N + pair * 16 + 4 * (lane >> 4)) = pk;
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int col = pair * 32 + h * 16 + 4 * (lane >> 4);
          if (col >= N) continue;
          const f32x4_t a = acc[i][q][h];
          uint2 pk;
          pk.x = pack2(f32_to_bf16(a[0]), f32_to_bf16(a[1]));
          pk.y = pack2(f32_to_bf16(a[2]), f32_to_bf16(a[3]));
          *reinterpret_cast<uint2*>(out + (size_t)row * N + col) = pk;
        }
      }
    }
  }
}

}  // namespace

bool gemm_path_ok(int K, int N, int max_rows) {
  return max_rows >= kGemmMinRows && K % kGK == 0 && N % 16 == 0;
}

template <bool GATED>
hipError_t launch_gemm_t(const bf16_t* x, const int32_t* gather, const int32_t* offsets, int G, int n_rows, int T,
                         const bf16_t* W, int K, int N, bf16_t* out, hipStream_t s) {
  const int n_pairs = GATED ? N / 16 : (N + 31) / 32;
  const int n_ntiles = (n_pairs + kGPairs - 1) / kGPairs;
  // M-tiles <= sum over groups of ceil(rows / 256) <= n_rows / 256 + G
  const int mtiles = n_rows / kGM + G;
  const long long blocks = 8LL * ((mtiles + 7) / 8) * n_ntiles;
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
