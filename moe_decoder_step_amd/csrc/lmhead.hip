// lmhead_argmax: argmax_v (h W_lm^T)[t, v] per row, ties to the lowest v.
//
// The 129,280 x 1280 bf16 LM head (331 MB, packed by moe_pack_weights so
// every load is 1 KB of consecutive bytes) is streamed from HBM exactly once
// per call and the logits never leave registers:
//   * a block of 4 wavefronts owns 128 vocabulary rows; wavefront w streams 32
//     of them (two 16-row MFMA blocks) as the A operand of
//     v_mfma_f32_16x16x32_bf16, two 128-element chunks in flight;
//   * the h rows (all T rows, up to 128 per pass) are the B operand, staged
//     through LDS in 128-element chunks and shared by the four wavefronts;
//   * each logit becomes a 64-bit key (order-preserving float bits, then
//     0xffffffff - v) so "largest logit, then lowest index" is a plain max;
//     keys are reduced over the block's rows with shuffles and LDS and one key
//     per (row, block) goes to the workspace;
//   * a second kernel takes the max over blocks for each row.
// Max is exact, so the result does not depend on reduction order.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "validate.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kNB = 2;               // 16-row vocabulary blocks per wavefront
constexpr int kKC = 128;             // K elements per LDS chunk
constexpr int kSteps = kKC / 32;
constexpr int kLdsRow = kKC + 8;
static_assert(kLmRowsPerBlock == 4 * kNB * 16, "block rows");

__device__ __forceinline__ unsigned long long make_key(float v, int idx) {
  return ((unsigned long long)float_key(v) << 32) | (uint32_t)(0xffffffffu - (uint32_t)idx);
}

template <int MB>
__global__ __launch_bounds__(kThreads) void lm_bf16_kernel(const bf16_t* __restrict__ h,
                                                           const bf16_t* __restrict__ W, int T, int H, int V,
                                                           unsigned long long* __restrict__ part, int nblk) {
  constexpr int MROWS = MB * 16;
  __shared__ __align__(16) bf16_t xl[2][MROWS][kLdsRow];
  __shared__ unsigned long long red[4][MROWS];

  const int blk = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int vbase = blk * kLmRowsPerBlock + wave * kNB * 16;
  // packed LM head: [pair of 32 rows][k-step][set][lane][8]; this wavefront's
  // 32 rows are one pair, each (pair, k-step) 2 KB of consecutive bytes
  const int nK = H / 32;
  const int n_pairs = (V + 31) / 32;
  const int pair = min(blk * 4 + wave, n_pairs - 1);  // past the vocabulary: a valid pair, masked below
  const bf16_t* wp[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) wp[nb] = W + (size_t)pair * nK * 1024 + nb * 512 + lane * 8;
  const int nC = (H + kKC - 1) / kKC;
  const int srow = threadIdx.x >> 4, sseg = (threadIdx.x & 15) * 8;

  for (int mstart = 0; mstart < T; mstart += MROWS) {
    const int mr = min(MROWS, T - mstart);
    // rows past T point at a valid row and are zeroed after the load: no
    // load is conditional, so the compiler can keep the weight stream in flight
    const bf16_t* src[MB];
    bool xvalid[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int row = srow + 16 * i;
      xvalid[i] = row < mr;
      src[i] = h + (size_t)(mstart + min(row, mr - 1)) * H;
    }
    f32x4_t acc[kNB][MB];
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
      for (int i = 0; i < MB; ++i) acc[nb][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    uint4 w0[kNB][kSteps], w1[kNB][kSteps], xst[MB];
    bool xok[MB];
    auto load_w = [&](int c, uint4 (*d)[kSteps]) __attribute__((always_inline)) {
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
        for (int s = 0; s < kSteps; ++s) d[nb][s] = ldg16_stream(wp[nb] + min(c * kSteps + s, nK - 1) * 1024);
    };
    auto load_x = [&](int c) __attribute__((always_inline)) {
      const int kofs = c * kKC + sseg;
      const bool kin = kofs < H;
      const int kc = min(kofs, H - 8);
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        xst[i] = ldg16(src[i] + kc);
        xok[i] = kin && xvalid[i];
      }
    };
    auto store_x = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const uint4 v = xst[i];
        const bool ok = xok[i];  // masked here, after the MFMAs, not at the load
        *reinterpret_cast<uint4*>(&xl[buf][srow + 16 * i][sseg]) =
            make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
      }
    };
    auto mma = [&](int buf, uint4 (*cw)[kSteps]) __attribute__((always_inline)) {
#pragma unroll
      for (int s = 0; s < kSteps; ++s)
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          const bf16x8_t bx = as_bf16x8(*reinterpret_cast<const uint4*>(
              &xl[buf][i * 16 + (lane & 15)][s * 32 + (lane >> 4) * 8]));
#pragma unroll
          for (int nb = 0; nb < kNB; ++nb) acc[nb][i] = mfma16x16x32(as_bf16x8(cw[nb][s]), bx, acc[nb][i]);
        }
    };
    auto step_pf = [&](int c, uint4 (*cw)[kSteps], uint4 (*nw)[kSteps]) __attribute__((always_inline)) {
      load_x(c + 1);
      load_w(c + 1, nw);
      __builtin_amdgcn_sched_barrier(0);  // issue the whole prefetch before any MFMA
      mma(c & 1, cw);
      __builtin_amdgcn_sched_barrier(0);
      store_x((c + 1) & 1);
      lds_barrier();
    };

    load_x(0);
    load_w(0, w0);
    store_x(0);
    lds_barrier();
    int c = 0;
    for (; c + 2 < nC; c += 2) {
      step_pf(c, w0, w1);
      step_pf(c + 1, w1, w0);
    }
    if (nC - c == 2) {
      step_pf(c, w0, w1);
      mma((c + 1) & 1, w1);
    } else {
      mma(c & 1, w0);
    }

    // lane holds D[vocab 4*(lane/16)+v][row lane%16] of each (nb, i) block
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      if (i * 16 < mr) {
        unsigned long long best = 0ull;
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int vocab = vbase + nb * 16 + 4 * (lane >> 4) + v;
            const unsigned long long key = vocab < V ? make_key(acc[nb][i][v], vocab) : 0ull;
            best = key > best ? key : best;
          }
        unsigned long long o = __shfl_xor(best, 16, kWave);
        best = o > best ? o : best;
        o = __shfl_xor(best, 32, kWave);
        best = o > best ? o : best;
        if (lane < 16) red[wave][i * 16 + lane] = best;
      }
    }
    lds_barrier();
    if (threadIdx.x < mr) {
      unsigned long long best = red[0][threadIdx.x];
#pragma unroll
      for (int w = 1; w < 4; ++w) best = red[w][threadIdx.x] > best ? red[w][threadIdx.x] : best;
      part[(size_t)(mstart + threadIdx.x) * nblk + blk] = best;
    }
    lds_barrier();
  }
}

// Streaming form (H % 128 == 0): a block of 8 wavefronts owns 256 vocabulary
// rows; wavefront w streams its pair of 16-row sets with a rotating register
// pipeline 4 k-steps deep that runs across the chunk barriers, so the
// weights never wait on the h staging.  h goes through LDS in 64-element
// chunks (2 k-steps, double buffered) in fragment order: the 1 KB B operand
// of token block i and k-step s is lane-ordered, so each read is one
// conflict-free ds_read_b128.  A chunk is loaded into registers two chunks
// ahead and written to LDS one chunk ahead; one barrier per chunk.
constexpr int kSWaves = 8;
constexpr int kSThreads = kSWaves * 64;
constexpr int kSRows = kSWaves * 32;      // vocabulary rows per block

template <int MB>
__global__ __launch_bounds__(kSThreads) void lm_stream_kernel(const bf16_t* __restrict__ h,
                                                              const bf16_t* __restrict__ W, int T, int H, int V,
                                                              unsigned long long* __restrict__ part, int nblk) {
  constexpr int MROWS = MB * 16;
  constexpr int NF = MB * 2;              // h fragments per chunk
  constexpr int FPT = (NF + kSWaves - 1) / kSWaves;  // fragments staged per thread
  __shared__ __align__(16) char xl[2][NF * 1024];
  __shared__ unsigned long long red[kSWaves][MROWS];

  const int blk = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nK = H / 32, nC = H / 64;
  const int n_pairs = (V + 31) / 32;
  const int pair = min(blk * kSWaves + wave, n_pairs - 1);  // past the vocabulary: a valid pair, masked below
  const int vbase = (blk * kSWaves + wave) * 32;
  const bf16_t* wa = W + (size_t)pair * nK * 1024 + lane * 8;
  const bf16_t* wb = wa + 512;

  {
    // token pass blockIdx.y: a grid dimension rather than a loop, so the
    // compiler does not hoist the first weight loads out of it (a copy of
    // the whole ring per pass, measured 248 -> 202 VGPRs at 128 tokens and
    // 120 -> 64 at 16)
    const int mstart = blockIdx.y * MROWS;
    const int mr = min(MROWS, T - mstart);
    // h staging: thread stages fragments f = wave + 8u (token block f/2,
    // k-step f%2 of the chunk), lane's token and 8-element segment
    const bf16_t* hsrc[FPT];
#pragma unroll
    for (int u = 0; u < FPT; ++u) {
      const int f = min(wave + kSWaves * u, NF - 1);
      const int tok = mstart + min(16 * (f >> 1) + (lane & 15), mr - 1);   // past T: a valid row, never stored
      hsrc[u] = h + (size_t)tok * H + 32 * (f & 1) + 8 * (lane >> 4);
    }
    uint4 hs[FPT];
    auto hload = [&](int c) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < FPT; ++u) hs[u] = ldg16(hsrc[u] + c * 64);
    };
    auto hstore = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < FPT; ++u)
        if (wave + kSWaves * u < NF) *reinterpret_cast<uint4*>(&xl[buf][(wave + kSWaves * u) * 1024 + lane * 16]) = hs[u];
    };

    f32x4_t acc[2][MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) acc[0][i] = acc[1][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    uint4 ra[4], rb[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      ra[d] = ldg16_stream(wa + min(d, nK - 1) * 1024);
      rb[d] = ldg16_stream(wb + min(d, nK - 1) * 1024);
    }
    hload(0);
    hstore(0);
    if (nC > 1) hload(1);
    lds_barrier();

    // one chunk: k-steps 2c, 2c+1 use ring slots S0, S0+1 and refill them 4 ahead
    auto chunk = [&](int c, auto S0) __attribute__((always_inline)) {
      constexpr int s0 = decltype(S0)::value;
      if (c + 1 < nC) hstore((c + 1) & 1);
      if (c + 2 < nC) hload(c + 2);
      const char* buf = xl[c & 1];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          const bf16x8_t bx = as_bf16x8(*reinterpret_cast<const uint4*>(buf + (i * 2 + ks) * 1024 + lane * 16));
          acc[0][i] = mfma16x16x32(as_bf16x8(ra[s0 + ks]), bx, acc[0][i]);
          acc[1][i] = mfma16x16x32(as_bf16x8(rb[s0 + ks]), bx, acc[1][i]);
        }
        const int kk = min(2 * c + ks + 4, nK - 1);
        ra[s0 + ks] = ldg16_stream(wa + kk * 1024);
        rb[s0 + ks] = ldg16_stream(wb + kk * 1024);
      }
      lds_barrier();
    };
    int c = 0;
    for (; c + 1 < nC; c += 2) {
      chunk(c, std::integral_constant<int, 0>());
      chunk(c + 1, std::integral_constant<int, 2>());
    }
    if (c < nC) chunk(c, std::integral_constant<int, 0>());

    // lane holds D[vocab 4*(lane/16)+v][token lane%16] of each (set, token block)
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      unsigned long long best = 0ull;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int vocab = vbase + st * 16 + 4 * (lane >> 4) + v;
          const unsigned long long key = vocab < V ? make_key(acc[st][i][v], vocab) : 0ull;
          best = key > best ? key : best;
        }
      unsigned long long o = __shfl_xor(best, 16, kWave);
      best = o > best ? o : best;
      o = __shfl_xor(best, 32, kWave);
      best = o > best ? o : best;
      if (lane < 16) red[wave][i * 16 + lane] = best;
    }
    lds_barrier();
    if (threadIdx.x < mr) {
      unsigned long long best = red[0][threadIdx.x];
#pragma unroll
      for (int w = 1; w < kSWaves; ++w) best = red[w][threadIdx.x] > best ? red[w][threadIdx.x] : best;
      part[(size_t)(mstart + threadIdx.x) * nblk + blk] = best;
    }
  }
}

// fp32 path: one thread per vocabulary row, plain sequential dot products.
__global__ __launch_bounds__(256) void lm_f32_kernel(const float* __restrict__ h, const float* __restrict__ W,
                                                     int T, int H, int V, unsigned long long* __restrict__ part,
                                                     int nblk) {
  __shared__ unsigned long long red[4];
  const int v = blockIdx.x * kLmF32RowsPerBlock + threadIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const float* w = W + (size_t)min(v, V - 1) * H;
  for (int t = 0; t < T; ++t) {
    const float* x = h + (size_t)t * H;
    float acc = 0.f;
    for (int j = 0; j < H; ++j) acc = fmaf(w[j], x[j], acc);
    unsigned long long key = v < V ? make_key(acc, v) : 0ull;
    key = wave_max_u64(key);
    if (lane == 0) red[wave] = key;
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned long long best = red[0];
      for (int i = 1; i < 4; ++i) best = red[i] > best ? red[i] : best;
      part[(size_t)t * nblk + blockIdx.x] = best;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(64) void lm_reduce_kernel(const unsigned long long* __restrict__ part, int nblk,
                                                       int32_t* __restrict__ ids, float* __restrict__ max_logit) {
  const int t = blockIdx.x;
  unsigned long long best = 0ull;
  // 8 keys per lane in flight at once (a loop of single loads waits out one
  // round trip per key)
  for (int i0 = threadIdx.x; i0 < nblk; i0 += 8 * kWave) {
    unsigned long long k[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * kWave;
      k[u] = i < nblk ? part[(size_t)t * nblk + i] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) best = k[u] > best ? k[u] : best;
  }
  best = wave_max_u64(best);
  if (threadIdx.x == 0) {
    ids[t] = (int32_t)(0xffffffffu - (uint32_t)(best & 0xffffffffull));
    if (max_logit) max_logit[t] = key_float((uint32_t)(best >> 32));
  }
}

template <int MB>
void launch_mb(const bf16_t* h, const bf16_t* W, int T, int H, int V, unsigned long long* part, int nblk,
               hipStream_t s) {
  if (H % 128 == 0)  // nblk = ceil(V / 256): one block per 256 vocabulary rows
    hipLaunchKernelGGL((lm_stream_kernel<MB>), dim3(nblk, (T + MB * 16 - 1) / (MB * 16)), dim3(kSThreads), 0, s, h,
                       W, T, H, V, part, nblk);
  else
    hipLaunchKernelGGL((lm_bf16_kernel<MB>), dim3(nblk), dim3(kThreads), 0, s, h, W, T, H, V, part, nblk);
}

}  // namespace

hipError_t launch_lmhead(const void* h, const void* w_lm, int T, int H, int V, int dtype,
                         int32_t* ids, float* max_logit, void* ws, hipStream_t s) {
  unsigned long long* part = static_cast<unsigned long long*>(ws);
  // the streaming bf16 form has half as many (256-row) blocks as the workspace is sized for
  const int nblk = dtype == kBf16 && H % 128 == 0 ? (V + kSRows - 1) / kSRows : lmhead_blocks(V, dtype);
  if (dtype == kF32) {
    hipLaunchKernelGGL(lm_f32_kernel, dim3(nblk), dim3(256), 0, s, static_cast<const float*>(h),
                       static_cast<const float*>(w_lm), T, H, V, part, nblk);
  } else {
    const bf16_t* hb = static_cast<const bf16_t*>(h);
    const bf16_t* wb = static_cast<const bf16_t*>(w_lm);
    if (T <= 16) launch_mb<1>(hb, wb, T, H, V, part, nblk, s);
    else if (T <= 32) launch_mb<2>(hb, wb, T, H, V, part, nblk, s);
    else if (T <= 64) launch_mb<4>(hb, wb, T, H, V, part, nblk, s);
    else launch_mb<8>(hb, wb, T, H, V, part, nblk, s);
  }
  hipLaunchKernelGGL(lm_reduce_kernel, dim3(T), dim3(64), 0, s, part, nblk, ids, max_logit);
  return hipGetLastError();
}

}  // namespace moe
