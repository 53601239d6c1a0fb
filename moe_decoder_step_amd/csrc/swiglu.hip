// moe_grouped_swiglu: per expert group, a = silu(W_g x) * (W_u x); y = W_d a.
//
// bf16 path (decode-sized groups): the expert weights are the bytes that
// matter -- each row of W is read once from HBM and used for every token of
// its group -- so the kernel is a weight stream feeding MFMA:
//   * a block of 4 wavefronts owns 64 output columns of one group; wavefront w
//     owns 16 of them (for the gated stage, its 16 gate rows and the matching
//     16 up rows) and streams those weight rows straight into registers as the
//     A operand of v_mfma_f32_16x16x32_bf16, three or four 32-wide k-steps in flight;
//   * the group's activation rows (gathered tokens, a few hundred KB that stay
//     in L2) are the B operand, loaded by each wavefront alongside its
//     weights -- no LDS and no barrier, so every wavefront streams on its own;
//   * a block covers up to 32 rows; larger groups are split over several
//     blocks on the same XCD, so they share its L2 copy of the weights;
//   * groups with no rows cost one early exit, so untouched experts are
//     never read.
// The fp32 reduction order along K is fixed (chunk by chunk, 32 per MFMA)
// and does not depend on how many rows a group has.
//
// fp32 path (the tiny fp32 configuration): one thread per output element,
// plain sequential fp32 dot products.
#include "common.hpp"
#include "kernels.hpp"
#include "validate.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kColsPerBlock = 64;

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// One wavefront's stream: 16 weight rows (with TWO, a second set of 16: the
// matching up rows, or the next 16 output rows) over the full reduction length K, against NM
// 16-row activation blocks.  Lane l supplies weight row l%16 and activation
// row l%16 at k-offset 8*(l/16) of every 32-wide MFMA step.  D steps of
// loads are kept in flight in rotating registers; the loop body has no
// conditional load (a conditional load makes the compiler drain every
// outstanding load), so the weight stream never stalls on a full drain.
template <int NM, int D, bool TWO>
__device__ __forceinline__ void stream_rows(const bf16_t* wa, const bf16_t* wb, const bf16_t* const* xp, int nK,
                                            f32x4_t* acc_a, f32x4_t* acc_b) {
  uint4 ra[D], rb[D], rx[D][NM];
  auto load = [&](int d, int kk) __attribute__((always_inline)) {
    ra[d] = ldg16(wa + kk * 32);
    if (TWO) rb[d] = ldg16(wb + kk * 32);
#pragma unroll
    for (int i = 0; i < NM; ++i) rx[d][i] = ldg16(xp[i] + kk * 32);
  };
  auto mma = [&](int d) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      const bf16x8_t bx = as_bf16x8(rx[d][i]);
      acc_a[i] = mfma16x16x32(as_bf16x8(ra[d]), bx, acc_a[i]);
      if (TWO) acc_b[i] = mfma16x16x32(as_bf16x8(rb[d]), bx, acc_b[i]);
    }
  };
#pragma unroll
  for (int d = 0; d < D; ++d) load(d, min(d, nK - 1));
  const int nfull = nK / D;
  for (int g = 0; g < nfull; ++g) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      mma(d);
      load(d, min((g + 1) * D + d, nK - 1));  // past the end: a repeat of the last step, never used
    }
  }
  const int rem = nK - nfull * D;
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (d < rem) mma(d);
}

// GATED: x = token rows [T,K] read through gather, W = [G, 2N, K] (gate rows
//        0..N-1, up rows N..2N-1), out = a [n_rows, N]; wavefront w owns output
//        columns 16w..16w+15 of a 64-column block tile (its 16 gate rows and
//        16 up rows are the two streamed row sets).
// plain: x = activation rows [n_rows, K] read directly, W = [G, N, K],
//        out = y [n_rows, N]; wavefront w owns output columns 32w..32w+31 of a
//        128-column block tile (two 16-row sets), so that every wavefront
//        streams as many bytes per k-step as in the gated stage.
// A block of 4 independent wavefronts owns one column tile of one group and
// one range of up to 32 rows.
template <bool GATED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void skinny_kernel(
    const bf16_t* __restrict__ x, const int32_t* __restrict__ gather,
    const int32_t* __restrict__ offsets, int G, int n_rows, int T,
    const bf16_t* __restrict__ W, int K, int N, int n_ctiles, int n_mranges,
    bf16_t* __restrict__ out) {
  constexpr int MROWS = 32;
  constexpr int D = 3;               // k-steps in flight: fits 4 wavefronts per SIMD without spills
  constexpr int WCOLS = GATED ? 16 : 32;  // output columns per wavefront
  // Block b runs on XCD b % 8.  (group, column tile) pair p lives on XCD
  // p % 8, so the row ranges of one pair share that XCD's L2 copy of the
  // weights.  The row range is the slowest-varying index: the first range of
  // every pair (the only non-empty one for a decode-sized group) comes first
  // and is dealt over all CUs of the XCD; later ranges, mostly empty, follow.
  const int b = blockIdx.x;
  const int xcd = b & 7, local = b >> 3;
  const int per_xcd = (G * n_ctiles + 7) / 8;
  const int mr_idx = local / per_xcd, q = local % per_xcd;
  const int p = xcd + 8 * q;
  if (p >= G * n_ctiles) return;
  const int g = p / n_ctiles, ct = p % n_ctiles;
  const int r_begin = clampi(offsets[g], 0, n_rows);
  const int r_end = clampi(offsets[g + 1], r_begin, n_rows);

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col0 = ct * (4 * WCOLS) + wave * WCOLS;
  if (col0 >= N) return;  // waves are independent: no block-wide sync below
  const size_t gstride = (GATED ? (size_t)2 * N : (size_t)N) * K;
  const bf16_t* wa = W + g * gstride + (size_t)(col0 + (lane & 15)) * K + (lane >> 4) * 8;
  // second row set: the up rows (gated) or the next 16 output columns (plain;
  // clamped to a valid row when N is not a multiple of 32 -- never stored)
  const bf16_t* wb = GATED ? wa + (size_t)N * K
                           : W + g * gstride + (size_t)min(col0 + 16 + (lane & 15), N - 1) * K + (lane >> 4) * 8;
  const int nK = K / 32;

  for (int mstart = r_begin + mr_idx * MROWS; mstart < r_end; mstart += n_mranges * MROWS) {
    const int mr = min(MROWS, r_end - mstart);
    // activation row of this lane in each 16-row block (rows past the group
    // read a valid row; their results are never stored)
    const bf16_t* xp[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = mstart + min(i * 16 + (lane & 15), mr - 1);
      int s;
      if (GATED) s = gather ? clampi(gather[r], 0, T - 1) : clampi(r - r_begin, 0, T - 1);
      else s = r;
      xp[i] = x + (size_t)s * K + (lane >> 4) * 8;
    }
    f32x4_t acc_a[2], acc_b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      acc_a[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      acc_b[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    if (mr <= 16) stream_rows<1, D, true>(wa, wb, xp, nK, acc_a, acc_b);
    else stream_rows<2, D, true>(wa, wb, xp, nK, acc_a, acc_b);

    // lane holds D[col 4*(lane/16)+v][row lane%16]: 4 consecutive output columns of one row
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = i * 16 + (lane & 15);
      if (row < mr) {
        bf16_t* orow = out + (size_t)(mstart + row) * N + col0 + 4 * (lane >> 4);
        if (GATED) {
          uint2 pk;
          pk.x = pack2(f32_to_bf16(silu(acc_a[i][0]) * acc_b[i][0]), f32_to_bf16(silu(acc_a[i][1]) * acc_b[i][1]));
          pk.y = pack2(f32_to_bf16(silu(acc_a[i][2]) * acc_b[i][2]), f32_to_bf16(silu(acc_a[i][3]) * acc_b[i][3]));
          *reinterpret_cast<uint2*>(orow) = pk;
        } else {
          uint2 pa, pb;
          pa.x = pack2(f32_to_bf16(acc_a[i][0]), f32_to_bf16(acc_a[i][1]));
          pa.y = pack2(f32_to_bf16(acc_a[i][2]), f32_to_bf16(acc_a[i][3]));
          pb.x = pack2(f32_to_bf16(acc_b[i][0]), f32_to_bf16(acc_b[i][1]));
          pb.y = pack2(f32_to_bf16(acc_b[i][2]), f32_to_bf16(acc_b[i][3]));
          *reinterpret_cast<uint2*>(orow) = pa;
          if (col0 + 16 < N) *reinterpret_cast<uint2*>(orow + 16) = pb;
        }
      }
    }
  }
}

hipError_t launch_bf16(const bf16_t* x, const int32_t* gather, const int32_t* offsets, int G, int n_rows,
                       const bf16_t* wgu, const bf16_t* wd, int T, int H, int I, int max_rows, bf16_t* act,
                       bf16_t* y, hipStream_t s) {
  const int n_mranges = max(1, (max_rows + 31) / 32);
  {
    const int n_ctiles = (I + kColsPerBlock - 1) / kColsPerBlock;
    const int blocks = 8 * ((G * n_ctiles + 7) / 8) * n_mranges;
    hipLaunchKernelGGL((skinny_kernel<true>), dim3(blocks), dim3(kThreads), 0, s, x, gather, offsets, G, n_rows,
                       T, wgu, H, I, n_ctiles, n_mranges, act);
  }
  {
    const int n_ctiles = (H + 2 * kColsPerBlock - 1) / (2 * kColsPerBlock);
    const int blocks = 8 * ((G * n_ctiles + 7) / 8) * n_mranges;
    hipLaunchKernelGGL((skinny_kernel<false>), dim3(blocks), dim3(kThreads), 0, s, act, nullptr, offsets, G,
                       n_rows, T, wd, I, H, n_ctiles, n_mranges, y);
  }
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

__global__ __launch_bounds__(256) void f32_gate_up_kernel(const float* __restrict__ x,
                                                          const int32_t* __restrict__ gather,
                                                          const int32_t* __restrict__ offsets, int G,
                                                          int n_rows, int T, const float* __restrict__ wgu,
                                                          int H, int I, float* __restrict__ act) {
  const int r = blockIdx.x;
  int r_begin = 0;
  const int g = find_group(offsets, G, n_rows, r, &r_begin);
  if (g < 0) return;
  const int t = gather ? clampi(gather[r], 0, T - 1) : clampi(r - r_begin, 0, T - 1);
  const float* xr = x + (size_t)t * H;
  for (int c = threadIdx.x; c < I; c += blockDim.x) {
    const float* wg = wgu + ((size_t)g * 2 * I + c) * H;
    const float* wu = wg + (size_t)I * H;
    float a = 0.f, u = 0.f;
    for (int h = 0; h < H; ++h) {
      a = fmaf(wg[h], xr[h], a);
      u = fmaf(wu[h], xr[h], u);
    }
    act[(size_t)r * I + c] = silu(a) * u;
  }
}

__global__ __launch_bounds__(256) void f32_down_kernel(const float* __restrict__ act,
                                                       const int32_t* __restrict__ offsets, int G, int n_rows,
                                                       const float* __restrict__ wd, int H, int I,
                                                       float* __restrict__ y) {
  const int r = blockIdx.x;
  int r_begin = 0;
  const int g = find_group(offsets, G, n_rows, r, &r_begin);
  if (g < 0) return;
  const float* ar = act + (size_t)r * I;
  for (int o = threadIdx.x; o < H; o += blockDim.x) {
    const float* w = wd + ((size_t)g * H + o) * I;
    float acc = 0.f;
    for (int c = 0; c < I; ++c) acc = fmaf(w[c], ar[c], acc);
    y[(size_t)r * H + o] = acc;
  }
}

}  // namespace

hipError_t launch_swiglu(const void* x, const int32_t* gather, const int32_t* offsets, int G,
                         int n_rows, const void* w_gate_up, const void* w_down, int T, int H, int I,
                         int max_rows, int dtype, void* y, void* ws, hipStream_t s) {
  if (dtype == kF32) {
    float* act = static_cast<float*>(ws);
    hipLaunchKernelGGL(f32_gate_up_kernel, dim3(n_rows), dim3(256), 0, s, static_cast<const float*>(x), gather,
                       offsets, G, n_rows, T, static_cast<const float*>(w_gate_up), H, I, act);
    hipLaunchKernelGGL(f32_down_kernel, dim3(n_rows), dim3(256), 0, s, act, offsets, G, n_rows,
                       static_cast<const float*>(w_down), H, I, static_cast<float*>(y));
    return hipGetLastError();
  }
  const bf16_t* xb = static_cast<const bf16_t*>(x);
  const bf16_t* wgu = static_cast<const bf16_t*>(w_gate_up);
  const bf16_t* wd = static_cast<const bf16_t*>(w_down);
  bf16_t* act = static_cast<bf16_t*>(ws);
  bf16_t* yb = static_cast<bf16_t*>(y);
  return launch_bf16(xb, gather, offsets, G, n_rows, wgu, wd, T, H, I, max_rows, act, yb, s);
}

}  // namespace moe
