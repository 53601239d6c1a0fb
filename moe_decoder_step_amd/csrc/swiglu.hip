// moe_grouped_swiglu: per expert group, a = silu(W_g x) * (W_u x); y = W_d a.
//
// bf16 path (decode-sized groups): the expert weights are the bytes that
// matter -- each row of W is read once from HBM and used for every token of
// its group -- so the kernel is a weight stream feeding MFMA:
//   * a block of 4 wavefronts owns 64 output columns of one group; wavefront w
//     owns 16 of them (for the gated stage, its 16 gate rows and the matching
//     16 up rows) and streams those weight rows straight into registers as the
//     A operand of v_mfma_f32_16x16x32_bf16, two 128-element chunks in flight;
//   * the group's activation rows (gathered tokens) are the B operand; they
//     are staged through LDS in 128-element chunks (double-buffered) and
//     shared by the block's four wavefronts;
//   * a block covers up to 32 rows; larger groups are split over several
//     blocks, and the row blocks of one (group, column tile) are placed on the
//     same XCD (consecutive blocks of that XCD) so they share its L2 copy of
//     the weights;
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
constexpr int kKC = 128;             // K elements per LDS chunk
constexpr int kSteps = kKC / 32;     // MFMA k-steps per chunk
constexpr int kLdsRow = kKC + 8;     // padded LDS row (bf16 elements)

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// GATED: x = token rows [T,K] read through gather, W = [G, 2N, K] (gate rows
//        0..N-1, up rows N..2N-1), out = a [n_rows, N].
// plain: x = activation rows [n_rows, K] read directly, W = [G, N, K],
//        out = y [n_rows, N].
template <int MB, bool GATED>
__global__ __launch_bounds__(kThreads) void skinny_kernel(
    const bf16_t* __restrict__ x, const int32_t* __restrict__ gather,
    const int32_t* __restrict__ offsets, int G, int n_rows, int T,
    const bf16_t* __restrict__ W, int K, int N, int n_ctiles, int n_mranges,
    bf16_t* __restrict__ out) {
  constexpr int MROWS = MB * 16;
  __shared__ __align__(16) bf16_t xl[2][MROWS][kLdsRow];

  // (group, column tile) pair p lives on XCD p % 8; its row ranges are
  // consecutive blocks of that XCD (block b runs on XCD b % 8).
  const int b = blockIdx.x;
  const int xcd = b & 7, local = b >> 3;
  const int q = local / n_mranges, mr_idx = local % n_mranges;
  const int p = xcd + 8 * q;
  if (p >= G * n_ctiles) return;
  const int g = p / n_ctiles, ct = p % n_ctiles;
  const int r_begin = clampi(offsets[g], 0, n_rows);
  const int r_end = clampi(offsets[g + 1], r_begin, n_rows);
  if (r_begin + mr_idx * MROWS >= r_end) return;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col0 = ct * kColsPerBlock + wave * 16;
  const bool active = col0 < N;
  const size_t gstride = (GATED ? (size_t)2 * N : (size_t)N) * K;
  const int wrow = min(col0 + (lane & 15), N - 1);
  const bf16_t* wa = W + g * gstride + (size_t)wrow * K + (lane >> 4) * 8;
  const bf16_t* wb = wa + (size_t)N * K;  // up rows (gated stage only)
  const int nK = K / 32;
  const int nC = (K + kKC - 1) / kKC;

  // LDS staging role of this thread: rows srow + 16 i, 8 elements at sseg
  const int srow = threadIdx.x >> 4, sseg = (threadIdx.x & 15) * 8;

  for (int mstart = r_begin + mr_idx * MROWS; mstart < r_end; mstart += n_mranges * MROWS) {
    const int mr = min(MROWS, r_end - mstart);
    const bf16_t* src[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int row = srow + 16 * i;
      src[i] = nullptr;
      if (row < mr) {
        const int r = mstart + row;
        int s;
        if (GATED) s = gather ? clampi(gather[r], 0, T - 1) : clampi(r - r_begin, 0, T - 1);
        else s = r;
        src[i] = x + (size_t)s * K + sseg;
      }
    }

    f32x4_t acc_a[MB], acc_b[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      acc_a[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      acc_b[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    uint4 w0a[kSteps], w0b[kSteps], w1a[kSteps], w1b[kSteps], xst[MB];

    auto load_w = [&](int c, uint4* da, uint4* db) __attribute__((always_inline)) {
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        const int kk = c * kSteps + s;
        if (active && kk < nK) {
          da[s] = ldg16_stream(wa + kk * 32);
          if (GATED) db[s] = ldg16_stream(wb + kk * 32);
        } else {
          da[s] = make_uint4(0u, 0u, 0u, 0u);
          if (GATED) db[s] = make_uint4(0u, 0u, 0u, 0u);
        }
      }
    };
    auto load_x = [&](int c) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int kofs = c * kKC + sseg;
        xst[i] = (src[i] && kofs < K) ? ldg16(src[i] + c * kKC) : make_uint4(0u, 0u, 0u, 0u);
      }
    };
    auto store_x = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < MB; ++i) *reinterpret_cast<uint4*>(&xl[buf][srow + 16 * i][sseg]) = xst[i];
    };
    // One chunk: prefetch chunk c+1 (activations first, so that waiting for
    // them before the LDS store leaves the weight loads in flight), run the
    // MFMAs of chunk c on (ca, cb), stage chunk c+1 into the other buffer.
    auto chunk = [&](int c, const uint4* ca, const uint4* cb, uint4* na, uint4* nb) __attribute__((always_inline)) {
      const bool more = c + 1 < nC;
      if (more) {
        load_x(c + 1);
        load_w(c + 1, na, nb);
      }
      const int buf = c & 1;
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        if (c * kSteps + s < nK) {
#pragma unroll
          for (int i = 0; i < MB; ++i) {
            if (i * 16 < mr) {
              const bf16x8_t bx = as_bf16x8(*reinterpret_cast<const uint4*>(
                  &xl[buf][i * 16 + (lane & 15)][s * 32 + (lane >> 4) * 8]));
              acc_a[i] = mfma16x16x32(as_bf16x8(ca[s]), bx, acc_a[i]);
              if (GATED) acc_b[i] = mfma16x16x32(as_bf16x8(cb[s]), bx, acc_b[i]);
            }
          }
        }
      }
      if (more) store_x(buf ^ 1);
      __syncthreads();
    };

    load_x(0);
    load_w(0, w0a, w0b);
    store_x(0);
    __syncthreads();
    for (int c = 0; c < nC; c += 2) {
      chunk(c, w0a, w0b, w1a, w1b);
      if (c + 1 < nC) chunk(c + 1, w1a, w1b, w0a, w0b);
    }

    // D[col 4*(lane/16)+v][row lane%16] -> 4 consecutive output columns of one row
    if (active) {
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int row = i * 16 + (lane & 15);
        if (i * 16 < mr && row < mr) {
          float o[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) o[v] = GATED ? silu(acc_a[i][v]) * acc_b[i][v] : acc_a[i][v];
          uint2 pk;
          pk.x = pack2(f32_to_bf16(o[0]), f32_to_bf16(o[1]));
          pk.y = pack2(f32_to_bf16(o[2]), f32_to_bf16(o[3]));
          *reinterpret_cast<uint2*>(out + (size_t)(mstart + row) * N + col0 + 4 * (lane >> 4)) = pk;
        }
      }
    }
  }
}

template <int MB>
hipError_t launch_bf16(const bf16_t* x, const int32_t* gather, const int32_t* offsets, int G, int n_rows,
                       const bf16_t* wgu, const bf16_t* wd, int T, int H, int I, int max_rows, bf16_t* act,
                       bf16_t* y, hipStream_t s) {
  const int mrows = MB * 16;
  const int n_mranges = max(1, (max_rows + mrows - 1) / mrows);
  {
    const int n_ctiles = (I + kColsPerBlock - 1) / kColsPerBlock;
    const int pairs = G * n_ctiles;
    const int blocks = 8 * ((pairs + 7) / 8) * n_mranges;
    hipLaunchKernelGGL((skinny_kernel<MB, true>), dim3(blocks), dim3(kThreads), 0, s, x, gather, offsets, G,
                       n_rows, T, wgu, H, I, n_ctiles, n_mranges, act);
  }
  {
    const int n_ctiles = (H + kColsPerBlock - 1) / kColsPerBlock;
    const int pairs = G * n_ctiles;
    const int blocks = 8 * ((pairs + 7) / 8) * n_mranges;
    hipLaunchKernelGGL((skinny_kernel<MB, false>), dim3(blocks), dim3(kThreads), 0, s, act, nullptr, offsets,
                       G, n_rows, T, wd, I, H, n_ctiles, n_mranges, y);
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
  if (max_rows <= 16)
    return launch_bf16<1>(xb, gather, offsets, G, n_rows, wgu, wd, T, H, I, max_rows, act, yb, s);
  return launch_bf16<2>(xb, gather, offsets, G, n_rows, wgu, wd, T, H, I, max_rows, act, yb, s);
}

}  // namespace moe
