// moe_pack_weights: logical bf16 weight matrices -> the streamed fragment layout.
//
// The weight-streaming kernels read a weight row set as the A operand of
// v_mfma_f32_16x16x32_bf16: lane l of a wavefront needs row l%16, elements
// 8*(l/16) .. 8*(l/16)+7 of every 32-wide k-step.  Stored row-major, one such
// load touches 64 bytes of 16 rows; the level-1 cache then sends half-line
// requests and halves the request throughput.  The packed layout stores every
// (row pair, k-step, set) fragment as 1 KB in lane order, so a load is 1 KB
// of consecutive bytes:
//
//   packed[g][p][s][h][l][j] = W[g][row(p, h, l % 16)][32 s + 8 (l / 16) + j]
//
// with p the pair index, s the k-step, h the set (0, 1), l the lane, j < 8:
//   MOE_PACK_GATE_UP: W is [G, 2N, K] (gate rows, then up rows); pair p holds
//                     gate rows 16p.. (set 0) and up rows N + 16p.. (set 1);
//   MOE_PACK_ROWS:    W is [G, N, K]; pair p holds rows 32p + 16h + (0..15);
//                     rows at or past N are zero.
//
// The fp32 router weight [G, E, K] (E <= 64 experts, one per lane) is packed
// as packed[g][q][e][j] = W[g][e][4q + j] (MOE_PACK_ROUTER; experts past E
// are zero), so a wavefront's 16-byte loads of four hidden elements for its
// 64 expert lanes are 1 KB of consecutive bytes.
#include "common.hpp"
#include "kernels.hpp"
#include "validate.hpp"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void pack_kernel(const bf16_t* __restrict__ src, bf16_t* __restrict__ dst,
                                                   int G, int N, int K, int kind, int n_pairs, long long total) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;  // one 16-byte piece
  if (idx >= total) return;
  const int nK = K / 32;
  const int l = (int)(idx % 64);
  long long r = idx / 64;
  const int h = (int)(r % 2);
  r /= 2;
  const int s = (int)(r % nK);
  r /= nK;
  const int p = (int)(r % n_pairs);
  const int g = (int)(r / n_pairs);
  int row;
  size_t rows_per_group;
  if (kind == 0) {
    row = h * N + 16 * p + (l & 15);
    rows_per_group = (size_t)2 * N;
  } else {
    row = 32 * p + 16 * h + (l & 15);
    rows_per_group = (size_t)N;
  }
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (kind != 0 ? row < N : true)
    v = ldg16(src + ((size_t)g * rows_per_group + row) * K + 32 * s + 8 * (l >> 4));
  *reinterpret_cast<uint4*>(dst + idx * 8) = v;
}

__global__ __launch_bounds__(256) void pack_router_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                                          int E, int K, long long total) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;  // one float4
  if (idx >= total) return;
  const int e = (int)(idx % 64);
  const long long r = idx / 64;
  const int q = (int)(r % (K / 4));
  const int g = (int)(r / (K / 4));
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (e < E) v = *reinterpret_cast<const float4*>(src + ((size_t)g * E + e) * K + 4 * q);
  *reinterpret_cast<float4*>(dst + idx * 4) = v;
}

}  // namespace

hipError_t launch_pack_router(const void* src, void* dst, int G, int E, int K, hipStream_t s) {
  const long long total = (long long)G * (K / 4) * 64;
  hipLaunchKernelGGL(pack_router_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                     static_cast<const float*>(src), static_cast<float*>(dst), E, K, total);
  return hipGetLastError();
}

hipError_t launch_pack(const void* src, void* dst, int G, int N, int K, int kind, hipStream_t s) {
  const int n_pairs = pack_pairs(N, kind);
  const long long total = (long long)G * n_pairs * (K / 32) * 2 * 64;
  const long long blocks = (total + 255) / 256;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<const bf16_t*>(src),
                     static_cast<bf16_t*>(dst), G, N, K, kind, n_pairs, total);
  return hipGetLastError();
}

}  // namespace moe
