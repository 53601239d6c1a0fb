// moe_combine: out[t] = residual[t] + sum_j w[t,j] y[inv(t,j)] + sum_s ys[s,t].
//
// One block per token row; each thread owns 8 consecutive hidden elements
// (one 16-byte vector for bf16) and sums its k routed rows and S shared rows
// in a fixed order in fp32, so a token's result never depends on the batch.
// The k row indices and weights are read once per block into LDS.
#include "common.hpp"
#include "kernels.hpp"
#include "validate.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;  // one thread per 8 elements of the row (H <= 2048 in one pass)

__device__ __forceinline__ void load8(const bf16_t* p, float* f) { unpack8(ldg16(p), f); }
__device__ __forceinline__ void load8(const float* p, float* f) {
  float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}
__device__ __forceinline__ void store8(bf16_t* p, const float* f) {
  uint4 o;
  o.x = pack2(f32_to_bf16(f[0]), f32_to_bf16(f[1]));
  o.y = pack2(f32_to_bf16(f[2]), f32_to_bf16(f[3]));
  o.z = pack2(f32_to_bf16(f[4]), f32_to_bf16(f[5]));
  o.w = pack2(f32_to_bf16(f[6]), f32_to_bf16(f[7]));
  *reinterpret_cast<uint4*>(p) = o;
}
__device__ __forceinline__ void store8(float* p, const float* f) {
  *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(f[4], f[5], f[6], f[7]);
}

template <typename St>
__global__ __launch_bounds__(kThreads) void combine_kernel(
    const St* __restrict__ y, const int32_t* __restrict__ inv, const float* __restrict__ w,
    const St* __restrict__ ys, int S, const St* res, int T, int H, int k, int n_rows, St* out,
    St* __restrict__ combined) {
  const int t = blockIdx.x;
  __shared__ int rows[kMaxExperts];
  __shared__ float wk[kMaxExperts];
  if (threadIdx.x < k) {
    rows[threadIdx.x] = clampi(inv[(size_t)t * k + threadIdx.x], 0, n_rows - 1);
    wk[threadIdx.x] = w[(size_t)t * k + threadIdx.x];
  }
  __syncthreads();
  for (int c = threadIdx.x * 8; c < H; c += kThreads * 8) {
    float acc[8], f[8];
    typename Row8<St>::raw rres{};
    if (res) rres = Row8<St>::load(res + (size_t)t * H + c);   // in flight with the expert rows
    combine8(y, rows, wk, k, ys, S, T, t, H, c, acc);
    if (combined) store8(combined + (size_t)t * H + c, acc);
    if (res) {
      Row8<St>::unpack(rres, f);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] += acc[i];
      store8(out + (size_t)t * H + c, f);
    } else {
      store8(out + (size_t)t * H + c, acc);
    }
  }
}

}  // namespace

hipError_t launch_combine(const void* y, const int32_t* inv, const float* topk_w,
                          const void* y_shared, int S, const void* residual, int T, int H, int k,
                          int n_rows, int dtype, void* out, void* combined, hipStream_t s) {
  if (dtype == kBf16)
    hipLaunchKernelGGL((combine_kernel<bf16_t>), dim3(T), dim3(kThreads), 0, s,
                       static_cast<const bf16_t*>(y), inv, topk_w, static_cast<const bf16_t*>(y_shared), S,
                       static_cast<const bf16_t*>(residual), T, H, k, n_rows, static_cast<bf16_t*>(out),
                       static_cast<bf16_t*>(combined));
  else
    hipLaunchKernelGGL((combine_kernel<float>), dim3(T), dim3(kThreads), 0, s,
                       static_cast<const float*>(y), inv, topk_w, static_cast<const float*>(y_shared), S,
                       static_cast<const float*>(residual), T, H, k, n_rows, static_cast<float*>(out),
                       static_cast<float*>(combined));
  return hipGetLastError();
}

}  // namespace moe
