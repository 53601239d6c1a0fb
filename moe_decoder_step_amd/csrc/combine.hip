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
  o.x = pack_bf16x2(f[0], f[1]);
  o.y = pack_bf16x2(f[2], f[3]);
  o.z = pack_bf16x2(f[4], f[5]);
  o.w = pack_bf16x2(f[6], f[7]);
  *reinterpret_cast<uint4*>(p) = o;
}
__device__ __forceinline__ void store8(float* p, const float* f) {
  *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(f[4], f[5], f[6], f[7]);
}

__device__ __forceinline__ bf16_t to_store8(float v, bf16_t*) { return f32_to_bf16(v); }
__device__ __forceinline__ float to_store8(float v, float*) { return v; }
__device__ __forceinline__ float from_store8(bf16_t v) { return __uint_as_float((uint32_t)v << 16); }
__device__ __forceinline__ float from_store8(float v) { return v; }
__device__ __forceinline__ void store8s(bf16_t* p, const bf16_t* v) {
  uint4 o;
  o.x = pack2(v[0], v[1]); o.y = pack2(v[2], v[3]); o.z = pack2(v[4], v[5]); o.w = pack2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = o;
}
__device__ __forceinline__ void store8s(float* p, const float* v) { store8(p, v); }

template <typename St>
__global__ __launch_bounds__(kThreads) void combine_kernel(
    const St* __restrict__ y, const int32_t* __restrict__ inv, const float* __restrict__ w,
    const St* __restrict__ ys, int S, const St* res, int T, int H, int k, int n_rows, St* out,
    St* __restrict__ combined, uint32_t* err) {
  const int t = blockIdx.x;
  __shared__ int rows[kMaxExperts];
  __shared__ float wk[kMaxExperts];
  if (threadIdx.x < k) {
    rows[threadIdx.x] = clamp_report(inv[(size_t)t * k + threadIdx.x], 0, n_rows - 1, err, kDataErrInv);
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

// The combine followed by the RMSNorm of the combined row (xn), one block
// per token: the rounded output row stays in registers, each thread's
// 8-element segment contributes its fp64 sum of squares to LDS, and
// wavefront 0 adds them in the order the plain row norm does (lane l:
// segments l, l+64, ..., then the wavefront butterfly), so xn has the same
// bits as moe_rmsnorm of the output.  H <= 2048: one segment per thread.
template <typename St>
__global__ __launch_bounds__(kThreads) void combine_norm_kernel(
    const St* __restrict__ y, const int32_t* __restrict__ inv, const float* __restrict__ w,
    const St* __restrict__ ys, int S, const St* res, int T, int H, int k, int n_rows, const float* __restrict__ gain,
    float eps, St* out, St* __restrict__ xn, uint32_t* err) {
  const int t = blockIdx.x;
  __shared__ int rows[kMaxExperts];
  __shared__ float wk[kMaxExperts];
  __shared__ double ssp[kThreads];
  __shared__ double s_scale;
  if (threadIdx.x < k) {
    rows[threadIdx.x] = clamp_report(inv[(size_t)t * k + threadIdx.x], 0, n_rows - 1, err, kDataErrInv);
    wk[threadIdx.x] = w[(size_t)t * k + threadIdx.x];
  }
  __syncthreads();
  const int c = threadIdx.x * 8;
  const bool mine = c < H;
  float f[8];
  if (mine) {
    float acc[8];
    typename Row8<St>::raw rres{};
    if (res) rres = Row8<St>::load(res + (size_t)t * H + c);
    combine8(y, rows, wk, k, ys, S, T, t, H, c, acc);
    if (res) {
      Row8<St>::unpack(rres, f);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] += acc[i];
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = acc[i];
    }
    store8(out + (size_t)t * H + c, f);
    // the stored values, as the norm reads them
    St o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = to_store8(f[i], (St*)nullptr);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = from_store8(o[i]);
    ssp[threadIdx.x] = seg_sumsq(f);
  }
  __syncthreads();
  if (threadIdx.x < kWave) {
    double ss = 0.0;
    for (int sg = threadIdx.x; sg < H / 8; sg += kWave) ss += ssp[sg];
    ss = wave_sum_f64(ss);
    if (threadIdx.x == 0) s_scale = 1.0 / sqrt(ss / (double)H + (double)eps);
  }
  __syncthreads();
  if (mine) {
    St o[8];
    norm8(f, s_scale, gain, c, o);
    store8s(xn + (size_t)t * H + c, o);
  }
}

}  // namespace

hipError_t launch_combine_norm(const void* y, const int32_t* inv, const float* topk_w, const void* y_shared, int S,
                               const void* residual, int T, int H, int k, int n_rows, const float* gain, float eps,
                               int dtype, void* out, void* xn, hipStream_t s) {
  if (dtype == kBf16)
    hipLaunchKernelGGL((combine_norm_kernel<bf16_t>), dim3(T), dim3(kThreads), 0, s,
                       static_cast<const bf16_t*>(y), inv, topk_w, static_cast<const bf16_t*>(y_shared), S,
                       static_cast<const bf16_t*>(residual), T, H, k, n_rows, gain, eps, static_cast<bf16_t*>(out),
                       static_cast<bf16_t*>(xn), data_error_word(s));
  else
    hipLaunchKernelGGL((combine_norm_kernel<float>), dim3(T), dim3(kThreads), 0, s,
                       static_cast<const float*>(y), inv, topk_w, static_cast<const float*>(y_shared), S,
                       static_cast<const float*>(residual), T, H, k, n_rows, gain, eps, static_cast<float*>(out),
                       static_cast<float*>(xn), data_error_word(s));
  return hipGetLastError();
}

hipError_t launch_combine(const void* y, const int32_t* inv, const float* topk_w,
                          const void* y_shared, int S, const void* residual, int T, int H, int k,
                          int n_rows, int dtype, void* out, void* combined, hipStream_t s) {
  if (dtype == kBf16)
    hipLaunchKernelGGL((combine_kernel<bf16_t>), dim3(T), dim3(kThreads), 0, s,
                       static_cast<const bf16_t*>(y), inv, topk_w, static_cast<const bf16_t*>(y_shared), S,
                       static_cast<const bf16_t*>(residual), T, H, k, n_rows, static_cast<bf16_t*>(out),
                       static_cast<bf16_t*>(combined), data_error_word(s));
  else
    hipLaunchKernelGGL((combine_kernel<float>), dim3(T), dim3(kThreads), 0, s,
                       static_cast<const float*>(y), inv, topk_w, static_cast<const float*>(y_shared), S,
                       static_cast<const float*>(residual), T, H, k, n_rows, static_cast<float*>(out),
                       static_cast<float*>(combined), data_error_word(s));
  return hipGetLastError();
}

}  // namespace moe
