// moe_route: pre-RMSNorm, fp32 router logits and top-k routing of each token.
//
// One block of 4 wavefronts handles 4*TPW tokens; each wavefront owns TPW
// tokens from the norm to the top-k, so the only block-wide traffic is the
// router weight, staged through LDS 64 hidden elements at a time and shared
// by all of the block's tokens.  In the logit and top-k phases lane e is
// expert e (E <= 64 routed experts), so the top-k is k rounds of a
// wavefront-wide max over (logit, lower id) keys and needs no sort.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "validate.hpp"

namespace moe {
namespace {

constexpr int kWaves = 4;
constexpr int kChunk = 64;        // hidden elements of the router weight per LDS pass
constexpr int kWtStride = 65;     // padded LDS row (conflict-free transpose)

template <typename St> struct Vec8;
template <> struct Vec8<bf16_t> {
  static __device__ __forceinline__ void load(const bf16_t* p, float* f) { unpack8(ldg16(p), f); }
};
template <> struct Vec8<float> {
  static __device__ __forceinline__ void load(const float* p, float* f) {
    float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
};

__device__ __forceinline__ void store8(bf16_t* p, const bf16_t* v) {
  uint4 o;
  o.x = pack2(v[0], v[1]); o.y = pack2(v[2], v[3]); o.z = pack2(v[4], v[5]); o.w = pack2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = o;
}
__device__ __forceinline__ void store8(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

__device__ __forceinline__ bf16_t round_store(double v, bf16_t*) { return f64_to_bf16(v); }
__device__ __forceinline__ float round_store(double v, float*) { return (float)v; }

__device__ __forceinline__ float lds_val(const bf16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ float lds_val(const float* p) { return *p; }

template <typename St, int TPW>
__global__ __launch_bounds__(256) void route_kernel(
    const St* __restrict__ h, const float* __restrict__ gain, float eps,
    const float* __restrict__ wr, const float* __restrict__ bias, int T, int H, int E, int k,
    int flags, St* __restrict__ xn, int32_t* __restrict__ ids, float* __restrict__ wts,
    float* __restrict__ logits) {
  constexpr int TPB = TPW * kWaves;
  extern __shared__ __align__(16) char smem[];
  St* xs = reinterpret_cast<St*>(smem);
  float* wt = reinterpret_cast<float*>(smem + ((TPB * H * (int)sizeof(St) + 15) & ~15));

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tbase = blockIdx.x * TPB + wave * TPW;

  // ---- RMSNorm: xn = h / sqrt(mean(h^2) + eps) * gain, scale in fp64, one rounding ----
  for (int i = 0; i < TPW; ++i) {
    const int t = tbase + i;
    if (t >= T) break;
    const St* hrow = h + (size_t)t * H;
    St* xrow = xs + (wave * TPW + i) * H;
    double scale = 1.0;
    const bool norm = (flags & 1) != 0;
    if (norm) {
      double ss = 0.0;
      for (int c = lane * 8; c < H; c += 8 * kWave) {
        float f[8];
        Vec8<St>::load(hrow + c, f);
#pragma unroll
        for (int j = 0; j < 8; ++j) ss += (double)f[j] * (double)f[j];
      }
      ss = __shfl(wave_sum_f64(ss), 0, kWave);
      scale = 1.0 / sqrt(ss / (double)H + (double)eps);
    }
    for (int c = lane * 8; c < H; c += 8 * kWave) {
      float f[8];
      St o[8];
      Vec8<St>::load(hrow + c, f);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        double v = (double)f[j];
        if (norm) {
          v *= scale;
          if (gain) v *= (double)gain[c + j];
        }
        o[j] = round_store(v, (St*)nullptr);
      }
      store8(xn + (size_t)t * H + c, o);
      store8(xrow + c, o);
    }
  }

  // ---- router logits: lane e accumulates l[t,e] over h in order, fp32 ----
  float acc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) acc[i] = 0.f;
  const int e = lane;
  for (int h0 = 0; h0 < H; h0 += kChunk) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < kChunk * kWave; idx += 256) {
      const int ee = idx / kChunk, hh = idx % kChunk;
      float v = 0.f;
      if (ee < E && h0 + hh < H) v = wr[(size_t)ee * H + h0 + hh];
      wt[hh * kWtStride + ee] = v;
    }
    __syncthreads();
    const int hn = min(kChunk, H - h0);
    for (int hh = 0; hh < hn; ++hh) {
      const float wv = wt[hh * kWtStride + e];
#pragma unroll
      for (int i = 0; i < TPW; ++i) acc[i] = fmaf(lds_val(xs + (wave * TPW + i) * H + h0 + hh), wv, acc[i]);
    }
  }

  // ---- top-k by (logit desc, expert id asc), then softmax weights ----
  for (int i = 0; i < TPW; ++i) {
    const int t = tbase + i;
    if (t >= T) break;
    const bool valid = e < E;
    const float l = valid ? acc[i] + (bias ? bias[e] : 0.f) : 0.f;
    if (logits && valid) logits[(size_t)t * E + e] = l;
    const unsigned long long key = valid ? (((unsigned long long)float_key(l) << 32) | (uint32_t)(255 - e)) : 0ull;
    int rank = -1;
    float lmax = 0.f;
    for (int j = 0; j < k; ++j) {
      const unsigned long long best = wave_max_u64(rank < 0 ? key : 0ull);
      if (j == 0) lmax = key_float((uint32_t)(best >> 32));
      if (e == 255 - (int)(best & 0xffu)) rank = j;
    }
    const float z = rank >= 0 ? expf(l - lmax) : 0.f;
    float den;
    if (flags & 2) den = wave_sum_f32(z);
    else den = wave_sum_f32(valid ? expf(l - lmax) : 0.f);
    den = __shfl(den, 0, kWave);
    if (rank >= 0) {
      ids[(size_t)t * k + rank] = e;
      wts[(size_t)t * k + rank] = z / den;
    }
  }
}

template <typename St, int TPW>
hipError_t launch_tpw(const void* h, const float* gain, float eps, const float* wr, const float* bias,
                      int T, int H, int E, int k, int flags, void* xn, int32_t* ids, float* w,
                      float* logits, hipStream_t s) {
  constexpr int TPB = TPW * kWaves;
  const size_t lds = ((TPB * H * sizeof(St) + 15) & ~size_t(15)) + kChunk * kWtStride * sizeof(float);
  const int grid = (T + TPB - 1) / TPB;
  hipLaunchKernelGGL((route_kernel<St, TPW>), dim3(grid), dim3(256), lds, s,
                     static_cast<const St*>(h), gain, eps, wr, bias, T, H, E, k, flags,
                     static_cast<St*>(xn), ids, w, logits);
  return hipGetLastError();
}

template <typename St>
hipError_t launch_st(const void* h, const float* gain, float eps, const float* wr, const float* bias,
                     int T, int H, int E, int k, int flags, void* xn, int32_t* ids, float* w,
                     float* logits, hipStream_t s) {
  // keep the block's normed rows within 40 KB of LDS
  const size_t row = (size_t)H * sizeof(St);
  if (16 * row <= 40 * 1024)
    return launch_tpw<St, 4>(h, gain, eps, wr, bias, T, H, E, k, flags, xn, ids, w, logits, s);
  if (8 * row <= 40 * 1024)
    return launch_tpw<St, 2>(h, gain, eps, wr, bias, T, H, E, k, flags, xn, ids, w, logits, s);
  return launch_tpw<St, 1>(h, gain, eps, wr, bias, T, H, E, k, flags, xn, ids, w, logits, s);
}

}  // namespace

hipError_t launch_route(const void* h, const float* gain, float eps, const float* w_router,
                        const float* bias, int T, int H, int E, int k, int flags, int dtype,
                        void* xn, int32_t* ids, float* w, float* logits, hipStream_t s) {
  if (dtype == kBf16)
    return launch_st<bf16_t>(h, gain, eps, w_router, bias, T, H, E, k, flags, xn, ids, w, logits, s);
  return launch_st<float>(h, gain, eps, w_router, bias, T, H, E, k, flags, xn, ids, w, logits, s);
}

}  // namespace moe
