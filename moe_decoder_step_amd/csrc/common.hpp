// Device helpers shared by the gfx950 kernels of the MoE verify step.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;  // CDNA wavefront width

// MFMA operand / accumulator vectors.
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

// bf16 is carried as its raw 16 bits.
typedef uint16_t bf16_t;

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.  One
// v_cvt_pk_bf16_f32 (gfx950); over random, denormal, tie and near-tie bit
// patterns it gives the same bits as the rounding done on the integer bits
// (add 0x7fff plus the lowest kept bit, keep the high half; NaN: set the
// quiet bit).
typedef float f32x2_cvt_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_cvt_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_cvt_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_cvt_t));
}
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return (bf16_t)(pack_bf16x2(f, 0.f) & 0xffffu); }

// silu(z) = z / (1 + e^-z) from the hardware exp2 and reciprocal (v_exp_f32,
// v_rcp_f32, about 1 ulp each; the product with the up projection is then
// rounded to bf16).  Every bf16 SwiGLU path uses this one function -- the
// weight-streaming kernel for decode-sized groups and the tiled GEMM for
// prefill-sized ones -- so, with the same MFMA k-order in both, a token row's
// activation does not depend on which path its batch size selects.
__device__ __forceinline__ float silu_bf16path(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.44269504088896341f));
}

// fp64 -> bf16 in a single rounding step (nearest, ties to even): the 45 low
// mantissa bits of the double are rounded away by an integer add, then the
// (now 8-significant-bit) value converts to fp32 exactly.  Normal range only.
__device__ __forceinline__ bf16_t f64_to_bf16(double d) {
  uint64_t u = (uint64_t)__double_as_longlong(d);
  u += 0x00000FFFFFFFFFFFull + ((u >> 45) & 1ull);
  u &= ~((1ull << 45) - 1ull);
  float f = (float)__longlong_as_double((long long)u);
  return (bf16_t)(__float_as_uint(f) >> 16);
}

// RMSNorm pieces shared by every kernel that normalises rows (route, the
// plain row norm, the fused combine + norm), so a row normalises to the same
// bits in all of them: the sum of squares in fp64 per 8-element segment, in
// order; the scale applied in fp64 with one rounding to the storage type.
__device__ __forceinline__ double seg_sumsq(const float* f) {
  double s = 0.0;
#pragma unroll
  for (int q = 0; q < 8; ++q) s += (double)f[q] * (double)f[q];
  return s;
}
__device__ __forceinline__ bf16_t round_store(double v, bf16_t*) { return f64_to_bf16(v); }
__device__ __forceinline__ float round_store(double v, float*) { return (float)v; }
// xn = f * scale (* gain[c+q]) in fp64, one rounding to the storage type
template <typename St>
__device__ __forceinline__ void norm8(const float* f, double scale, const float* gain, int c, St* o) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    double v = (double)f[q] * scale;
    if (gain) v *= (double)gain[c + q];
    o[q] = round_store(v, (St*)nullptr);
  }
}

// Unpack 8 bf16 (one 16-byte vector) into fp32.
__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
  f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
  f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
  f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xffff0000u);
  f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xffff0000u);
}

__device__ __forceinline__ uint32_t pack2(bf16_t lo, bf16_t hi) {
  return (uint32_t)lo | ((uint32_t)hi << 16);
}

// Wave-wide reductions (butterfly over all 64 lanes; every lane gets the result).
__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    unsigned long long w = __shfl_xor(v, o, kWave);
    v = w > v ? w : v;
  }
  return v;
}

// Wavefront-wide max / sum with DPP lane moves (no LDS round trip): quad
// swaps, half-row and row mirrors, then row broadcasts carry the result to
// lane 63, which every lane reads back.  The sum adds in a fixed tree order.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}

__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));        // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f32<0x4E>(v));        // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f32<0x141>(v));       // row_half_mirror
  v = fmaxf(v, dpp_f32<0x140>(v));       // row_mirror
  v = fmaxf(v, dpp_f32<0x142, 0xA>(v));  // row_bcast:15
  v = fmaxf(v, dpp_f32<0x143, 0xC>(v));  // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  v += dpp_f32<0x142, 0xA>(v);
  v += dpp_f32<0x143, 0xC>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// The same tree in fp64 (both halves of each double take the same lane
// move): the sum of squares of every RMSNorm, so all of them add in one order.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ double dpp_f64(double v) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  const int lo = (int)(uint32_t)u, hi = (int)(uint32_t)(u >> 32);
  const uint32_t l2 = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, ROW_MASK, 0xF, false);
  const uint32_t h2 = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROW_MASK, 0xF, false);
  return __longlong_as_double((long long)(((unsigned long long)h2 << 32) | l2));
}

// wavefront sum in fp64, the total in every lane
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<0xB1>(v);
  v += dpp_f64<0x4E>(v);
  v += dpp_f64<0x141>(v);
  v += dpp_f64<0x140>(v);
  v += dpp_f64<0x142, 0xA>(v);
  v += dpp_f64<0x143, 0xC>(v);
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 63);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// Order-preserving map of a float onto uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Device-side data errors (moestep.h MOE_DATA_ERR_*).  An index argument is
// always clamped before it addresses memory; when it was out of range the
// kernel also ORs the error's kind into the per-GPU word `err` (relaxed,
// device scope).  In-range data issues no memory operation here.
constexpr uint32_t kDataErrExpertId = 1u;   // MOE_DATA_ERR_EXPERT_ID
constexpr uint32_t kDataErrRowIndex = 2u;   // MOE_DATA_ERR_ROW_INDEX
constexpr uint32_t kDataErrOffsets = 4u;    // MOE_DATA_ERR_OFFSETS
constexpr uint32_t kDataErrInv = 8u;        // MOE_DATA_ERR_INV
constexpr uint32_t kDataErrLength = 16u;    // MOE_DATA_ERR_LENGTH
constexpr uint32_t kDataErrSequence = 32u;  // MOE_DATA_ERR_SEQUENCE
__device__ __forceinline__ void report_error(uint32_t* err, bool bad, uint32_t bit) {
  if (__builtin_expect(bad, false) && err) __hip_atomic_fetch_or(err, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// clampi that reports an argument outside [lo, hi]
__device__ __forceinline__ int clamp_report(int v, int lo, int hi, uint32_t* err, uint32_t bit) {
  report_error(err, v < lo || v > hi, bit);
  return clampi(v, lo, hi);
}

// 16x16x32 bf16 MFMA, fp32 accumulate.  Lane l supplies A[l%16][8*(l/16)+0..7]
// and B[8*(l/16)+0..7][l%16]; it receives D[4*(l/16)+v][l%16], v = 0..3.
__device__ __forceinline__ f32x4_t mfma16x16x32(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Streaming (read-once) 16-byte load: marked non-temporal so weight streams do
// not push reusable activations out of the caches.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldg16_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Block barrier for data exchanged through LDS only.  __syncthreads() carries
// a workgroup-scope fence over all memory, which waits for every outstanding
// global load; restricting the fence to LDS keeps a weight stream in flight
// across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---- the weighted combine of one token's expert rows, 8 hidden elements ----
// acc[q] = sum_j w[j] * y[rows[j]][c+q] (j ascending, fmaf) + sum_s ys[s*T+t][c+q]
// (s ascending), in fp32.  Every row load of the first batch of 8 routed rows
// and of the first 4 shared rows (1 for fp32 rows) is issued before any of
// the sums, so a bf16 token's rows cost one memory round trip (k <= 8,
// S <= 4), not one per row or per kind.  The expert rows are read once: non-temporal loads.
template <typename St> struct Row8;
template <> struct Row8<bf16_t> {
  typedef uint4 raw;
  static __device__ __forceinline__ raw load(const bf16_t* p) { return *reinterpret_cast<const uint4*>(p); }
  static __device__ __forceinline__ void unpack(const raw& r, float* f) { unpack8(r, f); }
};
template <> struct Row8<float> {
  struct raw { float4 a, b; };
  static __device__ __forceinline__ raw load(const float* p) {
    return raw{*reinterpret_cast<const float4*>(p), *reinterpret_cast<const float4*>(p + 4)};
  }
  static __device__ __forceinline__ void unpack(const raw& r, float* f) {
    f[0] = r.a.x; f[1] = r.a.y; f[2] = r.a.z; f[3] = r.a.w; f[4] = r.b.x; f[5] = r.b.y; f[6] = r.b.z; f[7] = r.b.w;
  }
};

template <typename St> struct RowNT;
template <> struct RowNT<bf16_t> {
  typedef uint4 raw;
  static __device__ __forceinline__ raw load(const bf16_t* p) { return ldg16_stream(p); }
};
template <> struct RowNT<float> {
  typedef Row8<float>::raw raw;
  static __device__ __forceinline__ raw load(const float* p) { return Row8<float>::load(p); }
};

template <typename St>
__device__ __forceinline__ void combine8(const St* y, const int* rows, const float* wk, int k, const St* ys, int S,
                                         int T, int t, int H, int c, float* acc) {
  // shared rows loaded with the first routed batch (1 for fp32 rows, which
  // take twice the registers)
  constexpr int kEarly = sizeof(St) == 2 ? 4 : 1;
  typename Row8<St>::raw rs[kEarly];
  if (S > 0) {
#pragma unroll
    for (int u = 0; u < kEarly; ++u) rs[u] = RowNT<St>::load(ys + ((size_t)min(u, S - 1) * T + t) * H + c);
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.f;
  for (int j0 = 0; j0 < k; j0 += 8) {
    typename Row8<St>::raw r[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) r[u] = RowNT<St>::load(y + (size_t)rows[min(j0 + u, k - 1)] * H + c);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (j0 + u < k) {
        float f[8];
        Row8<St>::unpack(r[u], f);
        const float wj = wk[j0 + u];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = fmaf(wj, f[q], acc[q]);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kEarly; ++u) {
    if (u < S) {
      float f[8];
      Row8<St>::unpack(rs[u], f);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] += f[q];
    }
  }
  for (int s0 = kEarly; s0 < S; s0 += 4) {
    typename Row8<St>::raw r[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) r[u] = RowNT<St>::load(ys + ((size_t)min(s0 + u, S - 1) * T + t) * H + c);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (s0 + u < S) {
        float f[8];
        Row8<St>::unpack(r[u], f);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] += f[q];
      }
    }
  }
}

}  // namespace moe
