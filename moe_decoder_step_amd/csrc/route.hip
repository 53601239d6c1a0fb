// moe_route: pre-RMSNorm, fp32 router logits and top-k routing of each token.
//
// A block of 16 wavefronts owns TPB tokens:
//   1. norm: wavefront w normalises tokens w, w+16, ... (fp64 scale, one
//      rounding to the storage type) into LDS and to xn;
//   2. logits: the hidden dimension is split in sixteen slices, one per
//      wavefront, and each slice in two halves; lane l accumulates experts
//      l % 32 and l % 32 + 32 (E <= 64) over half l / 32 of its wavefront's
//      slice for all TPB tokens in fp32, so every normed value read from LDS
//      (a broadcast) feeds two experts' FMAs; the router weights were loaded
//      into registers at kernel entry (they do not depend on the norm); the
//      two halves of an expert's slice are then added, half 0 + half 1;
//   3. top-k: wavefront w sums the sixteen slices in order (a fixed order that
//      does not depend on the batch), adds the bias and runs k rounds of a
//      DPP wavefront max followed by a ballot: the lowest lane holding the
//      maximum wins, which is the lower-id rule for equal logits; then the
//      softmax weights.
// Decode batches (up to 256 tokens) use one token per block: the block's
// work is a latency chain and the logits loop is VALU-bound, so 128 blocks
// of one token beat 64 of two (measured 10 us per 12-layer step at 128
// tokens); larger batches use 8, and prefill-sized ones 32 to
// amortise the router reads (then the normed rows and the slice partials
// share one LDS region, the rows being dead once the partials exist, and the
// router slice is read in the loop rather than held in registers).  The
// summation order of a logit is the same for every block size.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "validate.hpp"

namespace moe {
namespace {

constexpr int kWaves = 16;     // wavefronts per block (hidden split in 16 slices)
constexpr int kThreads = kWaves * 64;

// router-weight float4 per lane loaded at kernel entry (two per step of 4
// hidden elements: the lane's two experts); 16 tokens per block hold fewer,
// their accumulators taking the registers
template <int TPB> constexpr int pre_count() { return TPB <= 8 ? 20 : TPB <= 16 ? 8 : 0; }
// the slice partials reuse the normed rows' LDS, which then hold fp32 (exact
// copies of the stored values, converted once instead of at every use)
template <int TPB> constexpr bool lds_union() { return TPB > 16; }
// normed rows in LDS as fp32 where they fit: the logits loop then reads them
// with no unpacking (at decode sizes the bf16 unpacking was half of that
// loop's VALU work); bf16 rows at 8 and 16 tokens keep the LDS small
template <int TPB> constexpr bool lds_f32() { return lds_union<TPB>() || TPB <= 2; }   // 1 token per block at decode sizes
template <typename St, int TPB> using lds_row_t = typename std::conditional<lds_f32<TPB>(), float, St>::type;

__device__ __forceinline__ void load8(const bf16_t* p, float* f) { unpack8(ldg16(p), f); }
__device__ __forceinline__ void load8(const float* p, float* f) {
  float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}
__device__ __forceinline__ void store8(bf16_t* p, const bf16_t* v) {
  uint4 o;
  o.x = pack2(v[0], v[1]); o.y = pack2(v[2], v[3]); o.z = pack2(v[4], v[5]); o.w = pack2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = o;
}
__device__ __forceinline__ void store8(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}
__device__ __forceinline__ void store8(float* p, const bf16_t* v) {
  float f[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = __uint_as_float((uint32_t)v[j] << 16);
  store8(p, f);
}
__device__ __forceinline__ bf16_t to_store(float v, bf16_t*) { return f32_to_bf16(v); }
__device__ __forceinline__ float to_store(float v, float*) { return v; }

// four consecutive normed values of a token from LDS
__device__ __forceinline__ float4 lds4(const bf16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}
__device__ __forceinline__ float4 lds4(const float* p) { return *reinterpret_cast<const float4*>(p); }

template <typename St, int TPB, bool PACKED, bool COMBINE>
__global__ __launch_bounds__(kThreads) void route_kernel(
    const St* h, St* hout, CombineArgs ca, const float* __restrict__ gain, float eps,
    const float* __restrict__ wr, const float* __restrict__ bias, int T, int H, int E, int k,
    int flags, St* __restrict__ xn, int32_t* __restrict__ ids, float* __restrict__ wts,
    float* __restrict__ logits) {
  constexpr int kPre = pre_count<TPB>();
  using Xs = lds_row_t<St, TPB>;
  extern __shared__ __align__(16) char smem[];
  Xs* xs = reinterpret_cast<Xs*>(smem);
  float* part = reinterpret_cast<float*>(                        // [kWaves][TPB][64]
      smem + (lds_union<TPB>() ? 0 : ((TPB * H * (int)sizeof(Xs) + 15) & ~15)));

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * TPB;
  const int e = lane;

  // (fused) the token's expert row numbers and weights go out before the
  // router weights: loads retire in issue order, so behind the router loads
  // their wait would include the router loads' latency
  // (so are the norm gain's, staged through LDS before the first barrier)
  constexpr bool kEarly = TPB <= 8;
  int crow_g = 0;
  float cwt_g = 0.f, gv0 = 0.f, gv1 = 0.f;
  const bool use_gain = COMBINE && kEarly && (flags & 1) && gain;
  if constexpr (COMBINE) {
    static_assert(TPB * kMaxExperts <= kThreads, "one (token, slot) per thread");
    static_assert(kMaxHidden <= 2 * kThreads, "two gain values per thread");
    if ((int)threadIdx.x < TPB * ca.k) {
      const int t = min(t0 + (int)threadIdx.x / ca.k, T - 1), j = (int)threadIdx.x % ca.k;
      crow_g = ca.inv[(size_t)t * ca.k + j];
      cwt_g = ca.w[(size_t)t * ca.k + j];
    }
    if (use_gain) {
      if ((int)threadIdx.x < H) gv0 = gain[threadIdx.x];
      if ((int)threadIdx.x + kThreads < H) gv1 = gain[threadIdx.x + kThreads];
    }
    asm volatile("" ::: "memory");
  }

  // this wavefront's slice of the hidden dim; its router weights go out next
  // (they depend on nothing) and land while the combine and the norm run
  const int hq = ((H / kWaves + 3) / 4) * 4;
  const int h_lo = min(H, wave * hq), h_hi = min(H, h_lo + hq);
  // lane l: experts ea = l % 32 and ea + 32 over half hb = l / 32 of the
  // slice, [my_lo, my_hi) (the halves split at a multiple of 4)
  const int hb = lane >> 5, ea = lane & 31;
  const int h_mid = min(h_hi, h_lo + ((((h_hi - h_lo) >> 1) + 3) & ~3));
  const int my_lo = hb ? h_mid : h_lo, my_hi = hb ? h_hi : h_mid;
  // router weights of hidden elements hh..hh+3 for expert ex: packed, a
  // wavefront load is 2 x 512 consecutive bytes; row-major, it touches 32 rows
  auto wload = [&](int ex, int hh) __attribute__((always_inline)) -> float4 {
    if (PACKED) return *reinterpret_cast<const float4*>(wr + ((size_t)(hh >> 2) * kWave + ex) * 4);
    return *reinterpret_cast<const float4*>(wr + (size_t)min(ex, E - 1) * H + hh);
  };
  // float4 slot u of the prefetch: step u / 2, expert ea (+ 32 if u is odd)
  auto wpre_load = [&](int u) __attribute__((always_inline)) -> float4 {
    return wload(ea + 32 * (u & 1), min(my_lo + 4 * (u >> 1), H - 4));
  };
  // the fused form holds only the first kPreA of them in registers during
  // the combine (the combine's row loads need registers too), up to kPreB
  // go out as soon as the combine's rows are summed and the rest after the
  // norm (issuing all of them after the sums spilled registers)
  constexpr int kPreA = COMBINE ? (kPre < 8 ? kPre : 8) : kPre;
  constexpr int kPreB = COMBINE ? (kPre < 16 ? kPre : 16) : kPre;
  float4 wpre[kPre > 0 ? kPre : 1];
#pragma unroll
  for (int u = 0; u < kPreA; ++u) wpre[u] = wpre_load(u);
  // larger blocks stream the slice through a ring of kRing steps (2 float4
  // each), the first ones issued here so that they land while the norm runs
  // (a single load in flight made every 128 FMAs wait out an L2 round trip)
  constexpr int kRing = kPre > 0 ? 1 : 2;
  float4 wring[kRing][2];
  if constexpr (kPre == 0) {
#pragma unroll
    for (int d = 0; d < kRing; ++d)
#pragma unroll
      for (int x = 0; x < 2; ++x) wring[d][x] = wload(ea + 32 * x, min(my_lo + 4 * d, H - 4));
  }
  // up to 8 tokens per block the expert's bias is read here, not at the
  // top-k, and the fused norm's gain is staged through LDS (at 16 tokens the
  // extra live registers spilled)
  const float bias_e = kEarly && bias && e < E ? bias[e] : 0.f;

  // ---- 0. (fused) the previous layer's combine: h' = h + sum_j w_j y[inv] + sum_s ys,
  //         the same fixed-order fp32 sums as moe_combine, into h and the LDS rows ----
  if constexpr (COMBINE) {
    __shared__ int crow[TPB][kMaxExperts];
    __shared__ float cwt[TPB][kMaxExperts];
    __shared__ double s_scale[TPB];
    // the norm gain staged once into LDS (H <= 2 x kThreads), its loads
    // issued at entry
    __shared__ float s_gain[kEarly ? kMaxHidden : 1];
    double* ssp = reinterpret_cast<double*>(part);  // [TPB][H/8] segment sums (part is free until the logits)
    const St* y = static_cast<const St*>(ca.y);
    const St* ys = static_cast<const St*>(ca.ys);
    if ((int)threadIdx.x < TPB * ca.k) {
      const int i = (int)threadIdx.x / ca.k, j = (int)threadIdx.x % ca.k;
      crow[i][j] = clamp_report(crow_g, 0, ca.n_rows - 1, ca.err, kDataErrInv);
      cwt[i][j] = cwt_g;
    }
    if (use_gain) {
      if ((int)threadIdx.x < H) s_gain[threadIdx.x] = gv0;
      if ((int)threadIdx.x + kThreads < H) s_gain[threadIdx.x + kThreads] = gv1;
    }
    lds_barrier();
    const int nseg = H / 8;
    for (int idx = threadIdx.x; idx < TPB * nseg; idx += kThreads) {
      const int i = idx / nseg, c = (idx % nseg) * 8, t = t0 + i;
      if (t >= T) continue;
      float acc[8], f[8];
      const typename Row8<St>::raw rres = Row8<St>::load(h + (size_t)t * H + c);
      combine8(y, crow[i], cwt[i], ca.k, ys, ca.S, T, t, H, c, acc);
      Row8<St>::unpack(rres, f);
      St o[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) o[q] = to_store(f[q] + acc[q], (St*)nullptr);
      store8(hout + (size_t)t * H + c, o);
      store8(xs + i * H + c, o);
      float g[8];
      load8(o, g);
      ssp[idx] = seg_sumsq(g);   // this 8-element segment's sum of squares
    }
#pragma unroll
    for (int u = kPreA; u < kPreB; ++u) wpre[u] = wpre_load(u);
    lds_barrier();
    // scale per token from its segment sums, in the order the unfused norm uses
    for (int i = wave; i < TPB; i += kWaves) {
      if (t0 + i >= T) break;
      double ss = 0.0;
      for (int sg = lane; sg < nseg; sg += kWave) ss += ssp[i * nseg + sg];
      ss = wave_sum_f64(ss);
      if (lane == 0) s_scale[i] = (flags & 1) ? 1.0 / sqrt(ss / (double)H + (double)eps) : 1.0;
    }
    lds_barrier();
    for (int idx = threadIdx.x; idx < TPB * nseg; idx += kThreads) {
      const int i = idx / nseg, c = (idx % nseg) * 8, t = t0 + i;
      if (t >= T) continue;
      float f[8];
      St o[8];
      load8(xs + i * H + c, f);
      // the gain from LDS through an LDS pointer: a pointer that may point to
      // either LDS or global memory compiles to flat loads, and each of
      // those waits for every global load in flight (the router weights)
      if (use_gain) norm8(f, s_scale[i], s_gain, c, o);
      else norm8(f, s_scale[i], (flags & 1) ? gain : nullptr, c, o);
      store8(xn + (size_t)t * H + c, o);
      store8(xs + i * H + c, o);
    }
  }
#pragma unroll
  for (int u = kPreB; u < kPre; ++u) wpre[u] = wpre_load(u);

  // ---- 1. RMSNorm: xn = h / sqrt(mean(h^2) + eps) * gain, scale in fp64, one rounding ----
  // (the fused form did this above with the whole block).  The sum of squares
  // is taken per 8-element segment, lane l adding segments l, l+64, ... in
  // order, then a wavefront tree: the same order in both forms.
  if constexpr (!COMBINE) {
    const bool norm = (flags & 1) != 0;
    for (int i = wave; i < TPB; i += kWaves) {
      const int t = t0 + i;
      if (t >= T) break;
      const St* hrow = h + (size_t)t * H;
      Xs* xrow = xs + i * H;
      if constexpr (kPre == 0) {
        // (blocks of 32 tokens, no router registers held) the row's segments
        // of this lane (l, l + 64, ...): all loads in flight at once, kept
        // for the normalising pass
        constexpr int kSegs = (kMaxHidden + 8 * kWave - 1) / (8 * kWave);
        typename Row8<St>::raw rr[kSegs];
#pragma unroll
        for (int q = 0; q < kSegs; ++q) rr[q] = Row8<St>::load(hrow + min(lane * 8 + q * 8 * kWave, H - 8));
        double scale = 1.0;
        if (norm) {
          double ss = 0.0;
#pragma unroll
          for (int q = 0; q < kSegs; ++q) {
            if (lane * 8 + q * 8 * kWave < H) {
              float f[8];
              Row8<St>::unpack(rr[q], f);
              ss += seg_sumsq(f);
            }
          }
          ss = wave_sum_f64(ss);
          scale = 1.0 / sqrt(ss / (double)H + (double)eps);
        }
#pragma unroll
        for (int q = 0; q < kSegs; ++q) {
          const int c = lane * 8 + q * 8 * kWave;
          if (c < H) {
            float f[8];
            St o[8];
            Row8<St>::unpack(rr[q], f);
            norm8(f, scale, norm ? gain : nullptr, c, o);
            store8(xn + (size_t)t * H + c, o);
            store8(xrow + c, o);
          }
        }
      } else {
        double scale = 1.0;
        if (norm) {
          double ss = 0.0;
          for (int c = lane * 8; c < H; c += 8 * kWave) {
            float f[8];
            load8(hrow + c, f);
            ss += seg_sumsq(f);
          }
          ss = wave_sum_f64(ss);
          scale = 1.0 / sqrt(ss / (double)H + (double)eps);
        }
        for (int c = lane * 8; c < H; c += 8 * kWave) {
          float f[8];
          St o[8];
          load8(hrow + c, f);
          norm8(f, scale, norm ? gain : nullptr, c, o);
          store8(xn + (size_t)t * H + c, o);
          store8(xrow + c, o);
        }
      }
    }
  }
  lds_barrier();

  // ---- 2. partial logits: per expert and half slice, fp32, ascending h ----
  float acc[2][TPB];   // [expert ea, ea + 32][token]
#pragma unroll
  for (int i = 0; i < TPB; ++i) acc[0][i] = acc[1][i] = 0.f;
  auto fma4 = [&](const float4& w0, const float4& w1, int hh) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TPB; ++i) {
      const float4 x = lds4(xs + i * H + hh);
      acc[0][i] = fmaf(x.x, w0.x, acc[0][i]);
      acc[0][i] = fmaf(x.y, w0.y, acc[0][i]);
      acc[0][i] = fmaf(x.z, w0.z, acc[0][i]);
      acc[0][i] = fmaf(x.w, w0.w, acc[0][i]);
      acc[1][i] = fmaf(x.x, w1.x, acc[1][i]);
      acc[1][i] = fmaf(x.y, w1.y, acc[1][i]);
      acc[1][i] = fmaf(x.z, w1.z, acc[1][i]);
      acc[1][i] = fmaf(x.w, w1.w, acc[1][i]);
    }
  };
  if constexpr (kPre > 0) {
    constexpr int kPreSteps = kPre / 2;
#pragma unroll
    for (int u = 0; u < kPreSteps; ++u)
      if (my_lo + 4 * u < my_hi) fma4(wpre[2 * u], wpre[2 * u + 1], my_lo + 4 * u);
    for (int hh = my_lo + 4 * kPreSteps; hh < my_hi; hh += 4) fma4(wload(ea, hh), wload(ea + 32, hh), hh);
  } else {
    // slot d holds the step s with s % kRing == d; the refill kRing steps
    // ahead is unconditional (past the half: a valid address, never used)
    for (int s0 = 0; my_lo + 4 * s0 < my_hi; s0 += kRing) {
#pragma unroll
      for (int d = 0; d < kRing; ++d) {
        const int hh = my_lo + 4 * (s0 + d);
        if (hh < my_hi) fma4(wring[d][0], wring[d][1], hh);
#pragma unroll
        for (int x = 0; x < 2; ++x) wring[d][x] = wload(ea + 32 * x, min(my_lo + 4 * (s0 + d + kRing), H - 4));
      }
    }
  }
  // lane l ends with expert l's slice: half 0 (lane l % 32) + half 1 (lane
  // l % 32 + 32), the other half from lane l ^ 32
  float lsl[TPB];
#pragma unroll
  for (int i = 0; i < TPB; ++i) {
    const float o0 = __shfl_xor(acc[0][i], 32, kWave), o1 = __shfl_xor(acc[1][i], 32, kWave);
    lsl[i] = hb == 0 ? acc[0][i] + o0 : o1 + acc[1][i];
  }
  if (lds_union<TPB>()) lds_barrier();  // every wavefront is done with the normed rows
#pragma unroll
  for (int i = 0; i < TPB; ++i) part[(wave * TPB + i) * kWave + e] = lsl[i];
  lds_barrier();

  // ---- 3. top-k by (logit desc, expert id asc), then softmax weights ----
  for (int i = wave; i < TPB; i += kWaves) {
    const int t = t0 + i;
    if (t >= T) break;
    const bool valid = e < E;
    float l = part[i * kWave + e];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) l += part[(w * TPB + i) * kWave + e];
    if (bias && valid) l += kEarly ? bias_e : bias[e];
    if (logits && valid) logits[(size_t)t * E + e] = l;
    // k rounds: the largest remaining logit, then the lowest lane holding it
    float cur = valid ? l : -INFINITY;
    int rank = -1;
    float lmax = 0.f;
    for (int j = 0; j < k; ++j) {
      const float m = wave_max_dpp(cur);
      const unsigned long long hit = __ballot(cur == m);
      const int win = (int)__builtin_ctzll(hit);
      if (j == 0) lmax = m;
      if (e == win) {
        rank = j;
        cur = -INFINITY;
      }
    }
    const float z = rank >= 0 ? expf(l - lmax) : 0.f;
    const float den = (flags & 2) ? wave_sum_dpp(z) : wave_sum_dpp(valid ? expf(l - lmax) : 0.f);
    if (rank >= 0) {
      ids[(size_t)t * k + rank] = e;
      wts[(size_t)t * k + rank] = z / den;
    }
  }
}

template <typename St, int TPB>
size_t lds_bytes(int H) {
  const size_t rows = (TPB * H * sizeof(lds_row_t<St, TPB>) + 15) & ~size_t(15);
  const size_t parts = (size_t)kWaves * TPB * kWave * sizeof(float);
  return lds_union<TPB>() ? (rows > parts ? rows : parts) : rows + parts;
}

template <typename St, int TPB, bool PACKED, bool COMBINE>
hipError_t launch_one(const void* h, void* hout, const CombineArgs& ca, const float* gain, float eps,
                      const float* wr, const float* bias, int T, int H, int E, int k, int flags, void* xn,
                      int32_t* ids, float* w, float* logits, hipStream_t s) {
  const int grid = (T + TPB - 1) / TPB;
  const size_t lds = lds_bytes<St, TPB>(H);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&route_kernel<St, TPB, PACKED, COMBINE>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((route_kernel<St, TPB, PACKED, COMBINE>), dim3(grid), dim3(kThreads), lds, s,
                     static_cast<const St*>(h), static_cast<St*>(hout), ca, gain, eps, wr, bias, T, H, E, k, flags,
                     static_cast<St*>(xn), ids, w, logits);
  return hipGetLastError();
}

template <typename St, int TPB>
hipError_t launch_tpb(const void* h, void* hout, const CombineArgs* ca, const float* gain, float eps,
                      const float* wr, const float* bias, int T, int H, int E, int k, int flags, void* xn,
                      int32_t* ids, float* w, float* logits, hipStream_t s) {
  const CombineArgs none{};
  if constexpr (!lds_union<TPB>()) {
    if (ca) {
      if (flags & 4)
        return launch_one<St, TPB, true, true>(h, hout, *ca, gain, eps, wr, bias, T, H, E, k, flags, xn, ids, w,
                                               logits, s);
      return launch_one<St, TPB, false, true>(h, hout, *ca, gain, eps, wr, bias, T, H, E, k, flags, xn, ids, w,
                                              logits, s);
    }
  }
  if (flags & 4)
    return launch_one<St, TPB, true, false>(h, nullptr, none, gain, eps, wr, bias, T, H, E, k, flags, xn, ids, w,
                                            logits, s);
  return launch_one<St, TPB, false, false>(h, nullptr, none, gain, eps, wr, bias, T, H, E, k, flags, xn, ids, w,
                                           logits, s);
}

template <typename St>
hipError_t launch_st(const void* h, void* hout, const CombineArgs* ca, const float* gain, float eps,
                     const float* wr, const float* bias, int T, int H, int E, int k, int flags, void* xn,
                     int32_t* ids, float* w, float* logits, hipStream_t s) {
  constexpr size_t kLds = 64 * 1024;
  if (T >= 4096 && lds_bytes<St, 32>(H) <= 160 * 1024) {
    if (ca) {  // prefill-sized batches: the combine as its own launch, then the 32-token route
      hipError_t e = launch_combine(ca->y, ca->inv, ca->w, ca->ys, ca->S, h, T, H, ca->k, ca->n_rows,
                                    sizeof(St) == 2 ? kBf16 : kF32, hout, nullptr, s);
      if (e != hipSuccess) return e;
      h = hout;
    }
    return launch_tpb<St, 32>(h, nullptr, nullptr, gain, eps, wr, bias, T, H, E, k, flags, xn, ids, w, logits, s);
  }
  if (T > 256 && lds_bytes<St, 16>(H) <= kLds)
    return launch_tpb<St, 16>(h, hout, ca, gain, eps, wr, bias, T, H, E, k, flags, xn, ids, w, logits, s);
  if (T > 256 && lds_bytes<St, 8>(H) <= kLds)
    return launch_tpb<St, 8>(h, hout, ca, gain, eps, wr, bias, T, H, E, k, flags, xn, ids, w, logits, s);
  return launch_tpb<St, 1>(h, hout, ca, gain, eps, wr, bias, T, H, E, k, flags, xn, ids, w, logits, s);
}

// RMSNorm of rows (the draft block's inputs): one wavefront per output row,
// the same segment-order fp64 sum of squares and single rounding as the
// route kernel's norm, so a row normalises to the same bits in both.
template <typename St>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const St* __restrict__ x, const int32_t* __restrict__ rows,
                                                      int x_rows, int T, int H, const float* __restrict__ gain,
                                                      float eps, St* __restrict__ out, int out_stride,
                                                      uint32_t* err) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (t >= T) return;
  const int r = rows ? clamp_report(rows[t], 0, x_rows - 1, err, kDataErrRowIndex) : t;
  const St* xr = x + (size_t)r * H;
  double ss = 0.0;
  for (int c = lane * 8; c < H; c += 8 * kWave) {
    float f[8];
    load8(xr + c, f);
    ss += seg_sumsq(f);
  }
  ss = wave_sum_f64(ss);
  const double scale = 1.0 / sqrt(ss / (double)H + (double)eps);
  for (int c = lane * 8; c < H; c += 8 * kWave) {
    float f[8];
    St o[8];
    load8(xr + c, f);
    norm8(f, scale, gain, c, o);
    store8(out + (size_t)t * out_stride + c, o);
  }
}

}  // namespace

hipError_t launch_rmsnorm(const void* x, const int32_t* rows, int x_rows, int T, int H, const float* gain, float eps,
                          int dtype, void* out, int out_stride, hipStream_t s) {
  const dim3 grid((T + 3) / 4), block(256);
  if (dtype == kBf16)
    hipLaunchKernelGGL(rmsnorm_kernel<bf16_t>, grid, block, 0, s, static_cast<const bf16_t*>(x), rows, x_rows, T, H,
                       gain, eps, static_cast<bf16_t*>(out), out_stride, data_error_word(s));
  else
    hipLaunchKernelGGL(rmsnorm_kernel<float>, grid, block, 0, s, static_cast<const float*>(x), rows, x_rows, T, H,
                       gain, eps, static_cast<float*>(out), out_stride, data_error_word(s));
  return hipGetLastError();
}

hipError_t launch_route(const void* h, const float* gain, float eps, const float* w_router,
                        const float* bias, int T, int H, int E, int k, int flags, int dtype,
                        void* xn, int32_t* ids, float* w, float* logits, hipStream_t s) {
  if (dtype == kBf16)
    return launch_st<bf16_t>(h, nullptr, nullptr, gain, eps, w_router, bias, T, H, E, k, flags, xn, ids, w, logits,
                             s);
  return launch_st<float>(h, nullptr, nullptr, gain, eps, w_router, bias, T, H, E, k, flags, xn, ids, w, logits, s);
}

hipError_t launch_combine_route(const CombineArgs& ca, void* h, const float* gain, float eps, const float* w_router,
                                const float* bias, int T, int H, int E, int k, int flags, int dtype, void* xn,
                                int32_t* ids, float* w, float* logits, hipStream_t s) {
  CombineArgs c = ca;
  c.err = data_error_word(s);
  if (dtype == kBf16)
    return launch_st<bf16_t>(h, h, &c, gain, eps, w_router, bias, T, H, E, k, flags, xn, ids, w, logits, s);
  return launch_st<float>(h, h, &c, gain, eps, w_router, bias, T, H, E, k, flags, xn, ids, w, logits, s);
}

}  // namespace moe
