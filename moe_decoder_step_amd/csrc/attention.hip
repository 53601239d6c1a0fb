// Causal attention of the verify positions over a per-sequence KV cache.
//
// The verify pass of sequence b holds P positions at L_b .. L_b+P-1 (its last
// committed token, then the drafts).  Each layer:
//   rope_cache_kernel  q, k <- rotary(q, k) at their positions (angle and
//                      rotation in fp64, one rounding to bf16); k and v go
//                      into the cache at [b][head][L_b + i][0 / 1][d];
//   attn_split_kernel  flash-decoding: block (b, head, split) scores its span
//                      of cached keys for the P queries (q k^T on MFMA), with
//                      an online fp32 softmax, and writes (max, sum,
//                      unnormalised output); keys and values pass through LDS
//                      in 64-key tiles;
//   attn_merge_kernel  merges the splits of each (b, head, query), one
//                      rounding to bf16.
// Query i of sequence b sees keys 0 .. L_b + i: entries past that (drafts a
// previous pass wrote and the verifier rejected) are never read, so rolling
// back is only a matter of not advancing the length (spec_commit).
//
// The cache interleaves k and v per position (512 bytes: k then v), so a
// tile of keys is one contiguous stream rather than two (measured in the
// verify step at 2,241 positions x 32 sequences x 10 heads: 79.9 against
// 82.9 us per layer with separate k and v caches).
#include "common.hpp"
#include "kernels.hpp"
#include "validate.hpp"

namespace moe {
namespace {

constexpr int kD = kAttnHeadDim;      // 128
constexpr int kTile = 64;             // keys per LDS tile
constexpr int kRowPad = kD + 8;       // bf16 per LDS row (conflict-free column reads)

__global__ __launch_bounds__(256) void rope_cache_kernel(const bf16_t* __restrict__ qkv,
                                                         const int32_t* __restrict__ lengths, int B, int P,
                                                         int n_heads, int max_len, double log_base,
                                                         bf16_t* __restrict__ q, bf16_t* __restrict__ kv,
                                                         uint32_t* err) {
  // one thread per (token, head, rotation pair j < 64)
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int half = kD / 2;
  if (idx >= (long long)B * P * n_heads * half) return;
  const int j = (int)(idx % half);
  const int hd = (int)((idx / half) % n_heads);
  const int t = (int)(idx / ((long long)half * n_heads));
  const int b = t / P, i = t % P;
  // (one thread per sequence reports a length outside [0, max_len - P])
  const int pos = clamp_report(lengths[b], 0, max_len - P, i == 0 && hd == 0 && j == 0 ? err : nullptr,
                               kDataErrLength) + i;
  const int H = n_heads * kD;
  const double ang = (double)pos * exp(-(double)j / (double)half * log_base);
  const double c = cos(ang), s = sin(ang);
  const bf16_t* row = qkv + (size_t)t * 3 * H + hd * kD;
  auto bf = [](bf16_t v) { return (double)__uint_as_float((uint32_t)v << 16); };
  // q
  const double q1 = bf(row[j]), q2 = bf(row[j + half]);
  bf16_t* qo = q + (size_t)t * H + hd * kD;
  qo[j] = f64_to_bf16(q1 * c - q2 * s);
  qo[j + half] = f64_to_bf16(q1 * s + q2 * c);
  // k (rotated) and v (as it is) into the cache
  const double k1 = bf(row[H + j]), k2 = bf(row[H + j + half]);
  bf16_t* ck = kv + (((size_t)b * n_heads + hd) * max_len + pos) * (2 * kD);
  bf16_t* cv = ck + kD;
  ck[j] = f64_to_bf16(k1 * c - k2 * s);
  ck[j + half] = f64_to_bf16(k1 * s + k2 * c);
  cv[j] = row[2 * H + j];
  cv[j + half] = row[2 * H + j + half];
}

// block (b, head, split): keys [k0, k1) of sequence b, all P queries (P <= 16);
// wavefront w owns the softmax state of queries w, w+4, ...  Partials:
// ws[((b*nh + head)*nsplit + split)*P + i] = {max, sum, out[128]} (fp32).
// Both products run on v_mfma_f32_16x16x32_bf16 with 16 query slots:
//   scores: every wavefront computes the tile's 64 keys x 16 slots (keys the
//     A operand from LDS, the queries the B operand held in registers; bf16
//     products, fp32 sums in k-step order) and parks them in its own padded
//     LDS rows, so that lane = key for the online softmax;
//   values: the probabilities go to LDS in bf16 [slot][key], the value tile
//     sits in LDS transposed [dim][key], and wavefront w accumulates output
//     dims 32 w .. 32 w + 31 of every slot (the running sums rescaled by each
//     slot's correction first).
// Staging: wavefronts 0-1 copy the tile's key rows (8 16-byte segments per
// thread); wavefronts 2-3 each load an 8-key x 8-dim block of values and
// transpose it in registers into 8 16-byte dim rows.  The next tile's loads
// are in flight while the current one is scored.
__global__ __launch_bounds__(256) void attn_split_kernel(const bf16_t* __restrict__ q,
                                                         const bf16_t* __restrict__ kv,
                                                         const int32_t* __restrict__ lengths, int P, int n_heads,
                                                         int max_len, int max_keys, int split_keys, int nsplit,
                                                         float scale, float* __restrict__ ws, uint32_t* err) {
  constexpr int kVRow = kTile + 8;                                // bf16 per transposed value / probability row
  __shared__ __align__(16) bf16_t ks[kTile][kRowPad];             // keys [key][dim]
  __shared__ __align__(16) bf16_t vt[kD][kVRow];                  // values [dim][key]
  __shared__ __align__(16) float sc[4][kMaxAttnP / 4][kTile + 4]; // per wavefront: scores of its slots [u][key]
  __shared__ __align__(16) bf16_t pb[kMaxAttnP][kVRow];           // probabilities [slot][key]
  __shared__ float cs[kMaxAttnP];                                 // per slot: the running sums' rescale
  const int split = blockIdx.x % nsplit;
  const int hd = (blockIdx.x / nsplit) % n_heads;
  const int b = blockIdx.x / (nsplit * n_heads);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int H = n_heads * kD;
  // the grid covers keys < max_keys (<= max_len); a longer length is clamped
  const int L = clamp_report(lengths[b], 0, max_keys - P, threadIdx.x == 0 && split == 0 && hd == 0 ? err : nullptr,
                             kDataErrLength);
  const int k0 = split * split_keys, k1 = min(k0 + split_keys, L + P);
  const size_t base = ((size_t)b * n_heads + hd) * max_len;

  // the scores' B operand: lane l holds query slot l%16 (zero past P), dims
  // 32 kk + 8 (l/16) .. +7 of k-step kk
  bf16x8_t qf[kD / 32];
  {
    const int j = lane & 15;
#pragma unroll
    for (int kk = 0; kk < kD / 32; ++kk) {
      const uint4 v = j < P ? ldg16(q + (size_t)(b * P + j) * H + hd * kD + 32 * kk + 8 * (lane >> 4))
                            : make_uint4(0u, 0u, 0u, 0u);
      qf[kk] = as_bf16x8(v);
    }
  }
  // slots past P: zero probabilities and unit rescale (their outputs are never written)
  for (int idx = threadIdx.x; idx < kMaxAttnP * kVRow; idx += 256) (&pb[0][0])[idx] = (bf16_t)0;
  if (threadIdx.x < kMaxAttnP) cs[threadIdx.x] = 1.f;
  // softmax state of this wavefront's queries
  float m[4], l[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) { m[u] = -INFINITY; l[u] = 0.f; }
  // output dims 32 wave + 16 db + 4 (lane/16) + v of slot lane%16
  f32x4_t o[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};

  const bool stage_k = threadIdx.x < 128;                 // wavefronts 0-1 (uniform per wavefront)
  const int kt = threadIdx.x & 127;
  const int ksg = kt & 15, krow = kt >> 4;                 // keys: segment ksg of rows krow + 8 j
  const int vqb = kt & 7, vdb = kt >> 3;                   // values: keys 8 vqb .. +7, dims 8 vdb .. +7
  uint4 r8[8];
  auto fetch = [&](int t0) __attribute__((always_inline)) {
    const int nk = min(kTile, k1 - t0);                    // rows past the span repeat a valid key
    if (stage_k) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int key = t0 + min(krow + 8 * j, nk - 1);
        r8[j] = ldg16(kv + (base + key) * (2 * kD) + 8 * ksg);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int key = t0 + min(8 * vqb + j, nk - 1);
        r8[j] = ldg16(kv + (base + key) * (2 * kD) + kD + 8 * vdb);
      }
    }
  };
  auto store = [&]() __attribute__((always_inline)) {
    if (stage_k) {
#pragma unroll
      for (int j = 0; j < 8; ++j) *reinterpret_cast<uint4*>(&ks[krow + 8 * j][8 * ksg]) = r8[j];
    } else {
      // r8[j] holds dims 8 vdb .. +7 of key 8 vqb + j, two dims per word (even
      // dim low); row e of the transpose holds keys 8 vqb .. +7 of dim 8 vdb + e
      uint32_t w[8][4];
#pragma unroll
      for (int j = 0; j < 8; ++j) { w[j][0] = r8[j].x; w[j][1] = r8[j].y; w[j][2] = r8[j].z; w[j][3] = r8[j].w; }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int wi = e >> 1;
        uint32_t t[4];
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
          const uint32_t a = w[2 * mm][wi], c = w[2 * mm + 1][wi];
          t[mm] = (e & 1) ? ((a >> 16) | (c & 0xffff0000u)) : ((a & 0xffffu) | (c << 16));
        }
        *reinterpret_cast<uint4*>(&vt[8 * vdb + e][8 * vqb]) = make_uint4(t[0], t[1], t[2], t[3]);
      }
    }
  };
  if (k0 < k1) fetch(k0);

  for (int t0 = k0; t0 < k1; t0 += kTile) {
    const int nk = min(kTile, k1 - t0);
    store();
    lds_barrier();
    if (t0 + kTile < k1) fetch(t0 + kTile);
    {
      // S[key][slot]: lane l ends with keys 16 kb + 4 (l/16) + v of slot l%16;
      // 16-byte key-row reads, rows 272 bytes apart
      f32x4_t d[kTile / 16];
#pragma unroll
      for (int kb = 0; kb < kTile / 16; ++kb) d[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < kD / 32; ++kk)
#pragma unroll
        for (int kb = 0; kb < kTile / 16; ++kb) {
          const uint4 a = *reinterpret_cast<const uint4*>(&ks[16 * kb + (lane & 15)][32 * kk + 8 * (lane >> 4)]);
          d[kb] = mfma16x16x32(as_bf16x8(a), qf[kk], d[kb]);
        }
      // keep the slots this wavefront owns (slot = wave + 4 u)
      if ((lane & 3) == wave)
#pragma unroll
        for (int kb = 0; kb < kTile / 16; ++kb)
          *reinterpret_cast<f32x4_t*>(&sc[wave][(lane & 15) >> 2][16 * kb + 4 * (lane >> 4)]) = d[kb];
      // the wavefront's own LDS rows: only its lanes wrote them
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = wave + 4 * u;
      if (i >= P) break;
      // lane = key of the tile
      const int key = t0 + lane;
      float s = sc[wave][u][lane];
      const bool vis = lane < nk && key <= L + i;
      s = vis ? s * scale : -INFINITY;
      const float mt = wave_max_dpp(s);
      const float mn = fmaxf(m[u], mt);
      const float p = vis ? expf(s - mn) : 0.f;
      const float corr = m[u] == -INFINITY ? 0.f : expf(m[u] - mn);
      l[u] = l[u] * corr + wave_sum_dpp(p);
      m[u] = mn;
      pb[i][lane] = f32_to_bf16(p);
      if (lane == 0) cs[i] = corr;
    }
    lds_barrier();   // every slot's probabilities and rescale
    {
      const float c = cs[lane & 15];
#pragma unroll
      for (int db = 0; db < 2; ++db) o[db] *= c;
#pragma unroll
      for (int kk = 0; kk < kTile / 32; ++kk) {
        const uint4 pf = *reinterpret_cast<const uint4*>(&pb[lane & 15][32 * kk + 8 * (lane >> 4)]);
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const uint4 a =
              *reinterpret_cast<const uint4*>(&vt[32 * wave + 16 * db + (lane & 15)][32 * kk + 8 * (lane >> 4)]);
          o[db] = mfma16x16x32(as_bf16x8(a), as_bf16x8(pf), o[db]);
        }
      }
    }
    lds_barrier();   // the tile's buffers are free for the next one
  }
  const size_t wbase = (((size_t)b * n_heads + hd) * nsplit + split) * P;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = wave + 4 * u;
    if (i >= P) break;
    if (lane == 0) {
      ws[(wbase + i) * (kD + 2)] = m[u];
      ws[(wbase + i) * (kD + 2) + 1] = l[u];
    }
  }
  const int slot = lane & 15;
  if (slot < P) {
    float* w = ws + (wbase + slot) * (kD + 2) + 2 + 32 * wave + 4 * (lane >> 4);
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int v = 0; v < 4; ++v) w[16 * db + v] = o[db][v];
  }
}

// one wavefront per (b, head, query): merge the splits (nsplit <= 64), lane
// owns 2 dims.  Lane s first reads split s's (max, sum) so the global max and
// the scale of every split come from two wave reductions; the output sums
// then run over the splits in order with their loads batched.
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ ws, int B, int P, int n_heads,
                                                         int nsplit, bf16_t* __restrict__ o) {
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (gw >= B * n_heads * P) return;
  const int i = gw % P, hd = (gw / P) % n_heads, b = gw / (P * n_heads);
  const size_t stride = (size_t)P * (kD + 2);   // between splits
  const float* w0 = ws + ((((size_t)b * n_heads + hd) * nsplit) * P + i) * (kD + 2);
  float ms = -INFINITY, ls = 0.f;
  if (lane < nsplit) {
    ms = w0[lane * stride];
    ls = w0[lane * stride + 1];
  }
  const float M = wave_max_dpp(ms);
  const float fs = ms == -INFINITY ? 0.f : expf(ms - M);   // a split with no visible key weighs 0
  const float Ls = wave_sum_dpp(fs * ls);
  float a0 = 0.f, a1 = 0.f;
#pragma unroll 8
  for (int sp = 0; sp < nsplit; ++sp) {
    const float f = __shfl(fs, sp);
    const float2 v = *reinterpret_cast<const float2*>(w0 + sp * stride + 2 + 2 * lane);
    a0 = fmaf(f, v.x, a0);
    a1 = fmaf(f, v.y, a1);
  }
  const int H = n_heads * kD;
  bf16_t* out = o + (size_t)(b * P + i) * H + hd * kD + 2 * lane;
  *reinterpret_cast<uint32_t*>(out) = pack_bf16x2(a0 / Ls, a1 / Ls);
}

__global__ void commit_kernel(const int32_t* __restrict__ n_commit, int B, int32_t* __restrict__ lengths) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) lengths[b] += n_commit[b];
}

}  // namespace

hipError_t launch_rope_cache(const void* qkv, const int32_t* lengths, int B, int P, int n_heads, float rope_base,
                             int max_len, void* q, void* kv_cache, hipStream_t s) {
  const long long n = (long long)B * P * n_heads * (kD / 2);
  hipLaunchKernelGGL(rope_cache_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     static_cast<const bf16_t*>(qkv), lengths, B, P, n_heads, max_len, log((double)rope_base),
                     static_cast<bf16_t*>(q), static_cast<bf16_t*>(kv_cache), data_error_word(s));
  return hipGetLastError();
}

hipError_t launch_attention(const void* q, const void* kv_cache, const int32_t* lengths, int B, int P, int n_heads,
                            int max_len, int max_keys, void* o, void* ws, hipStream_t s) {
  const int sk = attn_split_keys(max_keys);
  const int nsplit = (max_keys + sk - 1) / sk;
  float* w = static_cast<float*>(ws);
  hipLaunchKernelGGL(attn_split_kernel, dim3(B * n_heads * nsplit), dim3(256), 0, s, static_cast<const bf16_t*>(q),
                     static_cast<const bf16_t*>(kv_cache), lengths, P, n_heads,
                     max_len, max_keys, sk, nsplit, 1.0f / sqrtf((float)kD), w, data_error_word(s));
  const int waves = B * n_heads * P;
  hipLaunchKernelGGL(attn_merge_kernel, dim3((waves + 3) / 4), dim3(256), 0, s, w, B, P, n_heads, nsplit,
                     static_cast<bf16_t*>(o));
  return hipGetLastError();
}

hipError_t launch_commit(const int32_t* n_commit, int B, int32_t* lengths, hipStream_t s) {
  hipLaunchKernelGGL(commit_kernel, dim3((B + 255) / 256), dim3(256), 0, s, n_commit, B, lengths);
  return hipGetLastError();
}

}  // namespace moe
