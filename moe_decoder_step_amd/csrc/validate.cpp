// Host-side argument checks and workspace sizes of the C ABI (no HIP).
#include "validate.hpp"

namespace moe {

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool valid_dtype(int dt) { return dt == kBf16 || dt == kF32; }
size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

}  // namespace

int pack_pairs(int N, int kind) { return kind == 0 ? N / 16 : (N + 31) / 32; }

size_t packed_bytes(int G, int N, int K, int kind) {
  if (G <= 0 || N <= 0 || K <= 0 || kind < 0 || kind > 2) return 0;
  if (kind == 2) return (size_t)G * (size_t)(K / 4) * kMaxExperts * 4 * sizeof(float);
  // per pair: K/32 steps x 2 sets x 1 KB fragment
  return (size_t)G * (size_t)pack_pairs(N, kind) * (size_t)(K / 32) * 2 * 1024;
}

int check_pack(const void* src, const void* dst, int G, int N, int K, int kind, int dtype) {
  if (kind < 0 || kind > 2) return kErrUnsupported;
  if (kind == 2) {  // router: fp32 [G, E, K], E <= 64
    if (dtype != kF32) return kErrUnsupported;
    if (G < 0 || N <= 0 || K <= 0 || K % 4 != 0) return kErrShape;
    if (N > kMaxExperts) return kErrUnsupported;
    if (G == 0) return kOk;
    if (!src || !dst) return kErrNull;
    if (!aligned16(src) || !aligned16(dst)) return kErrAlign;
    return kOk;
  }
  if (dtype != kBf16) return kErrUnsupported;  // fp32 expert weights stay row-major
  if (G < 0 || N <= 0 || K <= 0 || K % 32 != 0 || (kind == 0 && N % 16 != 0)) return kErrShape;
  if (G == 0) return kOk;
  if (!src || !dst) return kErrNull;
  if (!aligned16(src) || !aligned16(dst)) return kErrAlign;
  return kOk;
}

size_t permute_ws_bytes(int T, int k, int E) {
  if (T <= 0 || k <= 0 || E <= 0) return 0;
  long long slots = (long long)T * k;
  if (slots <= kPermuteChunk) return 0;   // one block, no workspace
  long long chunks = (slots + kPermuteChunkM - 1) / kPermuteChunkM;
  // per-chunk expert counts and per-chunk scatter bases
  return align256((size_t)(2 * chunks * E) * sizeof(int32_t));
}

size_t swiglu_ws_bytes(int n_rows, int I, int dtype) {
  if (n_rows <= 0 || I <= 0) return 0;
  size_t elem = dtype == kF32 ? 4 : 2;
  return align256((size_t)n_rows * (size_t)I * elem);  // SwiGLU activation rows
}

int lmhead_blocks(int V, int dtype) {
  int rows = dtype == kF32 ? kLmF32RowsPerBlock : kLmRowsPerBlock;
  return (int)(((long long)V + rows - 1) / rows);
}

size_t lmhead_ws_bytes(int T, int V, int dtype) {
  if (T <= 0 || V <= 0) return 0;
  // one (max logit, index) pair per row and vocabulary block
  return align256((size_t)T * (size_t)lmhead_blocks(V, dtype) * 8);
}

int check_advance(const int32_t* n_commit, const int32_t* committed, const int32_t* seq_ids, int B, int K, int S,
                  int target, const int32_t* total, const int32_t* steps, const int32_t* tokens, const int32_t* seq_out,
                  const int32_t* n_active) {
  if (B < 0 || K < 0 || S <= 0 || target <= 0 || B > S) return kErrShape;
  if (B > kAdvanceMaxB || K > kMaxDrafts) return kErrUnsupported;
  if (!n_active) return kErrNull;
  if (B == 0) return kOk;
  if (!n_commit || !committed || !seq_ids || !total || !steps || !tokens || !seq_out) return kErrNull;
  return kOk;
}

int check_gather_rows(const void* pool, const int32_t* seq_ids, const int32_t* steps, int B, int R, int J, int S,
                      int row_bytes, const void* out) {
  if (B < 0 || R <= 0 || J <= 0 || S <= 0 || row_bytes < 0) return kErrShape;
  if ((long long)B * R > 0x7fffffffLL) return kErrUnsupported;
  if (B == 0 || row_bytes == 0) return kOk;
  if (!pool || !seq_ids || !steps || !out) return kErrNull;
  return kOk;
}

int check_gate_up_routed(const void* x, const int32_t* ids, int T, int k, int E, int S, const void* w_gate_up, int H,
                         int I, int dtype, const void* act, const int32_t* offsets, const int32_t* inv) {
  if (!valid_dtype(dtype)) return kErrUnsupported;
  if (T < 0 || k <= 0 || E <= 0 || k > E || S < 0 || H <= 0 || I <= 0) return kErrShape;
  if (dtype != kBf16 || E > kMaxExperts || S > kMaxShared || (long long)T * k > kPermuteChunk) return kErrUnsupported;
  if (H % 32 != 0 || I % 32 != 0 || H > 4096 || I > 4096 || E + S > 128) return kErrUnsupported;
  if (!offsets) return kErrNull;
  if (T == 0) return kOk;
  if (!x || !ids || !w_gate_up || !act || !inv) return kErrNull;
  if (!aligned16(x) || !aligned16(w_gate_up) || !aligned16(act)) return kErrAlign;
  return kOk;
}

int check_rmsnorm(const void* x, const int32_t* rows, int x_rows, int T, int H, int dtype, const void* out,
                  int out_stride) {
  if (!valid_dtype(dtype)) return kErrUnsupported;
  if (T < 0 || H <= 0 || x_rows <= 0 || out_stride < H) return kErrShape;
  if (!rows && x_rows < T) return kErrShape;
  if (H % 8 != 0 || H > 8192) return kErrUnsupported;
  if (T == 0) return kOk;
  if (!x || !out) return kErrNull;
  const size_t es = dtype == kBf16 ? 2 : 4;
  if (!aligned16(x) || !aligned16(out) || ((size_t)out_stride * es) % 16 != 0) return kErrAlign;
  return kOk;
}

int check_combine_norm(const void* y, const int32_t* inv, const float* topk_w, const void* y_shared,
                       int S, const void* residual, int T, int H, int k, int n_rows, int dtype,
                       const void* out, const void* xn) {
  int st = check_combine(y, inv, topk_w, y_shared, S, residual, T, H, k, n_rows, dtype, out, nullptr);
  if (st != kOk) return st;
  if (H > 2048) return kErrUnsupported;
  if (T == 0) return kOk;
  if (!xn) return kErrNull;
  if (!aligned16(xn)) return kErrAlign;
  if (xn == out || (residual && xn == residual)) return kErrShape;
  return kOk;
}

int attn_split_keys(int max_keys) {
  // at most 64 splits per (sequence, head), at least 256 keys each, a multiple of the 64-key tile
  int sk = (max_keys + 63) / 64;
  sk = ((sk + 63) / 64) * 64;
  return sk < 256 ? 256 : sk;
}

int check_rope_cache(const void* qkv, const int32_t* lengths, int B, int P, int n_heads, int head_dim, float rope_base,
                     int max_len, int dtype, const void* q, const void* kv_cache) {
  if (!valid_dtype(dtype)) return kErrUnsupported;
  if (B < 0 || P <= 0 || n_heads <= 0 || max_len < P || !(rope_base > 1.f)) return kErrShape;
  if (dtype != kBf16 || head_dim != kAttnHeadDim || P > kMaxAttnP) return kErrUnsupported;
  if ((long long)B * n_heads * max_len * head_dim > (1LL << 40)) return kErrUnsupported;
  if (B == 0) return kOk;
  if (!qkv || !lengths || !q || !kv_cache) return kErrNull;
  return kOk;
}

int check_commit(const int32_t* n_commit, int B, const int32_t* lengths) {
  if (B < 0) return kErrShape;
  if (B == 0) return kOk;
  if (!n_commit || !lengths) return kErrNull;
  return kOk;
}

int check_attention(const void* q, const void* kv_cache, const int32_t* lengths, int B, int P, int n_heads,
                    int head_dim, int max_len, int max_keys, int dtype, const void* o) {
  if (!valid_dtype(dtype)) return kErrUnsupported;
  if (B < 0 || P <= 0 || n_heads <= 0 || max_len < P || max_keys < P || max_keys > max_len) return kErrShape;
  if (dtype != kBf16 || head_dim != kAttnHeadDim || P > kMaxAttnP) return kErrUnsupported;
  if ((long long)B * n_heads * max_len * head_dim > (1LL << 40)) return kErrUnsupported;
  if (B == 0) return kOk;
  if (!q || !kv_cache || !lengths || !o) return kErrNull;
  if (!aligned16(kv_cache)) return kErrAlign;
  return kOk;
}

size_t attention_ws_bytes(int B, int P, int n_heads, int head_dim, int max_keys) {
  if (B <= 0 || P <= 0 || n_heads <= 0 || max_keys <= 0) return 0;
  const int sk = attn_split_keys(max_keys);
  const size_t nsplit = (size_t)((max_keys + sk - 1) / sk);
  return align256((size_t)B * n_heads * nsplit * P * (head_dim + 2) * sizeof(float));
}

int check_route(const void* h, const float* w_router, int T, int H, int E, int k, int dtype,
                const void* xn, const int32_t* ids, const float* w) {
  if (!valid_dtype(dtype)) return kErrUnsupported;
  if (T < 0 || H <= 0 || E <= 0 || k <= 0 || k > E) return kErrShape;
  if (E > kMaxExperts || H > kMaxHidden || H % 8 != 0) return kErrUnsupported;
  if (T == 0) return kOk;
  if (!h || !w_router || !xn || !ids || !w) return kErrNull;
  if (!aligned16(h) || !aligned16(xn) || !aligned16(w_router)) return kErrAlign;
  return kOk;
}

int check_permute(const int32_t* ids, int T, int k, int E, int S, const int32_t* offsets,
                  const int32_t* gather, const int32_t* inv, const void* ws, size_t ws_bytes) {
  if (T < 0 || k <= 0 || E <= 0 || k > E || S < 0) return kErrShape;
  if (E > kMaxExperts || S > kMaxShared) return kErrUnsupported;
  if ((long long)T * (k + S) > 0x7fffffffLL) return kErrUnsupported;
  if (!offsets) return kErrNull;   // offsets are written even for T == 0
  if (T == 0) return kOk;
  if (!ids || !gather || !inv) return kErrNull;
  size_t need = permute_ws_bytes(T, k, E);
  if (need && (!ws || ws_bytes < need)) return kErrWorkspace;
  return kOk;
}

int check_expert_shape(int G, int n_rows, int T, int H, int I, int max_rows, int dtype) {
  if (!valid_dtype(dtype)) return kErrUnsupported;
  if (G <= 0 || n_rows < 0 || T < 0 || H <= 0 || I <= 0 || max_rows < 0) return kErrShape;
  if (dtype == kBf16 && (H % 32 != 0 || I % 32 != 0 || H > 4096 || I > 4096 || G > 128)) return kErrUnsupported;
  if (dtype == kF32 && (H % 4 != 0 || I % 4 != 0)) return kErrUnsupported;
  return kOk;
}

int check_gate_up(const void* x, const int32_t* offsets, int G, int n_rows, const void* w_gate_up, int T,
                  int H, int I, int max_rows, int dtype, const void* act) {
  int st = check_expert_shape(G, n_rows, T, H, I, max_rows, dtype);
  if (st != kOk || n_rows == 0 || T == 0) return st;
  if (!x || !offsets || !w_gate_up || !act) return kErrNull;
  if (!aligned16(x) || !aligned16(w_gate_up) || !aligned16(act)) return kErrAlign;
  return kOk;
}

int check_down_residual(const void* act, const int32_t* offsets, int G, int n_rows, const void* w_down, int H, int I,
                        int max_rows, int dtype, const void* residual, const void* y) {
  int st = check_down(act, offsets, G, n_rows, w_down, H, I, max_rows, dtype, y);
  if (st != kOk || n_rows == 0) return st;
  if (!residual) return kErrNull;
  if (!aligned16(residual)) return kErrAlign;
  return kOk;
}

int check_down(const void* act, const int32_t* offsets, int G, int n_rows, const void* w_down, int H, int I,
               int max_rows, int dtype, const void* y) {
  int st = check_expert_shape(G, n_rows, 1, H, I, max_rows, dtype);
  if (st != kOk || n_rows == 0) return st;
  if (!act || !offsets || !w_down || !y) return kErrNull;
  if (!aligned16(act) || !aligned16(w_down) || !aligned16(y)) return kErrAlign;
  return kOk;
}

int check_swiglu(const void* x, const int32_t* offsets, int G, int n_rows, const void* w_gate_up,
                 const void* w_down, int T, int H, int I, int max_rows, int dtype, const void* y,
                 const void* ws, size_t ws_bytes) {
  int st = check_expert_shape(G, n_rows, T, H, I, max_rows, dtype);
  if (st != kOk || n_rows == 0 || T == 0) return st;
  if (!x || !offsets || !w_gate_up || !w_down || !y) return kErrNull;
  if (!aligned16(x) || !aligned16(w_gate_up) || !aligned16(w_down) || !aligned16(y)) return kErrAlign;
  size_t need = swiglu_ws_bytes(n_rows, I, dtype);
  if (!ws || ws_bytes < need) return kErrWorkspace;
  if (!aligned16(ws)) return kErrAlign;
  return kOk;
}

int check_combine(const void* y, const int32_t* inv, const float* topk_w, const void* y_shared,
                  int S, const void* residual, int T, int H, int k, int n_rows, int dtype,
                  const void* out, const void* combined) {
  if (!valid_dtype(dtype)) return kErrUnsupported;
  if (T < 0 || H <= 0 || k < 0 || S < 0 || n_rows < 0) return kErrShape;
  if (H % 8 != 0 || k > kMaxExperts) return kErrUnsupported;
  if (k > 0 && n_rows <= 0 && T > 0) return kErrShape;
  if (S > 0 && !y_shared) return kErrNull;
  if (T == 0) return kOk;
  if (!out || (k > 0 && (!y || !inv || !topk_w))) return kErrNull;
  if ((y && !aligned16(y)) || (y_shared && !aligned16(y_shared)) || (residual && !aligned16(residual)) ||
      !aligned16(out) || (combined && !aligned16(combined)))
    return kErrAlign;
  return kOk;
}

int check_lmhead(const void* h, const void* w_lm, int T, int H, int V, int dtype,
                 const int32_t* ids, const void* ws, size_t ws_bytes) {
  if (!valid_dtype(dtype)) return kErrUnsupported;
  if (T < 0 || H <= 0 || V <= 0) return kErrShape;
  if (dtype == kBf16 && H % 32 != 0) return kErrUnsupported;
  if (dtype == kF32 && H % 4 != 0) return kErrUnsupported;
  if (T == 0) return kOk;
  if (!h || !w_lm || !ids) return kErrNull;
  if (!aligned16(h) || !aligned16(w_lm)) return kErrAlign;
  size_t need = lmhead_ws_bytes(T, V, dtype);
  if (!ws || ws_bytes < need) return kErrWorkspace;
  if (!aligned16(ws)) return kErrAlign;
  return kOk;
}

int check_verify(const int32_t* drafts, const int32_t* argmax_ids, int B, int K,
                 const int32_t* accepted, const int32_t* committed, const int32_t* n_commit) {
  if (B < 0 || K < 0) return kErrShape;
  if (K > kMaxDrafts) return kErrUnsupported;
  if (B == 0) return kOk;
  if ((K > 0 && !drafts) || !argmax_ids || !accepted || !committed || !n_commit) return kErrNull;
  return kOk;
}

int check_plant(const int32_t* argmax_ids, const uint8_t* keep, const int32_t* repl, int B, int K,
                int V, const int32_t* drafts) {
  if (B < 0 || K < 0 || V <= 1) return kErrShape;
  if (K > kMaxDrafts) return kErrUnsupported;
  if (B == 0 || K == 0) return kOk;
  if (!argmax_ids || !keep || !repl || !drafts) return kErrNull;
  return kOk;
}

}  // namespace moe
