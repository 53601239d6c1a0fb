// extern "C" entry points of libmoestep: host checks, then the launchers.
#include <hip/hip_runtime.h>

#include "../../include/moestep.h"
#include "kernels.hpp"
#include "validate.hpp"

namespace {

inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }
inline int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is negative or inconsistent";
    case MOE_ERR_UNSUPPORTED: return "shape or dtype not supported by the library";
    case MOE_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

size_t moe_packed_weights_bytes(int G, int N, int K, int kind) { return moe::packed_bytes(G, N, K, kind); }

int moe_pack_weights(const void* src, void* dst, int G, int N, int K, int kind, int dtype, void* stream) {
  int st = moe::check_pack(src, dst, G, N, K, kind, dtype);
  if (st != MOE_OK || G == 0) return st;
  if (kind == MOE_PACK_ROUTER) return hip_status(moe::launch_pack_router(src, dst, G, N, K, as_stream(stream)));
  return hip_status(moe::launch_pack(src, dst, G, N, K, kind, as_stream(stream)));
}

size_t moe_permute_workspace_bytes(int T, int k, int E) { return moe::permute_ws_bytes(T, k, E); }

size_t moe_grouped_swiglu_workspace_bytes(int n_rows, int I, int dtype) {
  return moe::swiglu_ws_bytes(n_rows, I, dtype);
}

size_t lmhead_argmax_workspace_bytes(int T, int V, int dtype) { return moe::lmhead_ws_bytes(T, V, dtype); }

int moe_route(const void* h, const float* gain, float eps, const float* w_router, const float* bias,
              int T, int H, int E, int k, int flags, int dtype, void* xn, int32_t* topk_ids,
              float* topk_w, float* logits, void* stream) {
  int st = moe::check_route(h, w_router, T, H, E, k, dtype, xn, topk_ids, topk_w);
  if (st != MOE_OK || T == 0) return st;
  return hip_status(moe::launch_route(h, gain, eps, w_router, bias, T, H, E, k, flags, dtype, xn, topk_ids,
                                      topk_w, logits, as_stream(stream)));
}

int moe_permute(const int32_t* topk_ids, int T, int k, int E, int S, int32_t* offsets, int32_t* gather,
                int32_t* inv, void* ws, size_t ws_bytes, void* stream) {
  int st = moe::check_permute(topk_ids, T, k, E, S, offsets, gather, inv, ws, ws_bytes);
  if (st != MOE_OK) return st;
  // T == 0 still writes offsets (all groups empty) with a kernel, not a memset
  return hip_status(moe::launch_permute(topk_ids, T, k, E, S, offsets, gather, inv, ws, as_stream(stream)));
}

int moe_grouped_swiglu(const void* x, const int32_t* gather, const int32_t* offsets, int G, int n_rows,
                       const void* w_gate_up, const void* w_down, int T, int H, int I, int max_rows,
                       int dtype, void* y, void* ws, size_t ws_bytes, void* stream) {
  int st = moe::check_swiglu(x, offsets, G, n_rows, w_gate_up, w_down, T, H, I, max_rows, dtype, y, ws,
                             ws_bytes);
  if (st != MOE_OK || n_rows == 0 || T == 0) return st;
  const hipError_t e = moe::launch_gate_up(x, gather, offsets, G, n_rows, w_gate_up, T, H, I, max_rows, dtype, ws,
                                           as_stream(stream));
  if (e != hipSuccess) return hip_status(e);
  return hip_status(moe::launch_down(ws, offsets, G, n_rows, w_down, H, I, max_rows, dtype, y, as_stream(stream)));
}

int moe_expert_gate_up(const void* x, const int32_t* gather, const int32_t* offsets, int G, int n_rows,
                       const void* w_gate_up, int T, int H, int I, int max_rows, int dtype, void* act,
                       void* stream) {
  int st = moe::check_gate_up(x, offsets, G, n_rows, w_gate_up, T, H, I, max_rows, dtype, act);
  if (st != MOE_OK || n_rows == 0 || T == 0) return st;
  return hip_status(moe::launch_gate_up(x, gather, offsets, G, n_rows, w_gate_up, T, H, I, max_rows, dtype, act,
                                        as_stream(stream)));
}

int moe_expert_gate_up_routed(const void* x, const int32_t* topk_ids, int T, int k, int E, int S,
                              const void* w_gate_up, int H, int I, int dtype, void* act, int32_t* offsets,
                              int32_t* inv, void* stream) {
  int st = moe::check_gate_up_routed(x, topk_ids, T, k, E, S, w_gate_up, H, I, dtype, act, offsets, inv);
  if (st != MOE_OK) return st;
  if (T == 0)  // every group empty: offsets all zero, written by moe_permute's kernel
    return hip_status(moe::launch_permute(topk_ids, 0, k, E, S, offsets, nullptr, nullptr, nullptr, as_stream(stream)));
  return hip_status(moe::launch_gate_up_routed(x, topk_ids, T, k, E, S, w_gate_up, H, I, act, offsets, inv,
                                               as_stream(stream)));
}

int moe_expert_down(const void* act, const int32_t* offsets, int G, int n_rows, const void* w_down, int H, int I,
                    int max_rows, int dtype, void* y, void* stream) {
  int st = moe::check_down(act, offsets, G, n_rows, w_down, H, I, max_rows, dtype, y);
  if (st != MOE_OK || n_rows == 0) return st;
  return hip_status(moe::launch_down(act, offsets, G, n_rows, w_down, H, I, max_rows, dtype, y, as_stream(stream)));
}

int moe_expert_down_residual(const void* act, const int32_t* offsets, int G, int n_rows, const void* w_down, int H,
                             int I, int max_rows, int dtype, const void* residual, void* y, void* stream) {
  int st = moe::check_down_residual(act, offsets, G, n_rows, w_down, H, I, max_rows, dtype, residual, y);
  if (st != MOE_OK || n_rows == 0) return st;
  return hip_status(moe::launch_down(act, offsets, G, n_rows, w_down, H, I, max_rows, dtype, y, as_stream(stream),
                                     residual));
}

int moe_combine(const void* y, const int32_t* inv, const float* topk_w, const void* y_shared, int S,
                const void* residual, int T, int H, int k, int n_rows, int dtype, void* out, void* combined,
                void* stream) {
  int st = moe::check_combine(y, inv, topk_w, y_shared, S, residual, T, H, k, n_rows, dtype, out, combined);
  if (st != MOE_OK || T == 0) return st;
  return hip_status(moe::launch_combine(y, inv, topk_w, y_shared, S, residual, T, H, k, n_rows, dtype, out,
                                        combined, as_stream(stream)));
}

int moe_combine_rmsnorm(const void* y, const int32_t* inv, const float* topk_w, const void* y_shared, int S,
                        const void* residual, int T, int H, int k, int n_rows, const float* gain, float eps,
                        int dtype, void* out, void* xn, void* stream) {
  int st = moe::check_combine_norm(y, inv, topk_w, y_shared, S, residual, T, H, k, n_rows, dtype, out, xn);
  if (st != MOE_OK || T == 0) return st;
  return hip_status(moe::launch_combine_norm(y, inv, topk_w, y_shared, S, residual, T, H, k, n_rows, gain, eps,
                                             dtype, out, xn, as_stream(stream)));
}

int lmhead_argmax(const void* h, const void* w_lm, int T, int H, int V, int dtype, int32_t* argmax_ids,
                  float* max_logit, void* ws, size_t ws_bytes, void* stream) {
  int st = moe::check_lmhead(h, w_lm, T, H, V, dtype, argmax_ids, ws, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  return hip_status(moe::launch_lmhead(h, w_lm, T, H, V, dtype, argmax_ids, max_logit, ws, as_stream(stream)));
}

int spec_verify(const int32_t* drafts, const int32_t* argmax_ids, int B, int K, int32_t* accepted,
                int32_t* committed, int32_t* n_commit, void* stream) {
  int st = moe::check_verify(drafts, argmax_ids, B, K, accepted, committed, n_commit);
  if (st != MOE_OK || B == 0) return st;
  return hip_status(moe::launch_verify(drafts, argmax_ids, B, K, accepted, committed, n_commit,
                                       as_stream(stream)));
}

int spec_plant_drafts(const int32_t* argmax_ids, const uint8_t* keep, const int32_t* repl, int B, int K, int V,
                      int32_t* drafts, void* stream) {
  int st = moe::check_plant(argmax_ids, keep, repl, B, K, V, drafts);
  if (st != MOE_OK || B == 0 || K == 0) return st;
  return hip_status(moe::launch_plant(argmax_ids, keep, repl, B, K, V, drafts, as_stream(stream)));
}

int moe_rmsnorm(const void* x, const int32_t* rows, int x_rows, int T, int H, const float* gain, float eps, int dtype,
                void* out, int out_stride, void* stream) {
  int st = moe::check_rmsnorm(x, rows, x_rows, T, H, dtype, out, out_stride);
  if (st != MOE_OK || T == 0) return st;
  return hip_status(moe::launch_rmsnorm(x, rows, x_rows, T, H, gain, eps, dtype, out, out_stride, as_stream(stream)));
}

int moe_combine_route(const void* y, const int32_t* inv, const float* topk_w_prev, const void* y_shared, int S,
                      int n_rows, int k_prev, void* h, int T, int H, const float* gain, float eps,
                      const float* w_router, const float* bias, int E, int k, int flags, int dtype, void* xn,
                      int32_t* topk_ids, float* topk_w, float* logits, void* stream) {
  int st = moe::check_combine(y, inv, topk_w_prev, y_shared, S, h, T, H, k_prev, n_rows, dtype, h, nullptr);
  if (st != MOE_OK) return st;
  st = moe::check_route(h, w_router, T, H, E, k, dtype, xn, topk_ids, topk_w);
  if (st != MOE_OK || T == 0) return st;
  const moe::CombineArgs ca{y, inv, topk_w_prev, y_shared, S, n_rows, k_prev};
  return hip_status(moe::launch_combine_route(ca, h, gain, eps, w_router, bias, T, H, E, k, flags, dtype, xn,
                                              topk_ids, topk_w, logits, as_stream(stream)));
}

int spec_advance(const int32_t* n_commit, const int32_t* committed, const int32_t* seq_ids, int B, int K, int S,
                 int target, int32_t* total, int32_t* steps, int32_t* tokens, int32_t* seq_ids_out,
                 int32_t* n_active, void* stream) {
  int st = moe::check_advance(n_commit, committed, seq_ids, B, K, S, target, total, steps, tokens, seq_ids_out,
                              n_active);
  if (st != MOE_OK) return st;
  // B == 0 still writes n_active = 0, with the same one-block kernel
  return hip_status(moe::launch_advance(n_commit, committed, seq_ids, B, K, S, target, total, steps, tokens,
                                        seq_ids_out, n_active, as_stream(stream)));
}

int spec_gather_rows(const void* pool, const int32_t* seq_ids, const int32_t* steps, int B, int R, int J, int S,
                     int row_bytes, void* out, void* stream) {
  int st = moe::check_gather_rows(pool, seq_ids, steps, B, R, J, S, row_bytes, out);
  if (st != MOE_OK || B == 0 || row_bytes == 0) return st;
  return hip_status(moe::launch_gather_rows(pool, seq_ids, steps, B, R, J, S, row_bytes, out, as_stream(stream)));
}

int moe_attn_rope_cache(const void* qkv, const int32_t* lengths, int B, int P, int n_heads, int head_dim,
                        float rope_base, int max_len, int dtype, void* q, void* kv_cache, void* stream) {
  int st = moe::check_rope_cache(qkv, lengths, B, P, n_heads, head_dim, rope_base, max_len, dtype, q, kv_cache);
  if (st != MOE_OK || B == 0) return st;
  return hip_status(moe::launch_rope_cache(qkv, lengths, B, P, n_heads, rope_base, max_len, q, kv_cache,
                                           as_stream(stream)));
}

size_t moe_attention_workspace_bytes(int B, int P, int n_heads, int head_dim, int max_keys) {
  return moe::attention_ws_bytes(B, P, n_heads, head_dim, max_keys);
}

int moe_attention(const void* q, const void* kv_cache, const int32_t* lengths, int B, int P, int n_heads,
                  int head_dim, int max_len, int max_keys, int dtype, void* o, void* ws, size_t ws_bytes,
                  void* stream) {
  int st = moe::check_attention(q, kv_cache, lengths, B, P, n_heads, head_dim, max_len, max_keys, dtype, o);
  if (st != MOE_OK || B == 0) return st;
  if (!ws || ws_bytes < moe::attention_ws_bytes(B, P, n_heads, head_dim, max_keys)) return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_attention(q, kv_cache, lengths, B, P, n_heads, max_len, max_keys, o, ws,
                                          as_stream(stream)));
}

int spec_commit(const int32_t* n_commit, int B, int32_t* lengths, void* stream) {
  int st = moe::check_commit(n_commit, B, lengths);
  if (st != MOE_OK || B == 0) return st;
  return hip_status(moe::launch_commit(n_commit, B, lengths, as_stream(stream)));
}

}  // extern "C"
