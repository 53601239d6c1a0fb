// Internal launchers of the gfx950 kernels (C++ linkage, not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// This GPU's data-error word (the stream's device; NULL stream: the current
// one), or NULL if its address cannot be found (errors then go unreported).
uint32_t* data_error_word(hipStream_t s);

hipError_t launch_pack(const void* src, void* dst, int G, int N, int K, int kind, hipStream_t s);
hipError_t launch_pack_router(const void* src, void* dst, int G, int E, int K, hipStream_t s);

// the previous layer's combine, fused in front of a route (moe_combine_route)
struct CombineArgs {
  const void* y;         // [n_rows, H] expert outputs, permuted order
  const int32_t* inv;    // [T, k] row of each (token, slot)
  const float* w;        // [T, k] routing weights
  const void* ys;        // [S*T, H] shared-expert outputs or NULL
  int S, n_rows, k;
  uint32_t* err = nullptr;  // the data-error word (set by the launcher)
};

hipError_t launch_combine_route(const CombineArgs& ca, void* h, const float* gain, float eps, const float* w_router,
                                const float* bias, int T, int H, int E, int k, int flags, int dtype, void* xn,
                                int32_t* ids, float* w, float* logits, hipStream_t s);

hipError_t launch_rmsnorm(const void* x, const int32_t* rows, int x_rows, int T, int H, const float* gain, float eps,
                          int dtype, void* out, int out_stride, hipStream_t s);

hipError_t launch_route(const void* h, const float* gain, float eps, const float* w_router,
                        const float* bias, int T, int H, int E, int k, int flags, int dtype,
                        void* xn, int32_t* ids, float* w, float* logits, hipStream_t s);

hipError_t launch_permute(const int32_t* ids, int T, int k, int E, int S, int32_t* offsets,
                          int32_t* gather, int32_t* inv, void* ws, hipStream_t s);

hipError_t launch_gate_up(const void* x, const int32_t* gather, const int32_t* offsets, int G, int n_rows,
                          const void* w_gate_up, int T, int H, int I, int max_rows, int dtype, void* act,
                          hipStream_t s);
// the gate/up stage deriving its rows from the expert ids (moe_permute's layout)
struct RoutedArgs {
  const int32_t* ids;  // [T, k] expert of each (token, slot)
  int k, E, S;
  int32_t* offsets;    // [E+S+1] out
  int32_t* inv;        // [T, k] out
};
hipError_t launch_gate_up_routed(const void* x, const int32_t* ids, int T, int k, int E, int S, const void* w_gate_up,
                                 int H, int I, void* act, int32_t* offsets, int32_t* inv, hipStream_t s);

// grouped expert GEMM (bf16, prefill-sized groups): gated = gate/up stage
bool gemm_path_ok(int K, int N, int max_rows);
hipError_t launch_gemm(bool gated, const void* x, const int32_t* gather, const int32_t* offsets, int G, int n_rows,
                       int T, const void* W, int K, int N, void* out, hipStream_t s);
hipError_t launch_down(const void* act, const int32_t* offsets, int G, int n_rows, const void* w_down, int H,
                       int I, int max_rows, int dtype, void* y, hipStream_t s, const void* residual = nullptr);

hipError_t launch_combine_norm(const void* y, const int32_t* inv, const float* topk_w, const void* y_shared, int S,
                               const void* residual, int T, int H, int k, int n_rows, const float* gain, float eps,
                               int dtype, void* out, void* xn, hipStream_t s);
hipError_t launch_combine(const void* y, const int32_t* inv, const float* topk_w,
                          const void* y_shared, int S, const void* residual, int T, int H, int k,
                          int n_rows, int dtype, void* out, void* combined, hipStream_t s);

hipError_t launch_lmhead(const void* h, const void* w_lm, int T, int H, int V, int dtype,
                         int32_t* ids, float* max_logit, void* ws, hipStream_t s);

hipError_t launch_verify(const int32_t* drafts, const int32_t* argmax_ids, int B, int K,
                         int32_t* accepted, int32_t* committed, int32_t* n_commit, hipStream_t s);

hipError_t launch_plant(const int32_t* argmax_ids, const uint8_t* keep, const int32_t* repl, int B,
                        int K, int V, int32_t* drafts, hipStream_t s);

hipError_t launch_advance(const int32_t* n_commit, const int32_t* committed, const int32_t* seq_ids, int B, int K,
                          int S, int target, int32_t* total, int32_t* steps, int32_t* tokens, int32_t* seq_out,
                          int32_t* n_active, hipStream_t s);

hipError_t launch_gather_rows(const void* pool, const int32_t* seq_ids, const int32_t* steps, int B, int R, int J,
                              int S, int row_bytes, void* out, hipStream_t s);

hipError_t launch_rope_cache(const void* qkv, const int32_t* lengths, int B, int P, int n_heads, float rope_base,
                             int max_len, void* q, void* kv_cache, hipStream_t s);
hipError_t launch_attention(const void* q, const void* kv_cache, const int32_t* lengths, int B, int P, int n_heads,
                            int max_len, int max_keys, void* o, void* ws, hipStream_t s);
hipError_t launch_commit(const int32_t* n_commit, int B, int32_t* lengths, hipStream_t s);

}  // namespace moe
