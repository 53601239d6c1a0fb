// Host-side argument checks and workspace sizes of the C ABI.
// Pure C++ (no HIP): these run before anything is enqueued.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace moe {

enum Status { kOk = 0, kErrNull = 1, kErrShape = 2, kErrUnsupported = 3, kErrAlign = 4,
              kErrWorkspace = 5, kErrHip = 6 };
enum Dtype { kBf16 = 0, kF32 = 1 };

constexpr int kMaxExperts = 64;      // one router lane per expert in a wavefront
constexpr int kMaxHidden = 2048;     // route kernel keeps a block's normed rows in LDS
constexpr int kMaxShared = 8;
constexpr int kMaxDrafts = 15;
constexpr int kPermuteChunk = 4096;  // slots of the one-block permutation (every decode batch)
constexpr int kPermuteChunkM = 1024; // slots per block of the multi-block permutation passes
constexpr int kAdvanceMaxB = 1024;   // sequences of one spec_advance call (one block)
constexpr int kAttnHeadDim = 128;    // attention head size
constexpr int kMaxAttnP = 16;        // verify positions per sequence in one attention call
constexpr int kGemmMinRows = 1024;   // max_rows from which the grouped SwiGLU runs as a tiled GEMM
constexpr int kLmRowsPerBlock = 128; // vocabulary rows per LM-head block (bf16 path)
constexpr int kLmF32RowsPerBlock = 256;

int pack_pairs(int N, int kind);
size_t packed_bytes(int G, int N, int K, int kind);
int check_pack(const void* src, const void* dst, int G, int N, int K, int kind, int dtype);

size_t permute_ws_bytes(int T, int k, int E);
size_t swiglu_ws_bytes(int n_rows, int I, int dtype);
size_t lmhead_ws_bytes(int T, int V, int dtype);
int lmhead_blocks(int V, int dtype);

int check_advance(const int32_t* n_commit, const int32_t* committed, const int32_t* seq_ids, int B, int K, int S,
                  int target, const int32_t* total, const int32_t* steps, const int32_t* tokens, const int32_t* seq_out,
                  const int32_t* n_active);
int check_gather_rows(const void* pool, const int32_t* seq_ids, const int32_t* steps, int B, int R, int J, int S,
                      int row_bytes, const void* out);
int check_gate_up_routed(const void* x, const int32_t* ids, int T, int k, int E, int S, const void* w_gate_up, int H,
                         int I, int dtype, const void* act, const int32_t* offsets, const int32_t* inv);
int check_rmsnorm(const void* x, const int32_t* rows, int x_rows, int T, int H, int dtype, const void* out,
                  int out_stride);
int attn_split_keys(int max_keys);
int check_rope_cache(const void* qkv, const int32_t* lengths, int B, int P, int n_heads, int head_dim, float rope_base,
                     int max_len, int dtype, const void* q, const void* kv_cache);
int check_commit(const int32_t* n_commit, int B, const int32_t* lengths);
int check_attention(const void* q, const void* kv_cache, const int32_t* lengths, int B, int P, int n_heads,
                    int head_dim, int max_len, int max_keys, int dtype, const void* o);
size_t attention_ws_bytes(int B, int P, int n_heads, int head_dim, int max_keys);
int check_route(const void* h, const float* w_router, int T, int H, int E, int k, int dtype,
                const void* xn, const int32_t* ids, const float* w);
int check_permute(const int32_t* ids, int T, int k, int E, int S, const int32_t* offsets,
                  const int32_t* gather, const int32_t* inv, const void* ws, size_t ws_bytes);
int check_expert_shape(int G, int n_rows, int T, int H, int I, int max_rows, int dtype);
int check_gate_up(const void* x, const int32_t* offsets, int G, int n_rows, const void* w_gate_up, int T,
                  int H, int I, int max_rows, int dtype, const void* act);
int check_down_residual(const void* act, const int32_t* offsets, int G, int n_rows, const void* w_down, int H, int I,
                        int max_rows, int dtype, const void* residual, const void* y);
int check_down(const void* act, const int32_t* offsets, int G, int n_rows, const void* w_down, int H, int I,
               int max_rows, int dtype, const void* y);
int check_swiglu(const void* x, const int32_t* offsets, int G, int n_rows, const void* w_gate_up,
                 const void* w_down, int T, int H, int I, int max_rows, int dtype, const void* y,
                 const void* ws, size_t ws_bytes);
int check_combine(const void* y, const int32_t* inv, const float* topk_w, const void* y_shared,
                  int S, const void* residual, int T, int H, int k, int n_rows, int dtype,
                  const void* out, const void* combined);
// moe_combine_rmsnorm: the checks of moe_combine, plus H <= 2048 (one block
// of 256 threads x 8 elements per row) and a distinct, aligned xn.
int check_combine_norm(const void* y, const int32_t* inv, const float* topk_w, const void* y_shared,
                       int S, const void* residual, int T, int H, int k, int n_rows, int dtype,
                       const void* out, const void* xn);
int check_lmhead(const void* h, const void* w_lm, int T, int H, int V, int dtype,
                 const int32_t* ids, const void* ws, size_t ws_bytes);
int check_verify(const int32_t* drafts, const int32_t* argmax_ids, int B, int K,
                 const int32_t* accepted, const int32_t* committed, const int32_t* n_commit);
int check_plant(const int32_t* argmax_ids, const uint8_t* keep, const int32_t* repl, int B, int K,
                int V, const int32_t* drafts);

}  // namespace moe
