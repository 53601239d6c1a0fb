/*
 * moestep.h -- C ABI of the MoE speculative verify step on MI355X (gfx950).
 *
 * The step is the verifier pass of the jina-ocr-v1 decoder (DeepSeek-3B-MoE:
 * hidden 1280, 64 routed + 2 shared experts, top-6 routing, vocabulary
 * 129,280 -- jina.ai/ko model card "jina-ocr-v1", architecture paragraph),
 * which checks K drafted tokens greedily and commits the longest agreeing
 * prefix plus one bonus token (jina.ai/de "jina-ocr-v1: Schnellere
 * Dokumentenanalyse auf kostenguenstigen GPUs", sections "Modell und
 * Training" and "Spekulatives Decoding auf einer L4").  Per layer:
 *
 *   moe_route -> moe_permute -> moe_grouped_swiglu -> moe_combine
 *
 * and once per verify pass: lmhead_argmax -> spec_verify.
 *
 * Conventions shared by every call
 * --------------------------------
 * - All tensor pointers are device memory owned by the caller.  The library
 *   never allocates, frees or synchronises; every call enqueues its kernels on
 *   `stream` (a hipStream_t passed as void*, NULL = the default stream) and
 *   returns at once.  Calls on one stream run in order.
 * - Layouts are row-major and contiguous.  Ids are int32.  `dtype` selects
 *   the storage type of activations and expert / LM-head weights (MOE_BF16 or
 *   MOE_F32); router weights, router bias and routing weights are always fp32.
 *   Arithmetic accumulates in fp32 (the RMSNorm scale in fp64).
 * - Activation and weight pointers must be 16-byte aligned (MOE_ERR_ALIGN).
 * - A size of 0 tokens (or sequences) is a no-op that returns MOE_OK.
 * - The return value is a moe_status.  Host-side argument checks run before
 *   anything is enqueued; a failed launch returns MOE_ERR_HIP.  Device-side
 *   data is never trusted for memory addressing: out-of-range ids, row
 *   indices, offsets and lengths are clamped into range (memory-safe), and
 *   the kernel that clamped also sets the matching MOE_DATA_ERR_* bit in a
 *   per-GPU word that moe_data_errors reads back (see there).
 * - Outputs are fully overwritten.  The only aliasing allowed is
 *   out == residual in moe_combine.
 * - Process-wide state: a per-device cache of the compute-unit count
 *   (atomics; racing threads store the same value); the data-error word, a
 *   static device variable per GPU, and a per-device cache of its address;
 *   for lmhead_argmax_noalloc a static device array per GPU and a per-device
 *   cache of its address (the address caches fill under a mutex).  Calls on different streams may
 *   run concurrently as long as they do not share output or workspace
 *   buffers (lmhead_argmax_noalloc calls share that array).
 */
#ifndef MOESTEP_H
#define MOESTEP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,         /* a required pointer is NULL */
  MOE_ERR_SHAPE = 2,        /* a size is negative or inconsistent */
  MOE_ERR_UNSUPPORTED = 3,  /* a valid shape the library does not handle (e.g. E > 64) */
  MOE_ERR_ALIGN = 4,        /* a tensor pointer is not 16-byte aligned */
  MOE_ERR_WORKSPACE = 5,    /* workspace missing or smaller than the query says */
  MOE_ERR_HIP = 6           /* the HIP runtime reported an error at launch */
} moe_status;

typedef enum { MOE_BF16 = 0, MOE_F32 = 1 } moe_dtype;

/* moe_pack_weights kinds */
#define MOE_PACK_GATE_UP 0  /* [G, 2N, K]: gate rows 0..N-1, up rows N..2N-1 */
#define MOE_PACK_ROWS 1     /* [G, N, K]: plain rows (down projection, LM head) */
#define MOE_PACK_ROUTER 2   /* fp32 router weight [G, E, K], E <= 64 */

/* moe_route flags */
#define MOE_ROUTE_NORM 1    /* apply RMSNorm before the router (else xn = h) */
#define MOE_ROUTE_RENORM 2  /* softmax over the k selected logits (else full-softmax probabilities) */
#define MOE_ROUTE_WPACKED 4 /* w_router is in the MOE_PACK_ROUTER layout (else row-major [E,H]) */

/* Version of this ABI (MOE_ABI_VERSION). */
int moe_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* moe_status_str(int status);

/* ---------------------------------------------------------------------------
 * moe_pack_weights -- convert row-major bf16 weights to the fragment layout
 * the weight-streaming kernels read (done once, when a model is loaded).
 *
 * The expert FFN and the LM head read weight rows as matrix-core A operands:
 * lane l of a wavefront takes row l%16, elements 8*(l/16)..+7 of each 32-wide
 * k-step.  The packed layout stores each such 16-row x 32 fragment as 1 KB
 * in lane order, two row sets side by side, so every load is 1 KB of
 * consecutive bytes:
 *   dst[g][p][s][h][l][j] = src[g][row][32*s + 8*(l/16) + j]
 *   MOE_PACK_GATE_UP: src [G, 2N, K]; row = h*N + 16p + l%16  (p < N/16)
 *   MOE_PACK_ROWS:    src [G, N, K];  row = 32p + 16h + l%16 (p < ceil(N/32));
 *                     rows at or past N are zero
 * src and dst: bf16, 16-byte aligned, not overlapping; dst holds
 * moe_packed_weights_bytes(G, N, K, kind) bytes.  MOE_F32 expert and LM-head
 * weights are used row-major and are not packed (MOE_ERR_UNSUPPORTED).
 * Limits: K % 32 == 0; N % 16 == 0 for MOE_PACK_GATE_UP.
 *
 * MOE_PACK_ROUTER (dtype MOE_F32): src is the router weight [G, E, K] with
 * E <= 64 experts (N = E) and K % 4 == 0; dst[g][q][e][j] = src[g][e][4q + j]
 * for e < E and 0 for E <= e < 64 (G * K/4 * 64 * 4 floats), the layout
 * moe_route reads with MOE_ROUTE_WPACKED: one expert per lane, four hidden
 * elements per 16-byte load, 1 KB per wavefront load.
 * ------------------------------------------------------------------------- */
size_t moe_packed_weights_bytes(int G, int N, int K, int kind);
int moe_pack_weights(const void* src, void* dst, int G, int N, int K, int kind, int dtype,
                     void* stream);

/* ---------------------------------------------------------------------------
 * moe_route -- pre-norm, router logits, top-k selection and routing weights.
 *
 * Per token t (the pages give top-6 of 64 routed experts -- alphasignal.ai
 * "Jina AI's 3.4B OCR model targets faster page parsing", section "A
 * compressed visual front end"; the norm and the routing function are not on
 * the pages, the readings are):
 *   xn[t]  = h[t] / sqrt(mean(h[t]^2) + eps) * gain     (if MOE_ROUTE_NORM)
 *            stored once, rounded to nearest-even from an fp64 scale
 *   l[t,e] = sum_h xn[t,h] * w_router[e,h] + bias[e]     fp32
 *   ids    = the k largest l[t,:], descending; equal logits -> lower expert id
 *   w[t,j] = exp(l[t,ids_j]) / sum_{i<k} exp(l[t,ids_i])  (MOE_ROUTE_RENORM)
 *            exp(l[t,ids_j]) / sum_e exp(l[t,e])          (otherwise)
 *
 * h        [T,H] dtype             in
 * gain     [H] fp32 or NULL (= 1)  in
 * w_router [E,H] fp32 row-major, or packed (MOE_PACK_ROUTER) with
 *          MOE_ROUTE_WPACKED;  bias [E] fp32 or NULL   in
 * xn       [T,H] dtype             out (the normed input the experts read)
 * topk_ids [T,k] int32, topk_w [T,k] fp32      out
 * logits   [T,E] fp32 or NULL      out (optional, for near-tie diagnostics)
 * Limits: 1 <= k <= E <= 64, 8 <= H <= 2048, H % 8 == 0.
 * ------------------------------------------------------------------------- */
int moe_route(const void* h, const float* gain, float eps,
              const float* w_router, const float* bias,
              int T, int H, int E, int k, int flags, int dtype,
              void* xn, int32_t* topk_ids, float* topk_w, float* logits,
              void* stream);

/* ---------------------------------------------------------------------------
 * moe_permute -- group the T*k (token, slot) pairs by expert.
 *
 * Why the step needs it: every token is sent to 6 of 64 routed experts and
 * to the 2 shared experts ("Jina AI's 3.4B OCR model targets faster page
 * parsing", section "A compressed visual front end"; jina.ai/ko model card
 * "jina-ocr-v1", architecture paragraph), so the rows an expert multiplies
 * are scattered over the batch; grouping them lets each expert's weights be
 * read once per call.  How the pairs are grouped is not on the pages: a
 * stable counting sort, so the order is unique.
 *
 * Slot s = t*k + j.  Routed expert e owns rows offsets[e] .. offsets[e+1]-1,
 * holding its slots in ascending token order (a stable counting sort).
 * When S > 0, shared expert s is appended as group E+s owning the T rows
 * T*k + s*T .. T*k + (s+1)*T - 1, one per token in order, so one grouped
 * SwiGLU call covers routed and shared experts.
 *
 * topk_ids [T,k] int32     in  (ids outside [0,E) are clamped into it and
 *                                reported: MOE_DATA_ERR_EXPERT_ID)
 * offsets  [E+S+1] int32   out (offsets[E+s] = T*k + s*T)
 * gather   [T*k + S*T] int32 out: token read by each row
 * inv      [T*k] int32     out: row of each slot
 * ws / ws_bytes            scratch of at least moe_permute_workspace_bytes()
 *                          bytes (may be NULL when that is 0)
 * Limits: 1 <= E <= 64, 1 <= k <= E, 0 <= S <= 8.
 * ------------------------------------------------------------------------- */
size_t moe_permute_workspace_bytes(int T, int k, int E);
int moe_permute(const int32_t* topk_ids, int T, int k, int E, int S,
                int32_t* offsets, int32_t* gather, int32_t* inv,
                void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * moe_grouped_swiglu -- SwiGLU expert FFN over groups of gathered rows.
 *
 * For each group g and each row r in offsets[g] .. offsets[g+1]-1, with
 * token t = gather[r] (or t = r - offsets[g] when gather is NULL):
 *   a[r] = silu(W_g[g] x[t]) * (W_u[g] x[t])    fp32 accumulate, stored in dtype
 *   y[r] = W_d[g] a[r]                          fp32 accumulate, stored in dtype
 * with silu(z) = z / (1 + exp(-z)).  Routed and shared experts are the same
 * operation (64 routed + 2 shared experts: jina.ai/ko model card, architecture
 * paragraph; the SwiGLU form is a reading, the pages do not give it).
 *
 * x         [T,H] dtype                 in
 * gather    [n_rows] int32 or NULL      in  (clamped into [0,T); MOE_DATA_ERR_ROW_INDEX)
 * offsets   [G+1] int32 (device)        in  (nondecreasing, offsets[G] <= n_rows;
 *                                            clamped into [0,n_rows];
 *                                            MOE_DATA_ERR_OFFSETS)
 * w_gate_up [G, 2I, H] dtype            in  rows 0..I-1 = W_g, I..2I-1 = W_u;
 *                                            MOE_BF16: packed (MOE_PACK_GATE_UP, N = I)
 * w_down    [G, H, I] dtype             in  MOE_BF16: packed (MOE_PACK_ROWS, N = H)
 * max_rows  host-side upper bound on any group's row count (e.g. T): a
 *           hint for choosing the kernel shape; any count is computed correctly
 * y         [n_rows, H] dtype           out (rows outside every group untouched)
 * ws        scratch of at least moe_grouped_swiglu_workspace_bytes() bytes
 * Limits: H % 32 == 0, I % 32 == 0, H <= 4096, I <= 4096 and G <= 128 for
 *         MOE_BF16 (a block keeps 16 activation rows of the full reduction
 *         length in LDS); H % 4 == 0 and I % 4 == 0 for MOE_F32; 1 <= G.
 * ------------------------------------------------------------------------- */
size_t moe_grouped_swiglu_workspace_bytes(int n_rows, int I, int dtype);
int moe_grouped_swiglu(const void* x, const int32_t* gather, const int32_t* offsets,
                       int G, int n_rows, const void* w_gate_up, const void* w_down,
                       int T, int H, int I, int max_rows, int dtype,
                       void* y, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * moe_expert_gate_up, moe_expert_down -- the two halves of moe_grouped_swiglu
 * as separate calls (same kernels, same results):
 *
 *   moe_expert_gate_up: act[r] = silu(W_g[g] x[t]) * (W_u[g] x[t])
 *   moe_expert_down:    y[r]   = W_d[g] act[r]
 *
 * for every row r of every group g, with t and the arguments as in
 * moe_grouped_swiglu.  act is [n_rows, I] in dtype (caller-owned, 16-byte
 * aligned); rows outside every group are untouched.  A caller that times or
 * overlaps the halves, or keeps act, uses these; moe_grouped_swiglu is
 * exactly moe_expert_gate_up into its workspace followed by moe_expert_down.
 * Limits and errors as for moe_grouped_swiglu.
 * ------------------------------------------------------------------------- */
int moe_expert_gate_up(const void* x, const int32_t* gather, const int32_t* offsets,
                       int G, int n_rows, const void* w_gate_up, int T, int H, int I,
                       int max_rows, int dtype, void* act, void* stream);
/* ---------------------------------------------------------------------------
 * moe_expert_gate_up_routed -- moe_permute and moe_expert_gate_up in one
 * launch for decode-sized batches: each block derives the rows it needs from
 * the expert ids (a histogram of the ids and a stable scan of its group's
 * (token, slot) pairs), so the permutation is never a launch of its own.
 * The rows, act and the outputs offsets and inv are exactly those of
 * moe_permute (E routed groups in expert order, then S shared groups of T
 * token-ordered rows) followed by moe_expert_gate_up; the gather list is not
 * produced.  offsets feeds moe_expert_down, inv feeds the combine.
 *
 * x         [T,H] bf16           in   normed tokens
 * topk_ids  [T,k] int32          in   (clamped into [0,E); MOE_DATA_ERR_EXPERT_ID)
 * w_gate_up [E+S, 2I, H] bf16    in   packed (MOE_PACK_GATE_UP, N = I)
 * act       [T*k + S*T, I] bf16  out
 * offsets   [E+S+1] int32        out  (written also for T = 0)
 * inv       [T,k] int32          out
 * Limits: MOE_BF16 only; T*k <= 4096; E <= 64, S <= 8, E+S <= 128; H, I as
 * for moe_grouped_swiglu.  Larger batches use moe_permute and
 * moe_expert_gate_up (MOE_ERR_UNSUPPORTED here).
 * ------------------------------------------------------------------------- */
int moe_expert_gate_up_routed(const void* x, const int32_t* topk_ids, int T, int k, int E, int S,
                              const void* w_gate_up, int H, int I, int dtype, void* act,
                              int32_t* offsets, int32_t* inv, void* stream);
int moe_expert_down(const void* act, const int32_t* offsets, int G, int n_rows,
                    const void* w_down, int H, int I, int max_rows, int dtype,
                    void* y, void* stream);
/* moe_expert_down_residual -- moe_expert_down with a residual added in the
 * epilogue: y[r] = residual[r] + round(W_d[g] act[r]), the product rounded to
 * dtype first and the sum rounded once (the same bits as moe_expert_down
 * followed by moe_combine with y as its one shared row and k = 0).  For the
 * dense layers around the MoE blocks: the draft block's FFN ("Jina AI's 3.4B
 * OCR model targets faster page parsing", section "FastMTP cuts decoding
 * work": one dense block) and the attention output projection (the
 * decoder's attention, jina.ai/ko model card, architecture paragraph, read
 * as a pre-norm residual block).  residual [n_rows, H] dtype, 16-byte aligned; it may
 * be y itself (in place).  Errors as moe_expert_down, plus MOE_ERR_NULL for
 * a NULL residual. */
int moe_expert_down_residual(const void* act, const int32_t* offsets, int G, int n_rows,
                             const void* w_down, int H, int I, int max_rows, int dtype,
                             const void* residual, void* y, void* stream);

/* ---------------------------------------------------------------------------
 * moe_combine -- weighted sum of the expert outputs plus the residual.
 *
 * Why the step needs it: a token's layer output joins its 6 routed experts
 * (top-6 of 64), weighted by the router, and its 2 shared experts ("Jina
 * AI's 3.4B OCR model targets faster page parsing", section "A compressed
 * visual front end"; jina.ai/ko model card "jina-ocr-v1", architecture
 * paragraph).  The pages do not give the weighting; the reading taken is
 * the router's softmax over the selected logits for routed experts, weight
 * 1 for shared ones, added to the block's input (a residual block).
 *
 *   c[t]   = sum_{j<k} topk_w[t,j] * y[inv[t*k+j]] + sum_{s<S} y_shared[s*T+t]
 *   out[t] = residual[t] + c[t]          (out = c[t] when residual is NULL)
 * fp32, summed in that fixed order, then stored in dtype.  Shared experts
 * carry weight 1.
 *
 * y        [n_rows, H] dtype (rows in permuted order)   in
 * inv      [T*k] int32  (clamped into [0,n_rows); MOE_DATA_ERR_INV)  in
 * topk_w   [T,k] fp32                                    in
 * y_shared [S*T, H] dtype or NULL (then S must be 0)     in
 * residual [T,H] dtype or NULL                           in
 * out      [T,H] dtype, may alias residual               out
 * combined [T,H] dtype or NULL: c[t] before the residual out
 * Limits: H % 8 == 0, 0 <= k <= 64.
 * ------------------------------------------------------------------------- */
int moe_combine(const void* y, const int32_t* inv, const float* topk_w,
                const void* y_shared, int S, const void* residual,
                int T, int H, int k, int n_rows, int dtype,
                void* out, void* combined, void* stream);

/* moe_combine_rmsnorm -- moe_combine (combined = NULL) followed by the
 * RMSNorm of each output row, in one launch: xn[t] = out[t] /
 * sqrt(mean(out[t]^2) + eps) (* gain), normalised from the stored (rounded)
 * out row, with the same bits as moe_combine then moe_rmsnorm.  For the
 * block that follows a combine and starts with a norm: the next layer's
 * attention (the MoE layers and attention of the decoder: jina.ai/ko model
 * card, architecture paragraph; pre-norm blocks).  Arguments as moe_combine,
 * plus gain [H] fp32 or NULL and xn [T, H] dtype (16-byte aligned, distinct
 * from out and residual; MOE_ERR_SHAPE otherwise).  out == residual is
 * allowed.  Limits: H % 8 == 0, H <= 2048, 0 <= k <= 64. */
int moe_combine_rmsnorm(const void* y, const int32_t* inv, const float* topk_w,
                        const void* y_shared, int S, const void* residual,
                        int T, int H, int k, int n_rows, const float* gain, float eps,
                        int dtype, void* out, void* xn, void* stream);

/* ---------------------------------------------------------------------------
 * moe_rmsnorm -- RMSNorm of rows: out[t] = x[r] / sqrt(mean(x[r]^2) + eps)
 * (* gain), r = rows[t] (a gather, e.g. of token embeddings; clamped into
 * [0, x_rows), MOE_DATA_ERR_ROW_INDEX) or t when rows is NULL.  The scale is fp64 with one rounding
 * to the storage type, in the same order as moe_route's norm, so a row
 * normalises to the same bits in both.  Used for the inputs of the draft
 * block ("Jina AI's 3.4B OCR model targets faster page parsing", section
 * "FastMTP cuts decoding work": one dense block applied recursively).
 *
 * x     [x_rows, H] dtype          in
 * rows  [T] int32 or NULL          in
 * gain  [H] fp32 or NULL           in
 * out   rows of H at stride out_stride elements (>= H; a multiple of 16 bytes)  out
 * Limits: H % 8 == 0, H <= 8192.
 * ------------------------------------------------------------------------- */
int moe_rmsnorm(const void* x, const int32_t* rows, int x_rows, int T, int H, const float* gain,
                float eps, int dtype, void* out, int out_stride, void* stream);

/* ---------------------------------------------------------------------------
 * moe_combine_route -- the end of one MoE block fused with the start of the
 * next: moe_combine of the previous layer in place on the hidden state,
 *   h[t] = h[t] + sum_j topk_w_prev[t,j] y[inv[t,j]] + sum_s y_shared[s*T+t]
 * (the same fixed-order fp32 sums and rounding as moe_combine), then
 * moe_route on the new h (RMSNorm, logits, top-k, weights), as the two calls
 * would compute them, bit for bit.  Each token's previous routing weights
 * are read before its new ones are written, so topk_w may alias
 * topk_w_prev; inv must not alias topk_ids.  Arguments as in moe_combine
 * (k_prev, n_rows, y, inv, y_shared, S) and moe_route (the rest); h is the
 * residual in and the combined hidden state out.  Batches of 4,096 tokens
 * or more run the combine as a launch of its own.
 * ------------------------------------------------------------------------- */
int moe_combine_route(const void* y, const int32_t* inv, const float* topk_w_prev,
                      const void* y_shared, int S, int n_rows, int k_prev, void* h, int T, int H,
                      const float* gain, float eps, const float* w_router, const float* bias,
                      int E, int k, int flags, int dtype, void* xn, int32_t* topk_ids,
                      float* topk_w, float* logits, void* stream);

/* ---------------------------------------------------------------------------
 * lmhead_argmax -- greedy next token of every row: argmax_v (h W_lm^T)[v].
 *
 * The logits (vocabulary 129,280: jina.ai/ko model card, architecture
 * paragraph) are never written out; each row gets the index of its largest
 * fp32 logit, equal logits going to the lowest index, and that logit.
 *
 * h          [T,H] dtype       in
 * w_lm       [V,H] dtype       in  MOE_BF16: packed (MOE_PACK_ROWS, G = 1, N = V)
 * argmax_ids [T] int32         out
 * max_logit  [T] fp32 or NULL  out
 * ws         scratch of at least lmhead_argmax_workspace_bytes() bytes
 * Limits: H % 32 == 0 (MOE_BF16) or H % 4 == 0 (MOE_F32); 1 <= V < 2^31.
 * ------------------------------------------------------------------------- */
size_t lmhead_argmax_workspace_bytes(int T, int V, int dtype);
int lmhead_argmax(const void* h, const void* w_lm, int T, int H, int V, int dtype,
                  int32_t* argmax_ids, float* max_logit,
                  void* ws, size_t ws_bytes, void* stream);

/* lmhead_argmax_noalloc -- lmhead_argmax for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid allocation.  Same kernels and results, bit for bit;
 * the workspace is a static device array of the library instead of `ws`.
 *
 * Each GPU holds its own copy of that array (MOE_NOALLOC_SCRATCH_BYTES) until
 * the process ends.  Its device address is looked up on the first call on a
 * device (the stream's device; hipGetSymbolAddress with that device current)
 * and cached.  Calls that overlap on one GPU (several streams or host
 * threads) share the array and race: serialise them.  Nothing is allocated,
 * freed or cleared.
 *
 * Arguments as lmhead_argmax without ws / ws_bytes.  Errors as
 * lmhead_argmax, plus MOE_ERR_WORKSPACE when
 * lmhead_argmax_workspace_bytes(T, V, dtype) > MOE_NOALLOC_SCRATCH_BYTES
 * (e.g. more than 519 rows at V = 129,280 in bf16), and MOE_ERR_HIP if the
 * array's address cannot be looked up or the launch fails. */
#define MOE_NOALLOC_SCRATCH_BYTES (4u << 20)
int lmhead_argmax_noalloc(const void* h, const void* w_lm, int T, int H, int V, int dtype,
                          int32_t* argmax_ids, float* max_logit, void* stream);

/* ---------------------------------------------------------------------------
 * spec_verify -- greedy longest-prefix acceptance plus the bonus token.
 *
 * Sequence b verified K+1 positions: its last committed token and K drafts.
 * argmax_ids[b,i] is the verifier's greedy token after position i, so
 * draft i is accepted while drafts[b,i'] == argmax_ids[b,i'] for every
 * i' <= i.  With n accepted drafts the step commits drafts[b,0..n-1] and
 * argmax_ids[b,n]: n+1 tokens, at most K+1 (jina.ai/de page, sections
 * "Modell und Training" and "Spekulatives Decoding auf einer L4").  K = 0
 * is plain greedy decoding.  A draft id outside the vocabulary is simply a
 * mismatch.
 *
 * drafts     [B,K] int32     in
 * argmax_ids [B,K+1] int32   in
 * accepted   [B] int32       out  n
 * committed  [B,K+1] int32   out  committed tokens, -1 padded
 * n_commit   [B] int32       out  n+1
 * Limits: 0 <= K <= 15.
 * ------------------------------------------------------------------------- */
int spec_verify(const int32_t* drafts, const int32_t* argmax_ids, int B, int K,
                int32_t* accepted, int32_t* committed, int32_t* n_commit,
                void* stream);

/* ---------------------------------------------------------------------------
 * spec_plant_drafts -- benchmark-harness stand-in for a draft head (not part
 * of the verify step).  Draft i of sequence b is argmax_ids[b,i] when
 * keep[b,i] != 0, else u + (u >= argmax_ids[b,i]) with u = repl[b,i] in
 * [0, V-1): a uniform draw over the other V-1 ids, so it never matches.
 *
 * argmax_ids [B,K+1] int32, keep [B,K] uint8, repl [B,K] int32   in
 * drafts     [B,K] int32                                          out
 * ------------------------------------------------------------------------- */
int spec_plant_drafts(const int32_t* argmax_ids, const uint8_t* keep, const int32_t* repl,
                      int B, int K, int V, int32_t* drafts, void* stream);

/* ---------------------------------------------------------------------------
 * Decode loop over a shrinking batch (the concurrency-32 document workload:
 * 32 pages decoded together, about 1,085 output tokens each -- alphasignal
 * page "Jina AI's 3.4B OCR model targets faster page parsing", section
 * "Quality and speed").  A pass verifies the B active sequences; afterwards
 * spec_advance appends each one's committed tokens to its stream, stops a
 * sequence at `target` tokens (the excess of its last pass is dropped) and
 * compacts the still-active sequence ids in their order.  The caller reads
 * n_active (one 4-byte copy per pass) to size a later pass; a pass may be
 * launched before that copy arrives, with the previous batch size: the slots
 * past n_active hold -1 and every call skips them.
 *
 * spec_advance:
 *   n_commit  [B] int32, committed [B,K+1] int32   in  (spec_verify's outputs)
 *   seq_ids   [B] int32                            in  sequence of each slot, in [0,S);
 *                                                      a negative id is an empty slot (skipped);
 *                                                      ids >= S and n_commit outside [0,K+1] are
 *                                                      clamped (MOE_DATA_ERR_SEQUENCE)
 *   total     [S] int32                            in/out tokens committed so far
 *   steps     [S] int32                            in/out passes taken so far
 *   tokens    [S,target] int32                     out committed streams
 *   seq_ids_out [B] int32                          out active sequences, in slot order,
 *                                                      then -1 up to slot B-1
 *   n_active  [1] int32                            out number of them
 *   Limits: 0 <= B <= min(S, 1024), 0 <= K <= 15, target >= 1.  The ids in
 *   seq_ids are distinct; seq_ids_out must not alias seq_ids.  B = 0 writes
 *   n_active = 0.
 *
 * spec_gather_rows: the per-pass inputs of the active sequences from pools
 * laid out [S, J, R] rows of row_bytes bytes (J passes per sequence, R rows
 * per pass):  out row i*R + r = pool row (seq_ids[i] * J + min(steps[s], J-1))
 * * R + r, with s = seq_ids[i] (an empty slot, id < 0, reads sequence 0's
 * row: its pass result is skipped; an id >= S is clamped to S-1 and reported,
 * MOE_DATA_ERR_SEQUENCE).  Used for the hidden states of the verify
 * positions (R = K+1 rows of H bf16) and the planting draws (R = 1 row of K
 * bytes or K int32).  row_bytes = 0 (K = 0 drafts) is a no-op.
 * ------------------------------------------------------------------------- */
int spec_advance(const int32_t* n_commit, const int32_t* committed, const int32_t* seq_ids,
                 int B, int K, int S, int target, int32_t* total, int32_t* steps,
                 int32_t* tokens, int32_t* seq_ids_out, int32_t* n_active, void* stream);
int spec_gather_rows(const void* pool, const int32_t* seq_ids, const int32_t* steps, int B,
                     int R, int J, int S, int row_bytes, void* out, void* stream);

/* ---------------------------------------------------------------------------
 * Causal self-attention of the verify positions over a per-sequence KV cache.
 *
 * The pages give the decoder's context limit (32,768 positions; jina.ai/ko
 * model card "jina-ocr-v1", architecture paragraph) but not its attention;
 * these calls read it as plain multi-head attention with head size 128 and
 * rotary positions (rotate-half form, angle pos * base^(-j/64), j < 64).
 * A verify pass of sequence b holds P = K+1 positions at L_b .. L_b+P-1,
 * L_b = lengths[b] (its last committed token, then the drafts); tokens are
 * laid out [B*P] sequence-major, H = n_heads * 128.  The cache holds k and v
 * interleaved per position: kv [B, n_heads, max_len, 2, 128] bf16, [..][0][..]
 * the rotated key, [..][1][..] the value (one 512-byte row per position, so
 * a span of positions is one contiguous stream).
 *
 * moe_attn_rope_cache: q, k, v = split(qkv) (columns [0,H), [H,2H), [2H,3H));
 *   q <- rope(q), written to q [B*P, H]; rope(k) and v are written into the
 *   cache at [b][head][L_b + i][0] and [1].  Rotation in fp64 from the stored
 *   bf16 inputs, one rounding to bf16.
 *   qkv [B*P, 3H] bf16                          in
 *   lengths [B] int32                           in   clamped to [0, max_len-P]
 *                                                    (MOE_DATA_ERR_LENGTH)
 *   q [B*P, H] bf16                             out
 *   kv [B, n_heads, max_len, 2, 128] bf16       in/out (P positions each)
 *
 * moe_attention: o_i = sum_{j <= L_b+i} softmax_j(q_i . k_j / sqrt(128)) v_j
 *   per head, over the cached keys (split over the key axis; fp32 scores,
 *   online softmax, fp32 merge of the splits, one rounding to bf16).
 *   Cache rows past L_b + i (drafts of an earlier pass that the verifier
 *   rejected) are never read, so rejecting drafts needs no cache write.
 *   max_keys bounds lengths[b] + P for every b (it sizes the grid and the
 *   workspace; a longer length is clamped to max_keys - P and reported,
 *   MOE_DATA_ERR_LENGTH).
 *   q [B*P, H] bf16, kv as above                in
 *   o [B*P, H] bf16                             out
 *   ws                                          scratch of
 *                                               moe_attention_workspace_bytes(B, P, n_heads, 128, max_keys)
 *
 * spec_commit: lengths[b] += n_commit[b] (spec_verify's output): the accepted
 *   drafts and the bonus token's predecessor become the committed prefix; the
 *   rest of the pass's cache rows are overwritten by the next pass.
 *
 * Limits: dtype MOE_BF16, head_dim 128, 1 <= P <= 16, P <= max_keys <=
 * max_len; the cache pointer 16-byte aligned.
 * ------------------------------------------------------------------------- */
int moe_attn_rope_cache(const void* qkv, const int32_t* lengths, int B, int P, int n_heads,
                        int head_dim, float rope_base, int max_len, int dtype, void* q,
                        void* kv_cache, void* stream);
size_t moe_attention_workspace_bytes(int B, int P, int n_heads, int head_dim, int max_keys);
int moe_attention(const void* q, const void* kv_cache, const int32_t* lengths, int B, int P,
                  int n_heads, int head_dim, int max_len, int max_keys, int dtype, void* o,
                  void* ws, size_t ws_bytes, void* stream);
int spec_commit(const int32_t* n_commit, int B, int32_t* lengths, void* stream);

/* ---------------------------------------------------------------------------
 * moe_data_errors -- device-side data errors seen since the last clear.
 *
 * The kernels clamp every index argument before it addresses memory; an
 * argument that needed clamping is a caller mistake, and the kernel that saw
 * it ORs its kind into a 32-bit word that each GPU holds for the library
 * (a static device variable; its address is looked up once per device and
 * cached).  The clamped call still completes and its outputs are those of
 * the clamped data.  Bits:
 *   MOE_DATA_ERR_EXPERT_ID  topk_ids entry outside [0, E)
 *                           (moe_permute, moe_expert_gate_up_routed)
 *   MOE_DATA_ERR_ROW_INDEX  gather / rows entry outside [0, T) or
 *                           [0, x_rows) (moe_grouped_swiglu,
 *                           moe_expert_gate_up, moe_rmsnorm)
 *   MOE_DATA_ERR_OFFSETS    offsets outside [0, n_rows] or decreasing, or an
 *                           identity-gathered group longer than T (the
 *                           expert FFN calls)
 *   MOE_DATA_ERR_INV        inv entry outside [0, n_rows) (moe_combine,
 *                           moe_combine_rmsnorm, moe_combine_route)
 *   MOE_DATA_ERR_LENGTH     lengths entry outside [0, max_len - P]
 *                           (moe_attn_rope_cache) or [0, max_keys - P]
 *                           (moe_attention)
 *   MOE_DATA_ERR_SEQUENCE   seq_ids entry >= S, or n_commit outside
 *                           [0, K+1] (spec_advance, spec_gather_rows)
 * A draft id outside the vocabulary is no error (a mismatch, spec_verify).
 *
 * Enqueues one single-thread kernel on `stream` that writes the word to
 * flags_out (device memory, 4-byte aligned) and, with clear != 0, clears the
 * bits it read.  Calls on one stream see the errors of every earlier call on
 * it; a call on another stream of the same GPU may set bits at any time
 * (the word is per GPU).  Returns MOE_ERR_NULL / MOE_ERR_ALIGN for a bad
 * flags_out, MOE_ERR_HIP if the word's address cannot be looked up or the
 * launch fails.
 * ------------------------------------------------------------------------- */
#define MOE_DATA_ERR_EXPERT_ID 1u
#define MOE_DATA_ERR_ROW_INDEX 2u
#define MOE_DATA_ERR_OFFSETS 4u
#define MOE_DATA_ERR_INV 8u
#define MOE_DATA_ERR_LENGTH 16u
#define MOE_DATA_ERR_SEQUENCE 32u
int moe_data_errors(uint32_t* flags_out, int clear, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOESTEP_H */
