/*
 * A plain C client of libmoestep: one verify pass of an MoE decoder layer
 * through the C ABI alone (include/moestep.h), with HIP's C runtime API for
 * device memory.  No Python, no torch.
 *
 *   verify_pass host
 *       host-side checks only (no GPU needed): version, status strings, the
 *       documented error codes of bad arguments; exit status 0 if all hold.
 *   verify_pass run DIR f32|bf16 T H E S k I V B K
 *       reads DIR/{h,w_router,w_gate_up,w_down,w_lm}.bin (row-major, the
 *       storage dtype; w_router fp32) and DIR/drafts.bin (int32 [B,K]), runs
 *         moe_pack_weights (bf16) -> moe_route -> moe_permute ->
 *         moe_grouped_swiglu -> moe_combine -> lmhead_argmax -> spec_verify
 *       and writes DIR/{xn,ids,topk_w,h_out,argmax,accepted,committed,
 *       n_commit,errors}.bin (h_out and xn in the storage dtype).
 * Exit status: 0 on success, 1 on a failed call (its name and status are
 * printed), 2 on bad usage or I/O.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "moestep.h"

static int fail(const char* what, int st) {
  fprintf(stderr, "%s: status %d (%s)\n", what, st, moe_status_str(st));
  return 1;
}

#define CALL(x)                      \
  do {                               \
    int st_ = (x);                   \
    if (st_ != MOE_OK) return fail(#x, st_); \
  } while (0)

#define HIP(x)                                                  \
  do {                                                          \
    hipError_t e_ = (x);                                        \
    if (e_ != hipSuccess) {                                     \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));   \
      return 1;                                                 \
    }                                                           \
  } while (0)

static int expect(const char* what, int got, int want) {
  if (got == want) return 0;
  fprintf(stderr, "%s: got status %d, expected %d\n", what, got, want);
  return 1;
}

static int host_checks(void) {
  int bad = 0;
  void* A = (void*)(uintptr_t)0x100000;   /* aligned, never dereferenced */
  void* MIS = (void*)(uintptr_t)0x100004; /* misaligned */
  bad |= expect("moe_abi_version", moe_abi_version(), MOE_ABI_VERSION);
  bad |= strcmp(moe_status_str(MOE_OK), moe_status_str(MOE_ERR_NULL)) == 0;
  bad |= expect("moe_route(h = NULL)",
                moe_route(NULL, NULL, 1e-6f, (const float*)A, NULL, 4, 128, 8, 2, 3, MOE_F32, A, (int32_t*)A,
                          (float*)A, NULL, NULL), MOE_ERR_NULL);
  bad |= expect("moe_route(k > E)",
                moe_route(A, NULL, 1e-6f, (const float*)A, NULL, 4, 128, 8, 9, 3, MOE_F32, A, (int32_t*)A,
                          (float*)A, NULL, NULL), MOE_ERR_SHAPE);
  bad |= expect("moe_route(E = 65)",
                moe_route(A, NULL, 1e-6f, (const float*)A, NULL, 4, 128, 65, 2, 3, MOE_F32, A, (int32_t*)A,
                          (float*)A, NULL, NULL), MOE_ERR_UNSUPPORTED);
  bad |= expect("moe_route(misaligned h)",
                moe_route(MIS, NULL, 1e-6f, (const float*)A, NULL, 4, 128, 8, 2, 3, MOE_F32, A, (int32_t*)A,
                          (float*)A, NULL, NULL), MOE_ERR_ALIGN);
  bad |= expect("moe_route(T = 0)",
                moe_route(NULL, NULL, 1e-6f, NULL, NULL, 0, 128, 8, 2, 3, MOE_F32, NULL, NULL, NULL, NULL, NULL),
                MOE_OK);
  bad |= expect("spec_verify(K = 16)",
                spec_verify((const int32_t*)A, (const int32_t*)A, 4, 16, (int32_t*)A, (int32_t*)A, (int32_t*)A,
                            NULL), MOE_ERR_UNSUPPORTED);
  bad |= expect("moe_data_errors(NULL)", moe_data_errors(NULL, 1, NULL), MOE_ERR_NULL);
  bad |= expect("lmhead_argmax(small workspace)",
                lmhead_argmax(A, A, 4, 128, 512, MOE_F32, (int32_t*)A, NULL, A,
                              lmhead_argmax_workspace_bytes(4, 512, MOE_F32) - 1, NULL), MOE_ERR_WORKSPACE);
  if (!bad) printf("host checks ok\n");
  return bad;
}

static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s.bin", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return NULL;
  void* p = malloc(bytes ? bytes : 1);
  size_t n = p ? fread(p, 1, bytes, f) : 0;
  fclose(f);
  if (n != bytes) {
    free(p);
    return NULL;
  }
  return p;
}

static int write_file(const char* dir, const char* name, const void* p, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s.bin", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f) return 2;
  size_t n = fwrite(p, 1, bytes, f);
  fclose(f);
  return n == bytes ? 0 : 2;
}

/* a device copy of DIR/name.bin */
static void* upload(const char* dir, const char* name, size_t bytes) {
  void* h = read_file(dir, name, bytes);
  void* d = NULL;
  if (!h) return NULL;
  if (hipMalloc(&d, bytes) != hipSuccess || hipMemcpy(d, h, bytes, hipMemcpyHostToDevice) != hipSuccess) d = NULL;
  free(h);
  return d;
}

/* device -> DIR/name.bin */
static int download(const char* dir, const char* name, const void* d, size_t bytes) {
  void* h = malloc(bytes);
  int r = 2;
  if (h && hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost) == hipSuccess) r = write_file(dir, name, h, bytes);
  free(h);
  return r;
}

static void* dalloc(size_t bytes) {
  void* d = NULL;
  return hipMalloc(&d, bytes ? bytes : 16) == hipSuccess ? d : NULL;
}

/* bf16 weights in the layout the streaming kernels read */
static void* packed(const void* src, int G, int N, int K, int kind) {
  void* dst = dalloc(moe_packed_weights_bytes(G, N, K, kind));
  if (!dst || moe_pack_weights(src, dst, G, N, K, kind, MOE_BF16, NULL) != MOE_OK) return NULL;
  return dst;
}

static int run(int argc, char** argv) {
  if (argc != 13) return 2;
  const char* dir = argv[2];
  const int bf16 = strcmp(argv[3], "bf16") == 0;
  const int T = atoi(argv[4]), H = atoi(argv[5]), E = atoi(argv[6]), S = atoi(argv[7]), k = atoi(argv[8]);
  const int I = atoi(argv[9]), V = atoi(argv[10]), B = atoi(argv[11]), K = atoi(argv[12]);
  const int dt = bf16 ? MOE_BF16 : MOE_F32;
  const size_t es = bf16 ? 2 : 4;
  const int G = E + S, n_routed = T * k, n_rows = T * k + S * T;
  if (T != B * (K + 1)) return 2;

  void* h = upload(dir, "h", (size_t)T * H * es);
  float* w_router = upload(dir, "w_router", (size_t)E * H * 4);
  void* w_gu = upload(dir, "w_gate_up", (size_t)G * 2 * I * H * es);
  void* w_dn = upload(dir, "w_down", (size_t)G * H * I * es);
  void* w_lm = upload(dir, "w_lm", (size_t)V * H * es);
  int32_t* drafts = upload(dir, "drafts", (size_t)B * K * 4);
  if (!h || !w_router || !w_gu || !w_dn || !w_lm || (K > 0 && !drafts)) return 2;
  if (bf16) {  /* expert and LM-head weights, packed once */
    w_gu = packed(w_gu, G, I, H, MOE_PACK_GATE_UP);
    w_dn = packed(w_dn, G, H, I, MOE_PACK_ROWS);
    w_lm = packed(w_lm, 1, V, H, MOE_PACK_ROWS);
    if (!w_gu || !w_dn || !w_lm) return fail("moe_pack_weights", MOE_ERR_HIP);
  }

  void* xn = dalloc((size_t)T * H * es);
  int32_t* ids = dalloc((size_t)T * k * 4);
  float* tw = dalloc((size_t)T * k * 4);
  int32_t* offsets = dalloc((size_t)(G + 1) * 4);
  int32_t* gather = dalloc((size_t)n_rows * 4);
  int32_t* inv = dalloc((size_t)T * k * 4);
  void* y = dalloc((size_t)n_rows * H * es);
  void* h_out = dalloc((size_t)T * H * es);
  int32_t* am = dalloc((size_t)T * 4);
  int32_t* acc = dalloc((size_t)B * 4);
  int32_t* com = dalloc((size_t)B * (K + 1) * 4);
  int32_t* nc = dalloc((size_t)B * 4);
  uint32_t* errs = dalloc(4);
  const size_t ws_p = moe_permute_workspace_bytes(T, k, E);
  const size_t ws_s = moe_grouped_swiglu_workspace_bytes(n_rows, I, dt);
  const size_t ws_l = lmhead_argmax_workspace_bytes(T, V, dt);
  void* ws_perm = ws_p ? dalloc(ws_p) : NULL;
  void* ws_ffn = dalloc(ws_s);
  void* ws_lm = dalloc(ws_l);
  if (!xn || !ids || !tw || !offsets || !gather || !inv || !y || !h_out || !am || !acc || !com || !nc || !errs ||
      (ws_p && !ws_perm) || !ws_ffn || !ws_lm)
    return fail("hipMalloc", MOE_ERR_HIP);

  CALL(moe_data_errors(errs, 1, NULL));   /* start from a clear word */
  CALL(moe_route(h, NULL, 1e-6f, w_router, NULL, T, H, E, k, MOE_ROUTE_NORM | MOE_ROUTE_RENORM, dt, xn, ids, tw,
                 NULL, NULL));
  CALL(moe_permute(ids, T, k, E, S, offsets, gather, inv, ws_perm, ws_p, NULL));
  CALL(moe_grouped_swiglu(xn, gather, offsets, G, n_rows, w_gu, w_dn, T, H, I, T, dt, y, ws_ffn, ws_s, NULL));
  CALL(moe_combine(y, inv, tw, (const char*)y + (size_t)n_routed * H * es, S, h, T, H, k, n_routed, dt, h_out,
                   NULL, NULL));
  CALL(lmhead_argmax(h_out, w_lm, T, H, V, dt, am, NULL, ws_lm, ws_l, NULL));
  CALL(spec_verify(drafts, am, B, K, acc, com, nc, NULL));
  CALL(moe_data_errors(errs, 0, NULL));
  HIP(hipDeviceSynchronize());

  int r = 0;
  r |= download(dir, "xn", xn, (size_t)T * H * es);
  r |= download(dir, "ids", ids, (size_t)T * k * 4);
  r |= download(dir, "topk_w", tw, (size_t)T * k * 4);
  r |= download(dir, "h_out", h_out, (size_t)T * H * es);
  r |= download(dir, "argmax", am, (size_t)T * 4);
  r |= download(dir, "accepted", acc, (size_t)B * 4);
  r |= download(dir, "committed", com, (size_t)B * (K + 1) * 4);
  r |= download(dir, "n_commit", nc, (size_t)B * 4);
  r |= download(dir, "errors", errs, 4);
  if (r) return 2;
  printf("verify pass ok: %d tokens, %d sequences\n", T, B);
  return 0;
}

int main(int argc, char** argv) {
  if (argc >= 2 && strcmp(argv[1], "host") == 0) return host_checks();
  if (argc >= 2 && strcmp(argv[1], "run") == 0) {
    int r = run(argc, argv);
    if (r == 2) fprintf(stderr, "usage: verify_pass run DIR f32|bf16 T H E S k I V B K (inputs readable)\n");
    return r;
  }
  fprintf(stderr, "usage: verify_pass host | run DIR f32|bf16 T H E S k I V B K\n");
  return 2;
}
