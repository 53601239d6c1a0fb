"""Python names of the C-ABI calls, taking torch tensors.

Argument marshalling only: every wrapper checks dtypes and devices, passes
data pointers and the current HIP stream to libmoestep, and raises MoeError on
a non-zero status.  Output tensors are passed in by the caller (the `*_alloc`
helpers allocate them with torch first, for tests and one-off calls).
"""

from __future__ import annotations

import ctypes

import torch

from . import _lib as L

__all__ = [
    "Packed", "pack_weights", "packed_weights_bytes", "moe_route", "moe_rmsnorm", "moe_combine_route", "moe_permute", "moe_grouped_swiglu", "moe_combine", "moe_combine_rmsnorm", "lmhead_argmax",
    "moe_expert_gate_up", "moe_expert_gate_up_routed", "moe_expert_down", "moe_expert_down_residual", "ROUTED_MAX_PAIRS", "spec_verify", "spec_plant_drafts", "spec_advance",
    "spec_gather_rows", "moe_data_errors", "data_errors", "moe_attn_rope_cache", "moe_attention", "attention_workspace_bytes", "kv_cache_alloc", "spec_commit",
    "permute_workspace_bytes", "swiglu_workspace_bytes",
    "lmhead_workspace_bytes", "lmhead_argmax_noalloc", "dtype_code", "expert_weights", "lm_weights", "router_weights", "route_alloc", "permute_alloc", "swiglu_alloc",
    "combine_alloc", "lmhead_alloc", "verify_alloc",
]


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return L.BF16
    if t.dtype == torch.float32:
        return L.F32
    raise TypeError(f"unsupported storage dtype {t.dtype}")


def _need(t, dtype, name):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class Packed:
    """Weights in the layout the streaming kernels read (moe_pack_weights):
    bf16 expert / LM-head fragments, or the fp32 router layout.  `shape` is
    the logical row-major shape."""

    def __init__(self, data: torch.Tensor, shape, kind: int):
        self.data = data
        self.shape = tuple(int(v) for v in shape)
        self.kind = kind
        self.dtype = data.dtype
        self.device = data.device
        self.is_cuda = data.is_cuda

    def data_ptr(self) -> int:
        return self.data.data_ptr()

    def is_contiguous(self) -> bool:
        return True


def packed_weights_bytes(G: int, N: int, K: int, kind: int) -> int:
    return int(L.load().moe_packed_weights_bytes(G, N, K, kind))


def pack_weights(w: torch.Tensor, kind: int) -> Packed:
    """Pack row-major bf16 weights: [G, 2N, K] (gate/up, kind PACK_GATE_UP),
    [G, N, K] or [N, K] (kind PACK_ROWS)."""
    _need(w, torch.bfloat16, "w")
    shape = tuple(w.shape)
    G, R, K = (1, *shape) if w.dim() == 2 else shape
    N = R // 2 if kind == L.PACK_GATE_UP else R
    nbytes = packed_weights_bytes(G, N, K, kind)
    out = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=w.device)
    L.check("moe_pack_weights", L.load().moe_pack_weights(
        _p(w), _p(out), G, N, K, kind, L.BF16, _stream(w)))
    return Packed(out, shape, kind)


def router_weights(w_router: torch.Tensor) -> Packed:
    """Pack an fp32 router weight [E, H] (E <= 64) for moe_route."""
    _need(w_router, torch.float32, "w_router")
    E, H = w_router.shape
    nbytes = packed_weights_bytes(1, E, H, L.PACK_ROUTER)
    out = torch.empty(nbytes // 4, dtype=torch.float32, device=w_router.device)
    L.check("moe_pack_weights", L.load().moe_pack_weights(
        _p(w_router), _p(out), 1, E, H, L.PACK_ROUTER, L.F32, _stream(w_router)))
    return Packed(out, (E, H), L.PACK_ROUTER)


def expert_weights(w_gate_up: torch.Tensor, w_down: torch.Tensor):
    """The weights the grouped SwiGLU reads: packed for bf16, as they are for fp32."""
    if w_gate_up.dtype == torch.bfloat16:
        return pack_weights(w_gate_up, L.PACK_GATE_UP), pack_weights(w_down, L.PACK_ROWS)
    return w_gate_up, w_down


def lm_weights(w_lm: torch.Tensor):
    """The LM-head weight lmhead_argmax reads: packed for bf16, as it is for fp32."""
    return pack_weights(w_lm, L.PACK_ROWS) if w_lm.dtype == torch.bfloat16 else w_lm


def permute_workspace_bytes(T: int, k: int, E: int) -> int:
    return int(L.load().moe_permute_workspace_bytes(T, k, E))


def swiglu_workspace_bytes(n_rows: int, I: int, dtype: torch.dtype) -> int:
    return int(L.load().moe_grouped_swiglu_workspace_bytes(n_rows, I, L.BF16 if dtype == torch.bfloat16 else L.F32))


def lmhead_workspace_bytes(T: int, V: int, dtype: torch.dtype) -> int:
    return int(L.load().lmhead_argmax_workspace_bytes(T, V, L.BF16 if dtype == torch.bfloat16 else L.F32))


def moe_route(h, w_router, bias, k, xn, topk_ids, topk_w, logits=None, gain=None, eps=1e-6,
              norm=True, renormalize=True):
    """RMSNorm + router logits + top-k + routing weights (see moe_route in moestep.h).
    `w_router` is the fp32 [E, H] weight, row-major or packed (router_weights)."""
    T, H = h.shape
    E = w_router.shape[0]
    packed = isinstance(w_router, Packed)
    if packed and w_router.kind != L.PACK_ROUTER:
        raise TypeError("w_router must be packed with router_weights")
    for t, d, n in ((h, None, "h"), (xn, h.dtype, "xn"), (w_router, torch.float32, "w_router"),
                    (bias, torch.float32, "bias"), (gain, torch.float32, "gain"),
                    (topk_ids, torch.int32, "topk_ids"), (topk_w, torch.float32, "topk_w"),
                    (logits, torch.float32, "logits")):
        _need(t, d, n)
    flags = ((L.ROUTE_NORM if norm else 0) | (L.ROUTE_RENORM if renormalize else 0)
             | (L.ROUTE_WPACKED if packed else 0))
    L.check("moe_route", L.load().moe_route(
        _p(h), _p(gain), float(eps), _p(w_router), _p(bias), T, H, E, k, flags, dtype_code(h),
        _p(xn), _p(topk_ids), _p(topk_w), _p(logits), _stream(h)))


def moe_rmsnorm(x, out, rows=None, gain=None, eps=1e-6):
    """out[t] = RMSNorm(x[rows[t]] or x[t]); `out` may be a strided view of
    rows (e.g. one half of a [T, 2H] buffer)."""
    x_rows, H = x.shape
    T = out.shape[0]
    if out.stride(1) != 1:
        raise ValueError("out rows must be contiguous")
    for t, d, n in ((x, None, "x"), (rows, torch.int32, "rows"), (gain, torch.float32, "gain")):
        _need(t, d, n)
    if out.dtype != x.dtype or not out.is_cuda:
        raise TypeError("out must be a device tensor of x's dtype")
    L.check("moe_rmsnorm", L.load().moe_rmsnorm(
        _p(x), _p(rows), x_rows, T, H, _p(gain), float(eps), dtype_code(x), _p(out), out.stride(0), _stream(x)))


def moe_combine_route(y, inv, topk_w_prev, y_shared, S, h, w_router, bias, k, xn, topk_ids, topk_w,
                      logits=None, gain=None, eps=1e-6, norm=True, renormalize=True):
    """The previous layer's moe_combine in place on h, then moe_route on it (one launch)."""
    T, H = h.shape
    E = w_router.shape[0]
    k_prev = topk_w_prev.shape[1]
    packed = isinstance(w_router, Packed)
    if packed and w_router.kind != L.PACK_ROUTER:
        raise TypeError("w_router must be packed with router_weights")
    for t, d, n in ((y, h.dtype, "y"), (inv, torch.int32, "inv"), (topk_w_prev, torch.float32, "topk_w_prev"),
                    (y_shared, h.dtype, "y_shared"), (h, None, "h"), (xn, h.dtype, "xn"),
                    (w_router, torch.float32, "w_router"), (bias, torch.float32, "bias"),
                    (gain, torch.float32, "gain"), (topk_ids, torch.int32, "topk_ids"),
                    (topk_w, torch.float32, "topk_w"), (logits, torch.float32, "logits")):
        _need(t, d, n)
    flags = ((L.ROUTE_NORM if norm else 0) | (L.ROUTE_RENORM if renormalize else 0)
             | (L.ROUTE_WPACKED if packed else 0))
    L.check("moe_combine_route", L.load().moe_combine_route(
        _p(y), _p(inv), _p(topk_w_prev), _p(y_shared), S, y.shape[0], k_prev, _p(h), T, H, _p(gain), float(eps),
        _p(w_router), _p(bias), E, k, flags, dtype_code(h), _p(xn), _p(topk_ids), _p(topk_w), _p(logits),
        _stream(h)))


def moe_permute(topk_ids, E, S, offsets, gather, inv, ws=None):
    """Stable counting sort of the (token, slot) pairs by expert (+ shared groups)."""
    T, k = topk_ids.shape
    for t, n in ((topk_ids, "topk_ids"), (offsets, "offsets"), (gather, "gather"), (inv, "inv")):
        _need(t, torch.int32, n)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    L.check("moe_permute", L.load().moe_permute(
        _p(topk_ids), T, k, E, S, _p(offsets), _p(gather), _p(inv), _p(ws), nbytes, _stream(topk_ids)))


def moe_grouped_swiglu(x, gather, offsets, w_gate_up, w_down, y, ws, max_rows=None):
    """SwiGLU expert FFN over the rows of each group (routed and shared alike)."""
    T, H = x.shape
    G, I2, _ = w_gate_up.shape
    n_rows = y.shape[0]
    if x.dtype == torch.bfloat16 and not (isinstance(w_gate_up, Packed) and w_gate_up.kind == L.PACK_GATE_UP
                                          and isinstance(w_down, Packed) and w_down.kind == L.PACK_ROWS):
        raise TypeError("bf16 expert weights must be packed (expert_weights / pack_weights)")
    for t, d, n in ((x, None, "x"), (gather, torch.int32, "gather"), (offsets, torch.int32, "offsets"),
                    (w_gate_up, x.dtype, "w_gate_up"), (w_down, x.dtype, "w_down"), (y, x.dtype, "y"), (ws, None, "ws")):
        _need(t, d, n)
    L.check("moe_grouped_swiglu", L.load().moe_grouped_swiglu(
        _p(x), _p(gather), _p(offsets), G, n_rows, _p(w_gate_up), _p(w_down), T, H, I2 // 2,
        T if max_rows is None else int(max_rows), dtype_code(x), _p(y), _p(ws),
        ws.numel() * ws.element_size(), _stream(x)))


def moe_expert_gate_up(x, gather, offsets, w_gate_up, act, max_rows=None):
    """First half of the grouped SwiGLU: act[r] = silu(x W_g^T) * (x W_u^T) per group."""
    T, H = x.shape
    G, I2, _ = w_gate_up.shape
    n_rows = act.shape[0]
    if x.dtype == torch.bfloat16 and not (isinstance(w_gate_up, Packed) and w_gate_up.kind == L.PACK_GATE_UP):
        raise TypeError("bf16 expert weights must be packed (expert_weights / pack_weights)")
    for t, d, n in ((x, None, "x"), (gather, torch.int32, "gather"), (offsets, torch.int32, "offsets"),
                    (w_gate_up, x.dtype, "w_gate_up"), (act, x.dtype, "act")):
        _need(t, d, n)
    L.check("moe_expert_gate_up", L.load().moe_expert_gate_up(
        _p(x), _p(gather), _p(offsets), G, n_rows, _p(w_gate_up), T, H, I2 // 2,
        T if max_rows is None else int(max_rows), dtype_code(x), _p(act), _stream(x)))


ROUTED_MAX_PAIRS = 4096   # T*k up to which moe_expert_gate_up_routed runs


def moe_expert_gate_up_routed(x, topk_ids, E, S, w_gate_up, act, offsets, inv):
    """moe_permute + moe_expert_gate_up in one launch (decode-sized batches):
    writes act, offsets and inv as the two calls would (no gather list)."""
    T, H = x.shape
    k = topk_ids.shape[1]
    I = w_gate_up.shape[1] // 2
    if not (isinstance(w_gate_up, Packed) and w_gate_up.kind == L.PACK_GATE_UP):
        raise TypeError("bf16 expert weights must be packed (expert_weights / pack_weights)")
    for t, d, n in ((x, torch.bfloat16, "x"), (topk_ids, torch.int32, "topk_ids"), (act, torch.bfloat16, "act"),
                    (offsets, torch.int32, "offsets"), (inv, torch.int32, "inv")):
        _need(t, d, n)
    L.check("moe_expert_gate_up_routed", L.load().moe_expert_gate_up_routed(
        _p(x), _p(topk_ids), T, k, E, S, _p(w_gate_up), H, I, dtype_code(x), _p(act), _p(offsets), _p(inv),
        _stream(x)))


def moe_expert_down(act, offsets, w_down, y, max_rows=None):
    """Second half of the grouped SwiGLU: y[r] = act[r] W_d^T per group."""
    n_rows, I = act.shape
    G, H, _ = w_down.shape
    if act.dtype == torch.bfloat16 and not (isinstance(w_down, Packed) and w_down.kind == L.PACK_ROWS):
        raise TypeError("bf16 expert weights must be packed (expert_weights / pack_weights)")
    for t, d, n in ((act, None, "act"), (offsets, torch.int32, "offsets"), (w_down, act.dtype, "w_down"),
                    (y, act.dtype, "y")):
        _need(t, d, n)
    L.check("moe_expert_down", L.load().moe_expert_down(
        _p(act), _p(offsets), G, n_rows, _p(w_down), H, I, n_rows if max_rows is None else int(max_rows),
        dtype_code(act), _p(y), _stream(act)))


def moe_expert_down_residual(act, offsets, w_down, residual, y, max_rows=None):
    """y[r] = residual[r] + round(W_d act[r]) per group (y may be residual)."""
    n_rows, I = act.shape
    G, H, _ = w_down.shape
    if act.dtype == torch.bfloat16 and not (isinstance(w_down, Packed) and w_down.kind == L.PACK_ROWS):
        raise TypeError("bf16 expert weights must be packed (expert_weights / pack_weights)")
    for t, d, n in ((act, None, "act"), (offsets, torch.int32, "offsets"), (w_down, act.dtype, "w_down"),
                    (residual, act.dtype, "residual"), (y, act.dtype, "y")):
        _need(t, d, n)
    if residual is None:
        raise ValueError("residual is required")
    L.check("moe_expert_down_residual", L.load().moe_expert_down_residual(
        _p(act), _p(offsets), G, n_rows, _p(w_down), H, I, n_rows if max_rows is None else int(max_rows),
        dtype_code(act), _p(residual), _p(y), _stream(act)))


def moe_combine(y, inv, topk_w, y_shared, S, residual, out, combined=None):
    """out = residual + sum_j w_j y[inv] + sum_s y_shared (fixed order, fp32)."""
    T, k = topk_w.shape
    H = out.shape[1]
    for t, d, n in ((y, out.dtype, "y"), (inv, torch.int32, "inv"), (topk_w, torch.float32, "topk_w"),
                    (y_shared, out.dtype, "y_shared"), (residual, out.dtype, "residual"), (out, None, "out"),
                    (combined, out.dtype, "combined")):
        _need(t, d, n)
    L.check("moe_combine", L.load().moe_combine(
        _p(y), _p(inv), _p(topk_w), _p(y_shared), S, _p(residual), T, H, k, 0 if y is None else y.shape[0],
        dtype_code(out), _p(out), _p(combined), _stream(out)))


def moe_combine_rmsnorm(y, inv, topk_w, y_shared, S, residual, out, xn, gain=None, eps=1e-6):
    """moe_combine, then xn = RMSNorm(out) (* gain), in one launch."""
    T, k = topk_w.shape
    H = out.shape[1]
    for t, d, n in ((y, out.dtype, "y"), (inv, torch.int32, "inv"), (topk_w, torch.float32, "topk_w"),
                    (y_shared, out.dtype, "y_shared"), (residual, out.dtype, "residual"), (out, None, "out"),
                    (xn, out.dtype, "xn"), (gain, torch.float32, "gain")):
        _need(t, d, n)
    if xn is None:
        raise ValueError("xn is required")
    L.check("moe_combine_rmsnorm", L.load().moe_combine_rmsnorm(
        _p(y), _p(inv), _p(topk_w), _p(y_shared), S, _p(residual), T, H, k, 0 if y is None else y.shape[0],
        _p(gain), float(eps), dtype_code(out), _p(out), _p(xn), _stream(out)))


def lmhead_argmax(h, w_lm, argmax_ids, max_logit, ws):
    """Greedy token per row: argmax of h @ W_lm^T, ties to the lowest id."""
    T, H = h.shape
    V = w_lm.shape[0]
    if h.dtype == torch.bfloat16 and not (isinstance(w_lm, Packed) and w_lm.kind == L.PACK_ROWS):
        raise TypeError("a bf16 LM head must be packed (lm_weights / pack_weights)")
    for t, d, n in ((h, None, "h"), (w_lm, h.dtype, "w_lm"), (argmax_ids, torch.int32, "argmax_ids"),
                    (max_logit, torch.float32, "max_logit"), (ws, None, "ws")):
        _need(t, d, n)
    L.check("lmhead_argmax", L.load().lmhead_argmax(
        _p(h), _p(w_lm), T, H, V, dtype_code(h), _p(argmax_ids), _p(max_logit), _p(ws),
        ws.numel() * ws.element_size(), _stream(h)))


def lmhead_argmax_noalloc(h, w_lm, argmax_ids, max_logit):
    """lmhead_argmax with the library's static per-GPU workspace (no caller
    buffer, nothing allocated); concurrent calls on one GPU race on it."""
    T, H = h.shape
    V = w_lm.shape[0]
    if h.dtype == torch.bfloat16 and not (isinstance(w_lm, Packed) and w_lm.kind == L.PACK_ROWS):
        raise TypeError("a bf16 LM head must be packed (lm_weights / pack_weights)")
    for t, d, n in ((h, None, "h"), (w_lm, h.dtype, "w_lm"), (argmax_ids, torch.int32, "argmax_ids"),
                    (max_logit, torch.float32, "max_logit")):
        _need(t, d, n)
    L.check("lmhead_argmax_noalloc", L.load().lmhead_argmax_noalloc(
        _p(h), _p(w_lm), T, H, V, dtype_code(h), _p(argmax_ids), _p(max_logit), _stream(h)))


def spec_verify(drafts, argmax_ids, accepted, committed, n_commit):
    """Greedy longest-prefix acceptance + bonus token per sequence."""
    B, K = drafts.shape
    for t, n in ((drafts, "drafts"), (argmax_ids, "argmax_ids"), (accepted, "accepted"),
                 (committed, "committed"), (n_commit, "n_commit")):
        _need(t, torch.int32, n)
    L.check("spec_verify", L.load().spec_verify(
        _p(drafts), _p(argmax_ids), B, K, _p(accepted), _p(committed), _p(n_commit), _stream(argmax_ids)))


def spec_plant_drafts(argmax_ids, keep, repl, V, drafts):
    """Benchmark harness: drafts equal to the verifier's tokens where `keep`, else a different id."""
    B, K = keep.shape
    _need(argmax_ids, torch.int32, "argmax_ids")
    _need(keep, torch.uint8, "keep")
    _need(repl, torch.int32, "repl")
    _need(drafts, torch.int32, "drafts")
    L.check("spec_plant_drafts", L.load().spec_plant_drafts(
        _p(argmax_ids), _p(keep), _p(repl), B, K, V, _p(drafts), _stream(argmax_ids)))


def spec_advance(n_commit, committed, seq_ids, target, total, steps, tokens, seq_ids_out, n_active):
    """Decode-loop bookkeeping after a pass: append committed tokens to each
    active sequence's stream (capped at `target`), compact the active ids."""
    B = seq_ids.shape[0]
    K = committed.shape[1] - 1
    S = total.shape[0]
    for t, n in ((n_commit, "n_commit"), (committed, "committed"), (seq_ids, "seq_ids"), (total, "total"),
                 (steps, "steps"), (tokens, "tokens"), (seq_ids_out, "seq_ids_out"), (n_active, "n_active")):
        _need(t, torch.int32, n)
    L.check("spec_advance", L.load().spec_advance(
        _p(n_commit), _p(committed), _p(seq_ids), B, K, S, int(target), _p(total), _p(steps), _p(tokens),
        _p(seq_ids_out), _p(n_active), _stream(total)))


def spec_gather_rows(pool, seq_ids, steps, out):
    """out[i] = pool[seq_ids[i], min(steps[seq_ids[i]], J-1)] for pools [S, J, ...]."""
    S, J = pool.shape[0], pool.shape[1]
    B = seq_ids.shape[0]
    R = pool.shape[2] if pool.dim() > 3 else 1
    row_bytes = pool[0, 0].numel() * pool.element_size() // R
    for t, d, n in ((pool, None, "pool"), (seq_ids, torch.int32, "seq_ids"), (steps, torch.int32, "steps"),
                    (out, pool.dtype, "out")):
        _need(t, d, n)
    if row_bytes == 0:
        return
    if out.numel() < B * R * row_bytes // pool.element_size():
        raise ValueError("out is too small")
    L.check("spec_gather_rows", L.load().spec_gather_rows(
        _p(pool), _p(seq_ids), _p(steps), B, R, J, S, row_bytes, _p(out), _stream(out)))


def _cache_shape(kv, B):
    if kv.dim() != 5 or kv.shape[0] < B or kv.shape[3] != 2:
        raise ValueError("the KV cache must be [B, n_heads, max_len, 2, head_dim] (k then v per position)")
    return kv.shape[1], kv.shape[2], kv.shape[4]


def kv_cache_alloc(B: int, n_heads: int, max_len: int, device, head_dim: int = 128, dtype=torch.bfloat16):
    """A zeroed KV cache [B, n_heads, max_len, 2, head_dim]."""
    return torch.zeros((B, n_heads, max_len, 2, head_dim), dtype=dtype, device=device)


def moe_attn_rope_cache(qkv, lengths, P, q, kv, rope_base=10000.0):
    """q <- rope(q); rope(k) and v into the cache at positions lengths[b] + i
    for the B*P verify tokens of qkv [B*P, 3H]."""
    B = lengths.shape[0]
    n_heads, max_len, d = _cache_shape(kv, B)
    for t, dt, n in ((qkv, None, "qkv"), (lengths, torch.int32, "lengths"), (q, qkv.dtype, "q"),
                     (kv, qkv.dtype, "kv")):
        _need(t, dt, n)
    if qkv.shape != (B * P, 3 * n_heads * d) or q.shape != (B * P, n_heads * d):
        raise ValueError("qkv must be [B*P, 3H] and q [B*P, H]")
    L.check("moe_attn_rope_cache", L.load().moe_attn_rope_cache(
        _p(qkv), _p(lengths), B, int(P), n_heads, d, float(rope_base), max_len, dtype_code(qkv), _p(q), _p(kv),
        _stream(q)))


def attention_workspace_bytes(B: int, P: int, n_heads: int, max_keys: int, head_dim: int = 128) -> int:
    return int(L.load().moe_attention_workspace_bytes(B, P, n_heads, head_dim, max_keys))


def moe_attention(q, kv, lengths, P, o, ws, max_keys=None):
    """o = causal softmax attention of the B*P queries over the cached keys
    0 .. lengths[b] + i (max_keys bounds lengths[b] + P; default max_len)."""
    B = lengths.shape[0]
    n_heads, max_len, d = _cache_shape(kv, B)
    max_keys = max_len if max_keys is None else int(max_keys)
    for t, dt, n in ((q, None, "q"), (kv, q.dtype, "kv"), (lengths, torch.int32, "lengths"), (o, q.dtype, "o"),
                     (ws, None, "ws")):
        _need(t, dt, n)
    if q.shape != (B * P, n_heads * d) or o.shape != q.shape:
        raise ValueError("q and o must be [B*P, H]")
    nbytes = ws.numel() * ws.element_size()
    L.check("moe_attention", L.load().moe_attention(
        _p(q), _p(kv), _p(lengths), B, int(P), n_heads, d, max_len, max_keys, dtype_code(q), _p(o), _p(ws),
        nbytes, _stream(q)))


def spec_commit(n_commit, lengths):
    """lengths[b] += n_commit[b]: the accepted prefix joins the cache."""
    B = lengths.shape[0]
    _need(n_commit, torch.int32, "n_commit")
    _need(lengths, torch.int32, "lengths")
    if n_commit.shape[0] < B:
        raise ValueError("n_commit is shorter than lengths")
    L.check("spec_commit", L.load().spec_commit(_p(n_commit), B, _p(lengths), _stream(lengths)))


def moe_data_errors(flags_out, clear=True):
    """Write the GPU's device-side data-error bits (MOE_DATA_ERR_*) into the
    one-element int32 tensor flags_out, on the current stream, and clear the
    bits read if `clear`."""
    _need(flags_out, torch.int32, "flags_out")
    if flags_out.numel() < 1:
        raise ValueError("flags_out needs one element")
    L.check("moe_data_errors", L.load().moe_data_errors(_p(flags_out), 1 if clear else 0, _stream(flags_out)))


def data_errors(device="cuda", clear=True) -> int:
    """The data-error bits as an int (allocates one word, synchronises the
    current stream)."""
    out = torch.zeros(1, dtype=torch.int32, device=device)
    moe_data_errors(out, clear)
    return int(out.item()) & 0xFFFFFFFF


# ------------------------------------------------------------------ allocating helpers

def route_alloc(h, w_router, bias, k, with_logits=True, **kw):
    T, H = h.shape
    E = w_router.shape[0]
    xn = torch.empty_like(h)
    ids = torch.empty((T, k), dtype=torch.int32, device=h.device)
    w = torch.empty((T, k), dtype=torch.float32, device=h.device)
    lg = torch.empty((T, E), dtype=torch.float32, device=h.device) if with_logits else None
    moe_route(h, w_router, bias, k, xn, ids, w, lg, **kw)
    return xn, ids, w, lg


def permute_alloc(topk_ids, E, S):
    T, k = topk_ids.shape
    dev = topk_ids.device
    offsets = torch.empty(E + S + 1, dtype=torch.int32, device=dev)
    gather = torch.empty(T * k + S * T, dtype=torch.int32, device=dev)
    inv = torch.empty(T * k, dtype=torch.int32, device=dev)
    nb = permute_workspace_bytes(T, k, E)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev) if nb else None
    moe_permute(topk_ids, E, S, offsets, gather, inv, ws)
    return offsets, gather, inv


def swiglu_alloc(x, gather, offsets, w_gate_up, w_down, n_rows, max_rows=None):
    I = w_down.shape[2]
    y = torch.zeros((n_rows, x.shape[1]), dtype=x.dtype, device=x.device)
    ws = torch.empty(max(swiglu_workspace_bytes(n_rows, I, x.dtype), 16), dtype=torch.uint8, device=x.device)
    moe_grouped_swiglu(x, gather, offsets, w_gate_up, w_down, y, ws, max_rows)
    return y


def combine_alloc(y, inv, topk_w, y_shared, S, residual, with_combined=True):
    T = topk_w.shape[0]
    H = y.shape[1]
    out = torch.empty((T, H), dtype=y.dtype, device=y.device)
    comb = torch.empty_like(out) if with_combined else None
    moe_combine(y, inv, topk_w, y_shared, S, residual, out, comb)
    return out, comb


def lmhead_alloc(h, w_lm):
    T = h.shape[0]
    ids = torch.empty(T, dtype=torch.int32, device=h.device)
    mx = torch.empty(T, dtype=torch.float32, device=h.device)
    ws = torch.empty(max(lmhead_workspace_bytes(T, w_lm.shape[0], h.dtype), 16), dtype=torch.uint8, device=h.device)
    lmhead_argmax(h, w_lm, ids, mx, ws)
    return ids, mx


def verify_alloc(drafts, argmax_ids):
    B, K = drafts.shape
    dev = drafts.device
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    com = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    nc = torch.empty(B, dtype=torch.int32, device=dev)
    spec_verify(drafts, argmax_ids, acc, com, nc)
    return acc, com, nc
