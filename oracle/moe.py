"""fp64 NumPy oracle of the MoE speculative verify step (test infrastructure).

Every function is the plain definition written out; loops and library
primitives (matmul, sort, argmax) only, no blocking or fusion.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "f64", "round_bf16", "round_f32", "store",
    "rmsnorm", "router_logits", "topk_ids", "topk_weights", "topk_gap", "route",
    "permute", "silu", "swiglu", "moe_layer", "lm_logits", "lm_argmax",
    "spec_verify", "plant_drafts", "greedy_decode", "speculative_decode",
    "verify_step", "rope", "rope_cache", "causal_attention", "attention_block", "draft_step", "draft_propose", "active_params", "total_params",
]


# ----------------------------------------------------------------------------
# storage formats
# ----------------------------------------------------------------------------

def f64(a) -> np.ndarray:
    """Exact fp64 value of an input array.

    uint16 arrays are bf16 bit patterns (the top half of an fp32), float32 and
    float64 arrays are taken as they are.  No rounding happens here.
    """
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def round_bf16(x) -> np.ndarray:
    """Nearest bf16 value of fp64 `x` (8 significant bits, ties to even), as fp64.

    One rounding step straight from fp64: x = m * 2**e with 0.5 <= |m| < 1, the
    mantissa is scaled to 8 integer bits, rounded half-to-even and scaled back.
    Finite, normal-range inputs only (the step never leaves that range).
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def round_f32(x) -> np.ndarray:
    """Nearest fp32 value of `x` (IEEE round-to-nearest-even), as fp64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def store(x, mode: str) -> np.ndarray:
    """Round `x` to the storage dtype `mode` ("bf16", "f32") or keep it ("exact")."""
    if mode == "bf16":
        return round_bf16(x)
    if mode == "f32":
        return round_f32(x)
    if mode == "exact":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(f"unknown storage mode {mode!r}")


# ----------------------------------------------------------------------------
# router
# ----------------------------------------------------------------------------

def rmsnorm(h, eps: float, gain=None) -> np.ndarray:
    """xn = h / sqrt(mean(h^2) + eps) (* gain).

    The pages do not name the decoder's norm; the reading is a pre-norm RMSNorm
    with eps 1e-6 and unit gain in front of each MoE block.
    """
    h = np.asarray(h, dtype=np.float64)
    ms = np.mean(h * h, axis=-1, keepdims=True)
    y = h / np.sqrt(ms + eps)
    return y if gain is None else y * np.asarray(gain, dtype=np.float64)


def router_logits(xn, w_router, bias=None) -> np.ndarray:
    """l = xn @ W_r^T + b: one logit per routed expert (64 routed experts,
    jina.ai/ko model card "jina-ocr-v1", architecture paragraph)."""
    lg = np.asarray(xn, np.float64) @ np.asarray(w_router, np.float64).T
    if bias is not None:
        lg = lg + np.asarray(bias, np.float64)
    return lg


def topk_ids(logits, k: int) -> np.ndarray:
    """The k experts with the largest logits, in descending logit order; equal
    logits go to the lower expert id (top-6 of 64: alphasignal.ai, section
    "A compressed visual front end").

    A stable sort of the negated logits keeps equal values in ascending id order.
    """
    order = np.argsort(-np.asarray(logits, np.float64), axis=-1, kind="stable")
    return order[..., :k].astype(np.int64)


def topk_weights(logits, ids, renormalize: bool = True) -> np.ndarray:
    """Routing weights of the selected experts.

    renormalize=True: softmax over the k selected logits (equal to the full
    softmax renormalised over the selected k).  renormalize=False: the full
    softmax probability of each selected expert.
    """
    lg = np.asarray(logits, np.float64)
    if renormalize:
        sel = np.take_along_axis(lg, ids, axis=-1)
        z = np.exp(sel - sel.max(axis=-1, keepdims=True))
        return z / z.sum(axis=-1, keepdims=True)
    z = np.exp(lg - lg.max(axis=-1, keepdims=True))
    p = z / z.sum(axis=-1, keepdims=True)
    return np.take_along_axis(p, ids, axis=-1)


def topk_gap(logits, k: int) -> np.ndarray:
    """Per token, the smallest gap between neighbours among the k+1 largest
    logits: below it, the selected set or its order is decided by a near-tie."""
    s = -np.sort(-np.asarray(logits, np.float64), axis=-1)
    kk = min(k, s.shape[-1] - 1)
    if kk <= 0:
        return np.full(s.shape[:-1], np.inf)
    return (s[..., :kk] - s[..., 1:kk + 1]).min(axis=-1)


def route(h, w_router, bias, k: int, eps: float, mode: str,
          renormalize: bool = True, norm: bool = True) -> dict:
    """Pre-norm, router logits, top-k selection and routing weights of a block."""
    h = f64(h)
    xn = store(rmsnorm(h, eps), mode) if norm else h
    lg = router_logits(xn, f64(w_router), None if bias is None else f64(bias))
    ids = topk_ids(lg, k)
    return {"xn": xn, "logits": lg, "ids": ids,
            "w": topk_weights(lg, ids, renormalize), "gap": topk_gap(lg, k)}


# ----------------------------------------------------------------------------
# permutation by expert
# ----------------------------------------------------------------------------

def permute(ids, E: int, S: int = 0):
    """Group the (token, slot) pairs by expert.

    Slot s = t*k + j.  Rows of routed expert e are offsets[e]..offsets[e+1]-1,
    holding its slots in ascending token order; shared expert s follows as
    group E+s with one row per token.  Returns (offsets [E+S+1],
    gather [T*k + S*T] = token of each row, inv [T*k] = row of each slot).
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + S + 1, dtype=np.int64)
    offsets[1:E + 1] = np.cumsum(counts)
    for s in range(S):
        offsets[E + 1 + s] = offsets[E + s] + T
    gather = np.empty(T * k + S * T, dtype=np.int64)
    gather[:T * k] = order // k
    for s in range(S):
        gather[T * k + s * T:T * k + (s + 1) * T] = np.arange(T)
    inv = np.empty(T * k, dtype=np.int64)
    inv[order] = np.arange(T * k)
    return offsets, gather, inv


# ----------------------------------------------------------------------------
# experts
# ----------------------------------------------------------------------------

def silu(z) -> np.ndarray:
    """silu(z) = z / (1 + exp(-z))."""
    z = np.asarray(z, np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu(x, w_gate_up, w_down, mode: str) -> np.ndarray:
    """One SwiGLU expert: y = W_d (silu(W_g x) * (W_u x)).

    w_gate_up [2I, H] holds W_g in rows 0..I-1 and W_u in rows I..2I-1,
    w_down is [H, I].  The activation is rounded to the storage dtype before
    the down projection, and y after it.  The pages name 64 routed and 2
    shared experts but not their form; SwiGLU without biases is the reading.
    """
    x = np.asarray(x, np.float64)
    wgu = f64(w_gate_up)
    wd = f64(w_down)
    I = wd.shape[1]
    gu = x @ wgu.T
    a = store(silu(gu[:, :I]) * gu[:, I:], mode)
    return store(a @ wd.T, mode)


def moe_layer(h, wts: dict, k: int, eps: float, mode: str,
              renormalize: bool = True, norm: bool = True) -> dict:
    """One decoder MoE block: h' = h + sum_j w_j y_j + sum_s ys_s.

    Routed experts are chosen per token by top-k of the router; the shared
    experts (weight 1) see every token (64 routed + 2 shared, top-6: jina.ai/ko
    model card "jina-ocr-v1", architecture paragraph).  Attention is omitted.
    Returns the route, per-slot routed outputs y [T,k,H], shared outputs
    ys [S,T,H], `combined` = sum_j w_j y_j + sum_s ys_s (fp64) and h_out.
    """
    h = f64(h)
    T, H = h.shape
    E = np.asarray(wts["w_router"]).shape[0]
    G = np.asarray(wts["w_gate_up"]).shape[0]
    S = G - E
    r = route(h, wts["w_router"], wts.get("bias"), k, eps, mode, renormalize, norm)
    xn, ids = r["xn"], r["ids"]
    y = np.zeros((T, k, H))
    for e in range(E):
        t_idx, j_idx = np.nonzero(ids == e)
        if t_idx.size:
            y[t_idx, j_idx] = swiglu(xn[t_idx], wts["w_gate_up"][e], wts["w_down"][e], mode)
    ys = np.zeros((S, T, H))
    for s in range(S):
        ys[s] = swiglu(xn, wts["w_gate_up"][E + s], wts["w_down"][E + s], mode)
    combined = np.einsum("tj,tjh->th", r["w"], y) + ys.sum(axis=0)
    return {"route": r, "y": y, "ys": ys, "combined": combined,
            "h_out": store(h + combined, mode)}


# ----------------------------------------------------------------------------
# LM head, acceptance
# ----------------------------------------------------------------------------

def lm_logits(h, w_lm) -> np.ndarray:
    """All logits h @ W_lm^T (small vocabularies only)."""
    return f64(h) @ f64(w_lm).T


def lm_argmax(h, w_lm, chunk: int = 4096):
    """Greedy next token per row: argmax_v (h @ W_lm^T)[v], ties to the lowest v.

    The vocabulary (129,280, jina.ai/ko model card, architecture paragraph) is
    walked in chunks to bound memory; a later chunk replaces the running best
    only when strictly larger.  Returns (ids, max logit, top-1 minus top-2 gap).
    """
    h = f64(h)
    T = h.shape[0]
    V = np.asarray(w_lm).shape[0]
    best = np.full(T, -np.inf)
    second = np.full(T, -np.inf)
    idx = np.zeros(T, dtype=np.int64)
    for v0 in range(0, V, chunk):
        lg = h @ f64(w_lm[v0:v0 + chunk]).T
        a = np.argmax(lg, axis=1)
        m = lg[np.arange(T), a]
        if lg.shape[1] > 1:
            top2 = -np.partition(-lg, 1, axis=1)[:, :2]
            c2 = top2.min(axis=1)
        else:
            c2 = np.full(T, -np.inf)
        better = m > best
        second = np.where(better, np.maximum(best, c2), np.maximum(second, m))
        idx = np.where(better, a + v0, idx)
        best = np.where(better, m, best)
    return idx, best, best - second


def spec_verify(drafts, g):
    """Greedy longest-prefix acceptance with the bonus token.

    Position 0 of a sequence is its last committed token and positions 1..K
    hold the drafts; g[i] is the verifier's greedy token after position i, so
    draft d[i] is accepted while d[i] == g[i] for all earlier i.  The step
    commits the n accepted drafts plus g[n]: n+1 tokens, at most K+1 (jina.ai/de
    page, sections "Modell und Training" and "Spekulatives Decoding auf einer L4").
    Returns (accepted [B], committed [B, K+1] padded with -1, n_commit [B]).
    """
    d = np.asarray(drafts, dtype=np.int64)
    g = np.asarray(g, dtype=np.int64)
    B, K = d.shape
    assert g.shape == (B, K + 1)
    accepted = np.zeros(B, dtype=np.int64)
    committed = np.full((B, K + 1), -1, dtype=np.int64)
    for b in range(B):
        n = 0
        while n < K and d[b, n] == g[b, n]:
            n += 1
        committed[b, :n] = d[b, :n]
        committed[b, n] = g[b, n]
        accepted[b] = n
    return accepted, committed, accepted + 1


def plant_drafts(g, keep, repl):
    """Harness model of a draft head with a given acceptance: draft i is the
    verifier's own token g[i] when keep[i], else a different token, uniform
    over the other V-1 ids (repl is uniform in [0, V-1); values at or above
    g[i] shift up by one)."""
    g = np.asarray(g, dtype=np.int64)
    keep = np.asarray(keep).astype(bool)
    u = np.asarray(repl, dtype=np.int64)
    K = keep.shape[-1]
    gi = g[..., :K]
    return np.where(keep, gi, u + (u >= gi))


def greedy_decode(first: int, n: int, next_tokens):
    """Plain greedy decoding: one token per pass, t_{i+1} = next_tokens([t_i])[0]."""
    seq = [int(first)]
    while len(seq) < n + 1:
        seq.append(int(next_tokens([seq[-1]])[0]))
    return seq


def speculative_decode(first: int, n: int, next_tokens, propose, K: int):
    """Speculative decoding with greedy verification.

    Each pass verifies [last committed token, d_1..d_K] in one call of
    `next_tokens`, then commits the accepted prefix and the bonus token.
    Returns (sequence of n+1 tokens, number of passes, list of n_commit).
    """
    seq = [int(first)]
    commits = []
    while len(seq) < n + 1:
        d = [int(x) for x in propose(seq, K)]
        g = np.asarray(next_tokens([seq[-1]] + d), dtype=np.int64)
        _, com, nc = spec_verify(np.asarray([d], dtype=np.int64).reshape(1, K), g[None])
        seq.extend(int(x) for x in com[0, :nc[0]])
        commits.append(int(nc[0]))
    return seq[:n + 1], len(commits), commits


def verify_step(h, layers, w_lm, drafts, k: int, eps: float, mode: str,
                layer_inputs=None, lm_input=None, renormalize: bool = True) -> dict:
    """One verify pass through the stack: L MoE blocks, LM-head argmax, acceptance.

    h is [B*(K+1), H] in sequence-major order.  Teacher forcing: with
    `layer_inputs` (a list of L arrays) block l reads layer_inputs[l] instead
    of the previous block's output, and with `lm_input` the LM head reads that
    array; each block's own output is still returned for comparison.
    """
    cur = f64(h)
    outs = []
    for li, wts in enumerate(layers):
        x = cur if layer_inputs is None else f64(layer_inputs[li])
        o = moe_layer(x, wts, k, eps, mode, renormalize)
        outs.append(o)
        cur = o["h_out"]
    ids, mx, gap = lm_argmax(cur if lm_input is None else f64(lm_input), w_lm)
    d = np.asarray(drafts, dtype=np.int64)
    B, K = d.shape
    acc, com, nc = spec_verify(d, ids.reshape(B, K + 1))
    return {"layers": outs, "argmax": ids, "max_logit": mx, "gap": gap,
            "accepted": acc, "committed": com, "n_commit": nc}


# ----------------------------------------------------------------------------
# attention over a KV cache (the verify positions)
# ----------------------------------------------------------------------------

def rope(x, pos, base: float = 10000.0) -> np.ndarray:
    """Rotary position embedding, rotate-half form, per head of d = 2m dims:
    (x_j, x_{j+m}) -> (x_j cos a - x_{j+m} sin a, x_j sin a + x_{j+m} cos a)
    with a = pos * base^(-j/m), j < m.  x [T, n_heads, d], pos [T]."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    m = d // 2
    inv = base ** (-np.arange(m, dtype=np.float64) / m)
    a = np.asarray(pos, np.float64)[:, None, None] * inv[None, None, :]
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[..., :m], x[..., m:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def causal_attention(q, cache_k, cache_v, lengths, P: int) -> np.ndarray:
    """o[b*P+i] = sum_{j <= L_b+i} softmax_j(q . k_j / sqrt(d)) v_j per head,
    in fp64 over the cache as it stands (rows past L_b + i are not read).
    q [B*P, n_heads, d]; caches [B, n_heads, max_len, d]; returns [B*P, n_heads, d]."""
    q = f64(q)
    T, n_heads, d = q.shape
    o = np.zeros((T, n_heads, d))
    for b in range(T // P):
        L = int(lengths[b])
        for i in range(P):
            t = b * P + i
            kk = f64(cache_k[b, :, :L + i + 1])            # [n_heads, keys, d]
            vv = f64(cache_v[b, :, :L + i + 1])
            sc = np.einsum("hd,hjd->hj", q[t], kk) / np.sqrt(d)
            sc -= sc.max(axis=1, keepdims=True)
            p = np.exp(sc)
            p /= p.sum(axis=1, keepdims=True)
            o[t] = np.einsum("hj,hjd->hd", p, vv)
    return o


def rope_cache(qkv, lengths, P: int, n_heads: int, cache_k, cache_v, mode: str, base: float = 10000.0):
    """Split stored qkv [B*P, 3H] into heads, rotate q and k at their
    positions L_b + i, store (round) them, and write k, v into the caches at
    [b, :, L_b + i] (in place).  Returns q, k, v [B*P, n_heads, d]."""
    qkv = f64(qkv)
    T, H3 = qkv.shape
    H = H3 // 3
    d = H // n_heads
    B = T // P
    pos = np.concatenate([np.arange(P) + int(lengths[b]) for b in range(B)])
    q = store(rope(qkv[:, :H].reshape(T, n_heads, d), pos, base), mode)
    k = store(rope(qkv[:, H:2 * H].reshape(T, n_heads, d), pos, base), mode)
    v = qkv[:, 2 * H:].reshape(T, n_heads, d)
    for b in range(B):
        L = int(lengths[b])
        for i in range(P):
            cache_k[b, :, L + i] = k[b * P + i]
            cache_v[b, :, L + i] = v[b * P + i]
    return q, k, v


def attention_block(h, w_qkv, w_o, cache_k, cache_v, lengths, P: int, n_heads: int, eps: float, mode: str) -> dict:
    """Pre-norm causal self-attention of the verify positions over a KV cache.

    The pages give the decoder's position limit (32,768; jina.ai/ko model
    card, architecture paragraph) but not its attention; the reading is plain
    multi-head attention with rotary positions:
        xa = rmsnorm(h);  q, k, v = split(xa W_qkv^T)  (n_heads heads of d)
        q, k <- rope(., position);  cache[b, :, L_b + i] <- k, v
        o_i = sum_{j <= L_b + i} softmax_j(q_i . k_j / sqrt(d)) v_j
        h' = h + o W_o^T
    h is [B*P, H] in sequence-major order: sequence b's position i sits at
    L_b + i (position 0 is its last committed token, then the drafts).
    cache_k / cache_v [B, n_heads, max_len, d] hold the committed prefix and
    are written in place.  Storage rounding at xa, q/k/v (after rope), o and
    h'.  Returns o and h'.
    """
    h = f64(h)
    T, H = h.shape
    xa = store(rmsnorm(h, eps), mode)
    qkv = store(xa @ f64(w_qkv).T, mode)
    q, k, v = rope_cache(qkv, lengths, P, n_heads, cache_k, cache_v, mode)
    o = store(causal_attention(q, cache_k, cache_v, lengths, P).reshape(T, H), mode)
    h_out = store(h + store(o @ f64(w_o).T, mode), mode)
    return {"xa": xa, "qkv": qkv, "q": q, "k": k, "v": v, "o": o, "h_out": h_out}


# ----------------------------------------------------------------------------
# the draft block (FastMTP)
# ----------------------------------------------------------------------------

def draft_step(h, tok, wts: dict, w_lm, eps: float, mode: str) -> dict:
    """One recursive step of the dense draft block.

    The pages describe FastMTP as one dense block applied recursively for K
    prediction steps, fed back its own hidden state ("Jina AI's 3.4B OCR model
    targets faster page parsing", section "FastMTP cuts decoding work";
    jina.ai/de page, sections "Modell und Training" and "Erste Schritte",
    where the head runs as vLLM's eagle method).  The block's inside is not
    given; the reading is a DeepSeek-style multi-token-prediction block with
    attention omitted (as in the verifier):

        x  = [rmsnorm(h) ; rmsnorm(E[tok])]          (2H)
        h0 = W_p x                                   (H)
        h1 = h0 + W_d (silu(W_g z) * (W_u z)),  z = rmsnorm(h0)
        draft = argmax_v (W_lm h1)[v]                (the verifier's LM head)

    wts: emb [V,H], w_proj [H,2H], w_gate_up [2I,H] (gate rows, then up),
    w_down [H,I].  Storage rounding (`mode`) at x, h0, z, the SwiGLU
    activation, the FFN output and h1.  Returns h1, the draft ids and the
    LM-head gaps (top-1 minus top-2).
    """
    h = f64(h)
    e = f64(np.asarray(wts["emb"])[np.asarray(tok, dtype=np.int64)])
    x = np.concatenate([store(rmsnorm(h, eps), mode), store(rmsnorm(e, eps), mode)], axis=1)
    h0 = store(x @ f64(wts["w_proj"]).T, mode)
    z = store(rmsnorm(h0, eps), mode)
    f = swiglu(z, wts["w_gate_up"], wts["w_down"], mode)
    h1 = store(h0 + f, mode)
    ids, mx, gap = lm_argmax(h1, w_lm)
    return {"x": x, "h0": h0, "z": z, "h1": h1, "ids": ids, "gap": gap}


def draft_propose(h, tok, wts: dict, w_lm, K: int, eps: float, mode: str) -> dict:
    """K recursive draft steps from the verifier's hidden state h [B,H] at the
    last committed token tok [B]: step i reads the previous step's output
    hidden state and draft token.  Returns drafts [B,K] and the steps."""
    steps = []
    cur_h, cur_t = f64(h), np.asarray(tok, dtype=np.int64)
    for _ in range(K):
        st = draft_step(cur_h, cur_t, wts, w_lm, eps, mode)
        steps.append(st)
        cur_h, cur_t = st["h1"], st["ids"]
    B = np.asarray(tok).shape[0]
    drafts = np.stack([st["ids"] for st in steps], axis=1) if K else np.zeros((B, 0), np.int64)
    return {"drafts": drafts, "steps": steps}


# ----------------------------------------------------------------------------
# parameter accounting
# ----------------------------------------------------------------------------

def active_params(H, E, k, S, I, V, L, attn_per_layer: int = 0) -> int:
    """Weights one token reads in one decoder pass: per layer the router (E*H),
    k routed + S shared SwiGLU experts (3*H*I each) and any attention weights;
    then the LM head (V*H).  The pages give about 570M active parameters per
    token (alphasignal.ai, intro)."""
    return L * ((k + S) * 3 * H * I + E * H + attn_per_layer) + V * H


def total_params(H, E, S, I, V, L, attn_per_layer: int = 0,
                 tied_embedding: bool = True, encoder: int = 0) -> int:
    """All decoder weights (+ encoder): every expert, router, attention, LM head
    and, when untied, the embedding.  The pages give 3.4B in total with a
    ~380M-parameter vision encoder (alphasignal.ai, intro and section
    "A compressed visual front end")."""
    n = L * ((E + S) * 3 * H * I + E * H + attn_per_layer) + V * H + encoder
    return n if tied_embedding else n + V * H
