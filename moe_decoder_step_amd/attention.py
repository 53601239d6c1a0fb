"""Causal self-attention of the verify positions over a KV cache, driven
through the C-ABI calls.

The pages give the decoder's context limit (32,768 positions; jina.ai/ko
model card "jina-ocr-v1", architecture paragraph) but not its attention.
The reading is pre-norm multi-head attention with rotary positions and
heads of 128:

    xa = rmsnorm(h)                         moe_rmsnorm (or the previous block's
                                            moe_combine_rmsnorm)
    qkv = xa W_qkv^T                        moe_expert_down, one group (H -> 3H)
    q, cache[L_b + i] <- rope(q), rope(k), v    moe_attn_rope_cache
    o = causal softmax(q k^T / sqrt(128)) v  moe_attention (split over keys + merge)
    h <- h + o W_o^T                        moe_expert_down_residual

A pass of sequence b holds P positions at L_b .. L_b + P - 1 (its last
committed token, then the drafts).  Query i reads cache rows 0 .. L_b + i
only, so the rows of rejected drafts need no clean-up: spec_commit advances
L_b by the committed count and the next pass overwrites them.
"""

from __future__ import annotations

import torch

from . import ops
from . import _lib as L

HEAD_DIM = 128


class AttentionBlock:
    def __init__(self, w: dict, n_heads: int, max_seqs: int, P: int, max_len: int, eps: float = 1e-6,
                 rope_base: float = 10000.0):
        """w: w_qkv [3H, H], w_o [H, H] bf16 row-major (packed here).  Holds
        this layer's cache kv [max_seqs, n_heads, max_len, 2, 128] (k then v
        per position; cache_k and cache_v are views of it) and the buffers
        of a pass of up to max_seqs * P tokens."""
        w_qkv, w_o = w["w_qkv"], w["w_o"]
        H = w_o.shape[0]
        if w_qkv.dtype != torch.bfloat16 or H != n_heads * HEAD_DIM or tuple(w_qkv.shape) != (3 * H, H):
            raise ValueError("attention needs bf16 w_qkv [3H, H] and w_o [H, H] with H = n_heads * 128")
        self.H, self.n_heads, self.P, self.max_len = H, n_heads, P, max_len
        self.eps, self.rope_base = eps, rope_base
        self.w_qkv = ops.pack_weights(w_qkv.reshape(1, 3 * H, H).contiguous(), L.PACK_ROWS)
        self.w_o = ops.pack_weights(w_o.reshape(1, H, H).contiguous(), L.PACK_ROWS)
        dev, dt = w_o.device, w_o.dtype
        T = max_seqs * P
        self.kv = ops.kv_cache_alloc(max_seqs, n_heads, max_len, dev, HEAD_DIM, dt)
        self.cache_k = self.kv[:, :, :, 0]
        self.cache_v = self.kv[:, :, :, 1]
        self.xa = torch.empty((T, H), dtype=dt, device=dev)
        self.qkv = torch.empty((T, 3 * H), dtype=dt, device=dev)
        self.q = torch.empty((T, H), dtype=dt, device=dev)
        self.o = torch.empty((T, H), dtype=dt, device=dev)
        nb = ops.attention_workspace_bytes(max_seqs, P, n_heads, max_len)
        self.ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
        self.offsets = torch.stack([torch.zeros(T + 1, dtype=torch.int32),
                                    torch.arange(T + 1, dtype=torch.int32)], 1).to(dev)

    def forward(self, h: torch.Tensor, lengths: torch.Tensor, max_keys: int | None = None,
                record: dict | None = None, normed: bool = False) -> None:
        """In place on h [B*P, H] (sequence-major); lengths [B] int32 device.
        max_keys bounds lengths[b] + P (default: the cache length).  normed:
        self.xa[:T] already holds RMSNorm(h) (written by the caller's
        moe_combine_rmsnorm), so the norm is not run again."""
        T = h.shape[0]
        B = lengths.shape[0]
        if T != B * self.P:
            raise ValueError(f"h has {T} rows, expected {B} sequences x {self.P} positions")
        off = self.offsets[T]
        if not normed:
            ops.moe_rmsnorm(h, self.xa[:T], eps=self.eps)
        ops.moe_expert_down(self.xa[:T], off, self.w_qkv, self.qkv[:T], max_rows=T)
        ops.moe_attn_rope_cache(self.qkv[:T], lengths, self.P, self.q[:T], self.kv[:B], self.rope_base)
        ops.moe_attention(self.q[:T], self.kv[:B], lengths, self.P, self.o[:T], self.ws,
                          max_keys or self.max_len)
        if record is not None:
            record.update({"attn_input": h.clone(), "qkv": self.qkv[:T].clone(), "q": self.q[:T].clone(),
                           "o": self.o[:T].clone()})
        ops.moe_expert_down_residual(self.o[:T], off, self.w_o, h, h, max_rows=T)
