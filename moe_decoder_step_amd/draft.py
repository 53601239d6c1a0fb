"""The dense draft block (FastMTP), driven through the C-ABI calls.

FastMTP proposes K draft tokens with one dense block applied recursively,
fed back its own hidden state ("Jina AI's 3.4B OCR model targets faster
page parsing", section "FastMTP cuts decoding work"; jina.ai/de page,
sections "Modell und Training" and "Erste Schritte").  Reading of the block,
with attention omitted as in the verifier:

    x  = [rmsnorm(h) ; rmsnorm(E[tok])]        moe_rmsnorm (twice, into halves of x)
    h0 = W_p x                                 moe_expert_down, one group (2H -> H)
    z  = rmsnorm(h0)                           moe_rmsnorm
    a  = silu(W_g z) * (W_u z)                 moe_expert_gate_up, one group
    h1 = h0 + W_d a                            moe_expert_down_residual
    draft = argmax W_lm h1                     lmhead_argmax (the verifier's head)

Step i + 1 reads h1 and the draft of step i.  Every step runs in libmoestep's
kernels (the weight-streaming expert kernels with a single group); the LM head
is the verifier's, passed in packed.
"""

from __future__ import annotations

import torch

from . import ops
from . import _lib as L


class DraftHead:
    def __init__(self, w: dict, w_lm, max_seqs: int, K: int, eps: float = 1e-6):
        """w: emb [V,H], w_proj [H,2H], w_gate_up [1,2I,H], w_down [1,H,I]
        (row-major; bf16 weights are packed here); w_lm: the verifier's LM
        head as lmhead_argmax takes it (ops.lm_weights)."""
        self.emb = w["emb"]
        V, H = self.emb.shape
        self.H, self.K, self.eps = H, K, eps
        self.I = w["w_down"].shape[2]
        proj = w["w_proj"].reshape(1, H, 2 * H).contiguous()
        self.w_proj = ops.pack_weights(proj, L.PACK_ROWS) if proj.dtype == torch.bfloat16 else proj
        self.w_gate_up, self.w_down = ops.expert_weights(w["w_gate_up"], w["w_down"])
        self.w_lm = w_lm
        dev, dt = self.emb.device, self.emb.dtype
        B = max_seqs
        self.x = torch.empty((B, 2 * H), dtype=dt, device=dev)
        self.h0 = torch.empty((B, H), dtype=dt, device=dev)
        self.z = torch.empty((B, H), dtype=dt, device=dev)
        self.act = torch.empty((B, self.I), dtype=dt, device=dev)
        self.h1 = [torch.empty((B, H), dtype=dt, device=dev) for _ in range(2)]
        self.drafts = torch.empty((K, B), dtype=torch.int32, device=dev)   # step-major: step i's tokens contiguous
        self.max_logit = torch.empty(B, dtype=torch.float32, device=dev)
        self.lws = torch.empty(max(ops.lmhead_workspace_bytes(B, V, dt), 16), dtype=torch.uint8, device=dev)
        # the one-group row ranges [0, b] for every batch size b <= B
        self.offsets = torch.stack([torch.zeros(B + 1, dtype=torch.int32),
                                    torch.arange(B + 1, dtype=torch.int32)], 1).to(dev)

    def propose(self, h: torch.Tensor, tok: torch.Tensor, record: list | None = None) -> torch.Tensor:
        """K draft tokens [B, K] (int32, a view) from the verifier's hidden
        state h [B, H] at each sequence's last committed token tok [B]."""
        B, H = h.shape
        off = self.offsets[B]
        cur_h, cur_t = h, tok
        for i in range(self.K):
            x = self.x[:B]
            ops.moe_rmsnorm(cur_h, x[:, :H], eps=self.eps)
            ops.moe_rmsnorm(self.emb, x[:, H:], rows=cur_t, eps=self.eps)
            ops.moe_expert_down(x, off, self.w_proj, self.h0[:B], max_rows=B)
            ops.moe_rmsnorm(self.h0[:B], self.z[:B], eps=self.eps)
            ops.moe_expert_gate_up(self.z[:B], None, off, self.w_gate_up, self.act[:B], max_rows=B)
            h1 = self.h1[i & 1][:B]
            ops.moe_expert_down_residual(self.act[:B], off, self.w_down, self.h0[:B], h1, max_rows=B)
            ops.lmhead_argmax(h1, self.w_lm, self.drafts[i, :B], self.max_logit[:B], self.lws)
            if record is not None:
                record.append({"h": cur_h.clone(), "tok": cur_t.clone(), "h0": self.h0[:B].clone(),
                               "h1": h1.clone(), "ids": self.drafts[i, :B].clone()})
            cur_h, cur_t = h1, self.drafts[i, :B]
        return self.drafts[:, :B].t()
