"""The speculative verify step, driven through the C-ABI calls.

A VerifyStack holds one model's device-resident weights and the buffers of
one batch (allocated once, for the largest batch it will see).  A verify
pass of T = B*(K+1) positions runs, per MoE layer,

    moe_route -> moe_permute -> moe_grouped_swiglu -> moe_combine

(the residual add is fused into the combine, in place on the hidden state),
then lmhead_argmax over all positions and spec_verify per sequence.  With
attention weights, each MoE block is preceded by causal attention over a
per-layer KV cache (attention.AttentionBlock) and spec_commit advances the
committed lengths after acceptance.  Every
step runs in libmoestep's HIP kernels; torch only owns memory and streams.
"""

from __future__ import annotations

import torch

from . import ops


class VerifyStack:
    def __init__(self, layers: list[dict], w_lm: torch.Tensor | None, E: int, k: int, S: int,
                 max_tokens: int, max_seqs: int = 0, K: int = 0, eps: float = 1e-6,
                 keep_logits: bool = False, attn: list[dict] | None = None, n_heads: int = 0,
                 max_len: int = 0):
        """layers: per layer w_router [E,H] fp32, bias [E] fp32 (or absent),
        w_gate_up [E+S, 2I, H], w_down [E+S, H, I] row-major; w_lm [V, H].
        bf16 expert and LM-head weights are packed here (moe_pack_weights)
        into the stack's own copies; the caller may drop its tensors.

        attn (optional): per layer w_qkv [3H, H], w_o [H, H]; each MoE block
        is then preceded by causal attention over a per-layer KV cache of
        max_len positions for max_seqs sequences of K+1 verify positions
        (AttentionBlock), and `lengths` holds each sequence's committed
        length (advanced by step() after acceptance)."""
        self.layers = []
        for w in layers:
            gu, dn = ops.expert_weights(w["w_gate_up"], w["w_down"])
            self.layers.append({"w_router": ops.router_weights(w["w_router"]), "bias": w.get("bias"), "w_gate_up": gu, "w_down": dn})
        self.w_lm = None if w_lm is None else ops.lm_weights(w_lm)
        self.V = None if w_lm is None else w_lm.shape[0]
        self.E, self.k, self.S, self.eps = E, k, S, eps
        wgu = layers[0]["w_gate_up"]
        self.dtype = wgu.dtype
        self.device = wgu.device
        self.H = wgu.shape[2]
        self.I = wgu.shape[1] // 2
        self.attn = None
        if attn:
            from .attention import AttentionBlock
            if len(attn) != len(layers) or not max_seqs or not max_len:
                raise ValueError("attention needs one block per layer, max_seqs and max_len")
            self.attn = [AttentionBlock(a, n_heads, max_seqs, K + 1, max_len, eps) for a in attn]
        self._alloc(max_tokens, max_seqs, K, keep_logits)

    def sibling(self, max_tokens: int, max_seqs: int = 0, K: int = 0, keep_logits: bool = False) -> "VerifyStack":
        """A stack over the same packed weights with buffers of its own, sized
        for another batch (e.g. a prefill batch next to the decode batch).
        Attention-free."""
        if self.attn is not None:
            raise ValueError("a sibling of a stack with attention is not supported")
        other = object.__new__(VerifyStack)
        for name in ("layers", "w_lm", "V", "E", "k", "S", "eps", "dtype", "device", "H", "I", "attn"):
            setattr(other, name, getattr(self, name))
        other._alloc(max_tokens, max_seqs, K, keep_logits)
        return other

    def _alloc(self, max_tokens: int, max_seqs: int, K: int, keep_logits: bool) -> None:
        """The buffers of one batch of up to max_tokens positions."""
        E, k, S = self.E, self.k, self.S
        # when a list: (start, end) torch.cuda.Event pairs around every expert
        # gate/up launch, recorded on the stream the kernels run on
        self.ffn_events = None
        # fuse each block's combine with the next block's routing, and (bf16,
        # decode-sized batches) the permutation into the gate/up launch
        self.fuse = True
        self.max_tokens = T = max_tokens
        dev, H = self.device, self.H
        i32 = dict(dtype=torch.int32, device=dev)
        self.h = torch.empty((T, H), dtype=self.dtype, device=dev)
        self.xn = torch.empty((T, H), dtype=self.dtype, device=dev)
        self.ids = torch.empty((T, k), **i32)
        self.tw = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.logits = torch.empty((T, E), dtype=torch.float32, device=dev) if keep_logits else None
        self.offsets = torch.empty(E + S + 1, **i32)
        self.gather = torch.empty(T * k + S * T, **i32)
        self.inv = torch.empty(T * k, **i32)
        nb = ops.permute_workspace_bytes(T, k, E)
        self.pws = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
        self.n_rows = T * k + S * T
        self.y = torch.empty((self.n_rows, H), dtype=self.dtype, device=dev)
        self.act = torch.empty((self.n_rows, self.I), dtype=self.dtype, device=dev)
        if self.w_lm is not None:
            self.argmax = torch.empty(T, **i32)
            self.max_logit = torch.empty(T, dtype=torch.float32, device=dev)
            self.lws = torch.empty(max(ops.lmhead_workspace_bytes(T, self.V, self.dtype), 16), dtype=torch.uint8,
                                   device=dev)
        if self.attn is not None:
            self.lengths = torch.zeros(max_seqs, **i32)
            self.max_keys = None        # a known bound on lengths + K + 1 (default: max_len)
        if max_seqs:
            self.accepted = torch.empty(max_seqs, **i32)
            self.committed = torch.empty((max_seqs, K + 1), **i32)
            self.n_commit = torch.empty(max_seqs, **i32)

    def _route(self, li: int, T: int, combine_prev: bool) -> None:
        """Layer li's routing of self.h[:T]; with combine_prev, layer li-1's
        combine runs in the same launch first (moe_combine_route)."""
        w = self.layers[li]
        lg = None if self.logits is None else self.logits[:T]
        if combine_prev:
            k, S = self.k, self.S
            y = self.y[:T * k + S * T]
            ops.moe_combine_route(y[:T * k], self.inv[:T * k], self.tw[:T], y[T * k:] if S else None, S,
                                  self.h[:T], w["w_router"], w.get("bias"), k, self.xn[:T], self.ids[:T],
                                  self.tw[:T], lg, eps=self.eps)
        else:
            ops.moe_route(self.h[:T], w["w_router"], w.get("bias"), self.k, self.xn[:T], self.ids[:T],
                          self.tw[:T], lg, eps=self.eps)

    def _experts(self, li: int, T: int) -> None:
        """Layer li's permutation and routed + shared expert FFN (y rows)."""
        E, k, S = self.E, self.k, self.S
        w = self.layers[li]
        n_rows = T * k + S * T
        act = self.act[:n_rows]
        routed = self.fuse and self.dtype == torch.bfloat16 and T * k <= ops.ROUTED_MAX_PAIRS
        if not routed:
            ops.moe_permute(self.ids[:T], E, S, self.offsets, self.gather[:n_rows], self.inv[:T * k], self.pws)
        if self.ffn_events is not None:
            ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            ev[0].record()
        if routed:  # the permutation is derived inside the gate/up launch
            ops.moe_expert_gate_up_routed(self.xn[:T], self.ids[:T], E, S, w["w_gate_up"], act, self.offsets,
                                          self.inv[:T * k].view(T, k))
        else:
            ops.moe_expert_gate_up(self.xn[:T], self.gather[:n_rows], self.offsets, w["w_gate_up"], act,
                                   max_rows=T)
        if self.ffn_events is not None:
            ev[1].record()
            self.ffn_events.append(ev)
        ops.moe_expert_down(act, self.offsets, w["w_down"], self.y[:n_rows], max_rows=T)

    def _combine(self, T: int) -> None:
        """The last routed layer's weighted combine + residual, in place on self.h[:T]."""
        k, S = self.k, self.S
        y = self.y[:T * k + S * T]
        h = self.h[:T]
        ops.moe_combine(y[:T * k], self.inv[:T * k], self.tw[:T], y[T * k:] if S else None, S, h, h)

    def layer(self, li: int, T: int) -> None:
        """One MoE block in place on self.h[:T], unfused (route, permute,
        experts, combine)."""
        self._route(li, T, False)
        self._experts(li, T)
        self._combine(T)

    def forward(self, h_in: torch.Tensor, record: list | None = None) -> torch.Tensor:
        """All MoE blocks on a copy of h_in; returns the final hidden state (a view).

        Block l's combine runs fused with block l+1's routing (moe_combine_route)
        unless self.fuse is False.  With `record` (a list), a copy of every
        block's input, expert ids, routing weights and output is appended to
        it (for teacher-forced comparison)."""
        T = h_in.shape[0]
        self.h[:T].copy_(h_in)
        if self.attn is not None:
            return self._forward_attn(T, record)
        L = len(self.layers)
        for li in range(L):
            if self.fuse:
                self._route(li, T, li > 0)
            else:
                if li > 0:
                    self._combine(T)
                self._route(li, T, False)
            if record is not None:
                inp = self.h[:T].clone()
                if li > 0:
                    record[-1]["output"] = inp
                record.append({"input": inp, "ids": self.ids[:T].clone(), "w": self.tw[:T].clone()})
            self._experts(li, T)
        self._combine(T)
        if record is not None:
            record[-1]["output"] = self.h[:T].clone()
        return self.h[:T]

    def _forward_attn(self, T: int, record: list | None) -> torch.Tensor:
        """Attention block then MoE block per layer, in place on self.h[:T].
        Attention sits between a combine and the next routing, so the combine
        fuses with the attention's input norm instead (moe_combine_rmsnorm
        writes the block's xa)."""
        B = T // self.attn[0].P
        lengths = self.lengths[:B]
        for li, blk in enumerate(self.attn):
            if li > 0:
                k, S = self.k, self.S
                y = self.y[:T * k + S * T]
                h = self.h[:T]
                ops.moe_combine_rmsnorm(y[:T * k], self.inv[:T * k], self.tw[:T], y[T * k:] if S else None, S,
                                        h, h, blk.xa[:T], eps=blk.eps)
            rec = None if record is None else {}
            if record is not None and li > 0:
                record[-1]["output"] = self.h[:T].clone()
            blk.forward(self.h[:T], lengths, self.max_keys, rec, normed=li > 0)
            self._route(li, T, False)
            if record is not None:
                rec.update({"input": self.h[:T].clone(), "ids": self.ids[:T].clone(), "w": self.tw[:T].clone()})
                record.append(rec)
            self._experts(li, T)
        self._combine(T)
        if record is not None:
            record[-1]["output"] = self.h[:T].clone()
        return self.h[:T]

    def commit(self, B: int) -> None:
        """Advance the committed lengths by the last verify's n_commit."""
        ops.spec_commit(self.n_commit[:B], self.lengths[:B])

    def head(self, T: int) -> None:
        ops.lmhead_argmax(self.h[:T], self.w_lm, self.argmax[:T], self.max_logit[:T], self.lws)

    def verify(self, drafts: torch.Tensor) -> None:
        B, K = drafts.shape
        ops.spec_verify(drafts, self.argmax[:B * (K + 1)].view(B, K + 1), self.accepted[:B],
                        self.committed[:B], self.n_commit[:B])

    def step_planted(self, h_in: torch.Tensor, keep: torch.Tensor, repl: torch.Tensor,
                     drafts: torch.Tensor) -> None:
        """One verify pass whose drafts are planted from the pass's own greedy
        tokens (keep[b, i] -> the verifier's token, else a different id drawn
        from repl): the synthetic stand-in for a draft model of a given
        acceptance rate.  The forward pass never reads the drafts (each
        position's hidden state is an input), so planting after the LM head
        is the same as planting before the pass.  Allocates nothing, so the
        whole pass can be captured in a graph."""
        T = h_in.shape[0]
        B, K = keep.shape
        self.forward(h_in)
        self.head(T)
        ops.spec_plant_drafts(self.argmax[:B * (K + 1)].view(B, K + 1), keep, repl, self.w_lm.shape[0], drafts)
        self.verify(drafts)
        if self.attn is not None:
            self.commit(B)

    def step(self, h_in: torch.Tensor, drafts: torch.Tensor, record: list | None = None) -> None:
        """One verify pass: blocks, LM-head argmax, acceptance (results in self.*)."""
        T = h_in.shape[0]
        self.forward(h_in, record)
        self.head(T)
        self.verify(drafts)
        if self.attn is not None:
            self.commit(drafts.shape[0])
