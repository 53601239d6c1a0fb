"""Prefill -> decode handoff for a batch of pages, driven through the C-ABI
calls.

The concurrency-32 document workload parses 32 pages together: each page's
prompt of up to 1,156 visual tokens goes through the decoder once (prefill),
then about 1,085 output tokens are decoded per page (alphasignal page "Jina
AI's 3.4B OCR model targets faster page parsing", sections "A compressed
visual front end" and "Quality and speed").  With attention omitted, as in
the verify configurations, the handoff from prefill to decode is the first
output token: the greedy token after each page's last prompt position.

    prefill   12 MoE layers over all S x Lp prompt tokens (the tiled-GEMM
              expert path at this size), one stack over the decode stack's
              packed weights
    handoff   spec_gather_rows picks each page's last prompt row;
              lmhead_argmax gives its greedy token, the first of the stream
    decode    DecodeLoop from those tokens to `target` tokens per page
"""

from __future__ import annotations

import torch

from . import ops
from .loop import DecodeLoop
from .step import VerifyStack


class PagePipeline:
    def __init__(self, stack: VerifyStack, prompt_len: int, loop: DecodeLoop):
        """stack: the decode stack (its packed weights are shared with the
        prefill); loop: the decode loop over the same S pages."""
        self.st, self.loop = stack, loop
        self.S, self.Lp = loop.S, int(prompt_len)
        T = self.S * self.Lp
        self.pre = stack.sibling(T)
        dev = stack.device
        i32 = dict(dtype=torch.int32, device=dev)
        self.seq = torch.arange(self.S, **i32)
        self.last = torch.full((self.S,), self.Lp - 1, **i32)
        self.h_last = torch.empty((self.S, stack.H), dtype=stack.dtype, device=dev)
        self.first = torch.empty(self.S, **i32)
        self.first_logit = torch.empty(self.S, dtype=torch.float32, device=dev)
        self.lws = torch.empty(max(ops.lmhead_workspace_bytes(self.S, stack.V, stack.dtype), 16),
                               dtype=torch.uint8, device=dev)

    def prefill(self, h_prompt: torch.Tensor, record: list | None = None) -> torch.Tensor:
        """h_prompt [S*Lp, H] (page-major): the stack over every prompt token,
        then the greedy token after each page's last one (returned, [S]).
        `record` is passed to VerifyStack.forward."""
        if h_prompt.shape != (self.S * self.Lp, self.st.H):
            raise ValueError("h_prompt must be [S * prompt_len, H]")
        h = self.pre.forward(h_prompt, record)
        ops.spec_gather_rows(h.view(self.S, self.Lp, 1, self.st.H), self.seq, self.last, self.h_last)
        ops.lmhead_argmax(self.h_last, self.st.w_lm, self.first, self.first_logit, self.lws)
        return self.first

    def run(self, h_prompt: torch.Tensor, record: dict | None = None) -> dict:
        """Prefill, then decode every page to the loop's target."""
        self.prefill(h_prompt)
        if record is not None:
            record["h_final"] = self.pre.h[:self.S * self.Lp].clone()
            record["first"] = self.first.clone()
            record["passes"] = []
        res = self.loop.run(None if record is None else record["passes"], first=self.first)
        return res
