"""A decode loop over a shrinking batch, driven through the C-ABI calls.

The concurrency-32 document workload decodes 32 pages together, about 1,085
output tokens each (alphasignal page "Jina AI's 3.4B OCR model targets
faster page parsing", section "Quality and speed").  Every pass verifies the
sequences still running, K + 1 positions each; a sequence stops once it has
`target` committed tokens (the excess of its last pass is dropped) and leaves
the batch, the others keeping their order.  With attention omitted, each
position's hidden state is an input: the loop reads pass j of sequence s
from pools laid out [S, J, ...], and drafts are planted from the pass's own
greedy tokens (VerifyStack.step_planted).

Per pass: spec_gather_rows (inputs of the active sequences) -> the verify
pass -> spec_advance (streams, stop, compaction) -> one 4-byte copy of the
number of active sequences to the host, which sizes a later pass.  The host
does not wait for that copy before it queues the next pass: pass j + 1 is
launched with the batch size known when it is queued (the count after pass
j - 1), so the GPU never idles on the round trip; spec_advance marks the slots
past the true count empty (-1) and every call skips them.  The tokens are the
same as with a wait after every pass; the lag costs the few slots that stopped
in pass j and still ride along in pass j + 1.
"""

from __future__ import annotations

import torch

from . import ops
from .step import VerifyStack


class DecodeLoop:
    def __init__(self, stack: VerifyStack, h_pool: torch.Tensor, keep_pool: torch.Tensor,
                 repl_pool: torch.Tensor, target: int):
        """h_pool [S, J, K+1, H] (the stack's dtype), keep_pool [S, J, K] uint8,
        repl_pool [S, J, K] int32; the stack must hold S sequences of K+1
        positions."""
        self.st = stack
        self.S, self.J, self.P, self.H = h_pool.shape
        self.K = self.P - 1
        if keep_pool.shape != (self.S, self.J, self.K) or repl_pool.shape != (self.S, self.J, self.K):
            raise ValueError("keep_pool / repl_pool must be [S, J, K]")
        if self.J < target:
            raise ValueError("pools must hold at least `target` passes per sequence")
        self.h_pool, self.keep_pool, self.repl_pool = h_pool, keep_pool, repl_pool
        self.target = int(target)
        dev = h_pool.device
        i32 = dict(dtype=torch.int32, device=dev)
        S, P, K = self.S, self.P, self.K
        self.h_in = torch.empty((S * P, self.H), dtype=h_pool.dtype, device=dev)
        self.keep = torch.empty((S, K), dtype=torch.uint8, device=dev)
        self.repl = torch.empty((S, K), **i32)
        self.drafts = torch.empty((S, K), **i32)
        self.seq = [torch.empty(S, **i32), torch.empty(S, **i32)]
        self.total = torch.empty(S, **i32)
        self.steps = torch.empty(S, **i32)
        self.tokens = torch.empty((S, self.target), **i32)
        self.n_active = torch.empty(1, **i32)

    def run(self, record: list | None = None, first: torch.Tensor | None = None) -> dict:
        """Decode every sequence to `target` tokens; returns the number of passes
        and the batch size of each.  With `record`, every pass's active ids,
        inputs and greedy tokens are appended to it.  With `first` [S] int32
        (the greedy token after each prompt, from the prefill), each stream
        starts with it and the loop commits the other target - 1 tokens."""
        S, P, K = self.S, self.P, self.K
        self.seq[0].copy_(torch.arange(S, dtype=torch.int32))
        self.steps.zero_()
        self.tokens.fill_(-1)
        if first is None:
            self.total.zero_()
        else:
            if self.target < 2 or first.shape != (S,) or first.dtype != torch.int32:
                raise ValueError("first must be [S] int32 and target at least 2")
            self.tokens[:, 0].copy_(first)
            self.total.fill_(1)
        if record is None:
            return self._run_lagged()
        cur, B, sizes = 0, S, []
        while B > 0:
            ids = self.seq[cur][:B]
            self._pass(ids, self.seq[1 - cur], record)
            sizes.append(B)
            B = int(self.n_active.item())
            cur = 1 - cur
        return {"passes": len(sizes), "batch_sizes": sizes}

    def _pass(self, ids: torch.Tensor, out: torch.Tensor, record: list | None = None) -> None:
        B, P = ids.shape[0], self.P
        ops.spec_gather_rows(self.h_pool, ids, self.steps, self.h_in)
        ops.spec_gather_rows(self.keep_pool, ids, self.steps, self.keep)
        ops.spec_gather_rows(self.repl_pool, ids, self.steps, self.repl)
        self.st.step_planted(self.h_in[:B * P], self.keep[:B], self.repl[:B], self.drafts[:B])
        if record is not None:
            record.append({"seq": ids.clone(), "h": self.h_in[:B * P].clone(),
                           "keep": self.keep[:B].clone(), "repl": self.repl[:B].clone(),
                           "argmax": self.st.argmax[:B * P].clone()})
        ops.spec_advance(self.st.n_commit[:B], self.st.committed[:B], ids, self.target, self.total,
                         self.steps, self.tokens, out, self.n_active)

    def _run_lagged(self) -> dict:
        """Pass j + 1 is queued before pass j's active count reaches the host.
        Launch sizes: L_0 = L_1 = S, L_{j+2} = n_j (the count after pass j);
        since n_j <= L_{j+1}, every launched slot was written by the previous
        spec_advance (an id, or -1).  Stops once some n_j is 0: pass j + 1 then
        held empty slots only and changed nothing."""
        S = self.S
        if not hasattr(self, "_pin"):
            self._pin = [torch.empty(1, dtype=torch.int32, pin_memory=True) for _ in range(2)]
            self._ev = [torch.cuda.Event(), torch.cuda.Event()]
        known, sizes, launched = [S], [], []   # known[j + 1] = n_j
        while True:
            # pass p = len(launched) may go once n_{p-2} is known
            while len(launched) <= len(known) and known[-1] > 0:
                p = len(launched)
                L = known[max(p - 1, 0)]
                self._pass(self.seq[p & 1][:L], self.seq[1 - (p & 1)])
                self._pin[p & 1].copy_(self.n_active, non_blocking=True)
                self._ev[p & 1].record()
                launched.append(L)
            r = len(known) - 1   # the pass whose count is read next
            if r >= len(launched):
                break
            self._ev[r & 1].synchronize()
            n = int(self._pin[r & 1][0])
            sizes.append(known[-1])
            known.append(n)
            if n == 0:
                break
        torch.cuda.current_stream().synchronize()
        return {"passes": len(sizes), "batch_sizes": sizes, "launched": launched}
