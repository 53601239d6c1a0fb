"""Speculative decoding commits exactly the tokens of step-by-step greedy
decoding, on the GPU through the C ABI.

The pages' central property of FastMTP with greedy verification: the output
is token-identical with speculation on or off ("Jina AI's 3.4B OCR model
targets faster page parsing", section "FastMTP cuts decoding work"; jina.ai/de
"jina-ocr-v1: Schnellere Dokumentenanalyse auf kostenguenstigen GPUs",
section "Modell und Training").  A token-driven model runs entirely in the
library's kernels: a token's input row is the RMSNorm of its embedding row
(moe_rmsnorm over gathered rows), then the stack's blocks, the LM-head argmax
and spec_verify.  Greedy decoding runs one position per sequence per pass;
speculative decoding runs the last committed token plus K drafts per
sequence.  Drafts are random (mostly rejected), planted from the greedy
continuation with keep probability 0.576, or the continuation itself (all
accepted).  Both loops are plain host loops over device passes.
"""

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def m():
    import moe_decoder_step_amd as mod
    mod.load()
    return mod


class TokenModel:
    """tokens -> rmsnorm(emb[tok]) -> stack blocks -> argmax -> acceptance."""

    def __init__(self, m, stack, emb, B, P):
        self.m, self.st, self.emb, self.B, self.P = m, stack, emb, B, P
        self.hin = torch.empty((B * P, emb.shape[1]), dtype=emb.dtype, device=DEV)

    def run(self, tokens: np.ndarray, drafts: np.ndarray):
        """One pass over tokens [B, P] (position 0 the last committed token,
        then the drafts [B, P-1]); returns (committed [B, P], n_commit [B])."""
        B, P = tokens.shape
        T = B * P
        rows = torch.from_numpy(tokens.reshape(-1).astype(np.int32)).to(DEV)
        self.m.moe_rmsnorm(self.emb, self.hin[:T], rows=rows)
        d = torch.from_numpy(drafts.astype(np.int32)).to(DEV).view(B, P - 1)
        self.st.step(self.hin[:T], d)
        com = self.st.committed[:B].cpu().numpy()
        nc = self.st.n_commit[:B].cpu().numpy()
        return com, nc


def greedy(model: TokenModel, first: np.ndarray, n: int):
    """n greedy tokens after `first` for every sequence, one per pass."""
    B = first.shape[0]
    seqs = [[int(t)] for t in first]
    for _ in range(n):
        last = np.array([[s[-1]] for s in seqs])
        com, nc = model.run(last, np.zeros((B, 0), np.int64))
        assert np.all(nc == 1)
        for b in range(B):
            seqs[b].append(int(com[b, 0]))
    return seqs


def speculative(model: TokenModel, first: np.ndarray, n: int, K: int, propose):
    """Speculative decoding until every sequence holds n tokens after `first`.
    Every sequence stays in the batch until the last one is done (its cache
    positions keep advancing; only the first n tokens are compared)."""
    B = first.shape[0]
    seqs = [[int(t)] for t in first]
    passes = 0
    commits = []
    while min(len(s) for s in seqs) < n + 1:
        d = np.array([propose(b, seqs[b], K) for b in range(B)], dtype=np.int64).reshape(B, K)
        tokens = np.concatenate([np.array([[s[-1]] for s in seqs]), d], axis=1)
        com, nc = model.run(tokens, d)
        assert np.all((nc >= 1) & (nc <= K + 1))
        for b in range(B):
            seqs[b].extend(int(x) for x in com[b, :nc[b]])
        commits.append(nc)
        passes += 1
    return [s[:n + 1] for s in seqs], passes, np.concatenate(commits)


def _proposers(V, ref, seed):
    rng = np.random.default_rng(seed)

    def rand(b, s, K):
        return rng.integers(0, V, K)

    def planted(b, s, K):
        truth = (ref[b][len(s):len(s) + K] + [0] * K)[:K]
        return [t if rng.random() < 0.576 else int(rng.integers(0, V)) for t in truth]

    def perfect(b, s, K):
        return (ref[b][len(s):len(s) + K] + [0] * K)[:K]
    return {"random": rand, "planted": planted, "perfect": perfect}


def _check(m, make_stack, emb, V, B, n, K, seed):
    g_model = TokenModel(m, make_stack(0), emb, B, 1)
    first = np.random.default_rng(seed).integers(0, V, B)
    ref = greedy(g_model, first, n)
    assert any(len(set(s)) > 3 for s in ref), "degenerate greedy streams"
    s_model_factory = lambda: TokenModel(m, make_stack(K), emb, B, K + 1)  # noqa: E731
    for name, prop in _proposers(V, ref, seed + 1).items():
        s_model = s_model_factory()
        got, passes, commits = speculative(s_model, first, n, K, prop)
        for b in range(B):
            assert got[b] == ref[b], f"{name} drafts: sequence {b} differs at {next(i for i in range(n + 1) if got[b][i] != ref[b][i])}"
        if name == "perfect":
            assert passes <= -(-n // (K + 1)) + 1
        if name == "planted":
            assert commits.mean() > 1.2
        del s_model
        torch.cuda.empty_cache()


def test_speculative_equals_greedy_tiny_f32(m):
    """The tiny fp32 model (1 layer, hidden 128, 8+2 experts, top-2, vocab
    512), 4 sequences, K = 3, 40 tokens each."""
    sh = synth.SHAPES["tiny"]
    layers = [synth.layer_weights(0, 0, sh, DEV)]
    w_lm = synth.lm_weight(0, sh, DEV)
    emb = synth.normal(synth.subseed(0, "emb"), (sh.V, sh.H), 1.0, torch.float32, DEV)
    B, K = 4, 3

    def make(Kp):
        return m.VerifyStack(layers, w_lm, sh.E, sh.k, sh.S, max_tokens=B * (Kp + 1), max_seqs=B, K=Kp)
    _check(m, make, emb, sh.V, B, 40, K, 3)


def test_speculative_equals_greedy_real_shape_12_layers(m):
    """The real-shape stack (12 layers, hidden 1280, 64+2 experts, top-6,
    vocabulary 129,280, bf16), 8 sequences, K = 3, 24 tokens each: greedy
    passes of 8 rows against verify passes of 32."""
    sh = synth.SHAPES["step128"]
    layers = [synth.layer_weights(0, l, sh, DEV) for l in range(sh.L)]
    w_lm = synth.lm_weight(0, sh, DEV)
    emb = synth.normal(synth.subseed(0, "emb"), (sh.V, sh.H), 1.0, torch.bfloat16, DEV)
    B, K = 8, 3
    base = m.VerifyStack(layers, w_lm, sh.E, sh.k, sh.S, max_tokens=B * (K + 1), max_seqs=B, K=K)
    del layers

    def make(Kp):
        return base.sibling(B * (Kp + 1), B, Kp)
    _check(m, make, emb, sh.V, B, 24, K, 5)


def test_speculative_equals_greedy_with_attention(m):
    """Two real-shape layers with causal attention over a KV cache before
    each MoE block (10 heads of 128), LM head 129,280: greedy passes of one
    position against verify passes of K + 1 = 4 positions whose rejected
    drafts are rolled back.  4 sequences from an empty cache, 20 tokens each."""
    sh = synth.SHAPES["step128"]
    nL, nh = 2, sh.H // synth.ATTN_HEAD_DIM
    layers = [synth.layer_weights(1, l, sh, DEV) for l in range(nL)]
    attn = [synth.attn_weights(1, l, sh, DEV) for l in range(nL)]
    w_lm = synth.lm_weight(1, sh, DEV)
    emb = synth.normal(synth.subseed(1, "emb"), (sh.V, sh.H), 1.0, torch.bfloat16, DEV)
    B, K, n = 4, 3, 20
    # the slowest sequence commits >= 1 token per pass and the loop runs until
    # it holds n, so a sequence's cache never passes (n + 1) (K + 1) + K + 1
    max_len = (n + 2) * (K + 1)

    def make(Kp):
        st = m.VerifyStack(layers, w_lm, sh.E, sh.k, sh.S, max_tokens=B * (Kp + 1), max_seqs=B, K=Kp, attn=attn,
                           n_heads=nh, max_len=max_len)
        st.lengths.zero_()
        return st
    _check(m, make, emb, sh.V, B, n, K, 7)
