"""Verify passes (batch 1 and 32 x 4 tokens) and the prefill layer captured
in a HIP graph and replayed.

The whole pass (12 MoE layers, LM-head argmax, draft planting, acceptance)
is captured once over static buffers.  Each replay gets new inputs copied
into those buffers; its outputs must equal an eager run of the same inputs
bit for bit, with eager work on the same stream between the replays.  The
accepted lengths are also checked against the oracle's planting and
acceptance rules applied to the GPU's own greedy tokens.
"""

import numpy as np
import pytest
import torch

import oracle as O
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def m():
    import moe_decoder_step_amd as mod
    mod.load()
    return mod


@pytest.mark.parametrize("shape,K", [("batch1", 3), ("batch1", 1), ("step128", 3)])
def test_graph_replay_matches_eager(m, shape, K):
    import dataclasses
    sh = dataclasses.replace(synth.SHAPES[shape], P=K + 1)
    layers = [synth.layer_weights(0, l, sh, DEV) for l in range(sh.L)]
    w_lm = synth.lm_weight(0, sh, DEV)
    st = m.VerifyStack(layers, w_lm, sh.E, sh.k, sh.S, max_tokens=sh.T, max_seqs=sh.B, K=sh.K)
    keep_all, repl_all = synth.plant_schedule(5, 4, sh.B, sh.K, sh.V, 0.576)
    h_s = synth.hidden(100, sh.T, sh.H, torch.bfloat16, DEV)
    keep_s, repl_s = keep_all[0].to(DEV), repl_all[0].to(DEV)
    drafts = torch.zeros((sh.B, sh.K), dtype=torch.int32, device=DEV)

    def outputs():
        return [t.clone() for t in (st.h[:sh.T], st.argmax[:sh.T], drafts, st.accepted[:sh.B],
                                    st.committed[:sh.B], st.n_commit[:sh.B])]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.step_planted(h_s, keep_s, repl_s, drafts)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st.step_planted(h_s, keep_s, repl_s, drafts)

    for i in range(4):
        h_i = synth.hidden(200 + i, sh.T, sh.H, torch.bfloat16, DEV)
        h_s.copy_(h_i)
        keep_s.copy_(keep_all[i].to(DEV))
        repl_s.copy_(repl_all[i].to(DEV))
        graph.replay()
        got = outputs()
        # eager run of the same inputs, on the same buffers
        st.step_planted(h_i, keep_all[i].to(DEV), repl_all[i].to(DEV), drafts)
        ref = outputs()
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"replay {i} differs from the eager pass"
        # planting and acceptance against the oracle, on the GPU's greedy tokens
        g = got[1].cpu().numpy().reshape(sh.B, sh.K + 1).astype(np.int64)
        d = O.plant_drafts(g, keep_all[i].numpy(), repl_all[i].numpy())
        np.testing.assert_array_equal(got[2].cpu().numpy(), d)
        acc, com, nc = O.spec_verify(d, g)
        np.testing.assert_array_equal(got[3].cpu().numpy(), acc)
        np.testing.assert_array_equal(got[4].cpu().numpy(), com)
        np.testing.assert_array_equal(got[5].cpu().numpy(), nc)
        lead = np.cumprod(keep_all[i].numpy().astype(bool), axis=1).sum(axis=1)
        np.testing.assert_array_equal(acc, lead)


def test_prefill_layer_graph_replay_matches_eager(m):
    """One 36,992-token layer (multi-pass permute, both MFMA GEMMs, 32-token
    route, combine) captured once; three replays on new hidden states, each
    equal bit for bit to an eager pass of the same input run between them."""
    sh = synth.SHAPES["prefill"]
    w = synth.layer_weights(1, 0, sh, DEV)
    st = m.VerifyStack([w], None, sh.E, sh.k, sh.S, max_tokens=sh.T)
    h_s = synth.hidden(300, sh.T, sh.H, torch.bfloat16, DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.forward(h_s)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st.forward(h_s)
    for i in range(3):
        h_i = synth.hidden(301 + i, sh.T, sh.H, torch.bfloat16, DEV)
        h_s.copy_(h_i)
        graph.replay()
        got = [t.clone() for t in (st.h[:sh.T], st.ids[:sh.T], st.tw[:sh.T])]
        st.forward(h_i)
        ref = [t.clone() for t in (st.h[:sh.T], st.ids[:sh.T], st.tw[:sh.T])]
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"replay {i} differs from the eager pass"
