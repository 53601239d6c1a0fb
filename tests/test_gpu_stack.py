"""Whole verify passes through the C ABI against the fp64 oracle.

Layer outputs are compared with the oracle run from the GPU's own stored
layer input (teacher forcing: a bf16 rounding difference in one layer would
otherwise be amplified by the next and make an exact-id comparison
meaningless), and the LM head from the GPU's final hidden state.  Expert ids,
argmax tokens and accepted lengths are bit-exact outside oracle near-ties.
"""

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests._util import BF16_TOL, F32_TOL, as_f64, assert_close, compare_ids, host

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def m():
    import moe_decoder_step_amd as mod
    mod.load()
    return mod


def _stack(m, sh, seed, T, device=DEV, L=None):
    layers = [synth.layer_weights(seed, l, sh, device) for l in range(L or sh.L)]
    w_lm = synth.lm_weight(seed, sh, device) if sh.V else None
    st = m.VerifyStack(layers, w_lm, sh.E, sh.k, sh.S, max_tokens=T, max_seqs=max(T // sh.P, 1), K=sh.K)
    return st, layers, w_lm


def _check_layers(record, layers, sh, mode):
    """Teacher-forced per-layer comparison; returns total near-tie flags."""
    tol = BF16_TOL if mode == "bf16" else F32_TOL
    flags = 0
    for li, (rec, w) in enumerate(zip(record, layers)):
        hw = {k: host(v) for k, v in w.items()}
        ref = O.moe_layer(host(rec["input"]), hw, sh.k, sh.eps, mode)
        n, flagged = compare_ids(rec["ids"].cpu().numpy(), ref["route"]["ids"], ref["route"]["gap"], f"layer {li} ids")
        flags += n
        ok = ~flagged
        assert_close(rec["w"].cpu().numpy()[ok], ref["route"]["w"][ok], F32_TOL, f"layer {li} weights")
        assert_close(as_f64(rec["output"])[ok], ref["h_out"][ok], tol, f"layer {li} output")
    return flags


def test_tiny_verify_pass(m):
    """1 layer, hidden 128, 8+2 experts (I=64), top-2, vocab 512, 4 x 4 tokens,
    fp32; drafts uniform from seed 0."""
    sh = synth.SHAPES["tiny"]
    st, layers, w_lm = _stack(m, sh, 0, sh.T)
    h = synth.hidden(0, sh.T, sh.H, torch.float32, DEV)
    drafts = synth.uniform_ids(0, (sh.B, sh.K), sh.V).to(DEV)
    rec = []
    st.step(h, drafts, rec)
    torch.cuda.synchronize()
    _check_layers(rec, layers, sh, "f32")
    rid, rmx, gap = O.lm_argmax(host(st.h[:sh.T]), host(w_lm))
    _, flagged = compare_ids(st.argmax[:sh.T].cpu().numpy(), rid, gap, "argmax")
    assert not flagged.any()
    racc, rcom, rnc = O.spec_verify(drafts.cpu().numpy(), rid.reshape(sh.B, sh.P))
    np.testing.assert_array_equal(st.accepted[:sh.B].cpu().numpy(), racc)
    np.testing.assert_array_equal(st.committed[:sh.B].cpu().numpy(), rcom)
    np.testing.assert_array_equal(st.n_commit[:sh.B].cpu().numpy(), rnc)
    # free-running oracle (no teacher forcing) agrees too at fp32
    full = O.verify_step(host(h), [{k: host(v) for k, v in w.items()} for w in layers], host(w_lm),
                         drafts.cpu().numpy(), sh.k, sh.eps, "f32")
    np.testing.assert_array_equal(full["argmax"], rid)
    assert_close(as_f64(st.h[:sh.T]), full["layers"][-1]["h_out"], F32_TOL, "final hidden (free-running)")


def test_real_shape_layer_128_tokens(m):
    """One real-shape layer (hidden 1280, 64+2 experts, I=896, top-6) at 32 x 4 tokens."""
    sh = synth.SHAPES["layer128"]
    st, layers, _ = _stack(m, sh, 1, sh.T)
    h = synth.hidden(2, sh.T, sh.H, torch.bfloat16, DEV)
    rec = []
    st.forward(h, rec)
    torch.cuda.synchronize()
    _check_layers(rec, layers, sh, "bf16")
    # every expert touched at least once at this batch size (the weight-bound regime)
    assert len(np.unique(rec[0]["ids"].cpu().numpy())) >= 60
    # the bf16 drift: the emulating oracle (bf16 at the storage points)
    # against the exact one (fp64 throughout), and the GPU against the exact
    # one, both at the bf16 bound, over the tokens whose experts and their
    # order are the same in both oracles (xn's bf16 rounding moves the
    # logits by ~1e-3 relative, enough to reorder close ones: 8 of 128 here)
    hw = {k: host(v) for k, v in layers[0].items()}
    emu = O.moe_layer(host(rec[0]["input"]), hw, sh.k, sh.eps, "bf16")
    exact = O.moe_layer(host(rec[0]["input"]), hw, sh.k, sh.eps, "exact")
    ok = (emu["route"]["gap"] >= 1e-6) & (exact["route"]["gap"] >= 1e-6) & \
        (emu["route"]["ids"] == exact["route"]["ids"]).all(axis=1)
    assert ok.sum() >= sh.T * 3 // 4
    assert_close(emu["h_out"][ok], exact["h_out"][ok], BF16_TOL, "bf16 drift: emulating vs exact oracle")
    assert_close(as_f64(rec[0]["output"])[ok], exact["h_out"][ok], BF16_TOL, "layer output vs exact oracle")


@pytest.mark.timeout(900)
def test_batch1_stack_teacher_forced_200_steps(m):
    """Batch-1 verify, 200 steps with seeds 0..199: 12 layers + LM head
    1280 x 129,280 at 1 x 4 tokens.  Every step's blocks are teacher-forced
    (the oracle reads each block's stored input), its argmax comes from the
    GPU's final hidden state, and its drafts are planted from the oracle's own
    argmax (keep probability 0.576).  Acceptance of all 200 steps runs as one
    spec_verify call over 200 sequences.  The oracle runs once per layer over
    the 800 rows of all steps."""
    sh = synth.SHAPES["batch1"]
    steps = 200
    st, layers, w_lm = _stack(m, sh, 0, sh.T)
    keep, repl = synth.plant_schedule(0, steps, sh.B, sh.K, sh.V, 0.576)
    recs, finals, am = [], [], []
    for s in range(steps):
        h = synth.hidden(s, sh.T, sh.H, torch.bfloat16, DEV, name="step_hidden")
        rec = []
        st.forward(h, rec)
        st.head(sh.T)
        recs.append(rec)
        finals.append(st.h[:sh.T].clone())
        am.append(st.argmax[:sh.T].clone())
    torch.cuda.synchronize()
    flags = 0
    bad_step = np.zeros(steps, dtype=bool)
    for li, w in enumerate(layers):
        hw = {key: host(v) for key, v in w.items()}
        inp = torch.cat([r[li]["input"] for r in recs])
        ref = O.moe_layer(host(inp), hw, sh.k, sh.eps, "bf16")
        n, flagged = compare_ids(torch.cat([r[li]["ids"] for r in recs]).cpu().numpy(), ref["route"]["ids"],
                                 ref["route"]["gap"], f"layer {li} ids")
        flags += n
        ok = ~flagged
        bad_step |= flagged.reshape(steps, sh.T).any(axis=1)
        assert_close(torch.cat([r[li]["w"] for r in recs]).cpu().numpy()[ok], ref["route"]["w"][ok], F32_TOL,
                     f"layer {li} weights")
        assert_close(as_f64(torch.cat([r[li]["output"] for r in recs]))[ok], ref["h_out"][ok], BF16_TOL,
                     f"layer {li} output")
    rid, rmx, gap = O.lm_argmax(host(torch.cat(finals)), host(w_lm))
    got = torch.cat(am).cpu().numpy()
    n, flagged = compare_ids(got, rid, gap, "argmax")
    flags += n
    bad_step |= flagged.reshape(steps, sh.T).any(axis=1)
    print(f"\nnear-tie flags over 200 steps: {flags}; steps excluded from acceptance: {int(bad_step.sum())}")
    g = rid.reshape(steps, sh.P)
    drafts = O.plant_drafts(g, keep[:, 0].numpy(), repl[:, 0].numpy())
    acc, com, nc = m.verify_alloc(torch.from_numpy(drafts.astype(np.int32)).to(DEV),
                                  torch.from_numpy(got.reshape(steps, sh.P).astype(np.int32)).to(DEV))
    torch.cuda.synchronize()
    racc, rcom, rnc = O.spec_verify(drafts, g)
    oks = ~bad_step
    np.testing.assert_array_equal(acc.cpu().numpy()[oks], racc[oks])
    np.testing.assert_array_equal(com.cpu().numpy()[oks], rcom[oks])
    np.testing.assert_array_equal(nc.cpu().numpy()[oks], rnc[oks])
    # planted drafts: accepted = leading keeps, whatever the model
    kp = keep[:, 0].numpy().astype(bool)
    lead = np.array([next((i for i in range(sh.K) if not kp[s, i]), sh.K) for s in range(steps)])
    np.testing.assert_array_equal(racc, lead)
    # committed per pass: mean within 3 standard errors of 1 + p + p^2 + p^3
    p = 0.576
    mean = 1 + p + p * p + p ** 3
    second = 1 + 3 * p + 5 * p * p + 7 * p ** 3          # E[(n+1)^2] for n = leading keeps of K = 3
    se = np.sqrt((second - mean * mean) / steps)
    assert abs(rnc.mean() - mean) < 3 * se, (rnc.mean(), mean, se)


def test_full_step_128_tokens(m):
    """The benchmarked workload: 12 layers + LM head + acceptance at 32 x 4 tokens."""
    sh = synth.SHAPES["step128"]
    st, layers, w_lm = _stack(m, sh, 0, sh.T)
    h = synth.hidden(0, sh.T, sh.H, torch.bfloat16, DEV, name="step_hidden")
    drafts = synth.uniform_ids(0, (sh.B, sh.K), sh.V).to(DEV)
    rec = []
    st.step(h, drafts, rec)
    torch.cuda.synchronize()
    _check_layers(rec, layers, sh, "bf16")
    rid, rmx, gap = O.lm_argmax(host(st.h[:sh.T]), host(w_lm))
    _, flagged = compare_ids(st.argmax[:sh.T].cpu().numpy(), rid, gap, "argmax")
    assert_close(st.max_logit[:sh.T].cpu().numpy()[~flagged], rmx[~flagged], F32_TOL, "max logit")
    racc, rcom, rnc = O.spec_verify(drafts.cpu().numpy(), st.argmax[:sh.T].cpu().numpy().reshape(sh.B, sh.P))
    np.testing.assert_array_equal(st.accepted[:sh.B].cpu().numpy(), racc)
    np.testing.assert_array_equal(st.n_commit[:sh.B].cpu().numpy(), rnc)


def test_determinism_and_batch_invariance(m):
    """Two runs are bit-identical, and a token's result does not depend on the
    other tokens of its batch (needed for speculative == greedy on the GPU)."""
    sh = synth.SHAPES["step128"]
    st, layers, w_lm = _stack(m, sh, 0, sh.T, L=3)
    h = synth.hidden(9, sh.T, sh.H, torch.bfloat16, DEV)
    st.forward(h)
    st.head(sh.T)
    out1, ids1 = st.h[:sh.T].clone(), st.argmax[:sh.T].clone()
    st.forward(h)
    st.head(sh.T)
    assert torch.equal(out1, st.h[:sh.T]) and torch.equal(ids1, st.argmax[:sh.T])
    for sub in (slice(0, 4), slice(60, 61), slice(100, 128)):
        hs = h[sub].contiguous()
        n = hs.shape[0]
        st.forward(hs)
        st.head(n)
        torch.cuda.synchronize()
        assert torch.equal(st.h[:n], out1[sub]), f"hidden of rows {sub} depends on the batch"
        assert torch.equal(st.argmax[:n], ids1[sub])


@pytest.mark.parametrize("shape,T,L", [("step128", 128, 3), ("step128", 4, 2), ("tiny", 16, 1), ("step128", 256, 2),
                                       ("step128", 300, 2)])
def test_fused_combine_route_matches_separate_calls(m, shape, T, L):
    """moe_combine_route (each block's combine fused with the next block's
    routing) gives the same hidden states, ids and weights as moe_combine
    followed by moe_route, bit for bit."""
    sh = synth.SHAPES[shape]
    st, layers, w_lm = _stack(m, sh, 2, T, L=L)
    h = synth.hidden(13, T, sh.H, sh.torch_dtype, DEV)
    outs = []
    for fuse in (True, False):
        st.fuse = fuse
        rec = []
        st.forward(h, rec)
        torch.cuda.synchronize()
        outs.append(rec)
    for a, b in zip(*outs):
        for key in ("input", "ids", "w", "output"):
            assert torch.equal(a[key], b[key]), key

