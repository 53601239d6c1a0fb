"""The decode loop over a shrinking batch (spec_gather_rows, the verify pass,
spec_advance) against a re-run of its bookkeeping on the CPU.

The greedy tokens of each pass are checked against the oracle (the tiny fp32
stack, teacher forced from the pass's gathered inputs, ids bit-exact outside
near-ties).  Given those tokens, everything else is integer work with one
right answer, so the CPU re-run is exact: which sequences run in each pass
and in what order, the inputs each one reads, its planted drafts and
accepted length, its committed stream cut at the target, its pass count.
"""

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests._util import compare_ids, host

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def m():
    import moe_decoder_step_amd as mod
    mod.load()
    return mod


def _reference_loop(passes, keep_pool, repl_pool, target, S, first=None):
    """Bookkeeping of the loop from each pass's greedy tokens g (oracle side);
    with `first`, every stream starts with that sequence's token."""
    K = keep_pool.shape[2]
    active = list(range(S))
    total = [0 if first is None else 1] * S
    steps = [0] * S
    streams = [[] if first is None else [int(first[s])] for s in range(S)]
    for p in passes:
        assert p["seq"].cpu().numpy().tolist() == active
        g = p["argmax"].cpu().numpy().reshape(len(active), K + 1).astype(np.int64)
        keep = np.stack([keep_pool[s, steps[s]] for s in active])
        repl = np.stack([repl_pool[s, steps[s]] for s in active])
        np.testing.assert_array_equal(p["keep"].cpu().numpy(), keep)
        np.testing.assert_array_equal(p["repl"].cpu().numpy(), repl)
        d = O.plant_drafts(g, keep, repl)
        _, com, nc = O.spec_verify(d, g)
        nxt = []
        for i, s in enumerate(active):
            take = min(int(nc[i]), target - total[s])
            streams[s].extend(int(t) for t in com[i, :take])
            total[s] += take
            steps[s] += 1
            if total[s] < target:
                nxt.append(s)
        active = nxt
    assert not active
    return streams, steps


@pytest.mark.parametrize("S,target,K", [(6, 20, 3), (5, 9, 1), (3, 7, 0)])
def test_decode_loop_matches_cpu_rerun(m, S, target, K):
    import dataclasses
    sh = dataclasses.replace(synth.SHAPES["tiny"], B=S, P=K + 1)
    layers = [synth.layer_weights(3, l, sh, DEV) for l in range(sh.L)]
    w_lm = synth.lm_weight(3, sh, DEV)
    st = m.VerifyStack(layers, w_lm, sh.E, sh.k, sh.S, max_tokens=sh.T, max_seqs=S, K=K)
    J = target
    h_pool = synth.normal(11, (S, J, K + 1, sh.H), 1.0, torch.float32, DEV)
    keep, repl = synth.plant_schedule(12, J, S, K, sh.V, 0.576)           # [J, S, K]
    keep_pool = keep.permute(1, 0, 2).contiguous()
    repl_pool = repl.permute(1, 0, 2).contiguous()
    loop = m.DecodeLoop(st, h_pool, keep_pool.to(DEV), repl_pool.to(DEV), target)
    rec = []
    res = loop.run(rec)
    torch.cuda.synchronize()
    assert res["passes"] == len(rec) and res["batch_sizes"][0] == S
    # every pass read the right inputs, and its greedy tokens match the oracle
    hp = host(h_pool)
    steps = [0] * S
    hw = [{k: host(v) for k, v in w.items()} for w in layers]
    for p in rec:
        ids = p["seq"].cpu().numpy()
        want = np.concatenate([hp[s, steps[s]] for s in ids])
        np.testing.assert_array_equal(host(p["h"]), want)
        ref = O.verify_step(want, hw, host(w_lm), np.zeros((len(ids), K), np.int64), sh.k, sh.eps, "f32")
        compare_ids(p["argmax"].cpu().numpy(), ref["argmax"], ref["gap"], "pass argmax")
        # steps advance for the sequences that ran (the CPU re-run checks the rest)
        for s in ids:
            steps[s] += 1
    streams, ref_steps = _reference_loop(rec, keep_pool.numpy(), repl_pool.numpy(), target, S)
    np.testing.assert_array_equal(loop.tokens.cpu().numpy(), np.array(streams))
    np.testing.assert_array_equal(loop.total.cpu().numpy(), np.full(S, target))
    np.testing.assert_array_equal(loop.steps.cpu().numpy(), np.array(ref_steps))


@pytest.mark.parametrize("S,target,K", [(6, 20, 3), (7, 11, 1), (4, 9, 0)])
def test_lagged_loop_matches_waiting_loop(m, S, target, K):
    """The loop that queues pass j + 1 before pass j's count is back (empty
    slots marked -1) commits the same streams in the same passes as the loop
    that waits after every pass; it launches at most one extra pass."""
    import dataclasses
    sh = dataclasses.replace(synth.SHAPES["tiny"], B=S, P=K + 1)
    layers = [synth.layer_weights(5, l, sh, DEV) for l in range(sh.L)]
    w_lm = synth.lm_weight(5, sh, DEV)
    st = m.VerifyStack(layers, w_lm, sh.E, sh.k, sh.S, max_tokens=sh.T, max_seqs=S, K=K)
    h_pool = synth.normal(13, (S, target, K + 1, sh.H), 1.0, torch.float32, DEV)
    keep, repl = synth.plant_schedule(14, target, S, K, sh.V, 0.576)
    loop = m.DecodeLoop(st, h_pool, keep.permute(1, 0, 2).contiguous().to(DEV),
                        repl.permute(1, 0, 2).contiguous().to(DEV), target)
    rec = []
    want = loop.run(rec)
    tok, tot, stp = (host(t).copy() for t in (loop.tokens, loop.total, loop.steps))
    for _ in range(2):   # twice: the second run reuses the pinned counts
        got = loop.run()
        assert got["passes"] == want["passes"] and got["batch_sizes"] == want["batch_sizes"]
        assert len(got["launched"]) <= want["passes"] + 1
        assert all(a >= b for a, b in zip(got["launched"], want["batch_sizes"]))
        np.testing.assert_array_equal(host(loop.tokens), tok)
        np.testing.assert_array_equal(host(loop.total), tot)
        np.testing.assert_array_equal(host(loop.steps), stp)
