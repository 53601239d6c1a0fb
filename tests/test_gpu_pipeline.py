"""Prefill -> decode handoff (PagePipeline) against the oracle.

The prefill runs the decoder stack over every prompt token; each page's
first output token is the greedy token after its last prompt position, and
the decode loop continues from it.  Positions are independent (attention is
omitted, as in the verify configurations), so the oracle can check any
subset of prompt rows on its own.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests._util import BF16_TOL, F32_TOL, as_f64, assert_close, compare_ids, host
from tests.test_gpu_loop import _reference_loop

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def m():
    import moe_decoder_step_amd as mod
    mod.load()
    return mod


def _pipeline(m, sh, S, K, Lp, target, seed):
    layers = [synth.layer_weights(seed, l, sh, DEV) for l in range(sh.L)]
    w_lm = synth.lm_weight(seed, sh, DEV)
    st = m.VerifyStack(layers, w_lm, sh.E, sh.k, sh.S, max_tokens=S * (K + 1), max_seqs=S, K=K)
    h_pool = synth.normal(seed + 1, (S, target, K + 1, sh.H), 1.0, sh.torch_dtype, DEV)
    keep, repl = synth.plant_schedule(seed + 2, target, S, K, sh.V, 0.576)
    keep_pool = keep.permute(1, 0, 2).contiguous()
    repl_pool = repl.permute(1, 0, 2).contiguous()
    loop = m.DecodeLoop(st, h_pool, keep_pool.to(DEV), repl_pool.to(DEV), target)
    pipe = m.PagePipeline(st, Lp, loop)
    h_prompt = synth.normal(seed + 3, (S * Lp, sh.H), 1.0, sh.torch_dtype, DEV)
    return pipe, layers, w_lm, h_prompt, keep_pool, repl_pool


def test_tiny_pipeline(m):
    """4 pages x 9 prompt tokens, then 12 tokens per page (fp32 tiny model):
    prefill free-running against the oracle, first tokens bit-exact, the
    streams against a CPU re-run of the loop that starts from them."""
    sh = synth.SHAPES["tiny"]
    S, K, Lp, target = 4, 3, 9, 12
    pipe, layers, w_lm, h_prompt, keep_pool, repl_pool = _pipeline(m, sh, S, K, Lp, target, 20)
    rec = {}
    res = pipe.run(h_prompt, rec)
    torch.cuda.synchronize()
    hw = [{k: host(v) for k, v in w.items()} for w in layers]
    ref = O.verify_step(host(h_prompt), hw, host(w_lm), np.zeros((S * Lp, 0), np.int64), sh.k, sh.eps, "f32")
    assert_close(as_f64(rec["h_final"]), ref["layers"][-1]["h_out"], F32_TOL, "prefill output")
    last = np.arange(S) * Lp + Lp - 1
    first = rec["first"].cpu().numpy()
    compare_ids(first, ref["argmax"][last], ref["gap"][last], "first tokens")
    tokens = pipe.loop.tokens.cpu().numpy()
    np.testing.assert_array_equal(tokens[:, 0], first)
    streams, steps = _reference_loop(rec["passes"], keep_pool.numpy(), repl_pool.numpy(), target, S, first)
    np.testing.assert_array_equal(tokens, np.array(streams))
    np.testing.assert_array_equal(pipe.loop.total.cpu().numpy(), np.full(S, target))
    assert res["passes"] == len(rec["passes"])


def test_real_shape_prefill_handoff(m):
    """32 pages x 1,156 prompt tokens through the 12-layer stack (36,992
    tokens, tiled-GEMM experts), each layer teacher-forced on every page's
    last prompt row, and the first tokens from the full-vocabulary head;
    then 6 decoded tokens per page."""
    sh = synth.SHAPES["step128"]
    S, K, Lp, target = 32, 3, 1156, 6
    pipe, layers, w_lm, h_prompt, keep_pool, repl_pool = _pipeline(m, sh, S, K, Lp, target, 30)
    rec = []
    first = pipe.prefill(h_prompt, rec).clone()
    torch.cuda.synchronize()
    last = torch.arange(S, device=DEV) * Lp + Lp - 1
    for li, (r, w) in enumerate(zip(rec, layers)):
        ref = O.moe_layer(host(r["input"][last]), {k: host(v) for k, v in w.items()}, sh.k, sh.eps, "bf16")
        _, flagged = compare_ids(r["ids"][last].cpu().numpy(), ref["route"]["ids"], ref["route"]["gap"],
                                 f"layer {li} ids")
        assert_close(as_f64(r["output"][last])[~flagged], ref["h_out"][~flagged], BF16_TOL, f"layer {li} output")
    rid, _, gap = O.lm_argmax(host(pipe.pre.h[last]), host(w_lm))
    compare_ids(first.cpu().numpy(), rid, gap, "first tokens")
    passes = []
    pipe.loop.run(passes, first=first)
    torch.cuda.synchronize()
    streams, _ = _reference_loop(passes, keep_pool.numpy(), repl_pool.numpy(), target, S, first.cpu().numpy())
    np.testing.assert_array_equal(pipe.loop.tokens.cpu().numpy(), np.array(streams))
