"""The dense draft block (FastMTP) and its row RMSNorm against the fp64 oracle.

Each recursive step is compared teacher-forced: the oracle runs the step
from the GPU's own stored inputs (hidden state and token), so a rounding
difference in one step cannot reach the next.  Draft ids are bit-exact
outside oracle near-ties (top-1 minus top-2 logit gap below 1e-6).
"""

import dataclasses

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


@pytest.mark.parametrize("dtype,H", [(torch.bfloat16, 1280), (torch.float32, 128), (torch.bfloat16, 136)])
def test_rmsnorm_rows(m, dtype, H):
    """Plain rows, gathered rows and a strided output, against the oracle's
    RMSNorm rounded once to the storage type (bit-exact)."""
    mode = "bf16" if dtype == torch.bfloat16 else "f32"
    x = synth.normal(5, (300, H), 1.0, dtype, DEV)
    out = torch.empty((300, 2 * H), dtype=dtype, device=DEV)
    m.moe_rmsnorm(x, out[:, :H])
    rows = torch.tensor(np.random.default_rng(6).integers(0, 300, 77), dtype=torch.int32, device=DEV)
    out2 = torch.empty((77, H), dtype=dtype, device=DEV)
    m.moe_rmsnorm(x, out2, rows=rows)
    torch.cuda.synchronize()
    ref = O.store(O.rmsnorm(O.f64(host(x)), 1e-6), mode)
    np.testing.assert_array_equal(as_f64(out[:, :H]), ref)
    np.testing.assert_array_equal(as_f64(out2), ref[rows.cpu().numpy()])


def test_rmsnorm_matches_route_norm(m):
    """moe_rmsnorm and moe_route's RMSNorm give the same bits."""
    sh = synth.SHAPES["layer128"]
    w = synth.layer_weights(1, 0, sh, DEV)
    h = synth.hidden(8, 128, sh.H, torch.bfloat16, DEV)
    xn, _, _, _ = m.route_alloc(h, w["w_router"], None, sh.k)
    out = torch.empty_like(h)
    m.moe_rmsnorm(h, out)
    torch.cuda.synchronize()
    assert torch.equal(out, xn)


@pytest.mark.parametrize("shape,B,K", [("step128", 32, 3), ("step128", 1, 3), ("tiny", 4, 2)])
def test_draft_steps_teacher_forced(m, shape, B, K):
    sh = synth.SHAPES[shape]
    I = synth.DRAFT_INTERMEDIATE if shape == "step128" else 64
    dw = synth.draft_weights(4, sh, DEV, I=I)
    w_lm = synth.lm_weight(4, sh, DEV)
    head = m.DraftHead(dw, m.lm_weights(w_lm), max_seqs=B, K=K)
    h = synth.hidden(9, B, sh.H, sh.torch_dtype, DEV)
    tok = synth.uniform_ids(10, (B,), sh.V).to(DEV)
    rec = []
    drafts = head.propose(h, tok, rec).contiguous()
    torch.cuda.synchronize()
    mode, tol = (sh.dtype, BF16_TOL if sh.dtype == "bf16" else F32_TOL)
    wts = {"emb": host(dw["emb"]), "w_proj": host(dw["w_proj"]), "w_gate_up": host(dw["w_gate_up"])[0],
           "w_down": host(dw["w_down"])[0]}
    wl = host(w_lm)
    assert len(rec) == K
    for i, st in enumerate(rec):
        ref = O.draft_step(host(st["h"]), st["tok"].cpu().numpy(), wts, wl, sh.eps, mode)
        assert_close(as_f64(st["h0"]), ref["h0"], tol, f"step {i} projection")
        assert_close(as_f64(st["h1"]), ref["h1"], tol, f"step {i} block output")
        compare_ids(st["ids"].cpu().numpy(), ref["ids"], ref["gap"], f"step {i} drafts")
        np.testing.assert_array_equal(drafts[:, i].cpu().numpy(), st["ids"].cpu().numpy())
        if i + 1 < K:   # recursion: the next step reads this step's output and draft
            assert torch.equal(rec[i + 1]["h"], st["h1"]) and torch.equal(rec[i + 1]["tok"], st["ids"])
