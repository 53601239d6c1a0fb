"""A token row's expert FFN and layer output do not depend on its batch.

The grouped SwiGLU has three forms chosen by batch size: the routed
weight-streaming launch (permutation derived in the gate/up kernel, up to
4,096 (token, slot) pairs), the weight-streaming launch over a separate
permutation (items of 16, 32 or 64 rows), and the tiled MFMA GEMM from 1,024
rows per group.  All use the same MFMA k-order and the same SiLU, so a
token row gets the same bits in each.  Speculative decoding verifies
B x (K+1) positions in a pass where greedy decoding runs B x 1, so the
committed tokens can only equal greedy decoding's if a row's result is
independent of the batch it rides in.
"""

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests._util import BF16_TOL, as_f64, assert_close, host

pytestmark = pytest.mark.gpu

DEV = "cuda"
ROW_TOKENS = 16        # the rows compared: the first 16 tokens of every batch


@pytest.fixture(scope="module")
def m():
    import moe_decoder_step_amd as mod
    mod.load()
    return mod


def _ffn(m, sh, xn, ids, wgu, wd, routed):
    """act and y of one batch through the chosen form; returns (act, y, inv)."""
    T = xn.shape[0]
    k, E, S = sh.k, sh.E, sh.S
    n_rows = T * k + S * T
    act = torch.full((n_rows, sh.I), float("nan"), dtype=torch.bfloat16, device=DEV)
    y = torch.full((n_rows, sh.H), float("nan"), dtype=torch.bfloat16, device=DEV)
    off = torch.empty(E + S + 1, dtype=torch.int32, device=DEV)
    inv = torch.empty(T * k, dtype=torch.int32, device=DEV)
    if routed:
        m.moe_expert_gate_up_routed(xn, ids, E, S, wgu, act, off, inv.view(T, k))
    else:
        gat = torch.empty(n_rows, dtype=torch.int32, device=DEV)
        nb = m.permute_workspace_bytes(T, k, E)
        ws = torch.empty(nb, dtype=torch.uint8, device=DEV) if nb else None
        m.moe_permute(ids, E, S, off, gat, inv, ws)
        m.moe_expert_gate_up(xn, gat, off, wgu, act, max_rows=T)
    m.moe_expert_down(act, off, wd, y, max_rows=T)
    torch.cuda.synchronize()
    return act, y, inv


def _token_rows(sh, T, inv, t):
    """Rows of token t: its k routed slots (through inv), then its S shared rows."""
    k = sh.k
    return [int(r) for r in inv[t * k:(t + 1) * k]] + [T * k + s * T + t for s in range(sh.S)]


def test_expert_rows_bit_identical_across_ffn_forms(m):
    """The first 16 tokens' activation and output rows are the same bits at
    16 tokens (routed streaming), 128 (routed, multi-row items for the shared
    experts), 700 (streaming over a permutation, 4,200 pairs), 1,024 and 2,048
    (tiled GEMM).  The 16-token result is also checked against the oracle."""
    import moe_decoder_step_amd.ops as ops
    sh = synth.SHAPES["layer128"]
    w = synth.layer_weights(4, 0, sh, DEV)
    wgu, wd = m.expert_weights(w["w_gate_up"], w["w_down"])
    Tmax = 2048
    h = synth.hidden(31, Tmax, sh.H, torch.bfloat16, DEV)
    xn, ids, tw, _ = m.route_alloc(h, w["w_router"], None, sh.k)
    torch.cuda.synchronize()
    ref = None
    forms = [(16, True), (16, False), (128, True), (700, False), (1024, False), (2048, False)]
    for T, routed in forms:
        assert not routed or T * sh.k <= ops.ROUTED_MAX_PAIRS
        act, y, inv = _ffn(m, sh, xn[:T].contiguous(), ids[:T].contiguous(), wgu, wd, routed)
        inv_h = inv.cpu().numpy()
        rows = [_token_rows(sh, T, inv_h, t) for t in range(ROW_TOKENS)]
        got_a = torch.stack([act[r] for rr in rows for r in rr])
        got_y = torch.stack([y[r] for rr in rows for r in rr])
        if ref is None:
            ref = (got_a, got_y)
            # the reference rows against the oracle, expert by expert
            ids_h = ids[:ROW_TOKENS].cpu().numpy()
            xh = O.f64(host(xn[:ROW_TOKENS]))
            n = 0
            for t in range(ROW_TOKENS):
                for g in list(ids_h[t]) + [sh.E + s for s in range(sh.S)]:
                    yr = O.swiglu(xh[[t]], host(w["w_gate_up"][g]), host(w["w_down"][g]), "bf16")
                    assert_close(as_f64(got_y[n:n + 1]), yr, BF16_TOL, f"token {t} expert {g}")
                    n += 1
            continue
        assert torch.equal(got_a, ref[0]), f"activation rows differ at T = {T} (routed = {routed})"
        assert torch.equal(got_y, ref[1]), f"expert output rows differ at T = {T} (routed = {routed})"


def test_layer_rows_bit_identical_across_batch_sizes(m):
    """Two whole layers (route, experts, combine) in a VerifyStack: the first 4
    tokens' hidden states are the same bits at 4, 700, 1,100 and 4,100 tokens
    (routed streaming, streaming, GEMM; 1, 8 and 32 tokens per route block)."""
    sh = synth.SHAPES["step128"]
    layers = [synth.layer_weights(5, l, sh, DEV) for l in range(2)]
    st = m.VerifyStack(layers, None, sh.E, sh.k, sh.S, max_tokens=4100)
    h = synth.hidden(32, 4100, sh.H, torch.bfloat16, DEV)
    ref = None
    for T in (4, 700, 1100, 4100):
        st.forward(h[:T].contiguous())
        torch.cuda.synchronize()
        got = st.h[:4].clone()
        if ref is None:
            ref = got
            continue
        assert torch.equal(got, ref), f"hidden rows of the first tokens differ at T = {T}"
