"""Prefill-sized MoE layers: the grouped SwiGLU's tiled-GEMM path and the
36,992-token layer (32 pages x 1,156 visual tokens) with Zipf(1.1) expert
popularity, against the fp64 oracle.

Sizes the oracle finishes in seconds are compared row by row; the full-size
layer is compared on its permutation (bit-exact, every row) and on sampled
tokens (routing and output rows), since every token's result depends only on
its own input row and the weights.
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests._util import BF16_TOL, F32_TOL, as_f64, assert_close, compare_ids, host

pytestmark = pytest.mark.gpu

DEV = "cuda"
GEMM_MIN_ROWS = 1024      # max_rows from which the library runs the grouped SwiGLU as a tiled GEMM
ZIPF = os.path.join(os.path.dirname(__file__), "golden", "zipf_bias_prefill.json")


@pytest.fixture(scope="module")
def m():
    import moe_decoder_step_amd as mod
    mod.load()
    return mod


def _zipf_bias():
    with open(ZIPF) as f:
        fx = json.load(f)
    return torch.tensor(fx["bias"], dtype=torch.float32), fx


def test_gemm_path_ragged_groups(m):
    """Identity gather, groups of 0, 1, 255, 256, 257, 600, 1500, 0 and 40 rows
    (ragged and multiple 256-row tiles), max_rows selecting the GEMM path."""
    H, I, T = 1280, 896, 1500
    counts = [0, 1, 255, 256, 257, 600, 1500, 0, 40]
    G = len(counts)
    gen = torch.Generator(device=DEV).manual_seed(21)
    x = torch.randn(T, H, generator=gen, device=DEV).to(torch.bfloat16)
    wgu = (torch.randn(G, 2 * I, H, generator=gen, device=DEV) * 0.02).to(torch.bfloat16)
    wd = (torch.randn(G, H, I, generator=gen, device=DEV) * 0.02).to(torch.bfloat16)
    off = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32, device=DEV)
    n_rows = int(sum(counts))
    wgu_p, wd_p = m.expert_weights(wgu, wd)
    y = m.swiglu_alloc(x, None, off, wgu_p, wd_p, n_rows, max_rows=max(counts))
    torch.cuda.synchronize()
    xh, yg = O.f64(host(x)), as_f64(y)
    wguh, wdh = host(wgu), host(wd)
    for g, c in enumerate(counts):
        a = int(off[g])
        if c:
            ref = O.swiglu(xh[:c], wguh[g], wdh[g], "bf16")
            assert_close(yg[a:a + c], ref, BF16_TOL, f"group {g} ({c} rows)")


def test_gemm_path_shortest_k_gathered(m):
    """The GEMM path at its shortest reduction (K = 256 for gate/up and down:
    8 stages, where the next tile's gathered row numbers are loaded in one
    pass of the stage loop and used in the next), rows gathered from a
    random map, groups of 0, 1, 300, 1100, 7, 0 and 513 rows: every row of
    both outputs against the oracle."""
    H, I, T = 256, 256, 1500
    counts = [0, 1, 300, 1100, 7, 0, 513]
    G = len(counts)
    n_rows = int(sum(counts))
    assert max(counts) >= GEMM_MIN_ROWS
    gen = torch.Generator().manual_seed(31)
    x = torch.randn(T, H, generator=gen).to(torch.bfloat16).to(DEV)
    wgu = (torch.randn(G, 2 * I, H, generator=gen) * 0.05).to(torch.bfloat16).to(DEV)
    wd = (torch.randn(G, H, I, generator=gen) * 0.05).to(torch.bfloat16).to(DEV)
    gat = torch.randint(0, T, (n_rows,), generator=gen, dtype=torch.int32).to(DEV)
    off = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32, device=DEV)
    wgu_p, wd_p = m.expert_weights(wgu, wd)
    act = torch.empty((n_rows, I), dtype=torch.bfloat16, device=DEV)
    y = torch.empty((n_rows, H), dtype=torch.bfloat16, device=DEV)
    m.moe_expert_gate_up(x, gat, off, wgu_p, act, max_rows=max(counts))
    m.moe_expert_down(act, off, wd_p, y, max_rows=max(counts))
    torch.cuda.synchronize()
    xh, gath = O.f64(host(x)), gat.cpu().numpy()
    wguh, wdh = host(wgu), host(wd)
    ag, yg = as_f64(act), as_f64(y)
    for g, c in enumerate(counts):
        a = int(sum(counts[:g]))
        if c:
            xa = xh[gath[a:a + c]]
            assert_close(ag[a:a + c], O.swiglu(xa, wguh[g], np.eye(I), "bf16"), BF16_TOL, f"act group {g} ({c} rows)")
            assert_close(yg[a:a + c], O.swiglu(xa, wguh[g], wdh[g], "bf16"), BF16_TOL, f"y group {g} ({c} rows)")


def test_gemm_path_routed_zipf_1024_tokens(m):
    """Route -> permute -> gate/up -> down at 1,024 tokens with the Zipf
    router bias (max_rows = T selects the GEMM path): activation rows and
    expert outputs of every group against the oracle."""
    sh = synth.SHAPES["prefill"]
    T = 1024
    assert T >= GEMM_MIN_ROWS
    w = synth.layer_weights(1, 0, sh, DEV)
    bias, _ = _zipf_bias()
    h = synth.hidden(5, T, sh.H, torch.bfloat16, DEV)
    xn, ids, tw, _ = m.route_alloc(h, w["w_router"], bias.to(DEV), sh.k)
    off, gat, inv = m.permute_alloc(ids, sh.E, sh.S)
    n_rows = T * sh.k + sh.S * T
    wgu_p, wd_p = m.expert_weights(w["w_gate_up"], w["w_down"])
    act = torch.empty((n_rows, sh.I), dtype=torch.bfloat16, device=DEV)
    y = torch.empty((n_rows, sh.H), dtype=torch.bfloat16, device=DEV)
    m.moe_expert_gate_up(xn, gat, off, wgu_p, act, max_rows=T)
    m.moe_expert_down(act, off, wd_p, y, max_rows=T)
    torch.cuda.synchronize()
    xh, offh, gath = O.f64(host(xn)), off.cpu().numpy(), gat.cpu().numpy()
    wgu, wd = host(w["w_gate_up"]), host(w["w_down"])
    ag, yg = as_f64(act), as_f64(y)
    sizes = np.diff(offh)
    assert sizes[:sh.E].max() > 3 * sizes[:sh.E].mean()     # the bias makes the groups unequal
    for g in range(sh.E + sh.S):
        a, b = offh[g], offh[g + 1]
        if a == b:
            continue
        xa = xh[gath[a:b]]
        assert_close(ag[a:b], O.swiglu(xa, wgu[g], np.eye(sh.I), "bf16"), BF16_TOL, f"act group {g}")
        assert_close(yg[a:b], O.swiglu(xa, wgu[g], wd[g], "bf16"), BF16_TOL, f"y group {g}")


@pytest.mark.timeout(900)
def test_prefill_layer_36992_tokens(m):
    """The full prefill layer (32 x 1,156 tokens, Zipf-biased router), every
    row: the permutation of every (token, slot) bit-exact; every token's
    expert ids (oracle near-ties flagged) and routing weights; every routed
    expert output row, group by group, and every shared-expert row against
    the oracle's per-slot SwiGLU outputs; every token's layer output (the
    combine plus residual).  Tokens with a flagged near-tie are left out of
    the float comparisons (their experts may differ)."""
    sh = synth.SHAPES["prefill"]
    T, k, E, S = sh.T, sh.k, sh.E, sh.S
    assert T == 36992
    w = synth.layer_weights(1, 0, sh, DEV)
    bias, fx = _zipf_bias()
    w["bias"] = bias.to(DEV)
    st = m.VerifyStack([w], None, E, k, S, max_tokens=T)
    h = synth.hidden(3, T, sh.H, torch.bfloat16, DEV)
    rec = []
    st.forward(h, rec)
    torch.cuda.synchronize()
    ids = rec[0]["ids"].cpu().numpy()
    # permutation: every row, against the oracle's stable counting sort of the GPU's ids
    roff, rgat, rinv = O.permute(ids, E, S)
    offs = st.offsets.cpu().numpy()
    inv = st.inv[:T * k].cpu().numpy()
    np.testing.assert_array_equal(offs, roff)
    np.testing.assert_array_equal(st.gather[:T * k + S * T].cpu().numpy(), rgat)
    np.testing.assert_array_equal(inv, rinv)
    load = np.bincount(ids.ravel(), minlength=E)
    order = np.argsort(-load, kind="stable")
    print(f"\nrealised expert load (desc): {load[order][:8].tolist()} ... {load[order][-4:].tolist()}")
    assert load.max() > 20 * load.min() > 0                  # Zipf-like skew, no starved expert
    hw = {key: host(v) for key, v in w.items()}
    ref = O.moe_layer(host(rec[0]["input"]), hw, k, sh.eps, "bf16")
    n_flag, flagged = compare_ids(ids, ref["route"]["ids"], ref["route"]["gap"], "ids")
    print(f"near-tie tokens flagged: {n_flag}")
    ok = ~flagged
    assert_close(rec[0]["w"].cpu().numpy()[ok], ref["route"]["w"][ok], F32_TOL, "routing weights")
    # routed expert rows, group by group: row r holds slot s = t k + j
    y = st.y[:T * k + S * T]
    slot_of_row = np.empty(T * k, dtype=np.int64)
    slot_of_row[inv] = np.arange(T * k)
    for g in range(E):
        a, b = int(offs[g]), int(offs[g + 1])
        if a == b:
            continue
        sl = slot_of_row[a:b]
        t, j = sl // k, sl % k
        keep = ok[t]
        got = as_f64(y[a:b])[keep]
        assert_close(got, ref["y"][t[keep], j[keep]], BF16_TOL, f"expert {g} rows ({b - a})")
    for sx in range(S):
        a = T * k + sx * T
        assert_close(as_f64(y[a:a + T])[ok], ref["ys"][sx][ok], BF16_TOL, f"shared expert {sx} rows")
    assert_close(as_f64(rec[0]["output"])[ok], ref["h_out"][ok], BF16_TOL, "layer output")
