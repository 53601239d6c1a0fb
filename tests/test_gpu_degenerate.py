"""The method's degenerate cases through the C ABI against the fp64 oracle:
every expert selected (k = E, a dense softmax mixture), a single routed
expert (k = E = 1, S = 0: the layer is one SwiGLU FFN with weight 1), no
shared experts, one token, and a router bias that sends every token to the
same k experts (k full groups, every other group empty).  Ids bit-exact
outside oracle near-ties, layer outputs within the storage dtype's bound."""

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
    assert torch.cuda.is_available(), "GPU tests need a device"
    return mod


def _layer(m, sh, T, seed, bias=None):
    """One MoE layer of shape sh on T tokens; checks it against the oracle and
    returns (GPU ids, oracle result)."""
    w = synth.layer_weights(seed, 0, sh, DEV)
    if bias is not None:
        w["bias"] = bias.to(DEV)
    st = m.VerifyStack([w], None, sh.E, sh.k, sh.S, max_tokens=T, max_seqs=1, K=0)
    h = synth.hidden(seed + 1, T, sh.H, sh.torch_dtype, DEV)
    rec = []
    st.forward(h, rec)
    torch.cuda.synchronize()
    mode = sh.dtype
    hw = {k: host(v) for k, v in w.items()}
    ref = O.moe_layer(host(rec[0]["input"]), hw, sh.k, sh.eps, mode)
    ids = rec[0]["ids"].cpu().numpy()
    _, flagged = compare_ids(ids, ref["route"]["ids"], ref["route"]["gap"], "ids")
    ok = ~flagged
    assert flagged.sum() <= max(1, T // 10), "too many near-tie rows"
    assert_close(rec[0]["w"].cpu().numpy()[ok], ref["route"]["w"][ok], F32_TOL, "routing weights")
    assert_close(as_f64(rec[0]["output"])[ok], ref["h_out"][ok], BF16_TOL if mode == "bf16" else F32_TOL,
                 "layer output")
    return ids, ref


@pytest.mark.parametrize("base,E,T", [("tiny", 8, 16), ("layer128", 16, 32)])
def test_every_expert_selected(m, base, E, T):
    """k = E: every token's ids are a permutation of the experts, by logit."""
    sh = dataclasses.replace(synth.SHAPES[base], E=E, k=E)
    ids, ref = _layer(m, sh, T, 40)
    assert (np.sort(ids, axis=1) == np.arange(E)).all()
    np.testing.assert_allclose(ref["route"]["w"].sum(axis=1), 1.0, rtol=1e-12)


@pytest.mark.parametrize("base,T", [("tiny", 16), ("layer128", 40)])
def test_single_expert_is_a_dense_ffn(m, base, T):
    """k = E = 1, S = 0: weight 1 on the one expert; h' = h + SwiGLU(xn)."""
    sh = dataclasses.replace(synth.SHAPES[base], E=1, k=1, S=0)
    ids, ref = _layer(m, sh, T, 41)
    assert (ids == 0).all()
    np.testing.assert_array_equal(ref["route"]["w"], np.ones((T, 1)))


@pytest.mark.parametrize("T", [1, 128])
def test_no_shared_experts(m, T):
    sh = dataclasses.replace(synth.SHAPES["layer128"], S=0)
    _layer(m, sh, T, 42)


def test_one_token_real_shape(m):
    _layer(m, synth.SHAPES["layer128"], 1, 43)


@pytest.mark.parametrize("T", [128, 700])   # routed gate/up, and the grouped path past 4,096 pairs
def test_all_tokens_to_the_same_experts(m, T):
    """A bias of 8 on experts 5..10 puts every token on those six: six groups
    of T rows, 58 empty ones.  (8 is far above the other logits, whose spread
    is about 0.7, and small enough that adding it in fp32 moves a logit by
    less than the near-tie bound.)"""
    sh = synth.SHAPES["layer128"]
    bias = torch.zeros(sh.E)
    bias[5:11] = 8.0
    ids, _ = _layer(m, sh, T, 44, bias)
    assert (np.sort(ids, axis=1) == np.arange(5, 11)).all()
