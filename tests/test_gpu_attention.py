"""Causal attention over the KV cache (rope + cache write, split attention,
commit) against the fp64 oracle.

The rotation and cache write are bit-exact (both sides rotate the stored
bf16 inputs in fp64 and round once).  Attention outputs are compared
teacher-forced, from the GPU's own stored queries and cache, within the bf16
tolerance; cache rows past each sequence's last position are filled with NaN
to show that they are never read.  Commit/rollback is checked bit-exact on
the GPU: a pass after spec_commit gives the same bits whatever the rejected
rows held.
"""

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests._util import BF16_TOL, F32_TOL, as_f64, assert_close, compare_ids, host

pytestmark = pytest.mark.gpu

DEV = "cuda"
D = 128


@pytest.fixture(scope="module")
def m():
    import moe_decoder_step_amd as mod
    mod.load()
    return mod


def _caches(seed, B, nh, max_len, lengths, P):
    """A committed prefix below each length, NaN from length + P on; the
    interleaved cache and its k and v views."""
    kv = synth.kv_prefix(seed, 0, (B, nh, max_len, 2, D), torch.bfloat16, DEV, "kv")
    for b, L in enumerate(lengths):
        kv[b, :, L + P:] = float("nan")
    return kv, kv[:, :, :, 0], kv[:, :, :, 1]


def _run(m, qkv, lengths, P, nh, kv, max_keys=None):
    T = qkv.shape[0]
    B = len(lengths)
    lt = torch.tensor(lengths, dtype=torch.int32, device=DEV)
    q = torch.empty((T, nh * D), dtype=torch.bfloat16, device=DEV)
    o = torch.empty_like(q)
    mk = max_keys or kv.shape[2]
    ws = torch.empty(max(m.attention_workspace_bytes(B, P, nh, mk), 256), dtype=torch.uint8, device=DEV)
    m.moe_attn_rope_cache(qkv, lt, P, q, kv)
    m.moe_attention(q, kv, lt, P, o, ws, mk)
    torch.cuda.synchronize()
    return q, o


@pytest.mark.parametrize("P,lengths,max_len", [
    (4, [0, 1, 63, 64, 65, 300, 1000, 2096], 2100),     # tile edges, several splits, a full cache
    (1, [0, 5, 511, 512], 513),
    (16, [0, 17, 240, 241], 257),                       # the largest pass
])
def test_rope_cache_bit_exact_and_attention(m, P, lengths, max_len):
    nh = 10
    H = nh * D
    B = len(lengths)
    qkv = synth.normal(1, (B * P, 3 * H), 1.0, torch.bfloat16, DEV)
    kv, ck, cv = _caches(2, B, nh, max_len, lengths, P)
    ck0, cv0 = host(ck), host(cv)
    q, o = _run(m, qkv, lengths, P, nh, kv)
    # rotation and cache write against the oracle, bit for bit; no other row changes
    rk, rv = O.f64(ck0), O.f64(cv0)
    rq, _, _ = O.rope_cache(host(qkv), lengths, P, nh, rk, rv, "bf16")
    np.testing.assert_array_equal(as_f64(q), rq.reshape(B * P, H))
    np.testing.assert_array_equal(as_f64(ck), rk)
    np.testing.assert_array_equal(as_f64(cv), rv)
    # attention, teacher-forced from the stored queries and cache
    ref = O.causal_attention(host(q).reshape(B * P, nh, D), host(ck), host(cv), lengths, P)
    got = as_f64(o)
    assert np.isfinite(got).all(), "a NaN row past a sequence's positions was read"
    assert_close(got, ref.reshape(B * P, H), BF16_TOL, "attention output")


def test_attention_32768_positions(m):
    """The decoder's context limit: one sequence whose last verify position is 32,767."""
    nh, P, max_len = 10, 4, 32768
    lengths = [max_len - P]
    qkv = synth.normal(3, (P, 3 * nh * D), 1.0, torch.bfloat16, DEV)
    kv, ck, cv = _caches(4, 1, nh, max_len, lengths, P)
    q, o = _run(m, qkv, lengths, P, nh, kv)
    ref = O.causal_attention(host(q).reshape(P, nh, D), host(ck), host(cv), lengths, P)
    assert_close(as_f64(o), ref.reshape(P, nh * D), BF16_TOL, "attention output at 32,768 positions")


def test_tighter_key_bound_same_result_within_tolerance(m):
    """max_keys only sizes the split grid: a tight bound and the full cache
    length both match the oracle."""
    nh, P, max_len = 10, 4, 4096
    lengths = [100, 900, 1020]
    qkv = synth.normal(5, (len(lengths) * P, 3 * nh * D), 1.0, torch.bfloat16, DEV)
    outs = []
    for mk in (1024, None):
        kv, ck, cv = _caches(6, len(lengths), nh, max_len, lengths, P)
        q, o = _run(m, qkv, lengths, P, nh, kv, mk)
        ref = O.causal_attention(host(q).reshape(-1, nh, D), host(ck), host(cv), lengths, P)
        assert_close(as_f64(o), ref.reshape(-1, nh * D), BF16_TOL, f"max_keys {mk}")
        outs.append(o)


def _block(m, seed, sh, B, P, max_len):
    w = synth.attn_weights(seed, 0, sh, DEV)
    blk = m.AttentionBlock(w, sh.H // D, B, P, max_len, sh.eps)
    return blk, w


def test_block_against_oracle(m):
    """rmsnorm -> qkv -> rope + cache -> attention -> o projection + residual
    at 32 sequences x 4 positions, hidden 1280 (10 heads), ragged lengths."""
    sh = synth.SHAPES["step128"]
    B, P, max_len = 32, 4, 1028
    blk, w = _block(m, 7, sh, B, P, max_len)
    lengths = np.random.default_rng(8).integers(0, max_len - P + 1, B)
    lengths[:3] = [0, max_len - P, 64]
    blk.cache_k.copy_(synth.kv_prefix(9, 0, blk.cache_k.shape, torch.bfloat16, DEV, "k"))
    blk.cache_v.copy_(synth.kv_prefix(9, 0, blk.cache_v.shape, torch.bfloat16, DEV, "v"))
    ck0, cv0 = O.f64(host(blk.cache_k)), O.f64(host(blk.cache_v))
    h = synth.hidden(10, B * P, sh.H, torch.bfloat16, DEV)
    h0 = host(h)
    rec = {}
    blk.forward(h, torch.tensor(lengths, dtype=torch.int32, device=DEV), record=rec)
    torch.cuda.synchronize()
    ref = O.attention_block(h0, host(w["w_qkv"]), host(w["w_o"]), ck0, cv0, lengths, P, sh.H // D, sh.eps, "bf16")
    assert_close(as_f64(rec["qkv"]), ref["qkv"], BF16_TOL, "qkv")
    assert_close(as_f64(rec["q"]), ref["q"].reshape(B * P, -1), BF16_TOL, "rotated q")
    assert_close(as_f64(rec["o"]), ref["o"], BF16_TOL, "attention output")
    assert_close(as_f64(h), ref["h_out"], BF16_TOL, "block output")
    assert_close(as_f64(blk.cache_k), ck0, BF16_TOL, "cache k")


def test_commit_then_next_pass_ignores_rejected_rows(m):
    """Pass 1 writes P rows per sequence; spec_commit keeps n of them; pass 2
    at the new lengths gives the same bits whatever the rejected rows held,
    and matches the oracle's two passes."""
    sh = synth.SHAPES["step128"]
    B, P, max_len = 6, 4, 300
    nh = sh.H // D
    outs = []
    n_commit = torch.tensor([1, 2, 3, 4, 1, 4], dtype=torch.int32, device=DEV)
    L0 = np.array([0, 10, 100, 200, 287, 63])
    h1 = synth.hidden(11, B * P, sh.H, torch.bfloat16, DEV)
    h2 = synth.hidden(12, B * P, sh.H, torch.bfloat16, DEV)
    for junk in (False, True):
        blk, w = _block(m, 13, sh, B, P, max_len)
        blk.cache_k.copy_(synth.kv_prefix(14, 0, blk.cache_k.shape, torch.bfloat16, DEV, "k"))
        blk.cache_v.copy_(synth.kv_prefix(14, 0, blk.cache_v.shape, torch.bfloat16, DEV, "v"))
        pre = (O.f64(host(blk.cache_k)), O.f64(host(blk.cache_v)))
        lengths = torch.tensor(L0, dtype=torch.int32, device=DEV)
        x1 = h1.clone()
        blk.forward(x1, lengths)
        m.spec_commit(n_commit, lengths)
        if junk:   # what pass 1 wrote past the committed rows: anything at all
            for b in range(B):
                s = int(L0[b] + n_commit[b])
                blk.cache_k[b, :, s:] = float("nan")
                blk.cache_v[b, :, s:] = -1e30
        x2 = h2.clone()
        blk.forward(x2, lengths)
        torch.cuda.synchronize()
        outs.append(x2)
        np.testing.assert_array_equal(lengths.cpu().numpy(), L0 + n_commit.cpu().numpy())
    assert torch.equal(outs[0], outs[1])
    # the oracle's two passes with its own cache
    ck, cv = pre
    wq, wo = host(w["w_qkv"]), host(w["w_o"])
    O.attention_block(host(h1), wq, wo, ck, cv, L0, P, nh, sh.eps, "bf16")
    ref = O.attention_block(host(h2), wq, wo, ck, cv, L0 + n_commit.cpu().numpy(), P, nh, sh.eps, "bf16")
    assert_close(as_f64(outs[0]), ref["h_out"], BF16_TOL, "pass 2 output")


def test_verify_stack_with_attention(m):
    """Two layers of attention + MoE, LM head, acceptance and commit over
    three passes at 32 x 4 tokens; every block teacher-forced."""
    sh = synth.SHAPES["step128"]
    nL, max_len, nh = 2, 512, sh.H // D
    layers = [synth.layer_weights(0, l, sh, DEV) for l in range(nL)]
    attn = [synth.attn_weights(0, l, sh, DEV) for l in range(nL)]
    w_lm = synth.lm_weight(0, sh, DEV)
    st = m.VerifyStack(layers, w_lm, sh.E, sh.k, sh.S, max_tokens=sh.T, max_seqs=sh.B, K=sh.K, attn=attn,
                       n_heads=nh, max_len=max_len)
    L0 = np.random.default_rng(15).integers(0, 300, sh.B).astype(np.int32)
    st.lengths[:sh.B].copy_(torch.from_numpy(L0))
    for li, blk in enumerate(st.attn):
        blk.cache_k.copy_(synth.kv_prefix(16, li, blk.cache_k.shape, torch.bfloat16, DEV, "k"))
        blk.cache_v.copy_(synth.kv_prefix(16, li, blk.cache_v.shape, torch.bfloat16, DEV, "v"))
    hw = [{k: host(v) for k, v in w.items()} for w in layers]
    for p in range(3):
        lengths = st.lengths[:sh.B].cpu().numpy().copy()
        h = synth.hidden(p, sh.T, sh.H, torch.bfloat16, DEV, name="step_hidden")
        drafts = synth.uniform_ids(p, (sh.B, sh.K), sh.V).to(DEV)
        rec = []
        st.step(h, drafts, rec)
        torch.cuda.synchronize()
        for li, (r, blk) in enumerate(zip(rec, st.attn)):
            ck, cv = host(blk.cache_k[:sh.B]), host(blk.cache_v[:sh.B])
            o = O.causal_attention(host(r["q"]).reshape(sh.T, nh, D), ck, cv, lengths, sh.P)
            assert_close(as_f64(r["o"]), o.reshape(sh.T, sh.H), BF16_TOL, f"pass {p} layer {li} attention")
            ref = O.moe_layer(host(r["input"]), hw[li], sh.k, sh.eps, "bf16")
            _, flagged = compare_ids(r["ids"].cpu().numpy(), ref["route"]["ids"], ref["route"]["gap"],
                                     f"pass {p} layer {li} ids")
            assert_close(as_f64(r["output"])[~flagged], ref["h_out"][~flagged], BF16_TOL, f"layer {li} output")
        rid, rmx, gap = O.lm_argmax(host(st.h[:sh.T]), host(w_lm))
        compare_ids(st.argmax[:sh.T].cpu().numpy(), rid, gap, f"pass {p} argmax")
        racc, rcom, rnc = O.spec_verify(drafts.cpu().numpy(), st.argmax[:sh.T].cpu().numpy().reshape(sh.B, sh.P))
        np.testing.assert_array_equal(st.n_commit[:sh.B].cpu().numpy(), rnc)
        np.testing.assert_array_equal(st.lengths[:sh.B].cpu().numpy(), lengths + rnc)
