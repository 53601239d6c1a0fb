"""Device-side data errors (moe_data_errors): every call that clamps an
out-of-range index argument completes, gives the outputs of the clamped data,
and sets its MOE_DATA_ERR_* bit; in-range data leaves the word clear.

The bad values are of the kinds the kernels clamp before any memory access
(ids, row indices, offsets, inv rows, lengths, sequence ids), so every access
stays in bounds."""

import numpy as np
import pytest
import torch

import oracle as O
import synth
from moe_decoder_step_amd import _lib as L

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def m():
    import moe_decoder_step_amd as mod
    mod.load()
    assert torch.cuda.is_available(), "GPU tests need a device"
    return mod


@pytest.fixture(autouse=True)
def clean_word(m):
    m.data_errors(DEV, clear=True)     # start every test from a clear word
    yield
    m.data_errors(DEV, clear=True)


def _ids(T, k, E, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.stack([torch.randperm(E, generator=g)[:k] for _ in range(T)]).to(torch.int32)


def test_clear_word_after_a_real_shape_layer(m):
    sh = synth.SHAPES["layer128"]
    w = synth.layer_weights(3, 0, sh, DEV)
    h = synth.hidden(4, 128, sh.H, sh.torch_dtype, DEV)
    xn, ids, tw, _ = m.route_alloc(h, w["w_router"], None, sh.k)
    off, gat, inv = m.permute_alloc(ids, sh.E, sh.S)
    wgu, wd = m.expert_weights(w["w_gate_up"], w["w_down"])
    y = m.swiglu_alloc(xn, gat, off, wgu, wd, 128 * sh.k + sh.S * 128, max_rows=128)
    m.combine_alloc(y[:128 * sh.k], inv, tw, y[128 * sh.k:], sh.S, h)
    assert m.data_errors(DEV) == 0


@pytest.mark.parametrize("T", [37, 5000])   # one-block permute, and count/scan/scatter passes
def test_permute_expert_id_out_of_range(m, T):
    E, S, k = 64, 2, 6
    ids = _ids(T, k, E, T)
    ids[0, 0], ids[T // 2, 3], ids[T - 1, 5] = -3, E, E + 100
    off, gat, inv = m.permute_alloc(ids.to(DEV), E, S)
    assert m.data_errors(DEV) == L.ERR_EXPERT_ID
    roff, rgat, rinv = O.permute(np.clip(ids.numpy(), 0, E - 1), E, S)
    np.testing.assert_array_equal(off.cpu().numpy(), roff)
    np.testing.assert_array_equal(gat.cpu().numpy(), rgat)
    np.testing.assert_array_equal(inv.cpu().numpy(), rinv)


def test_routed_gate_up_expert_id_out_of_range(m):
    sh = synth.SHAPES["layer128"]
    T = 16
    w = synth.layer_weights(5, 0, sh, DEV)
    wgu, _ = m.expert_weights(w["w_gate_up"], w["w_down"])
    x = synth.hidden(6, T, sh.H, sh.torch_dtype, DEV)
    ids = _ids(T, sh.k, sh.E, 7)
    bad = ids.clone()
    bad[1, 2], bad[9, 0] = -1, sh.E + 5
    n_rows = T * sh.k + sh.S * T

    def run(idv):
        act = torch.empty(n_rows, sh.I, dtype=sh.torch_dtype, device=DEV)
        off = torch.empty(sh.E + sh.S + 1, dtype=torch.int32, device=DEV)
        inv = torch.empty(T * sh.k, dtype=torch.int32, device=DEV)
        m.moe_expert_gate_up_routed(x, idv.to(DEV), sh.E, sh.S, wgu, act, off, inv)
        return act, off, inv
    got = run(bad)
    assert m.data_errors(DEV) == L.ERR_EXPERT_ID
    ref = run(bad.clamp(0, sh.E - 1))
    assert m.data_errors(DEV) == 0
    for a, b in zip(got, ref):
        assert torch.equal(a, b)


@pytest.mark.parametrize("max_rows", [600, 2048])   # weight-streaming kernel, MFMA GEMM (groups <= 500 rows)
def test_gate_up_gather_and_offsets_out_of_range(m, max_rows):
    sh = synth.SHAPES["layer128"]
    T, G = 1100, 3
    w = synth.layer_weights(8, 0, sh, DEV)
    wgu, _ = m.expert_weights(w["w_gate_up"][:G].contiguous(), w["w_down"][:G].contiguous())
    x = synth.hidden(9, T, sh.H, sh.torch_dtype, DEV)
    n_rows = 1200
    g = torch.Generator().manual_seed(10)
    gather = torch.randint(0, T, (n_rows,), generator=g, dtype=torch.int32)
    offsets = torch.tensor([0, 300, 700, n_rows], dtype=torch.int32)

    def run(gv, ov):
        act = torch.empty(n_rows, sh.I, dtype=sh.torch_dtype, device=DEV)
        m.moe_expert_gate_up(x, gv.to(DEV), ov.to(DEV), wgu, act, max_rows=max_rows)
        return act
    bad = gather.clone()
    bad[5], bad[650], bad[n_rows - 1] = -7, T, T + 999
    got = run(bad, offsets)
    assert m.data_errors(DEV) == L.ERR_ROW_INDEX
    ref = run(bad.clamp(0, T - 1), offsets)
    assert m.data_errors(DEV) == 0
    assert torch.equal(got, ref)
    # the last group ends past n_rows: clamped to n_rows
    long_off = offsets.clone()
    long_off[G] = n_rows + 40
    got = run(gather, long_off)
    assert m.data_errors(DEV) == L.ERR_OFFSETS
    assert torch.equal(got, run(gather, offsets))


def test_down_offsets_out_of_range(m):
    sh = synth.SHAPES["layer128"]
    G, n_rows = 4, 96
    w = synth.layer_weights(11, 0, sh, DEV)
    _, wd = m.expert_weights(w["w_gate_up"][:G].contiguous(), w["w_down"][:G].contiguous())
    act = synth.hidden(12, n_rows, sh.I, sh.torch_dtype, DEV)
    offsets = torch.tensor([0, 20, 50, 70, n_rows], dtype=torch.int32)

    def run(ov):
        y = torch.zeros(n_rows, sh.H, dtype=sh.torch_dtype, device=DEV)
        m.moe_expert_down(act, ov.to(DEV), wd, y)
        return y
    ref = run(offsets)
    assert m.data_errors(DEV) == 0
    bad = offsets.clone()
    bad[0] = -16          # clamped to 0
    got = run(bad)
    assert m.data_errors(DEV) == L.ERR_OFFSETS
    assert torch.equal(got, ref)


def test_combine_inv_out_of_range(m):
    sh = synth.SHAPES["layer128"]
    T, k, S = 24, sh.k, sh.S
    n_rows = T * k
    y = synth.hidden(13, n_rows, sh.H, sh.torch_dtype, DEV)
    ys = synth.hidden(14, S * T, sh.H, sh.torch_dtype, DEV)
    h = synth.hidden(15, T, sh.H, sh.torch_dtype, DEV)
    tw = torch.rand(T, k, generator=torch.Generator().manual_seed(16)).to(DEV)
    inv = torch.randperm(n_rows, generator=torch.Generator().manual_seed(17)).to(torch.int32)
    bad = inv.clone()
    bad[3], bad[40] = n_rows, -2
    got, _ = m.combine_alloc(y, bad.to(DEV), tw, ys, S, h)
    assert m.data_errors(DEV) == L.ERR_INV
    ref, _ = m.combine_alloc(y, bad.clamp(0, n_rows - 1).to(DEV), tw, ys, S, h)
    assert torch.equal(got, ref)
    # the fused combine + route reports the same
    w = synth.layer_weights(18, 0, sh, DEV)
    hh = h.clone()
    xn = torch.empty_like(h)
    ids = torch.empty(T, k, dtype=torch.int32, device=DEV)
    w2 = torch.empty(T, k, dtype=torch.float32, device=DEV)
    m.moe_combine_route(y, bad.to(DEV), tw, ys, S, hh, w["w_router"], None, k, xn, ids, w2)
    assert m.data_errors(DEV) == L.ERR_INV
    assert torch.equal(hh, got)


def test_rmsnorm_rows_out_of_range(m):
    x = synth.hidden(19, 50, 1280, torch.bfloat16, DEV)
    rows = torch.tensor([0, 49, 50, -1, 7], dtype=torch.int32)
    out = torch.empty(5, 1280, dtype=torch.bfloat16, device=DEV)
    m.moe_rmsnorm(x, out, rows=rows.to(DEV))
    assert m.data_errors(DEV) == L.ERR_ROW_INDEX
    ref = torch.empty_like(out)
    m.moe_rmsnorm(x, ref, rows=rows.clamp(0, 49).to(DEV))
    assert m.data_errors(DEV) == 0
    assert torch.equal(out, ref)


def test_attention_length_out_of_range(m):
    B, P, nh, max_len = 2, 4, 2, 64
    H = nh * 128
    qkv = synth.hidden(20, B * P, 3 * H, torch.bfloat16, DEV)
    lengths = torch.tensor([10, max_len], dtype=torch.int32)    # the second leaves no room for P positions

    def run(lv):
        q = torch.empty(B * P, H, dtype=torch.bfloat16, device=DEV)
        kv = m.kv_cache_alloc(B, nh, max_len, DEV)
        m.moe_attn_rope_cache(qkv, lv.to(DEV), P, q, kv)
        return q, kv
    got = run(lengths)
    assert m.data_errors(DEV) == L.ERR_LENGTH
    ref = run(lengths.clamp(0, max_len - P))
    assert m.data_errors(DEV) == 0
    for a, b in zip(got, ref):
        assert torch.equal(a, b)


def test_loop_sequence_out_of_range(m):
    B, K, S, target = 3, 3, 4, 8
    committed = torch.arange(B * (K + 1), dtype=torch.int32).reshape(B, K + 1).to(DEV)
    n_commit = torch.tensor([2, 9, 1], dtype=torch.int32, device=DEV)    # 9 > K + 1
    seq_ids = torch.tensor([0, 1, 2], dtype=torch.int32, device=DEV)
    z = lambda *s: torch.zeros(*s, dtype=torch.int32, device=DEV)       # noqa: E731
    total, steps, tokens, out, n_act = z(S), z(S), z(S, target), z(B), z(1)
    m.spec_advance(n_commit, committed, seq_ids, target, total, steps, tokens, out, n_act)
    assert m.data_errors(DEV) == L.ERR_SEQUENCE
    assert total.tolist() == [2, 4, 1, 0]       # the bad count taken as K + 1
    # an id >= S in the row gather (a negative id is an empty slot, not an error)
    pool = torch.arange(S * 2 * 4, dtype=torch.int32, device=DEV).reshape(S, 2, 4)
    o = z(3, 4)
    m.spec_gather_rows(pool, torch.tensor([-1, 1, 2], dtype=torch.int32, device=DEV), z(S), o)
    assert m.data_errors(DEV) == 0
    m.spec_gather_rows(pool, torch.tensor([0, S + 3, 2], dtype=torch.int32, device=DEV), z(S), o)
    assert m.data_errors(DEV) == L.ERR_SEQUENCE
    assert o[1].tolist() == pool[S - 1, 0].tolist()


def test_bits_accumulate_until_cleared(m):
    ids = _ids(8, 2, 8, 21)
    ids[0, 0] = 9
    m.permute_alloc(ids.to(DEV), 8, 0)
    x = synth.hidden(22, 4, 128, torch.float32, DEV)
    out = torch.empty(2, 128, dtype=torch.float32, device=DEV)
    m.moe_rmsnorm(x, out, rows=torch.tensor([0, 4], dtype=torch.int32, device=DEV))
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    m.moe_data_errors(flags, clear=False)
    assert int(flags.item()) == L.ERR_EXPERT_ID | L.ERR_ROW_INDEX
    m.moe_data_errors(flags, clear=True)
    assert int(flags.item()) == L.ERR_EXPERT_ID | L.ERR_ROW_INDEX
    m.moe_data_errors(flags, clear=True)
    assert int(flags.item()) == 0
