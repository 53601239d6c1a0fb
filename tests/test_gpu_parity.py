"""Per-op and per-layer parity of the HIP path against the fp64 oracle.

Every call goes through the C ABI (via the Python binding) on seeded
synthetic inputs and is compared element by element with the oracle in the
rounding mode of its storage dtype: ids, permutations and accepted lengths
bit-exact (oracle near-ties below 1e-6 flagged), floating-point outputs within
max|d|/max(1,|ref|) <= 2e-2 (bf16) or 1e-4 (fp32).
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
    assert torch.cuda.is_available(), "GPU tests need a device"
    return mod


def _layer(sh, seed, device=DEV):
    return synth.layer_weights(seed, 0, sh, device)


def _host_layer(w):
    return {k: host(v) for k, v in w.items()}


# --------------------------------------------------------------------------- weight packing

def _pack_reference(w, kind):
    """The packed layout written out with numpy index arithmetic (test side)."""
    w = np.asarray(w)
    if w.ndim == 2:
        w = w[None]
    G, R, K = w.shape
    N = R // 2 if kind == 0 else R
    P = N // 16 if kind == 0 else (N + 31) // 32
    out = np.zeros((G, P, K // 32, 2, 64, 8), dtype=w.dtype)
    for p in range(P):
        for h in range(2):
            for l in range(64):
                row = h * N + 16 * p + l % 16 if kind == 0 else 32 * p + 16 * h + l % 16
                if kind == 1 and row >= N:
                    continue
                for s in range(K // 32):
                    c = 32 * s + 8 * (l // 16)
                    out[:, p, s, h, l, :] = w[:, row, c:c + 8]
    return out.reshape(-1)


@pytest.mark.parametrize("kind,shape", [(0, (3, 64, 96)), (1, (2, 96, 64)), (1, (77, 64)), (0, (1, 32, 32))])
def test_pack_weights_layout(m, kind, shape):
    w = (torch.randn(shape, device=DEV) * 0.02).to(torch.bfloat16)
    pk = m.pack_weights(w, kind)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(pk.data), _pack_reference(host(w), kind))


# --------------------------------------------------------------------------- route

@pytest.mark.parametrize("shape,T", [("tiny", 16), ("layer128", 128), ("layer128", 1), ("layer128", 37),
                                     ("layer128", 256), ("layer128", 257), ("layer128", 300), ("layer128", 4100),
                                     ("tiny", 4100)])
@pytest.mark.parametrize("packed", [False, True])
def test_route(m, shape, T, packed):
    sh = synth.SHAPES[shape]
    w = _layer(sh, 1)
    h = synth.hidden(2, T, sh.H, sh.torch_dtype, DEV)
    bias = synth.normal(5, (sh.E,), 0.01, torch.float32, "cpu").to(DEV)   # non-zero bias exercises the add
    wr = m.router_weights(w["w_router"]) if packed else w["w_router"]
    xn, ids, tw, lg = m.route_alloc(h, wr, bias, sh.k)
    torch.cuda.synchronize()
    mode = sh.dtype
    ref = O.route(host(h), host(w["w_router"]), host(bias), sh.k, sh.eps, mode)
    # xn is the correctly rounded RMSNorm: bit-exact against the oracle's rounding
    np.testing.assert_array_equal(as_f64(xn), ref["xn"])
    # logits: fp32 accumulation of the same inputs
    lref = O.router_logits(ref["xn"], O.f64(host(w["w_router"])), O.f64(host(bias)))
    assert_close(as_f64(lg), lref, F32_TOL, "logits")
    nflag, flagged = compare_ids(ids.cpu().numpy(), ref["ids"], ref["gap"], "topk ids")
    ok = ~flagged
    assert_close(tw.cpu().numpy()[ok], ref["w"][ok], F32_TOL, "topk weights")


def test_route_batch_invariance(m):
    """The same rows routed inside batches tiled 1, 8 and 32 tokens per block
    give the same normed rows, logits, ids and weights, bit for bit (one
    summation order for every tiling)."""
    sh = synth.SHAPES["layer128"]
    w = _layer(sh, 3)
    wr = m.router_weights(w["w_router"])
    h = synth.hidden(9, 4100, sh.H, torch.bfloat16, DEV)
    outs = {}
    for T in (37, 256, 300, 4100):
        outs[T] = m.route_alloc(h[:T].contiguous(), wr, None, sh.k)
    torch.cuda.synchronize()
    for T in (256, 300, 4100):
        for a, b in zip(outs[37], outs[T]):
            assert torch.equal(a, b[:37]), T


def test_route_full_softmax_and_no_norm(m):
    sh = synth.SHAPES["layer128"]
    w = _layer(sh, 1)
    h = synth.hidden(3, 64, sh.H, torch.bfloat16, DEV)
    xn, ids, tw, _ = m.route_alloc(h, w["w_router"], None, 6, renormalize=False)
    ref = O.route(host(h), host(w["w_router"]), None, 6, sh.eps, "bf16", renormalize=False)
    _, flagged = compare_ids(ids.cpu().numpy(), ref["ids"], ref["gap"], "ids")
    assert_close(tw.cpu().numpy()[~flagged], ref["w"][~flagged], F32_TOL, "full-softmax weights")
    xn2, ids2, tw2, _ = m.route_alloc(h, w["w_router"], None, 6, norm=False)
    torch.cuda.synchronize()
    assert torch.equal(xn2, h)
    ref2 = O.route(host(h), host(w["w_router"]), None, 6, sh.eps, "bf16", norm=False)
    compare_ids(ids2.cpu().numpy(), ref2["ids"], ref2["gap"], "ids without norm")


@pytest.mark.parametrize("E,H", [(64, 1280), (8, 128), (17, 1288)])
def test_pack_router_layout(m, E, H):
    wr = synth.normal(9, (E, H), 0.02, torch.float32, "cpu")
    p = m.router_weights(wr.to(DEV))
    torch.cuda.synchronize()
    got = p.data.cpu().numpy().reshape(H // 4, 64, 4)
    ref = np.zeros((H // 4, 64, 4), np.float32)
    ref[:, :E, :] = wr.numpy().reshape(E, H // 4, 4).transpose(1, 0, 2)
    np.testing.assert_array_equal(got, ref)


def test_route_zero_router_tie_rule(m):
    """All logits equal: experts 0..k-1, weights 1/k (the lower-id tie rule)."""
    h = synth.hidden(4, 9, 1280, torch.bfloat16, DEV)
    wr = torch.zeros(64, 1280, device=DEV)
    _, ids, tw, _ = m.route_alloc(h, wr, None, 6)
    assert (ids.cpu() == torch.arange(6, dtype=torch.int32)).all()
    assert torch.allclose(tw.cpu(), torch.full((9, 6), 1 / 6))


# --------------------------------------------------------------------------- permute

@pytest.mark.parametrize("T,k,E,S", [(16, 2, 8, 2), (128, 6, 64, 2), (1, 6, 64, 2), (37, 6, 64, 0),
                                     (700, 6, 64, 2), (4096, 6, 64, 2), (5000, 3, 17, 1)])
def test_permute(m, T, k, E, S):
    g = torch.Generator().manual_seed(T * 131 + E)
    ids = torch.stack([torch.randperm(E, generator=g)[:k] for _ in range(T)]).to(torch.int32)
    if T > 64:   # skewed load: a few hot experts
        hot = torch.randint(0, 3, (T,), generator=g)
        ids[:, 0] = torch.where(hot == 0, ids[:, 0], ids[:, 0] % 4)   # may repeat an id within a token
    off, gat, inv = m.permute_alloc(ids.to(DEV), E, S)
    roff, rgat, rinv = O.permute(ids.numpy(), E, S)
    np.testing.assert_array_equal(off.cpu().numpy(), roff)
    np.testing.assert_array_equal(gat.cpu().numpy(), rgat)
    np.testing.assert_array_equal(inv.cpu().numpy(), rinv)


# --------------------------------------------------------------------------- grouped SwiGLU

@pytest.mark.parametrize("shape,T", [("tiny", 16), ("layer128", 128), ("layer128", 4), ("layer128", 37),
                                     ("layer128", 200)])
def test_grouped_swiglu(m, shape, T):
    sh = synth.SHAPES[shape]
    w = _layer(sh, 1)
    h = synth.hidden(2, T, sh.H, sh.torch_dtype, DEV)
    xn, ids, tw, _ = m.route_alloc(h, w["w_router"], None, sh.k)
    off, gat, inv = m.permute_alloc(ids, sh.E, sh.S)
    n_rows = T * sh.k + sh.S * T
    wgu_p, wd_p = m.expert_weights(w["w_gate_up"], w["w_down"])
    y = m.swiglu_alloc(xn, gat, off, wgu_p, wd_p, n_rows, max_rows=T)
    torch.cuda.synchronize()
    # oracle: every group on the GPU's own xn and permutation
    xh = O.f64(host(xn))
    offh, gath = off.cpu().numpy(), gat.cpu().numpy()
    wgu, wd = host(w["w_gate_up"]), host(w["w_down"])
    yg = as_f64(y)
    for g in range(sh.E + sh.S):
        a, b = offh[g], offh[g + 1]
        if a == b:
            continue
        ref = O.swiglu(xh[gath[a:b]], wgu[g], wd[g], sh.dtype)
        assert_close(yg[a:b], ref, BF16_TOL if sh.dtype == "bf16" else F32_TOL, f"group {g}")


@pytest.mark.parametrize("shape,T", [("layer128", 37), ("tiny", 16)])
def test_expert_halves(m, shape, T):
    """moe_expert_gate_up + moe_expert_down: the activation rows against the
    oracle (its SwiGLU with an identity down projection returns them), and y
    bit-identical to moe_grouped_swiglu."""
    sh = synth.SHAPES[shape]
    w = _layer(sh, 3)
    h = synth.hidden(4, T, sh.H, sh.torch_dtype, DEV)
    xn, ids, tw, _ = m.route_alloc(h, w["w_router"], None, sh.k)
    off, gat, inv = m.permute_alloc(ids, sh.E, sh.S)
    n_rows = T * sh.k + sh.S * T
    wgu_p, wd_p = m.expert_weights(w["w_gate_up"], w["w_down"])
    act = torch.full((n_rows, sh.I), float("nan"), dtype=sh.torch_dtype, device=DEV)
    y = torch.empty((n_rows, sh.H), dtype=sh.torch_dtype, device=DEV)
    m.moe_expert_gate_up(xn, gat, off, wgu_p, act, max_rows=T)
    m.moe_expert_down(act, off, wd_p, y, max_rows=T)
    y_fused = m.swiglu_alloc(xn, gat, off, wgu_p, wd_p, n_rows, max_rows=T)
    torch.cuda.synchronize()
    assert torch.equal(y, y_fused)
    xh, offh, gath = O.f64(host(xn)), off.cpu().numpy(), gat.cpu().numpy()
    wgu, eye = host(w["w_gate_up"]), np.eye(sh.I)
    ag = as_f64(act)
    tol = BF16_TOL if sh.dtype == "bf16" else F32_TOL
    for g in range(sh.E + sh.S):
        a, b = offh[g], offh[g + 1]
        if a < b:
            assert_close(ag[a:b], O.swiglu(xh[gath[a:b]], wgu[g], eye, sh.dtype), tol, f"act group {g}")


@pytest.mark.parametrize("T", [1, 4, 37, 128, 300, 682])
def test_gate_up_routed_matches_permute_path(m, T):
    """moe_expert_gate_up_routed: activation rows, offsets and inv identical to
    moe_permute + moe_expert_gate_up (bit for bit); 682 tokens x 6 slots is
    the largest batch it takes (4,092 pairs)."""
    sh = synth.SHAPES["layer128"]
    w = _layer(sh, 4)
    h = synth.hidden(6, T, sh.H, torch.bfloat16, DEV)
    xn, ids, tw, _ = m.route_alloc(h, w["w_router"], None, sh.k)
    off, gat, inv = m.permute_alloc(ids, sh.E, sh.S)
    n_rows = T * sh.k + sh.S * T
    wgu_p, _ = m.expert_weights(w["w_gate_up"], w["w_down"])
    act = torch.empty((n_rows, sh.I), dtype=torch.bfloat16, device=DEV)
    m.moe_expert_gate_up(xn, gat, off, wgu_p, act, max_rows=T)
    act2 = torch.full_like(act, float("nan"))
    off2 = torch.full_like(off, -7)
    inv2 = torch.full((T, sh.k), -7, dtype=torch.int32, device=DEV)
    m.moe_expert_gate_up_routed(xn, ids, sh.E, sh.S, wgu_p, act2, off2, inv2)
    torch.cuda.synchronize()
    assert torch.equal(off2, off)
    assert torch.equal(inv2.view(-1), inv)
    assert torch.equal(act2, act)


def test_grouped_swiglu_long_reduction(m):
    """A reduction length of 2,560 (its 16 staged rows need 82 KB of LDS, more
    than the default 64 KB a launch gets) in both stages."""
    H, I, T = 2560, 2560, 20
    counts = [7, 13]
    gen = torch.Generator(device=DEV).manual_seed(17)
    x = torch.randn(T, H, generator=gen, device=DEV).to(torch.bfloat16)
    wgu = (torch.randn(2, 2 * I, H, generator=gen, device=DEV) * 0.02).to(torch.bfloat16)
    wd = (torch.randn(2, H, I, generator=gen, device=DEV) * 0.02).to(torch.bfloat16)
    off = torch.tensor([0, 7, 20], dtype=torch.int32, device=DEV)
    wgu_p, wd_p = m.expert_weights(wgu, wd)
    y = m.swiglu_alloc(x, None, off, wgu_p, wd_p, T, max_rows=13)
    torch.cuda.synchronize()
    xh, yg = O.f64(host(x)), as_f64(y)
    for g, (a, c) in enumerate(zip([0, 7], counts)):
        ref = O.swiglu(xh[:c], host(wgu[g]), host(wd[g]), "bf16")
        assert_close(yg[a:a + c], ref, BF16_TOL, f"group {g}")


def test_grouped_swiglu_identity_gather_and_skewed_groups(m):
    """gather = NULL (row r of a group reads token r - offsets[g]); groups of
    0, 1, 15, 16, 17, 33, 100 rows (ragged M-blocks, several row blocks)."""
    H, I, T = 1280, 896, 100
    counts = [0, 1, 15, 16, 17, 33, 100, 0]
    G = len(counts)
    gen = torch.Generator(device=DEV).manual_seed(7)
    x = (torch.randn(T, H, generator=gen, device=DEV)).to(torch.bfloat16)
    wgu = (torch.randn(G, 2 * I, H, generator=gen, device=DEV) * 0.02).to(torch.bfloat16)
    wd = (torch.randn(G, H, I, generator=gen, device=DEV) * 0.02).to(torch.bfloat16)
    off = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32, device=DEV)
    n_rows = int(sum(counts))
    wgu_p, wd_p = m.expert_weights(wgu, wd)
    for max_rows in (16, 100):
        y = m.swiglu_alloc(x, None, off, wgu_p, wd_p, n_rows, max_rows=max_rows)
        torch.cuda.synchronize()
        xh, yg = O.f64(host(x)), as_f64(y)
        for g, c in enumerate(counts):
            a = int(off[g])
            if c:
                ref = O.swiglu(xh[:c], host(wgu[g]), host(wd[g]), "bf16")
                assert_close(yg[a:a + c], ref, BF16_TOL, f"group {g} ({c} rows, max_rows {max_rows})")


# --------------------------------------------------------------------------- combine

@pytest.mark.parametrize("dtype,T,k,S", [(torch.bfloat16, 128, 6, 2), (torch.float32, 16, 2, 2),
                                         (torch.bfloat16, 5, 6, 0), (torch.bfloat16, 3, 1, 1)])
def test_combine(m, dtype, T, k, S):
    H = 1280 if dtype == torch.bfloat16 else 128
    gen = torch.Generator(device=DEV).manual_seed(11)
    n_rows = T * k + S * T
    y = torch.randn(n_rows, H, generator=gen, device=DEV).to(dtype)
    inv = torch.randperm(T * k, generator=gen, device=DEV).to(torch.int32)
    tw = torch.rand(T, k, generator=gen, device=DEV)
    res = torch.randn(T, H, generator=gen, device=DEV).to(dtype)
    out, comb = m.combine_alloc(y[:T * k], inv, tw, y[T * k:] if S else None, S, res)
    torch.cuda.synchronize()
    yh, rh = O.f64(host(y)), O.f64(host(res))
    invh, twh = inv.cpu().numpy(), tw.cpu().numpy().astype(np.float64)
    c = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            c[t] += twh[t, j] * yh[invh[t * k + j]]
        for s in range(S):
            c[t] += yh[T * k + s * T + t]
    mode = "bf16" if dtype == torch.bfloat16 else "f32"
    tol = BF16_TOL if dtype == torch.bfloat16 else F32_TOL
    assert_close(as_f64(comb), O.store(c, mode), tol, "combined")
    assert_close(as_f64(out), O.store(rh + c, mode), tol, "out")
    # in place: out aliases residual
    res2 = res.clone()
    m.moe_combine(y[:T * k], inv, tw, y[T * k:] if S else None, S, res2, res2)
    torch.cuda.synchronize()
    assert torch.equal(res2, out)


@pytest.mark.parametrize("dtype,T,H,k,S,gain,resid", [
    (torch.bfloat16, 128, 1280, 6, 2, False, True), (torch.bfloat16, 37, 1280, 0, 1, True, True),
    (torch.bfloat16, 5, 2048, 6, 2, True, False), (torch.float32, 16, 128, 2, 2, True, True),
    (torch.bfloat16, 3, 136, 1, 0, False, True)])
def test_combine_rmsnorm(m, dtype, T, H, k, S, gain, resid):
    """The fused combine + RMSNorm gives the bits of moe_combine followed by
    moe_rmsnorm of its output, and xn matches the oracle's RMSNorm of the
    stored row; also in place (out is the residual)."""
    mode = "bf16" if dtype == torch.bfloat16 else "f32"
    gen = torch.Generator(device=DEV).manual_seed(13)
    y = torch.randn(T * k + S * T, H, generator=gen, device=DEV).to(dtype)
    inv = torch.randperm(T * k, generator=gen, device=DEV).to(torch.int32)
    tw = torch.rand(T, k, generator=gen, device=DEV)
    res = torch.randn(T, H, generator=gen, device=DEV).to(dtype) if resid else None
    g = (torch.rand(H, generator=gen, device=DEV) + 0.5) if gain else None
    yk, ys = (y[:T * k] if k else None), (y[T * k:] if S else None)
    ref_out = torch.empty((T, H), dtype=dtype, device=DEV)
    ref_xn = torch.empty_like(ref_out)
    m.moe_combine(yk, inv if k else None, tw, ys, S, res, ref_out)
    m.moe_rmsnorm(ref_out, ref_xn, gain=g)
    out = torch.full_like(ref_out, float("nan"))
    xn = torch.full_like(ref_out, float("nan"))
    m.moe_combine_rmsnorm(yk, inv if k else None, tw, ys, S, res, out, xn, gain=g)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)
    assert torch.equal(xn, ref_xn)
    gh = None if g is None else g.cpu().numpy().astype(np.float64)
    assert_close(as_f64(xn), O.store(O.rmsnorm(as_f64(out), 1e-6, gh), mode),
                 BF16_TOL if dtype == torch.bfloat16 else F32_TOL, "xn")
    if resid:
        h = res.clone()
        xn2 = torch.empty_like(xn)
        m.moe_combine_rmsnorm(yk, inv if k else None, tw, ys, S, h, h, xn2, gain=g)
        torch.cuda.synchronize()
        assert torch.equal(h, ref_out) and torch.equal(xn2, ref_xn)


# --------------------------------------------------------------------------- LM head

@pytest.mark.parametrize("dtype,T,H,V", [(torch.float32, 16, 128, 512), (torch.bfloat16, 4, 1280, 129280),
                                         (torch.bfloat16, 128, 1280, 20000), (torch.bfloat16, 37, 1280, 1003),
                                         (torch.bfloat16, 1, 64, 77), (torch.bfloat16, 200, 256, 5000),
                                         (torch.bfloat16, 65, 512, 4099)])
def test_lmhead_argmax(m, dtype, T, H, V):
    gen = torch.Generator(device=DEV).manual_seed(T + V)
    h = torch.randn(T, H, generator=gen, device=DEV).to(dtype)
    W = (torch.randn(V, H, generator=gen, device=DEV) * 0.02).to(dtype)
    ids, mx = m.lmhead_alloc(h, m.lm_weights(W))
    torch.cuda.synchronize()
    rid, rmx, gap = O.lm_argmax(host(h), host(W))
    nflag, flagged = compare_ids(ids.cpu().numpy(), rid, gap, "argmax")
    assert_close(mx.cpu().numpy()[~flagged], rmx[~flagged], F32_TOL, "max logit")


def test_lmhead_ties_go_to_lowest_id(m):
    H, V = 256, 3000
    gen = torch.Generator(device=DEV).manual_seed(3)
    W = (torch.randn(V, H, generator=gen, device=DEV) * 0.02).to(torch.bfloat16)
    W[2900] = W[17]
    W[1500] = W[17]
    h = (W[17:18].float() * 50).to(torch.bfloat16).repeat(3, 1)
    ids, _ = m.lmhead_alloc(h, m.lm_weights(W))
    assert (ids.cpu() == 17).all()


# --------------------------------------------------------------------------- verify / plant

@pytest.mark.parametrize("B,K", [(32, 3), (1, 3), (7, 0), (100, 1), (3, 15)])
def test_spec_verify_and_plant(m, B, K):
    g = torch.Generator().manual_seed(B * 17 + K)
    V = 5
    argmax = torch.randint(0, V, (B, K + 1), generator=g, dtype=torch.int32)
    drafts = torch.randint(0, V, (B, K), generator=g, dtype=torch.int32)
    acc, com, nc = m.verify_alloc(drafts.to(DEV), argmax.to(DEV))
    racc, rcom, rnc = O.spec_verify(drafts.numpy(), argmax.numpy())
    np.testing.assert_array_equal(acc.cpu().numpy(), racc)
    np.testing.assert_array_equal(com.cpu().numpy(), rcom)
    np.testing.assert_array_equal(nc.cpu().numpy(), rnc)
    if K:
        keep = (torch.rand(B, K, generator=g) < 0.576).to(torch.uint8)
        repl = torch.randint(0, V - 1, (B, K), generator=g, dtype=torch.int32)
        d = torch.empty(B, K, dtype=torch.int32, device=DEV)
        m.spec_plant_drafts(argmax.to(DEV), keep.to(DEV), repl.to(DEV), V, d)
        np.testing.assert_array_equal(d.cpu().numpy(), O.plant_drafts(argmax.numpy(), keep.numpy(), repl.numpy()))


def test_out_of_vocab_draft_is_a_mismatch(m):
    argmax = torch.tensor([[5, 6, 7, 8]], dtype=torch.int32, device=DEV)
    drafts = torch.tensor([[5, 2 ** 31 - 1, 7]], dtype=torch.int32, device=DEV)
    acc, com, nc = m.verify_alloc(drafts, argmax)
    assert acc.item() == 1 and nc.item() == 2 and com.cpu().tolist() == [[5, 6, -1, -1]]


@pytest.mark.parametrize("gated,N,K", [
    (False, 1312, 896),    # K split in 4, the last column tile half idle
    (False, 1280, 3584),   # K split in 8 (the draft block's down projection)
    (False, 3840, 1280),   # the attention qkv projection
    (True, 3584, 1280),    # K split in 4 (the draft block's gate/up)
    (False, 128, 256),     # too short to split
])
def test_one_group_dense_launches(m, gated, N, K):
    """One-group (dense) launches split the reduction across a block's
    wavefronts: outputs against the oracle's product, and a row's result is
    the same bits whatever the number of rows (the split depends on the
    weight shape only)."""
    Wrows = 2 * N if gated else N
    w = synth.normal(21, (1, Wrows, K), 0.02, torch.bfloat16, DEV)
    wp = m.pack_weights(w, m._lib.PACK_GATE_UP if gated else m._lib.PACK_ROWS)
    x = synth.normal(22, (130, K), 1.0, torch.bfloat16, DEV)
    wh = O.f64(host(w[0]))
    first = None
    for rows in (1, 17, 130):
        xr = x[:rows].contiguous()
        out = torch.full((rows, N), float("nan"), dtype=torch.bfloat16, device=DEV)
        off = torch.tensor([0, rows], dtype=torch.int32, device=DEV)
        if gated:
            m.moe_expert_gate_up(xr, None, off, wp, out, max_rows=rows)
        else:
            m.moe_expert_down(xr, off, wp, out, max_rows=rows)
        torch.cuda.synchronize()
        xh = O.f64(host(xr))
        if gated:
            ref = O.swiglu(xh, wh, np.eye(N), "bf16")
        else:
            ref = O.store(xh @ wh.T, "bf16")
        assert_close(as_f64(out), ref, BF16_TOL, f"rows {rows}")
        if first is None:
            first = out[0].clone()
        else:
            assert torch.equal(out[0], first), f"row 0 depends on the number of rows ({rows})"


@pytest.mark.parametrize("dtype,G,N,K,rows", [
    (torch.bfloat16, 1, 1280, 1280, 1), (torch.bfloat16, 1, 1280, 1280, 130), (torch.bfloat16, 1, 1280, 896, 37),
    (torch.bfloat16, 3, 1280, 896, 77), (torch.float32, 2, 128, 96, 40)])
def test_expert_down_residual(m, dtype, G, N, K, rows):
    """moe_expert_down_residual gives the bits of moe_expert_down followed by
    moe_combine with the product as its one shared row; also in place."""
    w = synth.normal(23, (G, N, K), 0.02, dtype, DEV)
    wp = m.pack_weights(w, m._lib.PACK_ROWS) if dtype == torch.bfloat16 else w
    x = synth.normal(24, (rows, K), 1.0, dtype, DEV)
    res = synth.normal(25, (rows, N), 1.0, dtype, DEV)
    cuts = np.sort(np.random.default_rng(26).integers(0, rows + 1, G - 1))
    off = torch.tensor([0, *cuts, rows], dtype=torch.int32, device=DEV)
    prod = torch.empty((rows, N), dtype=dtype, device=DEV)
    m.moe_expert_down(x, off, wp, prod, max_rows=rows)
    ref = torch.empty_like(prod)
    m.moe_combine(None, None, torch.empty((rows, 0), device=DEV), prod, 1, res, ref)
    y = torch.full_like(prod, float("nan"))
    m.moe_expert_down_residual(x, off, wp, res, y, max_rows=rows)
    h = res.clone()
    m.moe_expert_down_residual(x, off, wp, h, h, max_rows=rows)
    torch.cuda.synchronize()
    assert torch.equal(y, ref)
    assert torch.equal(h, ref)
    # and against the oracle: residual + the product rounded to the storage type
    mode = "bf16" if dtype == torch.bfloat16 else "f32"
    xh, wh, offh = O.f64(host(x)), O.f64(host(w)), off.cpu().numpy()
    pr = np.zeros((rows, N))
    for g in range(G):
        pr[offh[g]:offh[g + 1]] = xh[offh[g]:offh[g + 1]] @ wh[g].T
    assert_close(as_f64(y), O.store(O.f64(host(res)) + O.store(pr, mode), mode),
                 BF16_TOL if dtype == torch.bfloat16 else F32_TOL, "y")
