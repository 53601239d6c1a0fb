"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks one oracle function against something other than itself:
a closed form, a hand-worked case, a brute-force enumeration written
differently, a library routine, or a number printed on the pages.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def facts():
    with open(os.path.join(GOLDEN, "page_facts.json")) as f:
        return {k: v["value"] for k, v in json.load(f).items() if not k.startswith("_")}


# --------------------------------------------------------------------------
# storage rounding
# --------------------------------------------------------------------------

def test_round_bf16_matches_torch_cast():
    """For fp32 inputs, one RNE step to bf16 equals torch's fp32->bf16 cast."""
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 1.0, 37.0, 1e4)]).astype(np.float32)
    # exact halfway cases (low 16 bits = 0x8000) in both parities
    bits = rng.integers(0x3F000000, 0x43000000, 4000, dtype=np.uint32)
    halfway = ((bits & 0xFFFF0000) | 0x8000).view(np.float32)
    x = np.concatenate([x, halfway, -halfway])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_bf16(x.astype(np.float64)), ref)


def test_round_bf16_hand_cases():
    # bf16 keeps 8 significant bits: the spacing just above 1.0 is 2^-7
    assert O.round_bf16(1.0 + 2.0 ** -8) == 1.0                    # tie -> even (1.0)
    assert O.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6     # tie -> even (up)
    assert O.round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7  # just above the tie
    assert O.round_bf16(-3.0) == -3.0
    assert O.round_bf16(0.0) == 0.0
    # a value whose fp32 rounding would land on a bf16 tie: one step from fp64 is not two
    x = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert O.round_bf16(x) == 1.0 + 2.0 ** -7
    assert O.round_bf16(O.round_f32(x)) == 1.0   # the double rounding the oracle avoids


def test_f64_reads_bf16_bits_exactly():
    t = torch.randn(1000).to(torch.bfloat16)
    bits = t.view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(O.f64(bits), t.to(torch.float64).numpy())


def test_round_f32_is_numpy_cast():
    assert O.round_f32(1.0 + 2.0 ** -24) == 1.0
    assert O.round_f32(1.0 + 3 * 2.0 ** -24) == 1.0 + 2.0 ** -22


# --------------------------------------------------------------------------
# RMSNorm
# --------------------------------------------------------------------------

def test_rmsnorm_constant_vector_closed_form():
    # h = c * ones(H): mean(h^2) = c^2, so xn = c / sqrt(c^2 + eps)
    for c, eps in [(3.0, 0.5), (-2.0, 1e-6), (0.25, 0.1)]:
        xn = O.rmsnorm(np.full((1, 7), c), eps)
        np.testing.assert_allclose(xn, c / math.sqrt(c * c + eps), rtol=1e-15)


def test_rmsnorm_loops_and_scale_invariance():
    rng = np.random.default_rng(1)
    h = rng.standard_normal((3, 5))
    eps = 0.3
    for t in range(3):
        ms = sum(v * v for v in h[t]) / 5
        for i in range(5):
            assert math.isclose(O.rmsnorm(h, eps)[t, i], h[t, i] / math.sqrt(ms + eps), rel_tol=1e-14)
    # eps -> 0: RMSNorm ignores a positive scale, and mean(xn^2) = 1
    np.testing.assert_allclose(O.rmsnorm(4.0 * h, 0.0), O.rmsnorm(h, 0.0), rtol=1e-14)
    np.testing.assert_allclose((O.rmsnorm(h, 0.0) ** 2).mean(-1), 1.0, rtol=1e-14)


# --------------------------------------------------------------------------
# router
# --------------------------------------------------------------------------

def test_router_logits_loops():
    rng = np.random.default_rng(2)
    xn, W, b = rng.standard_normal((2, 5)), rng.standard_normal((3, 5)), rng.standard_normal(3)
    lg = O.router_logits(xn, W, b)
    for t in range(2):
        for e in range(3):
            assert math.isclose(lg[t, e], sum(xn[t, h] * W[e, h] for h in range(5)) + b[e], rel_tol=1e-13)


def _brute_topk(row, k):
    """Subset with the largest logit sum, lexicographically smallest ids on ties,
    listed by descending logit (ties by ascending id)."""
    best, best_key = None, None
    for sub in itertools.combinations(range(len(row)), k):
        key = (sum(row[i] for i in sub), [-i for i in sub])
        if best_key is None or key > best_key:
            best, best_key = sub, key
    return sorted(best, key=lambda i: (-row[i], i))


def test_topk_bruteforce_all_subsets():
    """All C(8,2) = 28 subsets per token at the tiny shape, plus k = 3 and ties."""
    rng = np.random.default_rng(3)
    rows = [rng.standard_normal(8) for _ in range(200)]
    rows += [np.round(rng.standard_normal(8) * 2) / 2 for _ in range(200)]   # many exact ties
    rows += [np.zeros(8), np.ones(8)]
    for k in (1, 2, 3, 6):
        got = O.topk_ids(np.asarray(rows), k)
        for r, g in zip(rows, got):
            assert list(g) == _brute_topk(list(r), k)


def test_topk_weights_identities():
    # hand-worked: logits log(1..4), top-2 = ids 3,2 with weights 4/7, 3/7
    lg = np.log(np.array([[1.0, 2.0, 3.0, 4.0]]))
    ids = O.topk_ids(lg, 2)
    assert list(ids[0]) == [3, 2]
    np.testing.assert_allclose(O.topk_weights(lg, ids, True), [[4 / 7, 3 / 7]], rtol=1e-15)
    np.testing.assert_allclose(O.topk_weights(lg, ids, False), [[4 / 10, 3 / 10]], rtol=1e-15)
    # renormalised full softmax == softmax over the selected logits; sum is 1
    rng = np.random.default_rng(4)
    lg = rng.standard_normal((50, 64)) * 3
    ids = O.topk_ids(lg, 6)
    full = O.topk_weights(lg, ids, False)
    np.testing.assert_allclose(full / full.sum(-1, keepdims=True), O.topk_weights(lg, ids, True), rtol=1e-13)
    np.testing.assert_allclose(O.topk_weights(lg, ids, True).sum(-1), 1.0, rtol=1e-14)
    assert np.all(np.diff(O.topk_weights(lg, ids, True), axis=-1) <= 0)   # descending order


def test_zero_router_picks_lowest_ids_uniformly():
    wts = {"w_router": np.zeros((8, 16)), "bias": np.zeros(8)}
    r = O.route(np.random.default_rng(5).standard_normal((4, 16)), wts["w_router"], wts["bias"], 2, 1e-6, "exact")
    assert (r["ids"] == [[0, 1]] * 4).all()
    np.testing.assert_allclose(r["w"], 0.5)
    assert (r["gap"] == 0).all()


def test_topk_gap():
    lg = np.array([[5.0, 1.0, 4.0, 4.5, 0.0]])
    # sorted 5, 4.5, 4, 1, 0; k=2: gaps 0.5 (5-4.5), 0.5 (4.5-4) -> 0.5
    assert O.topk_gap(lg, 2)[0] == 0.5
    assert O.topk_gap(lg, 3)[0] == 0.5
    lg = np.array([[5.0, 4.999, 1.0]])
    assert math.isclose(O.topk_gap(lg, 1)[0], 0.001, rel_tol=1e-9)


# --------------------------------------------------------------------------
# permutation
# --------------------------------------------------------------------------

def test_permute_hand_case():
    ids = np.array([[2, 0], [0, 1], [2, 1]])     # T=3, k=2, E=3
    off, gat, inv = O.permute(ids, 3, S=1)
    # expert 0: slots 1 (t0), 2 (t1); expert 1: slots 3 (t1), 5 (t2); expert 2: slots 0 (t0), 4 (t2)
    assert list(off) == [0, 2, 4, 6, 9]
    assert list(gat) == [0, 1, 1, 2, 0, 2, 0, 1, 2]
    assert list(inv) == [4, 0, 1, 2, 5, 3]


def test_permute_invariants():
    rng = np.random.default_rng(6)
    for T, k, E, S in [(16, 2, 8, 2), (128, 6, 64, 2), (5, 6, 64, 0), (1, 1, 1, 0)]:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
        off, gat, inv = O.permute(ids, E, S)
        assert off[0] == 0 and np.all(np.diff(off) >= 0) and off[-1] == T * k + S * T
        assert off[E] == T * k
        assert np.array_equal(np.diff(off[:E + 1]), np.bincount(ids.ravel(), minlength=E))
        assert sorted(inv) == list(range(T * k))                       # bijection
        for slot in range(T * k):
            t, j = divmod(slot, k)
            r = inv[slot]
            assert gat[r] == t and off[ids[t, j]] <= r < off[ids[t, j] + 1]
        for e in range(E):
            rows = gat[off[e]:off[e + 1]]
            assert np.all(np.diff(rows) > 0)                            # stable: ascending tokens
        for s in range(S):
            assert np.array_equal(gat[off[E + s]:off[E + s + 1]], np.arange(T))


# --------------------------------------------------------------------------
# experts and the block
# --------------------------------------------------------------------------

def test_silu_closed_forms():
    assert O.silu(0.0) == 0.0
    assert math.isclose(float(O.silu(1.0)), 1.0 / (1.0 + math.exp(-1.0)), rel_tol=1e-15)
    z = np.linspace(-8, 8, 101)
    np.testing.assert_allclose(O.silu(-z), O.silu(z) - z, atol=1e-14)   # silu(-z) = silu(z) - z
    assert math.isclose(float(O.silu(50.0)), 50.0, rel_tol=1e-15)


def _dense_swiglu_loops(x, wg, wu, wd):
    H, I = len(x), len(wg)
    g = [sum(wg[i][h] * x[h] for h in range(H)) for i in range(I)]
    u = [sum(wu[i][h] * x[h] for h in range(H)) for i in range(I)]
    a = [g[i] / (1 + math.exp(-g[i])) * u[i] for i in range(I)]
    return [sum(wd[o][i] * a[i] for i in range(I)) for o in range(H)]


def test_single_expert_block_is_dense_swiglu():
    """E=1, k=1, S=0: the block reduces to h + W_d(silu(W_g xn) * W_u xn)."""
    rng = np.random.default_rng(7)
    H, I, eps = 6, 4, 1e-6
    h = rng.standard_normal((3, H))
    wts = {"w_router": rng.standard_normal((1, H)), "bias": np.zeros(1),
           "w_gate_up": rng.standard_normal((1, 2 * I, H)) * 0.5,
           "w_down": rng.standard_normal((1, H, I)) * 0.5}
    out = O.moe_layer(h, wts, 1, eps, "exact")
    for t in range(3):
        ms = sum(v * v for v in h[t]) / H
        xn = [v / math.sqrt(ms + eps) for v in h[t]]
        y = _dense_swiglu_loops(xn, wts["w_gate_up"][0][:I], wts["w_gate_up"][0][I:], wts["w_down"][0])
        np.testing.assert_allclose(out["h_out"][t], h[t] + np.array(y), rtol=1e-12, atol=1e-13)
        assert out["route"]["w"][t, 0] == 1.0


def test_block_with_shared_expert_loops():
    """E=3, k=2, S=1 at tiny size: h + sum_j w_j y_j + y_shared, written as loops."""
    rng = np.random.default_rng(8)
    H, I, E, k, eps = 5, 3, 3, 2, 1e-6
    h = rng.standard_normal((4, H))
    wts = {"w_router": rng.standard_normal((E, H)), "bias": rng.standard_normal(E),
           "w_gate_up": rng.standard_normal((E + 1, 2 * I, H)) * 0.5,
           "w_down": rng.standard_normal((E + 1, H, I)) * 0.5}
    out = O.moe_layer(h, wts, k, eps, "exact")
    for t in range(4):
        ms = sum(v * v for v in h[t]) / H
        xn = [v / math.sqrt(ms + eps) for v in h[t]]
        lg = [sum(xn[j] * wts["w_router"][e][j] for j in range(H)) + wts["bias"][e] for e in range(E)]
        sel = sorted(range(E), key=lambda e: (-lg[e], e))[:k]
        z = [math.exp(lg[e] - lg[sel[0]]) for e in sel]
        w = [v / sum(z) for v in z]
        acc = np.zeros(H)
        for wj, e in zip(w, sel):
            acc += wj * np.array(_dense_swiglu_loops(xn, wts["w_gate_up"][e][:I], wts["w_gate_up"][e][I:], wts["w_down"][e]))
        acc += np.array(_dense_swiglu_loops(xn, wts["w_gate_up"][E][:I], wts["w_gate_up"][E][I:], wts["w_down"][E]))
        np.testing.assert_allclose(out["h_out"][t], h[t] + acc, rtol=1e-12, atol=1e-13)
        assert list(out["route"]["ids"][t]) == sel


def test_identical_experts_make_routing_irrelevant():
    rng = np.random.default_rng(9)
    H, I, E, k = 16, 8, 8, 2
    h = rng.standard_normal((10, H))
    one_gu, one_d = rng.standard_normal((2 * I, H)) * 0.3, rng.standard_normal((H, I)) * 0.3
    wts = {"w_router": rng.standard_normal((E, H)), "bias": np.zeros(E),
           "w_gate_up": np.broadcast_to(one_gu, (E, 2 * I, H)).copy(),
           "w_down": np.broadcast_to(one_d, (E, H, I)).copy()}
    out = O.moe_layer(h, wts, k, 1e-6, "exact")
    y = O.swiglu(O.rmsnorm(h, 1e-6), one_gu, one_d, "exact")
    np.testing.assert_allclose(out["combined"], y, rtol=1e-12, atol=1e-14)


def test_bf16_mode_rounds_at_storage_points():
    rng = np.random.default_rng(10)
    H, I, E = 32, 16, 4
    tb = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    wts = {"w_router": rng.standard_normal((E, H)).astype(np.float32) * 0.02, "bias": np.zeros(E, np.float32),
           "w_gate_up": tb(rng.standard_normal((E + 2, 2 * I, H)) * 0.02), "w_down": tb(rng.standard_normal((E + 2, H, I)) * 0.02)}
    h = tb(rng.standard_normal((8, H)))
    out = O.moe_layer(h, wts, 2, 1e-6, "bf16")
    for a in (out["route"]["xn"], out["y"], out["ys"], out["h_out"]):
        np.testing.assert_array_equal(O.round_bf16(a), a)
    ex = O.moe_layer(h, wts, 2, 1e-6, "exact")
    # storage rounding moves the block output by at most a few bf16 ulps
    assert np.max(np.abs(out["h_out"] - ex["h_out"])) < 0.05


# --------------------------------------------------------------------------
# LM head
# --------------------------------------------------------------------------

def test_lm_argmax_bruteforce_with_ties_across_chunks():
    rng = np.random.default_rng(11)
    T, H, V = 6, 5, 50
    h = rng.standard_normal((T, H))
    W = rng.standard_normal((V, H))
    W[37] = W[12]              # exact tie between ids 12 and 37 (different chunks of 7)
    h[0] = W[12] * 10          # row 0 very likely peaks at the tied pair
    ids, mx, gap = O.lm_argmax(h, W, chunk=7)
    for t in range(T):
        lg = [sum(h[t, j] * W[v, j] for j in range(H)) for v in range(V)]
        best = 0
        for v in range(1, V):
            if lg[v] > lg[best]:
                best = v
        assert ids[t] == best
        assert math.isclose(mx[t], lg[best], rel_tol=1e-12)
        s = sorted(lg, reverse=True)
        assert math.isclose(gap[t], s[0] - s[1], abs_tol=1e-12)
    assert ids[0] == 12 and gap[0] == 0.0


def test_lm_argmax_one_hot_selects_weight_column():
    rng = np.random.default_rng(12)
    V, H = 300, 16
    W = rng.standard_normal((V, H))
    h = np.eye(H)
    ids, _, _ = O.lm_argmax(h, W, chunk=64)
    np.testing.assert_array_equal(ids, np.argmax(W, axis=0))


# --------------------------------------------------------------------------
# acceptance
# --------------------------------------------------------------------------

def test_spec_verify_bruteforce_v3_k3():
    """All 3^3 drafts x 3^4 verifier outputs (2,187 cases) against a prefix-slice
    formulation: the accepted count is the longest m with d[:m] == g[:m]."""
    cases = list(itertools.product(itertools.product(range(3), repeat=3), itertools.product(range(3), repeat=4)))
    assert len(cases) == 2187
    D = np.array([c[0] for c in cases])
    G = np.array([c[1] for c in cases])
    acc, com, nc = O.spec_verify(D, G)
    for i, (d, g) in enumerate(cases):
        m = max(m for m in range(4) if list(d[:m]) == list(g[:m]))
        assert acc[i] == m and nc[i] == m + 1 <= 4
        assert list(com[i]) == list(d[:m]) + [g[m]] + [-1] * (3 - m)


def test_spec_verify_k0_is_greedy():
    g = np.array([[5], [7], [0]])
    acc, com, nc = O.spec_verify(np.zeros((3, 0), np.int64), g)
    assert list(acc) == [0, 0, 0] and list(nc) == [1, 1, 1] and list(com[:, 0]) == [5, 7, 0]


def test_plant_drafts_leading_keeps():
    rng = np.random.default_rng(13)
    V, B, K = 97, 2000, 3
    g = rng.integers(0, V, (B, K + 1))
    keep = rng.random((B, K)) < 0.576
    repl = rng.integers(0, V - 1, (B, K))
    d = O.plant_drafts(g, keep, repl)
    assert np.all((d == g[:, :K]) == keep)             # a replaced draft never matches
    assert d.min() >= 0 and d.max() < V
    acc, _, nc = O.spec_verify(d, g)
    lead = np.array([next((i for i in range(K) if not keep[b, i]), K) for b in range(B)])
    np.testing.assert_array_equal(acc, lead)


def test_planted_tau_closed_form():
    """n+1 with independent keeps has mean 1+p+p^2+p^3; the pages' tau = 1 + K*alpha
    relation holds for their printed acceptance 57.6% and tau 2.73."""
    f = facts()
    p, K = f["acceptance_rate_K3"], f["draft_tokens_K"]
    rng = np.random.default_rng(14)
    n_s = 200000
    keep = rng.random((n_s, K)) < p
    g = np.zeros((n_s, K + 1), np.int64)
    d = O.plant_drafts(g, keep, rng.integers(0, 10, (n_s, K)))
    _, _, nc = O.spec_verify(d, g)
    expect = 1 + p + p ** 2 + p ** 3
    se = nc.std() / math.sqrt(n_s)
    assert abs(nc.mean() - expect) < 4 * se
    assert abs((1 + K * p) - f["tau_eager_K3"]) < 0.005            # 2.728 vs 2.73
    assert abs(f["tau_eager_K3"] / f["speedup_eager_K3"] - f["cost_eager"]) < 0.005   # c = tau / speedup
    assert abs(f["spec_tok_s_eager"] / f["ar_tok_s_eager"] - f["speedup_eager_K3"]) < 0.01


def test_tau_matched_keep_probability():
    """The secondary planting: the keep probability q whose mean commits per
    pass, 1 + q + q^2 + q^3, equal the pages' printed tau of 2.73 is 0.749
    (to 3 decimals); planted at q, the oracle's mean n+1 matches it."""
    f = facts()
    K = f["draft_tokens_K"]
    tau = f["tau_eager_K3"]
    lo, hi = 0.0, 1.0
    for _ in range(60):   # bisection: 1 + q + q^2 + q^3 is increasing on [0, 1]
        mid = (lo + hi) / 2
        lo, hi = (mid, hi) if sum(mid ** i for i in range(K + 1)) < tau else (lo, mid)
    assert round(lo, 3) == 0.749
    q = 0.749
    rng = np.random.default_rng(15)
    n_s = 200000
    keep = rng.random((n_s, K)) < q
    g = np.zeros((n_s, K + 1), np.int64)
    d = O.plant_drafts(g, keep, rng.integers(0, 10, (n_s, K)))
    _, _, nc = O.spec_verify(d, g)
    se = nc.std() / math.sqrt(n_s)
    assert abs(nc.mean() - sum(q ** i for i in range(K + 1))) < 4 * se
    assert abs(sum(q ** i for i in range(K + 1)) - tau) < 0.005


# --------------------------------------------------------------------------
# speculative decoding is token-identical to greedy decoding
# --------------------------------------------------------------------------

def _tiny_token_model(seed=0):
    """Token-driven tiny model: embedding 512x128 -> one tiny MoE block -> LM head 512."""
    rng = np.random.default_rng(seed)
    V, H, I, E, k = 512, 128, 64, 8, 2
    emb = rng.standard_normal((V, H))
    wts = {"w_router": rng.standard_normal((E, H)) * 0.02, "bias": np.zeros(E),
           "w_gate_up": rng.standard_normal((E + 2, 2 * I, H)) * 0.02,
           "w_down": rng.standard_normal((E + 2, H, I)) * 0.02}
    w_lm = rng.standard_normal((V, H)) * 0.02
    cache = {}

    def next_tokens(tokens):
        out = []
        for t in tokens:
            if t not in cache:
                hout = O.moe_layer(emb[[t]], wts, k, 1e-6, "exact")["h_out"]
                cache[t] = int(O.lm_argmax(hout, w_lm)[0][0])
            out.append(cache[t])
        return out
    return next_tokens, V


@pytest.mark.parametrize("K", [0, 1, 2, 3])
def test_speculative_equals_greedy(K):
    next_tokens, V = _tiny_token_model()
    rng = np.random.default_rng(100 + K)
    n = 60
    ref = O.greedy_decode(7, n, next_tokens)
    # random proposals
    seq, passes, commits = O.speculative_decode(7, n, next_tokens, lambda s, K: rng.integers(0, V, K), K)
    assert seq == ref and all(1 <= c <= K + 1 for c in commits)
    # planted proposals (keep the true continuation with probability 0.576)
    def planted(s, K):
        pos = len(s) - 1
        truth = ref[pos + 1:pos + 1 + K] + [0] * K
        return [truth[i] if rng.random() < 0.576 else int(rng.integers(0, V)) for i in range(K)]
    seq, passes, commits = O.speculative_decode(7, n, next_tokens, planted, K)
    assert seq == ref
    # perfect proposals commit K+1 per pass
    seq, passes, commits = O.speculative_decode(
        7, n, next_tokens, lambda s, K: (ref[len(s):len(s) + K] + [0] * K)[:K], K)
    assert seq == ref and all(c == K + 1 for c in commits[:-1])


def test_verify_step_composition_by_hand():
    """verify_step chains L blocks, takes the LM-head argmax of every row and
    judges each sequence's drafts against its own K+1 rows (sequence-major).
    Recomputed here per row: the blocks as loops over tokens, the full logits
    with a linear scan, and acceptance by walking each sequence; drafts are
    planted from that scan so that some sequences accept 0, some 1..K."""
    rng = np.random.default_rng(41)
    B, K, H, I, E, k, V = 4, 3, 16, 8, 4, 2, 37
    layers = [{"w_router": rng.standard_normal((E, H)) * 0.3, "bias": np.zeros(E),
               "w_gate_up": rng.standard_normal((E + 1, 2 * I, H)) * 0.3,
               "w_down": rng.standard_normal((E + 1, H, I)) * 0.3} for _ in range(2)]
    w_lm = rng.standard_normal((V, H))
    h = rng.standard_normal((B * (K + 1), H))
    # per-row reference: each token alone through the two blocks
    cur = h.copy()
    for wts in layers:
        cur = np.stack([O.moe_layer(cur[[t]], wts, k, 1e-6, "exact")["h_out"][0] for t in range(B * (K + 1))])
    g = []
    for t in range(B * (K + 1)):
        lg = [float(w_lm[v] @ cur[t]) for v in range(V)]
        g.append(max(range(V), key=lambda v: (lg[v], -v)))
    g = np.array(g).reshape(B, K + 1)
    n_keep = [0, 1, 3, 2]
    drafts = np.zeros((B, K), dtype=np.int64)
    for b in range(B):
        for i in range(K):
            drafts[b, i] = g[b, i] if i < n_keep[b] else (g[b, i] + 1) % V
    out = O.verify_step(h, layers, w_lm, drafts, k, 1e-6, "exact")
    np.testing.assert_allclose(out["layers"][-1]["h_out"], cur, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(out["argmax"], g.reshape(-1))
    np.testing.assert_array_equal(out["accepted"], n_keep)
    np.testing.assert_array_equal(out["n_commit"], np.array(n_keep) + 1)
    for b in range(B):
        n = n_keep[b]
        want = list(drafts[b, :n]) + [g[b, n]] + [-1] * (K - n)
        assert list(out["committed"][b]) == want
    # teacher forcing with the free-running inputs reproduces the free run
    ins = [h] + [o["h_out"] for o in out["layers"][:-1]]
    tf = O.verify_step(h, layers, w_lm, drafts, k, 1e-6, "exact", layer_inputs=ins,
                       lm_input=out["layers"][-1]["h_out"])
    np.testing.assert_array_equal(tf["argmax"], out["argmax"])


# --------------------------------------------------------------------------
# attention over a KV cache
# --------------------------------------------------------------------------

def test_rope_position_zero_is_identity_and_rotations_keep_norms():
    rng = np.random.default_rng(31)
    x = rng.standard_normal((5, 3, 16))
    np.testing.assert_allclose(O.rope(x, np.zeros(5)), x, rtol=0, atol=0)
    y = O.rope(x, rng.integers(0, 30000, 5))
    n_x = x[..., :8] ** 2 + x[..., 8:] ** 2
    n_y = y[..., :8] ** 2 + y[..., 8:] ** 2
    np.testing.assert_allclose(n_y, n_x, rtol=1e-12)


def test_rope_scores_depend_only_on_the_position_difference():
    rng = np.random.default_rng(32)
    q, k = rng.standard_normal((1, 2, 32)), rng.standard_normal((1, 2, 32))
    for shift in (1, 17, 4000):
        for dp in (0, 3, 250):
            a = (O.rope(q, [dp + 5]) * O.rope(k, [5])).sum(-1)
            b = (O.rope(q, [dp + 5 + shift]) * O.rope(k, [5 + shift])).sum(-1)
            np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-9)


def test_rope_closed_form_d4_position_1():
    """d = 4 (m = 2) at position 1: the angles are 1 * 10000^(-j/2), i.e. 1 and
    0.01.  Unit vectors rotate by hand: e0 -> (cos 1, 0, sin 1, 0),
    e1 -> (0, cos .01, 0, sin .01), e2 -> (-sin 1, 0, cos 1, 0),
    e3 -> (0, -sin .01, 0, cos .01).  A wrong frequency schedule or a reversed
    rotation fails it."""
    c1, s1, c2, s2 = math.cos(1.0), math.sin(1.0), math.cos(0.01), math.sin(0.01)
    want = np.array([[c1, 0, s1, 0], [0, c2, 0, s2], [-s1, 0, c1, 0], [0, -s2, 0, c2]])
    got = O.rope(np.eye(4)[:, None, :], np.ones(4))[:, 0, :]
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-15)


def test_rope_closed_form_head_128_far_position():
    """The decoder's head of 128 dims (m = 64): component j pairs with j + 64 and
    turns by pos * 10000^(-j/64).  Checked for a few j at position 20,000 by
    direct cos/sin of the angle written out."""
    pos = 20000
    for j in (0, 1, 17, 63):
        x = np.zeros((1, 1, 128))
        x[0, 0, j] = 2.0
        x[0, 0, j + 64] = -0.5
        a = pos * 10000.0 ** (-j / 64.0)
        got = O.rope(x, [pos])[0, 0]
        want = np.zeros(128)
        want[j] = 2.0 * math.cos(a) + 0.5 * math.sin(a)
        want[j + 64] = 2.0 * math.sin(a) - 0.5 * math.cos(a)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def _attn_weights(rng, H, n_heads):
    return rng.standard_normal((3 * H, H)) * 0.05, rng.standard_normal((H, H)) * 0.05


def test_attention_first_position_returns_its_own_value():
    """An empty cache and one position: softmax over one key is 1, so the
    output is the value of the position itself."""
    rng = np.random.default_rng(33)
    H, nh = 64, 4
    wqkv, wo = _attn_weights(rng, H, nh)
    ck, cv = np.zeros((2, nh, 8, 16)), np.zeros((2, nh, 8, 16))
    out = O.attention_block(rng.standard_normal((2, H)), wqkv, wo, ck, cv, [0, 0], 1, nh, 1e-6, "exact")
    np.testing.assert_allclose(out["o"], out["v"].reshape(2, H), rtol=1e-12)


def test_attention_zero_queries_average_the_values():
    """q = 0 makes every score equal: the output is the plain mean of the
    visible values, over the cached prefix and the causal part of the pass."""
    rng = np.random.default_rng(34)
    H, nh, P = 64, 4, 3
    wqkv, wo = _attn_weights(rng, H, nh)
    wqkv[:H] = 0.0
    ck = rng.standard_normal((1, nh, 20, 16))
    cv = rng.standard_normal((1, nh, 20, 16))
    cv0 = cv.copy()
    out = O.attention_block(rng.standard_normal((P, H)), wqkv, wo, ck, cv, [5], P, nh, 1e-6, "exact")
    v = out["v"]
    for i in range(P):
        vis = np.concatenate([cv0[0, :, :5], np.moveaxis(v[:i + 1], 0, 1)], axis=1)   # [nh, 5+i+1, d]
        np.testing.assert_allclose(out["o"][i].reshape(nh, 16), vis.mean(axis=1), rtol=1e-10, atol=1e-12)


def test_attention_two_keys_closed_form():
    """One head, d = 4, one cached key k1 = e0 with value v1, and the pass's own
    position with key k2 = 0 and value v2.  A query (a, 0, 0, 0) scores a/sqrt(4)
    and 0, so o = sigmoid(a/2) v1 + (1 - sigmoid(a/2)) v2.  A missing or wrong
    score scale fails it."""
    rng = np.random.default_rng(37)
    for a in (-3.0, 0.7, 5.0):
        ck, cv = np.zeros((1, 1, 4, 4)), np.zeros((1, 1, 4, 4))
        ck[0, 0, 0] = [1.0, 0, 0, 0]
        v1, v2 = rng.standard_normal(4), rng.standard_normal(4)
        cv[0, 0, 0], cv[0, 0, 1] = v1, v2        # row 1 is the pass's own position (L = 1)
        q = np.array([[[a, 0.0, 0.0, 0.0]]])
        o = O.causal_attention(q, ck, cv, [1], 1)[0, 0]
        w = 1.0 / (1.0 + math.exp(-a / 2.0))
        np.testing.assert_allclose(o, w * v1 + (1 - w) * v2, rtol=1e-13, atol=1e-15)


def test_attention_three_keys_d16_closed_form():
    """d = 16 (scale 1/4): three visible keys with scores s_j = q . k_j / 4 set by
    hand, two heads with different queries, two positions of one pass.  The
    weights are exp(s_j) / sum exp(s), written out per key."""
    d, nh = 16, 2
    ck, cv = np.zeros((1, nh, 8, d)), np.zeros((1, nh, 8, d))
    rng = np.random.default_rng(38)
    ck[0, :, 0, 0] = 1.0          # key 0 = e0
    ck[0, :, 1, 1] = 2.0          # key 1 = 2 e1
    ck[0, :, 2, 0] = -1.0         # key 2 = -e0 + e2 (the pass's first position)
    ck[0, :, 2, 2] = 1.0
    ck[0, :, 3, 3] = 1.0          # key 3 = e3 (the pass's second position)
    cv[0, :, :4] = rng.standard_normal((nh, 4, d))
    q = np.zeros((2, nh, d))
    q[:, 0, :4] = [2.0, 1.0, 3.0, 0.5]
    q[:, 1, :4] = [-1.0, 0.0, 0.5, 4.0]
    o = O.causal_attention(q, ck, cv, [2], 2)
    for i in range(2):
        for hd in range(nh):
            qq = q[i, hd]
            n_vis = 3 + i
            s = [float(qq @ ck[0, hd, j]) / 4.0 for j in range(n_vis)]
            z = [math.exp(x) for x in s]
            want = sum(z[j] / sum(z) * cv[0, hd, j] for j in range(n_vis))
            np.testing.assert_allclose(o[i, hd], want, rtol=1e-12, atol=1e-14)


def test_attention_ignores_cache_entries_past_each_position():
    """Causality, and rollback for free: entries past L+i (rejected drafts of
    an earlier pass) never change the result."""
    rng = np.random.default_rng(35)
    H, nh, P = 64, 4, 4
    wqkv, wo = _attn_weights(rng, H, nh)
    h = rng.standard_normal((2 * P, H))
    base_k = rng.standard_normal((2, nh, 40, 16))
    base_v = rng.standard_normal((2, nh, 40, 16))
    outs = []
    for junk in (0.0, 1e3):
        ck, cv = base_k.copy(), base_v.copy()
        ck[:, :, 12:] += junk
        cv[:, :, 12:] -= junk
        outs.append(O.attention_block(h, wqkv, wo, ck, cv, [12, 7], P, nh, 1e-6, "exact"))
    np.testing.assert_allclose(outs[0]["h_out"], outs[1]["h_out"], rtol=1e-12, atol=1e-12)


def test_attention_commit_then_next_pass_equals_prefix_only_cache():
    """Pass 1 writes P positions; only n+1 are committed; pass 2 starts at the
    committed length and overwrites the rest.  Its result equals running pass
    2 on a cache holding the committed prefix alone."""
    rng = np.random.default_rng(36)
    H, nh, P = 64, 4, 4
    wqkv, wo = _attn_weights(rng, H, nh)
    ck, cv = np.zeros((1, nh, 32, 16)), np.zeros((1, nh, 32, 16))
    ck[:, :, :6] = rng.standard_normal((1, nh, 6, 16))
    cv[:, :, :6] = rng.standard_normal((1, nh, 6, 16))
    pre_k, pre_v = ck.copy(), cv.copy()
    h1 = rng.standard_normal((P, H))
    O.attention_block(h1, wqkv, wo, ck, cv, [6], P, nh, 1e-6, "exact")   # writes 6..9
    n_commit = 2                                                            # 6, 7 kept; 8, 9 rejected
    h2 = rng.standard_normal((P, H))
    a = O.attention_block(h2, wqkv, wo, ck, cv, [6 + n_commit], P, nh, 1e-6, "exact")
    # reference: a fresh cache with the prefix and the two committed positions only
    fk, fv = pre_k.copy(), pre_v.copy()
    O.attention_block(h1[:n_commit], wqkv, wo, fk, fv, [6], n_commit, nh, 1e-6, "exact")
    fk[:, :, 8:], fv[:, :, 8:] = 0.0, 0.0
    b = O.attention_block(h2, wqkv, wo, fk, fv, [6 + n_commit], P, nh, 1e-6, "exact")
    np.testing.assert_allclose(a["h_out"], b["h_out"], rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# the dense draft block
# --------------------------------------------------------------------------

def _draft_tiny(rng, V=97, H=64, I=48):
    return {"emb": rng.standard_normal((V, H)), "w_proj": rng.standard_normal((H, 2 * H)) * 0.02,
            "w_gate_up": rng.standard_normal((2 * I, H)) * 0.02, "w_down": rng.standard_normal((H, I)) * 0.02}


def test_draft_identity_projection_reduces_to_greedy_head():
    """W_p = [I | 0] and a zero FFN: each step's hidden state is the normed
    input, so every draft is the LM head's argmax of rmsnorm(h), and feeding
    the hidden state back (rmsnorm of a normed row is the row) repeats it."""
    rng = np.random.default_rng(21)
    V, H = 97, 64
    w = _draft_tiny(rng, V, H)
    w["w_proj"] = np.concatenate([np.eye(H), np.zeros((H, H))], axis=1)
    w["w_down"] = np.zeros_like(w["w_down"])
    w_lm = rng.standard_normal((V, H))
    h = rng.standard_normal((5, H)) * 3.0
    tok = rng.integers(0, V, 5)
    out = O.draft_propose(h, tok, w, w_lm, 3, 1e-6, "exact")
    ref, _, gap = O.lm_argmax(O.rmsnorm(h, 1e-6), w_lm)
    ok = gap > 1e-9
    np.testing.assert_allclose(out["steps"][0]["h1"], O.rmsnorm(h, 1e-6), rtol=1e-14, atol=0)
    for i in range(3):
        np.testing.assert_array_equal(out["drafts"][ok, i], ref[ok])
        # a normed row has mean square 1 - O(eps), so renorming moves it by O(eps)
        np.testing.assert_allclose(out["steps"][i]["h1"], O.rmsnorm(h, 1e-6), rtol=1e-5, atol=0)


def test_draft_token_projection_copies_the_token():
    """W_p = [0 | I], zero FFN and the LM head tied to the embedding: the
    draft is the token whose embedding best matches rmsnorm(E[tok]), i.e. tok
    itself for random high-dimensional embeddings; the recursion feeds each
    draft back as the next input token, so all K drafts repeat it."""
    rng = np.random.default_rng(22)
    V, H = 97, 64
    w = _draft_tiny(rng, V, H)
    w["w_proj"] = np.concatenate([np.zeros((H, H)), np.eye(H)], axis=1)
    w["w_down"] = np.zeros_like(w["w_down"])
    h = rng.standard_normal((6, H))
    tok = rng.integers(0, V, 6)
    # embeddings with equal norms so the best match is the token itself
    w["emb"] = w["emb"] / np.linalg.norm(w["emb"], axis=1, keepdims=True)
    out = O.draft_propose(h, tok, w, w["emb"], 4, 1e-6, "exact")
    np.testing.assert_array_equal(out["drafts"], np.repeat(tok[:, None], 4, axis=1))


def test_draft_block_ffn_is_the_residual_swiglu():
    """A zero projection makes h0 = 0, whose RMSNorm is 0, so the FFN adds
    silu(0) * 0 = 0: h1 = 0 and the draft is the lowest vocabulary id (all
    logits equal) -- the tie rule through the whole block."""
    rng = np.random.default_rng(23)
    w = _draft_tiny(rng)
    w["w_proj"] = np.zeros_like(w["w_proj"])
    out = O.draft_step(rng.standard_normal((3, 64)), np.array([1, 2, 3]), w, rng.standard_normal((97, 64)),
                       1e-6, "bf16")
    assert not out["h1"].any()
    np.testing.assert_array_equal(out["ids"], [0, 0, 0])


def _rms_loop(v, eps):
    ms = sum(float(x) * float(x) for x in v) / len(v)
    return [float(x) / math.sqrt(ms + eps) for x in v]


def test_draft_step_nonzero_ffn_written_as_loops():
    """A draft step with every weight non-zero, recomputed with plain loops:
    x = [rmsnorm(h); rmsnorm(E[tok])], h0 = W_p x, z = rmsnorm(h0),
    f = W_d (silu(W_g z) * W_u z), h1 = h0 + f, draft = argmax of W_lm h1.
    W_p is small, so h0 is far from unit RMS and the FFN fed h0 (or x) instead
    of z fails; so does a dropped residual."""
    rng = np.random.default_rng(24)
    V, H, I = 23, 12, 10
    w = _draft_tiny(rng, V, H, I)
    w["w_gate_up"] = w["w_gate_up"] * 40.0     # make the FFN term comparable to h0
    w["w_down"] = w["w_down"] * 40.0
    w_lm = rng.standard_normal((V, H))
    h = rng.standard_normal((3, H)) * 2.0
    tok = np.array([4, 0, 22])
    eps = 1e-6
    out = O.draft_step(h, tok, w, w_lm, eps, "exact")
    for t in range(3):
        x = _rms_loop(h[t], eps) + _rms_loop(w["emb"][tok[t]], eps)
        h0 = [sum(w["w_proj"][r][c] * x[c] for c in range(2 * H)) for r in range(H)]
        z = _rms_loop(h0, eps)
        g = [sum(w["w_gate_up"][r][c] * z[c] for c in range(H)) for r in range(I)]
        u = [sum(w["w_gate_up"][I + r][c] * z[c] for c in range(H)) for r in range(I)]
        a = [g[r] / (1.0 + math.exp(-g[r])) * u[r] for r in range(I)]
        f = [sum(w["w_down"][r][c] * a[c] for c in range(I)) for r in range(H)]
        h1 = [h0[r] + f[r] for r in range(H)]
        np.testing.assert_allclose(out["x"][t], x, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(out["h0"][t], h0, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(out["z"][t], z, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(out["h1"][t], h1, rtol=1e-12, atol=1e-14)
        logits = [sum(w_lm[v][c] * h1[c] for c in range(H)) for v in range(V)]
        best = max(range(V), key=lambda v: (logits[v], -v))
        assert out["ids"][t] == best
        # the FFN contributes: h1 differs from h0 by more than rounding
        assert max(abs(f[r]) for r in range(H)) > 0.05 * max(abs(v) for v in h0)


@pytest.mark.parametrize("K", [1, 3])
def test_speculation_with_draft_block_proposals_equals_greedy(K):
    """Drafts from the (untrained, random) draft block: the committed
    sequence is still exactly the greedy one."""
    next_tokens, V = _tiny_token_model()
    rng = np.random.default_rng(300 + K)
    H = 128
    w = _draft_tiny(rng, V, H, 64)
    w_lm = rng.standard_normal((V, H)) * 0.02
    emb = rng.standard_normal((V, H))

    def propose(s, K):
        out = O.draft_propose(emb[[s[-1]]], np.array([s[-1]]), w, w_lm, K, 1e-6, "exact")
        return [int(d) for d in out["drafts"][0]]
    ref = O.greedy_decode(7, 40, next_tokens)
    seq, passes, commits = O.speculative_decode(7, 40, next_tokens, propose, K)
    assert seq == ref and all(1 <= c <= K + 1 for c in commits)


# --------------------------------------------------------------------------
# parameter accounting against the pages
# --------------------------------------------------------------------------

def test_active_and_total_params_match_pages():
    f = facts()
    H, E, k, S, V, L = f["hidden"], f["routed_experts"], f["top_k"], f["shared_experts"], f["vocab"], f["decoder_layers"]
    I = 896          # synthetic intermediate size (the pages do not give it)
    attn = 4 * H * H  # attention projections q,k,v,o, omitted from the hot path
    moe_only = O.active_params(H, E, k, S, I, V, L)
    assert moe_only == 496_762_880
    act = O.active_params(H, E, k, S, I, V, L, attn_per_layer=attn)
    assert abs(act / f["active_params_approx"] - 1) < 0.015           # 575.4M vs ~570M
    tot = O.total_params(H, E, S, I, V, L, attn_per_layer=attn, encoder=f["encoder_params_approx"])
    assert abs(tot / f["total_params_approx"] - 1) < 0.03              # 3.35B vs 3.4B
    assert abs(f["total_params_approx"] * 2 / 1e9 - f["weights_bf16_gb_approx"]) < 0.05
    # visual token budget: 256 base + 9 tiles x 100
    assert f["visual_tokens_base"] + f["visual_tiles_max"] * f["visual_tokens_per_tile"] == f["visual_tokens_max"]
    # throughput arithmetic on the A100 run
    assert abs(f["pages_per_s_a100"] * f["tokens_per_page"] / f["tokens_per_s_a100"] - 1) < 0.005


# ---------------------------------------------------------------- Zipf router bias (prefill layer)

def test_zipf_bias_fixture_reproduces_its_counts():
    """The stored prefill router bias: its targets are the water-filled Zipf(1.1)
    counts (sum 6 T, capped at T, ratio ((r+1)/r)^1.1 below the cap), and the
    oracle's own routing of the calibration batch with that bias gives the
    stored realised counts, which follow the targets."""
    import synth
    from tests.golden.make_zipf_bias import counts, zipf_targets
    with open(os.path.join(os.path.dirname(__file__), "golden", "zipf_bias_prefill.json")) as f:
        fx = json.load(f)
    cal = fx["calibration"]
    T, k, E = cal["tokens"], 6, 64
    tgt = np.array(fx["target_counts_by_rank"])
    np.testing.assert_allclose(tgt, zipf_targets(T, k, E, cal["zipf_s"]))
    assert abs(tgt.sum() - k * T) < 1e-6 * T and tgt.max() <= T
    free = tgt < T
    r = np.arange(1, E + 1)[free]
    np.testing.assert_allclose(tgt[free][:-1] / tgt[free][1:], ((r[1:]) / r[:-1]) ** cal["zipf_s"], rtol=1e-9)
    assert sorted(fx["rank_to_expert"]) == list(range(E))
    sh = synth.SHAPES["prefill"]
    wr = synth.router_weight(fx["router_weight"]["seed"], fx["router_weight"]["layer"], sh).numpy()
    h = synth.bf16_bits(synth.hidden(cal["seed"], T, sh.H, torch.bfloat16, name=cal["hidden_name"]))
    xn = O.store(O.rmsnorm(O.f64(h), sh.eps), "bf16")
    n = counts(xn, wr, np.array(fx["bias"], np.float32).astype(np.float64), k, E)
    by_rank = n[fx["rank_to_expert"]]
    np.testing.assert_array_equal(by_rank, fx["realised_counts_by_rank"])
    assert n.sum() == k * T
    assert np.all(np.abs(by_rank - tgt) <= 0.1 * tgt + 10)
