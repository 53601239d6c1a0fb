"""Router bias for the 36,992-token prefill layer: Zipf(1.1) expert popularity.

    python tests/golden/make_zipf_bias.py      # writes tests/golden/zipf_bias_prefill.json

The prefill workload asks for expert popularity that follows Zipf with
exponent 1.1 over the 64 routed experts, so that the grouped GEMM sees
strongly unequal groups.  An exact Zipf share cannot be met with top-6
routing: rank 1 would need about a quarter of all assignments, and an expert
can be chosen by at most every token (one sixth).  The reading taken:

* target assignment counts c_r = min(T, lam * r**-1.1) for ranks r = 1..64,
  with lam chosen (by bisection) so that sum_r c_r = 6 T ("water-filled");
* ranks are given to experts by a seeded permutation;
* the router bias b (added to the logits before selection) is fitted on a
  separate calibration batch of 8,192 tokens (seed 99) by a fixed number of
  log-ratio steps  b_e += eta * (ln c_e - ln max(n_e, 0.5)),  where n_e is the
  number of tokens whose top-6 holds expert e under the current bias.

Every routing decision here is the oracle's (RMSNorm in the bf16 storage
mode, fp64 router logits with the bias, top-k with the lower-id tie rule);
this script draws its inputs from `synth` and calls nothing else.
"""

from __future__ import annotations

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
import synth  # noqa: E402

OUT = os.path.join(HERE, "zipf_bias_prefill.json")
WEIGHT_SEED, LAYER = 1, 0          # the router of the real-shape layer
CAL_SEED, CAL_TOKENS = 99, 8192
ZIPF_S = 1.1
ITERS, ETA = 300, 0.25


def zipf_targets(T: int, k: int, E: int, s: float) -> np.ndarray:
    """Water-filled counts c_r = min(T, lam r^-s) with sum = k T, by rank."""
    w = np.arange(1, E + 1, dtype=np.float64) ** -s
    lo, hi = 0.0, k * T / w[-1]
    for _ in range(200):
        lam = 0.5 * (lo + hi)
        if np.minimum(T, lam * w).sum() < k * T:
            lo = lam
        else:
            hi = lam
    return np.minimum(T, 0.5 * (lo + hi) * w)


def counts(xn, wr, bias, k: int, E: int) -> np.ndarray:
    ids = O.topk_ids(O.router_logits(xn, wr, bias), k)
    return np.bincount(ids.ravel(), minlength=E)


def main() -> None:
    sh = synth.SHAPES["prefill"]
    wr = synth.router_weight(WEIGHT_SEED, LAYER, sh).numpy()
    h = synth.bf16_bits(synth.hidden(CAL_SEED, CAL_TOKENS, sh.H, synth.SHAPES["layer128"].torch_dtype,
                                     name="zipf_calibration"))
    xn = O.store(O.rmsnorm(O.f64(h), sh.eps), "bf16")
    rank_perm = np.random.Generator(np.random.PCG64(CAL_SEED)).permutation(sh.E)   # expert of rank r+1
    by_rank = zipf_targets(CAL_TOKENS, sh.k, sh.E, ZIPF_S)
    target = np.empty(sh.E)
    target[rank_perm] = by_rank
    bias = np.zeros(sh.E)
    for it in range(ITERS):
        n = counts(xn, wr, bias, sh.k, sh.E)
        bias += ETA * (np.log(target) - np.log(np.maximum(n, 0.5)))
        bias -= bias.mean()
    bias32 = bias.astype(np.float32)
    n = counts(xn, wr, bias32.astype(np.float64), sh.k, sh.E)
    out = {
        "what": "router bias [64] (fp32) giving Zipf(1.1)-like expert popularity under top-6 routing",
        "recipe": "tests/golden/make_zipf_bias.py",
        "router_weight": {"seed": WEIGHT_SEED, "layer": LAYER, "shape": [sh.E, sh.H]},
        "calibration": {"seed": CAL_SEED, "tokens": CAL_TOKENS, "hidden_name": "zipf_calibration",
                        "iterations": ITERS, "eta": ETA, "zipf_s": ZIPF_S},
        "rank_to_expert": [int(e) for e in rank_perm],
        "target_counts_by_rank": [float(c) for c in by_rank],
        "realised_counts_by_rank": [int(n[e]) for e in rank_perm],
        "bias": [float(b) for b in bias32],
    }
    with open(OUT, "w") as f:
        json.dump(out, f, indent=1)
    print(f"wrote {OUT}")
    print("targets  :", np.round(by_rank[:8]).astype(int), "...", np.round(by_rank[-3:]).astype(int))
    print("realised :", [int(n[e]) for e in rank_perm[:8]], "...", [int(n[e]) for e in rank_perm[-3:]])


if __name__ == "__main__":
    main()
