"""Plain, slow fp64 CPU oracle of the MoE speculative verify step.

TEST INFRASTRUCTURE.  Only the tests, the smoke check of the entry module and
the CPU-baseline leg of the benchmark may import, call or execute anything in
this package.  The product path (the HIP library and its Python binding) never
does, and this package imports nothing from it: the two share no kernels,
headers, helpers, tables or constants.  Both sides only share the seeded input
generators in ``synth`` (random draws, no method arithmetic).

What it computes and where each step comes from:

* decoder block shape (12 layers, hidden 1280, 64 routed + 2 shared experts,
  top-6 routing, vocabulary 129,280): jina.ai/ko model card "jina-ocr-v1",
  architecture paragraph; aikraft.ru "Jina OCR v1: ...", section
  "01 Архитектура и эффективность"; alphasignal.ai "Jina AI's 3.4B OCR model
  targets faster page parsing", section "A compressed visual front end".
* greedy verification that accepts the longest prefix on which draft and
  verifier agree, so the committed sequence equals the verifier's greedy
  sequence: jina.ai/de "jina-ocr-v1: Schnellere Dokumentenanalyse auf
  kostengünstigen GPUs", section "Modell und Training".
* a committed count per speculative step that includes the bonus token:
  same page, section "Spekulatives Decoding auf einer L4".

The pages are silent on the norm, the routing function, the expert form and
the precision; the readings taken here (pre-RMSNorm eps 1e-6 with unit gain,
softmax over biased fp32 logits renormalised over the selected k with ties to
the lower expert id, SwiGLU experts without biases, shared experts weighted 1,
no final norm before the LM head, argmax ties to the lowest id) are listed in
the design notes of the repository.

Two modes: ``"exact"`` keeps fp64 everywhere (the mathematical definition);
``"bf16"`` / ``"f32"`` accumulate in fp64 but round to the storage dtype at the
storage points of the step (xn after the norm, the SwiGLU activation before
the down projection, each expert output, the layer output).  Parity of the GPU
path is judged against the rounding mode of its storage dtype.

Pin status (what fixes each function other than itself; tests/test_oracle_*):
  round_bf16 ......... torch's fp32->bf16 cast; hand-worked tie cases
  rmsnorm ............ constant-vector closed form; scale invariance
  topk_ids ........... brute force over every k-subset (max sum, lexicographic ties)
  topk_weights ....... sum 1; renormalised-full-softmax identity; zero-logit case
  permute ............ bijection / stability / offsets invariants
  swiglu / moe_layer . E=1,k=1 reduces to a dense SwiGLU FFN written as loops;
                       identical experts make routing irrelevant
  lm_argmax .......... brute-force scan; one-hot input selects a weight column
  spec_verify ........ brute force over V=3, K=3 against a prefix-slice
                       formulation; K=0 is greedy; n_commit = n+1 <= K+1
  speculative loop ... token-identical to step-by-step greedy decoding
  plant_drafts ....... accepted count = leading keeps; E[n+1] = 1+p+p^2+p^3
  active_params ...... the pages' ~570M active per token and 3.4B total
  verify_step ........ rows chained through the blocks one token at a time, a
                       linear argmax scan and acceptance walked per sequence
  rope ............... hand rotations of unit vectors at d = 4 (angles 1, 0.01)
                       and at d = 128 (pos * 10000^(-j/64)); position 0 is the
                       identity; norms kept; scores depend on distance only
  causal_attention ... two and three visible keys with scores set by hand
                       (softmax weights in closed form, scale 1/sqrt(d));
                       causality; zero queries average the values
  draft_step ......... every weight non-zero, recomputed with loops (FFN on
                       z = rmsnorm(h0), residual h0); identity and token
                       projections reduce to the greedy head / copy the token
Numerical values at the real shapes are otherwise parity unpinned: the pages
print no tensors, logits or token ids.
"""

from .moe import *  # noqa: F401,F403
from .moe import __all__  # noqa: F401
