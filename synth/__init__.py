"""Seeded synthetic inputs shared by the oracle-side tests and the GPU path.

This module draws random numbers and nothing else: it holds none of the MoE
step's arithmetic (no norm, routing, expert FFN, combine, LM head or
acceptance).  Every tensor is a pure function of (seed, name, layer, shape,
device), so a run can be repeated exactly.

Recipe (the model's shapes follow the jina.ai/ko model card "jina-ocr-v1",
architecture paragraph: hidden 1280, 64 routed + 2 shared experts, top-6,
vocabulary 129,280, 12 decoder layers; the expert intermediate size 896 is a
synthetic choice, the pages do not give it):

* expert and LM-head weights ~ N(0, 0.02), rounded to the storage dtype
  (bf16 round-to-nearest-even via torch's cast, or fp32);
* router weight ~ N(0, 0.02) in fp32; router bias 0 unless a calibrated bias
  is supplied by the caller;
* hidden states ~ N(0, 1) in the storage dtype;
* drafts: uniform ids, or planted from a keep mask (Bernoulli(p) per
  position) and a uniform replacement draw u in [0, V-1).

Router weights, biases, masks and draws are always generated on the CPU
generator (they are small) so that CPU-side calibration and GPU runs see the
same values; large tensors are generated on the requested device.
"""

from __future__ import annotations

import hashlib
from dataclasses import dataclass

import torch

__all__ = [
    "Shape", "SHAPES", "subseed", "normal", "router_weight", "layer_weights", "lm_weight",
    "DRAFT_INTERMEDIATE", "draft_weights", "ATTN_HEAD_DIM", "attn_weights", "kv_prefix",
    "hidden", "uniform_ids", "plant_schedule", "bf16_bits",
]


@dataclass(frozen=True)
class Shape:
    """Sizes of one verify workload (tokens = seqs * positions)."""
    name: str
    H: int          # hidden size
    E: int          # routed experts
    k: int          # experts selected per token
    S: int          # shared experts
    I: int          # expert intermediate size
    V: int          # vocabulary (0 = no LM head)
    L: int          # MoE layers
    B: int          # sequences
    P: int          # positions per sequence (1 committed + K drafts)
    dtype: str      # "bf16" or "f32" storage dtype
    eps: float = 1e-6

    @property
    def T(self) -> int:
        return self.B * self.P

    @property
    def K(self) -> int:
        return self.P - 1

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


SHAPES = {
    # tiny verify: 1 layer, hidden 128, 8+2 experts (I=64), top-2, vocab 512, 4x4 tokens, fp32
    "tiny": Shape("tiny", H=128, E=8, k=2, S=2, I=64, V=512, L=1, B=4, P=4, dtype="f32"),
    # one real-shape layer at 32 sequences x 4 positions
    "layer128": Shape("layer128", H=1280, E=64, k=6, S=2, I=896, V=0, L=1, B=32, P=4, dtype="bf16"),
    # batch-1 verify through 12 layers + LM head
    "batch1": Shape("batch1", H=1280, E=64, k=6, S=2, I=896, V=129280, L=12, B=1, P=4, dtype="bf16"),
    # prefill-sized layer: 32 pages x 1,156 visual tokens
    "prefill": Shape("prefill", H=1280, E=64, k=6, S=2, I=896, V=0, L=1, B=32, P=1156, dtype="bf16"),
    # full verify step at concurrency 32: 12 layers + LM head + verify, 32 x 4 tokens
    "step128": Shape("step128", H=1280, E=64, k=6, S=2, I=896, V=129280, L=12, B=32, P=4, dtype="bf16"),
}


def subseed(seed: int, name: str, layer: int = -1) -> int:
    """A 63-bit seed derived from (seed, tensor name, layer)."""
    d = hashlib.sha256(f"{int(seed)}/{name}/{int(layer)}".encode()).digest()
    return int.from_bytes(d[:8], "little") & ((1 << 63) - 1)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(seed: int, shape, std: float, dtype, device="cpu") -> torch.Tensor:
    """std * N(0,1) drawn in fp32 on `device`, then cast to `dtype`."""
    dev = torch.device(device)
    x = torch.randn(tuple(shape), generator=_gen(seed, dev), device=dev, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def router_weight(seed: int, layer: int, sh: Shape) -> torch.Tensor:
    """Router weight [E, H] fp32 ~N(0, 0.02), always drawn on the CPU."""
    return normal(subseed(seed, "w_router", layer), (sh.E, sh.H), 0.02, torch.float32, "cpu")


def layer_weights(seed: int, layer: int, sh: Shape, device="cpu") -> dict:
    """Weights of one MoE layer.

    Layout (the kernels' HBM layout, row-major):
      w_router   [E, H]        fp32
      bias       [E]           fp32 (zeros)
      w_gate_up  [E+S, 2I, H]  storage dtype; rows 0..I-1 gate, I..2I-1 up;
                               routed experts first, shared experts last
      w_down     [E+S, H, I]   storage dtype
    """
    G = sh.E + sh.S
    dt = sh.torch_dtype
    w_router = router_weight(seed, layer, sh)
    return {
        "w_router": w_router.to(device),
        "bias": torch.zeros(sh.E, dtype=torch.float32, device=device),
        "w_gate_up": normal(subseed(seed, "w_gate_up", layer), (G, 2 * sh.I, sh.H), 0.02, dt, device),
        "w_down": normal(subseed(seed, "w_down", layer), (G, sh.H, sh.I), 0.02, dt, device),
    }


DRAFT_INTERMEDIATE = 3584   # dense draft-block FFN width (a synthetic choice: 4 x 896)


def draft_weights(seed: int, sh: Shape, device="cpu", I: int = DRAFT_INTERMEDIATE) -> dict:
    """Weights of the dense draft block (storage dtype):
      emb        [V, H]     token embedding ~N(0, 1)
      w_proj     [H, 2H]    projection of [norm(h); norm(emb)] ~N(0, 0.02)
      w_gate_up  [1, 2I, H] dense SwiGLU gate rows then up rows ~N(0, 0.02)
      w_down     [1, H, I]  ~N(0, 0.02)
    """
    dt = sh.torch_dtype
    return {
        "emb": normal(subseed(seed, "draft_emb"), (sh.V, sh.H), 1.0, dt, device),
        "w_proj": normal(subseed(seed, "draft_proj"), (sh.H, 2 * sh.H), 0.02, dt, device),
        "w_gate_up": normal(subseed(seed, "draft_gate_up"), (1, 2 * I, sh.H), 0.02, dt, device),
        "w_down": normal(subseed(seed, "draft_down"), (1, sh.H, I), 0.02, dt, device),
    }


ATTN_HEAD_DIM = 128   # attention head size (a synthetic choice: hidden 1280 = 10 heads x 128)


def attn_weights(seed: int, layer: int, sh: Shape, device="cpu") -> dict:
    """Weights of one attention block (storage dtype, row-major):
      w_qkv  [3H, H]  q rows, then k rows, then v rows ~N(0, 0.04)
      w_o    [H, H]   ~N(0, 0.02)
    The q/k scale gives attention scores of standard deviation about 2 on
    normed inputs at H = 1280 (a softmax that is neither flat nor one-hot)."""
    dt = sh.torch_dtype
    return {
        "w_qkv": normal(subseed(seed, "w_qkv", layer), (3 * sh.H, sh.H), 0.04, dt, device),
        "w_o": normal(subseed(seed, "w_o", layer), (sh.H, sh.H), 0.02, dt, device),
    }


def kv_prefix(seed: int, layer: int, shape, dtype, device="cpu", name: str = "k") -> torch.Tensor:
    """A committed KV-cache prefix [B, n_heads, max_len, d] ~N(0, 1.4^2): the
    spread of the rotated keys and values the block writes itself."""
    return normal(subseed(seed, "kv_" + name, layer), shape, 1.4, dtype, device)


def lm_weight(seed: int, sh: Shape, device="cpu") -> torch.Tensor:
    """LM head weight [V, H] in the storage dtype, ~N(0, 0.02)."""
    return normal(subseed(seed, "w_lm"), (sh.V, sh.H), 0.02, sh.torch_dtype, device)


def hidden(seed: int, T: int, H: int, dtype, device="cpu", name: str = "hidden") -> torch.Tensor:
    """Hidden states [T, H] ~N(0, 1) in `dtype`."""
    return normal(subseed(seed, name), (T, H), 1.0, dtype, device)


def uniform_ids(seed: int, shape, V: int, name: str = "drafts") -> torch.Tensor:
    """Uniform int32 ids in [0, V) (CPU)."""
    g = _gen(subseed(seed, name), "cpu")
    return torch.randint(0, V, tuple(shape), generator=g, dtype=torch.int64).to(torch.int32)


def plant_schedule(seed: int, n_steps: int, B: int, K: int, V: int, p: float):
    """Draft-planting draws for `n_steps` verify passes (CPU tensors).

    keep[s, b, i] ~ Bernoulli(p) (uint8) and repl[s, b, i] uniform in [0, V-1)
    (int32).  How a draft is formed from them is the harness's business; this
    module only draws the numbers.
    """
    g = _gen(subseed(seed, "plant"), "cpu")
    keep = (torch.rand((n_steps, B, K), generator=g, dtype=torch.float64) < p).to(torch.uint8)
    repl = torch.randint(0, max(V - 1, 1), (n_steps, B, K), generator=g, dtype=torch.int64).to(torch.int32)
    return keep, repl


def bf16_bits(t: torch.Tensor):
    """Raw uint16 bit patterns of a bf16 tensor as a NumPy array (host copy)."""
    import numpy as np
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
