"""lmhead_argmax_noalloc (the LM head with the library's static per-GPU
workspace) against lmhead_argmax with a caller workspace, through the C ABI:
two calls in a row, the second with a smaller batch, each bit-identical to
the allocating call on the same inputs."""

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def m():
    import moe_decoder_step_amd as mod
    mod.load()
    return mod


def _pair(m, h, w, ws):
    T = h.shape[0]
    ids_a = torch.full((T,), -5, dtype=torch.int32, device=DEV)
    mx_a = torch.full((T,), float("nan"), dtype=torch.float32, device=DEV)
    m.lmhead_argmax(h, w, ids_a, mx_a, ws)
    ids_b = torch.full((T,), -7, dtype=torch.int32, device=DEV)
    mx_b = torch.full((T,), float("nan"), dtype=torch.float32, device=DEV)
    m.lmhead_argmax_noalloc(h, w, ids_b, mx_b)
    torch.cuda.synchronize()
    return ids_a, mx_a, ids_b, mx_b


@pytest.mark.parametrize("shape", ["step128", "tiny"])
def test_noalloc_lmhead_matches_workspace_call(m, shape):
    sh = synth.SHAPES[shape]
    w_lm = synth.lm_weight(3, sh, DEV)
    w = m.lm_weights(w_lm)
    big = 512 if sh.dtype == "bf16" else 64          # 512 rows: 4.1 MB of the 4 MiB array at V = 129,280
    h = synth.hidden(41, big, sh.H, sh.torch_dtype, DEV)
    ws = torch.empty(m.lmhead_workspace_bytes(big, sh.V, sh.torch_dtype), dtype=torch.uint8, device=DEV)
    for T in (big, 5):                               # the second call smaller than the first
        ids_a, mx_a, ids_b, mx_b = _pair(m, h[:T].contiguous(), w, ws)
        assert torch.equal(ids_a, ids_b), f"argmax differs at T = {T}"
        assert torch.equal(mx_a, mx_b), f"max logit differs at T = {T}"
        assert int(ids_b.min()) >= 0 and int(ids_b.max()) < sh.V
