"""One verify pass through the C ABI from a plain C program (no Python, no
torch in the process that runs it): tests/c_client/verify_pass reads seeded
synthetic inputs, runs moe_route -> moe_permute -> moe_grouped_swiglu ->
moe_combine -> lmhead_argmax -> spec_verify (packing the bf16 weights with
moe_pack_weights first), and writes its outputs; they are checked here
against the fp64 oracle: ids, argmax tokens and acceptance bit-exact outside
oracle near-ties, the layer output within the storage dtype's bound."""

import dataclasses
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle as O
import synth
from moe_decoder_step_amd import build as B
from tests._util import BF16_TOL, F32_TOL, assert_close, compare_ids

pytestmark = pytest.mark.gpu


def _raw(t: torch.Tensor) -> bytes:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.numpy().tobytes()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_c_client_verify_pass(tmp_path, dtype):
    assert os.path.exists(B.C_CLIENT), "the C client is built with the library (python -m moe_decoder_step_amd.build)"
    sh = dataclasses.replace(synth.SHAPES["tiny"], dtype=dtype)
    T, H, E, S, k, I, V, Bs, K = sh.T, sh.H, sh.E, sh.S, sh.k, sh.I, sh.V, sh.B, sh.K
    w = synth.layer_weights(50, 0, sh)
    w_lm = synth.lm_weight(50, sh)
    h = synth.hidden(51, T, H, sh.torch_dtype)
    drafts = synth.uniform_ids(52, (Bs, K), V)
    for name, t in (("h", h), ("w_router", w["w_router"]), ("w_gate_up", w["w_gate_up"]), ("w_down", w["w_down"]),
                    ("w_lm", w_lm), ("drafts", drafts.to(torch.int32))):
        (tmp_path / f"{name}.bin").write_bytes(_raw(t))
    args = [B.C_CLIENT, "run", str(tmp_path), dtype] + [str(v) for v in (T, H, E, S, k, I, V, Bs, K)]
    print("C client:", " ".join(args), flush=True)
    r = subprocess.run(args, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr

    def out(name, dt, shape):
        a = np.frombuffer((tmp_path / f"{name}.bin").read_bytes(), dtype=dt).reshape(shape)
        return a.view(np.uint16) if dt == np.int16 else a
    store = np.int16 if dtype == "bf16" else np.float32
    ids = out("ids", np.int32, (T, k))
    tw = out("topk_w", np.float32, (T, k))
    h_out = out("h_out", store, (T, H))
    argmax = out("argmax", np.int32, (T,))
    hostw = {n: (v.view(torch.int16).numpy().view(np.uint16) if v.dtype == torch.bfloat16 else v.numpy())
             for n, v in w.items()}
    h_host = h.view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else h.numpy()
    ref = O.moe_layer(h_host, hostw, k, sh.eps, dtype)
    _, flagged = compare_ids(ids, ref["route"]["ids"], ref["route"]["gap"], "ids")
    ok = ~flagged
    assert_close(tw[ok], ref["route"]["w"][ok], F32_TOL, "routing weights")
    got_h = O.f64(h_out)
    assert_close(got_h[ok], ref["h_out"][ok], BF16_TOL if dtype == "bf16" else F32_TOL, "layer output")
    # LM head on the client's own output (teacher forcing), then acceptance
    w_lm_host = w_lm.view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else w_lm.numpy()
    rid, _, gap = O.lm_argmax(h_out, w_lm_host)
    compare_ids(argmax, rid, gap, "argmax")
    racc, rcom, rnc = O.spec_verify(drafts.numpy(), argmax.reshape(Bs, K + 1))
    np.testing.assert_array_equal(out("accepted", np.int32, (Bs,)), racc)
    np.testing.assert_array_equal(out("committed", np.int32, (Bs, K + 1)), rcom)
    np.testing.assert_array_equal(out("n_commit", np.int32, (Bs,)), rnc)
    assert int(out("errors", np.uint32, (1,))[0]) == 0
