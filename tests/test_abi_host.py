"""The C-ABI library on the host: it loads, exports every function the header
declares, and its argument checks return the documented status codes before
anything reaches the GPU (no compute calls here)."""

import ctypes
import re

import pytest

import moe_decoder_step_amd as m
from moe_decoder_step_amd import _lib as L

P = ctypes.c_void_p
A = P(0x100000)        # aligned, never dereferenced: checks fail before any use
MIS = P(0x100004)      # misaligned


@pytest.fixture(scope="module")
def lib():
    return L.load()


def test_exports_every_declared_function(lib):
    names = L.header_functions()
    assert len(names) == 29
    assert set(names) == set(L.SIGNATURES)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.moe_abi_version() == 1
    for s in range(7):
        assert lib.moe_status_str(s)
    assert lib.moe_status_str(99) == b"unknown status"


def test_data_errors_checks(lib):
    f = lib.moe_data_errors
    assert f(None, 1, None) == L.ERR_NULL
    assert f(P(0x100002), 1, None) == L.ERR_ALIGN     # the flag word is 4-byte aligned
    # the binding's bits are the header's
    with open(L.HEADER) as fh:
        bits = dict((n, int(v)) for n, v in re.findall(r"#define MOE_DATA_ERR_(\w+) (\d+)u", fh.read()))
    assert bits == {"EXPERT_ID": L.ERR_EXPERT_ID, "ROW_INDEX": L.ERR_ROW_INDEX, "OFFSETS": L.ERR_OFFSETS,
                    "INV": L.ERR_INV, "LENGTH": L.ERR_LENGTH, "SEQUENCE": L.ERR_SEQUENCE}


def test_workspace_queries(lib):
    assert lib.moe_permute_workspace_bytes(128, 6, 64) == 0            # one chunk: no scratch
    n_chunks = (36992 * 6 + 4095) // 4096
    assert lib.moe_permute_workspace_bytes(36992, 6, 64) >= 2 * n_chunks * 64 * 4
    assert lib.moe_grouped_swiglu_workspace_bytes(1024, 896, m.BF16) >= 1024 * 896 * 2
    assert lib.moe_grouped_swiglu_workspace_bytes(1024, 896, m.F32) >= 1024 * 896 * 4
    assert lib.lmhead_argmax_workspace_bytes(128, 129280, m.BF16) >= 128 * 1010 * 8
    assert lib.lmhead_argmax_workspace_bytes(0, 129280, m.BF16) == 0


def test_pack_checks(lib):
    f = lib.moe_pack_weights
    assert lib.moe_packed_weights_bytes(66, 896, 1280, 0) == 66 * 2 * 896 * 1280 * 2
    assert lib.moe_packed_weights_bytes(1, 77, 64, 1) == 3 * 2 * 2 * 1024   # rows padded to pairs of 32
    assert f(A, A, 66, 896, 1280, 0, m.F32, None) == L.ERR_UNSUPPORTED       # fp32 weights stay row-major
    assert f(A, A, 66, 896, 1280, 2, m.BF16, None) == L.ERR_UNSUPPORTED      # router layout is fp32
    assert f(A, A, 66, 896, 1280, 3, m.BF16, None) == L.ERR_UNSUPPORTED
    assert lib.moe_packed_weights_bytes(12, 64, 1280, L.PACK_ROUTER) == 12 * 1280 * 64 * 4
    assert lib.moe_packed_weights_bytes(1, 8, 128, L.PACK_ROUTER) == 128 * 64 * 4   # padded to 64 experts
    assert f(A, A, 1, 65, 1280, L.PACK_ROUTER, m.F32, None) == L.ERR_UNSUPPORTED
    assert f(A, A, 1, 64, 1282, L.PACK_ROUTER, m.F32, None) == L.ERR_SHAPE
    assert f(MIS, A, 1, 64, 1280, L.PACK_ROUTER, m.F32, None) == L.ERR_ALIGN
    assert f(A, A, 1, 64, 1280, L.PACK_ROUTER, m.BF16, None) == L.ERR_UNSUPPORTED
    assert f(A, A, 66, 896, 1290, 0, m.BF16, None) == L.ERR_SHAPE
    assert f(A, A, 66, 900, 1280, 0, m.BF16, None) == L.ERR_SHAPE
    assert f(None, A, 66, 896, 1280, 0, m.BF16, None) == L.ERR_NULL
    assert f(MIS, A, 66, 896, 1280, 0, m.BF16, None) == L.ERR_ALIGN
    assert f(None, None, 0, 896, 1280, 0, m.BF16, None) == L.OK


def test_route_checks(lib):
    f = lib.moe_route
    base = dict(h=A, gain=None, eps=1e-6, w=A, b=None, T=4, H=128, E=8, k=2, flags=3, dt=m.BF16,
                xn=A, ids=A, tw=A, lg=None, s=None)

    def call(**kw):
        a = {**base, **kw}
        return f(a["h"], a["gain"], a["eps"], a["w"], a["b"], a["T"], a["H"], a["E"], a["k"], a["flags"],
                 a["dt"], a["xn"], a["ids"], a["tw"], a["lg"], a["s"])
    assert call(h=None) == L.ERR_NULL
    assert call(ids=None) == L.ERR_NULL
    assert call(T=-1) == L.ERR_SHAPE
    assert call(k=9) == L.ERR_SHAPE
    assert call(k=0) == L.ERR_SHAPE
    assert call(E=65, k=6) == L.ERR_UNSUPPORTED
    assert call(H=100) == L.ERR_UNSUPPORTED
    assert call(H=4096) == L.ERR_UNSUPPORTED
    assert call(dt=7) == L.ERR_UNSUPPORTED
    assert call(h=MIS) == L.ERR_ALIGN
    assert call(T=0, h=None) == L.OK        # empty batch: no-op


def test_permute_checks(lib):
    f = lib.moe_permute
    assert f(A, 4, 2, 8, 2, None, A, A, None, 0, None) == L.ERR_NULL
    assert f(None, 4, 2, 8, 2, A, A, A, None, 0, None) == L.ERR_NULL
    assert f(A, 4, 9, 8, 2, A, A, A, None, 0, None) == L.ERR_SHAPE
    assert f(A, 4, 2, 8, -1, A, A, A, None, 0, None) == L.ERR_SHAPE
    assert f(A, 4, 2, 80, 2, A, A, A, None, 0, None) == L.ERR_UNSUPPORTED
    assert f(A, 4, 2, 8, 9, A, A, A, None, 0, None) == L.ERR_UNSUPPORTED
    # multi-chunk sizes need a workspace
    assert f(A, 36992, 6, 64, 2, A, A, A, None, 0, None) == L.ERR_WORKSPACE
    assert f(A, 36992, 6, 64, 2, A, A, A, A, 16, None) == L.ERR_WORKSPACE


def test_swiglu_checks(lib):
    f = lib.moe_grouped_swiglu
    need = lib.moe_grouped_swiglu_workspace_bytes(40, 896, m.BF16)

    def call(x=A, off=A, G=66, n=40, wgu=A, wd=A, T=4, H=1280, I=896, mr=4, dt=m.BF16, y=A, ws=A, wsb=need):
        return f(x, None, off, G, n, wgu, wd, T, H, I, mr, dt, y, ws, wsb, None)
    assert call(off=None) == L.ERR_NULL
    assert call(y=None) == L.ERR_NULL
    assert call(G=0) == L.ERR_SHAPE
    assert call(n=-1) == L.ERR_SHAPE
    assert call(H=1288) == L.ERR_UNSUPPORTED          # bf16 needs H % 32 == 0
    assert call(I=900) == L.ERR_UNSUPPORTED
    assert call(I=4128) == L.ERR_UNSUPPORTED          # LDS holds 16 rows of the reduction length
    assert call(G=129) == L.ERR_UNSUPPORTED
    assert call(wgu=MIS) == L.ERR_ALIGN
    assert call(ws=None) == L.ERR_WORKSPACE
    assert call(wsb=need - 1) == L.ERR_WORKSPACE
    assert call(n=0, x=None) == L.OK


def test_expert_halves_checks(lib):
    gu, dn = lib.moe_expert_gate_up, lib.moe_expert_down
    assert gu(A, None, A, 66, 40, A, 4, 1280, 896, 4, m.BF16, None, None) == L.ERR_NULL
    assert gu(A, None, A, 66, 40, MIS, 4, 1280, 896, 4, m.BF16, A, None) == L.ERR_ALIGN
    assert gu(A, None, A, 66, 40, A, 4, 1288, 896, 4, m.BF16, A, None) == L.ERR_UNSUPPORTED
    assert gu(None, None, None, 66, 0, None, 4, 1280, 896, 4, m.BF16, None, None) == L.OK
    assert dn(A, A, 66, 40, A, 1280, 896, 4, m.BF16, None, None) == L.ERR_NULL
    assert dn(A, A, 0, 40, A, 1280, 896, 4, m.BF16, A, None) == L.ERR_SHAPE
    assert dn(MIS, A, 66, 40, A, 1280, 896, 4, m.BF16, A, None) == L.ERR_ALIGN
    assert dn(None, None, 66, 0, None, 1280, 896, 4, m.BF16, None, None) == L.OK
    dr = lib.moe_expert_down_residual
    assert dr(A, A, 1, 40, A, 1280, 1280, 40, m.BF16, None, A, None) == L.ERR_NULL
    assert dr(A, A, 1, 40, A, 1280, 1280, 40, m.BF16, MIS, A, None) == L.ERR_ALIGN
    assert dr(A, A, 1, 40, A, 1280, 1280, 40, m.BF16, A, None, None) == L.ERR_NULL
    assert dr(A, A, 0, 40, A, 1280, 1280, 40, m.BF16, A, A, None) == L.ERR_SHAPE
    assert dr(None, None, 1, 0, None, 1280, 1280, 40, m.BF16, None, None, None) == L.OK


def test_rmsnorm_checks(lib):
    f = lib.moe_rmsnorm
    # x, rows, x_rows, T, H, gain, eps, dtype, out, out_stride, stream
    assert f(A, None, 10, 10, 1280, None, 1e-6, m.BF16, None, 1280, None) == L.ERR_NULL
    assert f(A, None, 10, 11, 1280, None, 1e-6, m.BF16, A, 1280, None) == L.ERR_SHAPE     # more rows than x has
    assert f(A, None, 10, 10, 1280, None, 1e-6, m.BF16, A, 1000, None) == L.ERR_SHAPE     # stride < H
    assert f(A, None, 10, 10, 1284, None, 1e-6, m.BF16, A, 1284, None) == L.ERR_UNSUPPORTED
    assert f(A, None, 10, 10, 1280, None, 1e-6, m.BF16, A, 1284, None) == L.ERR_ALIGN     # 2568-byte stride
    assert f(None, None, 10, 0, 1280, None, 1e-6, m.BF16, None, 1280, None) == L.OK


def test_gate_up_routed_checks(lib):
    f = lib.moe_expert_gate_up_routed
    # x, ids, T, k, E, S, wgu, H, I, dtype, act, offsets, inv, stream
    assert f(A, A, 128, 6, 64, 2, A, 1280, 896, m.BF16, A, None, A, None) == L.ERR_NULL
    assert f(A, A, 128, 6, 64, 2, A, 1280, 896, m.F32, A, A, A, None) == L.ERR_UNSUPPORTED   # bf16 only
    assert f(A, A, 683, 6, 64, 2, A, 1280, 896, m.BF16, A, A, A, None) == L.ERR_UNSUPPORTED  # > 4096 pairs
    assert f(A, A, 128, 7, 6, 2, A, 1280, 896, m.BF16, A, A, A, None) == L.ERR_SHAPE
    assert f(A, A, 128, 6, 64, 2, MIS, 1280, 896, m.BF16, A, A, A, None) == L.ERR_ALIGN
    assert f(A, A, 128, 6, 64, 2, A, 1280, 896, m.BF16, A, A, None, None) == L.ERR_NULL


def test_combine_route_checks(lib):
    f = lib.moe_combine_route
    # y, inv, w_prev, ys, S, n_rows, k_prev, h, T, H, gain, eps, wr, bias, E, k, flags, dtype, xn, ids, w, lg, s
    base = [A, A, A, A, 2, 1024, 6, A, 128, 1280, None, 1e-6, A, None, 64, 6, 3, m.BF16, A, A, A, None, None]

    def call(**kw):
        a = list(base)
        names = ["y", "inv", "wp", "ys", "S", "n_rows", "kp", "h", "T", "H", "gain", "eps", "wr", "b", "E", "k",
                 "flags", "dt", "xn", "ids", "w", "lg", "s"]
        for key, v in kw.items():
            a[names.index(key)] = v
        return f(*a)
    assert call(inv=None) == L.ERR_NULL
    assert call(ids=None) == L.ERR_NULL
    assert call(H=1284) == L.ERR_UNSUPPORTED
    assert call(E=65) == L.ERR_UNSUPPORTED
    assert call(k=7, E=6) == L.ERR_SHAPE
    assert call(h=MIS) == L.ERR_ALIGN
    assert call(T=0) == L.OK


def test_advance_and_gather_checks(lib):
    adv, gat = lib.spec_advance, lib.spec_gather_rows
    # n_commit, committed, seq_ids, B, K, S, target, total, steps, tokens, seq_out, n_active, stream
    assert adv(A, A, A, 4, 3, 32, 1085, A, A, A, A, None, None) == L.ERR_NULL
    assert adv(A, A, A, 33, 3, 32, 1085, A, A, A, A, A, None) == L.ERR_SHAPE      # more slots than sequences
    assert adv(A, A, A, 4, 3, 32, 0, A, A, A, A, A, None) == L.ERR_SHAPE
    assert adv(A, A, A, 4, 16, 32, 10, A, A, A, A, A, None) == L.ERR_UNSUPPORTED   # K <= 15
    assert adv(A, A, A, 1025, 3, 2000, 10, A, A, A, A, A, None) == L.ERR_UNSUPPORTED
    assert adv(A, None, A, 4, 3, 32, 10, A, A, A, A, A, None) == L.ERR_NULL
    # pool, seq_ids, steps, B, R, J, S, row_bytes, out, stream
    assert gat(A, A, A, 4, 4, 10, 32, 2560, None, None) == L.ERR_NULL
    assert gat(A, A, A, 4, 0, 10, 32, 2560, A, None) == L.ERR_SHAPE
    assert gat(None, None, None, 0, 4, 10, 32, 2560, None, None) == L.OK
    assert gat(A, A, A, 4, 1, 10, 32, 0, A, None) == L.OK           # K = 0 drafts: nothing to gather
    assert gat(A, A, A, 4, 1, 10, 32, -1, A, None) == L.ERR_SHAPE


def test_attention_checks(lib):
    rope, att, com = lib.moe_attn_rope_cache, lib.moe_attention, lib.spec_commit
    ws = lib.moe_attention_workspace_bytes
    # one split per 256 keys up to 64 splits: 32 x 4 queries x 10 heads at 2,048 keys -> 8 splits
    assert ws(32, 4, 10, 128, 2048) == 32 * 10 * 8 * 4 * 130 * 4
    assert ws(1, 4, 10, 128, 32768) == 10 * 64 * 4 * 130 * 4          # 512 keys per split
    assert ws(0, 4, 10, 128, 2048) == 0
    # qkv, lengths, B, P, n_heads, head_dim, base, max_len, dtype, q, kv, stream
    assert rope(A, A, 2, 4, 10, 128, 1e4, 64, m.BF16, A, None, None) == L.ERR_NULL
    assert rope(A, A, 2, 4, 10, 64, 1e4, 64, m.BF16, A, A, None) == L.ERR_UNSUPPORTED    # head size 128
    assert rope(A, A, 2, 17, 10, 128, 1e4, 64, m.BF16, A, A, None) == L.ERR_UNSUPPORTED  # P <= 16
    assert rope(A, A, 2, 4, 10, 128, 1e4, 64, m.F32, A, A, None) == L.ERR_UNSUPPORTED
    assert rope(A, A, 2, 4, 10, 128, 1e4, 3, m.BF16, A, A, None) == L.ERR_SHAPE           # max_len < P
    assert rope(A, A, 2, 4, 10, 128, 1.0, 64, m.BF16, A, A, None) == L.ERR_SHAPE
    assert rope(None, None, 0, 4, 10, 128, 1e4, 64, m.BF16, None, None, None) == L.OK
    # q, kv, lengths, B, P, n_heads, head_dim, max_len, max_keys, dtype, o, ws, ws_bytes, stream
    need = ws(2, 4, 10, 128, 64)
    assert att(A, A, A, 2, 4, 10, 128, 64, 64, m.BF16, A, A, need - 1, None) == L.ERR_WORKSPACE
    assert att(A, A, A, 2, 4, 10, 128, 64, 64, m.BF16, A, None, need, None) == L.ERR_WORKSPACE
    assert att(A, MIS, A, 2, 4, 10, 128, 64, 64, m.BF16, A, A, need, None) == L.ERR_ALIGN
    assert att(A, A, A, 2, 4, 10, 128, 64, 65, m.BF16, A, A, need, None) == L.ERR_SHAPE  # max_keys > max_len
    assert att(A, A, A, 2, 4, 10, 128, 64, 3, m.BF16, A, A, need, None) == L.ERR_SHAPE   # max_keys < P
    assert att(A, A, None, 2, 4, 10, 128, 64, 64, m.BF16, A, A, need, None) == L.ERR_NULL
    assert att(None, None, None, 0, 4, 10, 128, 64, 64, m.BF16, None, None, 0, None) == L.OK
    assert com(A, -1, A, None) == L.ERR_SHAPE
    assert com(None, 4, A, None) == L.ERR_NULL
    assert com(None, 0, None, None) == L.OK


def test_combine_lmhead_verify_plant_checks(lib):
    assert lib.moe_combine(A, A, A, None, 2, A, 4, 1280, 6, 40, m.BF16, A, None, None) == L.ERR_NULL
    assert lib.moe_combine(A, None, A, A, 2, A, 4, 1280, 6, 40, m.BF16, A, None, None) == L.ERR_NULL
    assert lib.moe_combine(A, A, A, A, 2, A, 4, 1284, 6, 40, m.BF16, A, None, None) == L.ERR_UNSUPPORTED
    assert lib.moe_combine(A, A, A, A, 2, A, 4, 1280, 6, 40, m.BF16, MIS, None, None) == L.ERR_ALIGN
    assert lib.moe_combine(A, A, A, A, 2, A, 4, 1280, 65, 40, m.BF16, A, None, None) == L.ERR_UNSUPPORTED
    assert lib.moe_combine(A, A, A, A, 2, A, 0, 1280, 6, 40, m.BF16, A, None, None) == L.OK
    cn = lib.moe_combine_rmsnorm
    B = P(0x200000)
    assert cn(A, A, A, A, 2, A, 4, 1280, 6, 40, None, 1e-6, m.BF16, A, None, None) == L.ERR_NULL
    assert cn(A, A, A, A, 2, A, 4, 1280, 6, 40, None, 1e-6, m.BF16, A, A, None) == L.ERR_SHAPE     # xn == out
    assert cn(A, A, A, A, 2, B, 4, 1280, 6, 40, None, 1e-6, m.BF16, A, B, None) == L.ERR_SHAPE     # xn == residual
    assert cn(A, A, A, A, 2, A, 4, 1280, 6, 40, None, 1e-6, m.BF16, A, MIS, None) == L.ERR_ALIGN
    assert cn(A, A, A, A, 2, A, 4, 2056, 6, 40, None, 1e-6, m.BF16, A, B, None) == L.ERR_UNSUPPORTED
    assert cn(A, A, A, None, 2, A, 4, 1280, 6, 40, None, 1e-6, m.BF16, A, B, None) == L.ERR_NULL
    assert cn(None, None, None, None, 0, None, 0, 1280, 6, 40, None, 1e-6, m.BF16, None, None, None) == L.OK
    need = lib.lmhead_argmax_workspace_bytes(4, 129280, m.BF16)
    assert lib.lmhead_argmax(A, A, 4, 1280, 129280, m.BF16, A, None, A, need - 8, None) == L.ERR_WORKSPACE
    assert lib.lmhead_argmax(A, None, 4, 1280, 129280, m.BF16, A, None, A, need, None) == L.ERR_NULL
    assert lib.lmhead_argmax(A, A, 4, 1280, 0, m.BF16, A, None, A, need, None) == L.ERR_SHAPE
    assert lib.spec_verify(A, A, 4, 16, A, A, A, None) == L.ERR_UNSUPPORTED
    assert lib.spec_verify(A, A, 4, -1, A, A, A, None) == L.ERR_SHAPE
    assert lib.spec_verify(None, A, 4, 3, A, A, A, None) == L.ERR_NULL
    assert lib.spec_verify(None, A, 0, 3, None, None, None, None) == L.OK
    assert lib.spec_plant_drafts(A, A, A, 4, 3, 1, A, None) == L.ERR_SHAPE
    assert lib.spec_plant_drafts(A, None, A, 4, 3, 10, A, None) == L.ERR_NULL


def test_binding_raises_without_gpu_tensors():
    import torch
    h = torch.zeros(4, 128)
    with pytest.raises(ValueError):
        m.moe_route(h, torch.zeros(8, 128), None, 2, torch.zeros_like(h), torch.zeros(4, 2, dtype=torch.int32),
                    torch.zeros(4, 2))


def test_lmhead_noalloc_checks(lib):
    """The allocation-free LM head: argument checks as lmhead_argmax, and a
    batch whose workspace would exceed the static array is rejected."""
    f = lib.lmhead_argmax_noalloc
    V = 129280
    assert f(None, A, 4, 1280, V, m.BF16, A, None, None) == L.ERR_NULL
    assert f(A, A, 4, 1280, V, m.BF16, None, None, None) == L.ERR_NULL
    assert f(MIS, A, 4, 1280, V, m.BF16, A, None, None) == L.ERR_ALIGN
    assert f(A, A, 4, 1290, V, m.BF16, A, None, None) == L.ERR_UNSUPPORTED
    assert f(A, A, -1, 1280, V, m.BF16, A, None, None) == L.ERR_SHAPE
    assert f(A, A, 0, 1280, V, m.BF16, A, None, None) == L.OK
    assert lib.lmhead_argmax_workspace_bytes(519, V, m.BF16) <= L.NOALLOC_SCRATCH_BYTES
    assert lib.lmhead_argmax_workspace_bytes(520, V, m.BF16) > L.NOALLOC_SCRATCH_BYTES
    assert f(A, A, 520, 1280, V, m.BF16, A, None, None) == L.ERR_WORKSPACE
