"""ctypes loader of libmoestep.so (the HIP kernels behind the C ABI).

There is no fallback: if the library is missing, loading raises.
"""

from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
# MOESTEP_LIB names another build of the same library (the host-sanitizer
# build of the host checks); by default the in-tree one.
LIB_PATH = os.environ.get("MOESTEP_LIB") or os.path.join(HERE, "libmoestep.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "moestep.h")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_ALIGN, ERR_WORKSPACE, ERR_HIP = range(7)
BF16, F32 = 0, 1
ROUTE_NORM, ROUTE_RENORM, ROUTE_WPACKED = 1, 2, 4
PACK_GATE_UP, PACK_ROWS, PACK_ROUTER = 0, 1, 2
NOALLOC_SCRATCH_BYTES = 4 << 20   # MOE_NOALLOC_SCRATCH_BYTES
# MOE_DATA_ERR_* bits (moe_data_errors)
ERR_EXPERT_ID, ERR_ROW_INDEX, ERR_OFFSETS, ERR_INV, ERR_LENGTH, ERR_SEQUENCE = 1, 2, 4, 8, 16, 32

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_Z = ctypes.c_size_t

# name -> (restype, argtypes); must match include/moestep.h
SIGNATURES = {
    "moe_abi_version": (_I, []),
    "moe_status_str": (ctypes.c_char_p, [_I]),
    "moe_packed_weights_bytes": (_Z, [_I, _I, _I, _I]),
    "moe_pack_weights": (_I, [_P, _P, _I, _I, _I, _I, _I, _P]),
    "moe_permute_workspace_bytes": (_Z, [_I, _I, _I]),
    "moe_grouped_swiglu_workspace_bytes": (_Z, [_I, _I, _I]),
    "lmhead_argmax_workspace_bytes": (_Z, [_I, _I, _I]),
    "moe_route": (_I, [_P, _P, _F, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P]),
    "moe_permute": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _P, _Z, _P]),
    "moe_grouped_swiglu": (_I, [_P, _P, _P, _I, _I, _P, _P, _I, _I, _I, _I, _I, _P, _P, _Z, _P]),
    "moe_expert_gate_up": (_I, [_P, _P, _P, _I, _I, _P, _I, _I, _I, _I, _I, _P, _P]),
    "moe_expert_gate_up_routed": (_I, [_P, _P, _I, _I, _I, _I, _P, _I, _I, _I, _P, _P, _P, _P]),
    "moe_expert_down": (_I, [_P, _P, _I, _I, _P, _I, _I, _I, _I, _P, _P]),
    "moe_expert_down_residual": (_I, [_P, _P, _I, _I, _P, _I, _I, _I, _I, _P, _P, _P]),
    "moe_combine": (_I, [_P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _P, _P, _P]),
    "moe_combine_rmsnorm": (_I, [_P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _P, _F, _I, _P, _P, _P]),
    "moe_rmsnorm": (_I, [_P, _P, _I, _I, _I, _P, _F, _I, _P, _I, _P]),
    "moe_combine_route": (_I, [_P, _P, _P, _P, _I, _I, _I, _P, _I, _I, _P, _F, _P, _P, _I, _I, _I, _I,
                               _P, _P, _P, _P, _P]),
    "lmhead_argmax": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P, _Z, _P]),
    "lmhead_argmax_noalloc": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P]),
    "spec_verify": (_I, [_P, _P, _I, _I, _P, _P, _P, _P]),
    "spec_plant_drafts": (_I, [_P, _P, _P, _I, _I, _I, _P, _P]),
    "spec_advance": (_I, [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P]),
    "spec_gather_rows": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P]),
    "moe_attn_rope_cache": (_I, [_P, _P, _I, _I, _I, _I, _F, _I, _I, _P, _P, _P]),
    "moe_attention_workspace_bytes": (_Z, [_I, _I, _I, _I, _I]),
    "moe_attention": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _Z, _P]),
    "spec_commit": (_I, [_P, _I, _P, _P]),
    "moe_data_errors": (_I, [_P, _I, _P]),
}

_lib = None


class MoeError(RuntimeError):
    """A C-ABI call returned a non-zero moe_status."""

    def __init__(self, name: str, status: int, msg: str):
        super().__init__(f"{name} failed with status {status}: {msg}")
        self.status = status


def header_functions() -> list[str]:
    """Names of the functions include/moestep.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:int|size_t|const char\s*\*)\s+(\w+)\s*\(", text, flags=re.M)


def load():
    """Load libmoestep.so (once) and declare every entry point."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m moe_decoder_step_amd.build` "
                               "(the HIP library is required, there is no fallback)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(name: str, status: int) -> None:
    if status != OK:
        raise MoeError(name, status, load().moe_status_str(status).decode())
