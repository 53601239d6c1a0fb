"""MI355X-native speculative verify step of an MoE decoder (jina-ocr-v1's
DeepSeek-3B-MoE: hidden 1280, 64 routed + 2 shared experts, top-6,
vocabulary 129,280).

The hot path is hand-written HIP for gfx950 in libmoestep.so behind a C ABI
(include/moestep.h); this package is its thin Python binding.  There is no
CPU fallback: the calls raise if the library is not built.
"""

from ._lib import (BF16, F32, MoeError, ROUTE_NORM, ROUTE_RENORM, LIB_PATH, header_functions,  # noqa: F401
                   load)
from .ops import *  # noqa: F401,F403
from .step import VerifyStack  # noqa: F401
from .loop import DecodeLoop  # noqa: F401
from .draft import DraftHead  # noqa: F401
from .attention import AttentionBlock  # noqa: F401
from .pipeline import PagePipeline  # noqa: F401
