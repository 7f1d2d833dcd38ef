"""MI355X (gfx950) gated delta rule forward with FP8-E4M3 state QDQ.

The compute lives in libgdn.so (HIP kernels behind the C ABI of
include/gdn.h); this package only marshals torch device tensors into it.
"""
from ._lib import (GDN_BF16, GDN_F32, GDN_QDQ_CHUNK, GDN_QDQ_WRITE, GdnError,  # noqa: F401
                   LIB_PATH)
from .api import chunk_fwd, decode_step, state_qdq  # noqa: F401
