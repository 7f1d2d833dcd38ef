"""ctypes view of the C ABI in include/gdn.h (libgdn.so built from csrc/).

Loading fails loudly when the library has not been built: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

# GDN_LIB: another build of the same sources (the host-sanitized one)
LIB_PATH = os.environ.get("GDN_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn.so")

GDN_OK = 0
GDN_ERR_INVALID_ARG = 1
GDN_ERR_UNSUPPORTED = 2
GDN_ERR_DEVICE = 3

GDN_F32 = 0
GDN_BF16 = 1

GDN_QDQ_CHUNK = 1
GDN_QDQ_WRITE = 2
GDN_QDQ_W = 4        # W QDQ in every chunk of the chunked prefix
GDN_QDQ_INT8 = 8     # decode step: INT8 block-32 per-write QDQ instead of FP8 per tile

GDN_SCHEDULE_AUTO = 0
GDN_SCHEDULE_SPLIT = 1
GDN_SCHEDULE_FUSED = 2
GDN_SCHEDULE_FUSED_NO_PRODUCERS = 3   # test hook: every wait for a ready flag runs out

NOALLOC_SCRATCH_BYTES = 64 << 20   # GDN_NOALLOC_SCRATCH_BYTES

EXPORTS = ("gdn_chunk_fwd", "gdn_chunk_fwd_noalloc", "gdn_chunk_fwd_workspace_bytes", "gdn_workspace_status",
           "gdn_state_qdq",
           "gdn_state_qdq_int8", "gdn_decode_step", "gdn_chunk_bwd_dh", "gdn_chunk_bwd_workspace_bytes",
           "gdn_status_string", "gdn_last_error")


class GdnShape(ctypes.Structure):
    _fields_ = [
        ("n_seqs", ctypes.c_int32),
        ("n_heads", ctypes.c_int32),
        ("dk", ctypes.c_int32),
        ("dv", ctypes.c_int32),
        ("total_tokens", ctypes.c_int64),
        ("io_dtype", ctypes.c_int32),
        ("o_dtype", ctypes.c_int32),
        ("gate_per_channel", ctypes.c_int32),
        ("qdq_flags", ctypes.c_uint32),
        ("gate_grid_log2", ctypes.c_int32),
    ]


class GdnDebug(ctypes.Structure):
    _fields_ = [
        ("bound_offsets", ctypes.c_void_p),
        ("bound_pre", ctypes.c_void_p),
        ("bound_post", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("kernel_start", ctypes.c_void_p),
        ("kernel_end", ctypes.c_void_p),
        ("schedule", ctypes.c_int32),
        ("w_pre", ctypes.c_void_p),
        ("w_post", ctypes.c_void_p),
        ("suffix_offsets", ctypes.c_void_p),
        ("suffix_pre", ctypes.c_void_p),
        ("suffix_post", ctypes.c_void_p),
        ("status", ctypes.c_void_p),
    ]


class GdnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{status_string(status)}: {detail}")


_lib = None
_vp = ctypes.c_void_p


def lib():
    """The loaded library (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"HIP library {LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; "
            "g.build()'` (or python fp8_state_qat_amd/build.py)")
    L = ctypes.CDLL(LIB_PATH)
    L.gdn_chunk_fwd.argtypes = [ctypes.POINTER(GdnShape), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                _vp, _vp, _vp, _vp, ctypes.c_size_t, ctypes.POINTER(GdnDebug), _vp]
    L.gdn_chunk_fwd.restype = ctypes.c_int
    L.gdn_chunk_fwd_noalloc.argtypes = [ctypes.POINTER(GdnShape), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                        _vp, _vp, _vp, ctypes.POINTER(GdnDebug), _vp]
    L.gdn_chunk_fwd_noalloc.restype = ctypes.c_int
    L.gdn_chunk_fwd_workspace_bytes.argtypes = [ctypes.POINTER(GdnShape)]
    L.gdn_chunk_fwd_workspace_bytes.restype = ctypes.c_size_t
    L.gdn_state_qdq.argtypes = [_vp, _vp, _vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _vp]
    L.gdn_state_qdq.restype = ctypes.c_int
    L.gdn_chunk_bwd_dh.argtypes = [ctypes.POINTER(GdnShape)] + [_vp] * 11 + [_vp, ctypes.c_size_t, _vp]
    L.gdn_chunk_bwd_dh.restype = ctypes.c_int
    L.gdn_chunk_bwd_workspace_bytes.argtypes = [ctypes.POINTER(GdnShape)]
    L.gdn_chunk_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.gdn_state_qdq_int8.argtypes = [_vp, _vp, _vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _vp]
    L.gdn_state_qdq_int8.restype = ctypes.c_int
    L.gdn_decode_step.argtypes = [ctypes.POINTER(GdnShape), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                  _vp, _vp, _vp]
    L.gdn_workspace_status.argtypes = [_vp, _vp]
    L.gdn_workspace_status.restype = ctypes.c_int
    L.gdn_decode_step.restype = ctypes.c_int
    L.gdn_status_string.argtypes = [ctypes.c_int]
    L.gdn_status_string.restype = ctypes.c_char_p
    L.gdn_last_error.argtypes = []
    L.gdn_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().gdn_status_string(int(status)).decode()


def last_error() -> str:
    return lib().gdn_last_error().decode()


def check(status: int) -> None:
    if status != GDN_OK:
        raise GdnError(status, last_error())
