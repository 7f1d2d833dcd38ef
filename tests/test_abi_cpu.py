"""C ABI checks that need no GPU: the library loads, exports every entry point
that include/gdn.h declares, and rejects bad arguments on the host before
touching a device."""
import ctypes
import os
import re

import pytest
import torch

from fp8_state_qat_amd import _lib
from fp8_state_qat_amd._lib import GdnDebug, GdnShape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HAS_GPU = torch.cuda.is_available()


def _declared():
    with open(os.path.join(ROOT, "include", "gdn.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(gdn_\w+)\s*\(", text, re.M)))


def test_header_declares_expected_entry_points():
    assert _declared() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    for name in _declared():
        assert hasattr(L, name), name
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value


def test_status_strings():
    assert _lib.status_string(0) == "GDN_OK"
    assert _lib.status_string(1) == "GDN_ERR_INVALID_ARG"
    assert _lib.status_string(2) == "GDN_ERR_UNSUPPORTED"
    assert _lib.status_string(3) == "GDN_ERR_DEVICE"


FAKE = 0x10000  # 64 KiB-aligned stand-in address; never dereferenced on the host


def _shape(**kw):
    d = dict(n_seqs=2, n_heads=4, dk=128, dv=128, total_tokens=100, io_dtype=1, o_dtype=1,
             gate_per_channel=0, qdq_flags=3)
    d.update(kw)
    return GdnShape(**d)


def _ws(shape):
    return _lib.lib().gdn_chunk_fwd_workspace_bytes(ctypes.byref(shape))


def _chunk(shape, q=FAKE, beta=FAKE, cu=FAKE, fin=FAKE, dbg=None, ws=FAKE, ws_bytes=None):
    p = ctypes.c_void_p
    if ws_bytes is None:
        ws_bytes = _ws(shape) if shape is not None else 0
    return _lib.lib().gdn_chunk_fwd(ctypes.byref(shape) if shape is not None else None,
                                    p(q), p(FAKE), p(FAKE), p(beta), p(FAKE), p(cu), None, None,
                                    None, p(FAKE), p(fin), p(ws), ws_bytes, dbg, None)


@pytest.mark.parametrize("kw,status", [
    (dict(n_seqs=0), 1), (dict(n_heads=0), 1), (dict(dv=96), 1), (dict(dk=96), 2),
    (dict(dk=32), 2), (dict(dv=512), 2), (dict(total_tokens=-1), 1), (dict(io_dtype=7), 1),
    (dict(o_dtype=-1), 1), (dict(gate_per_channel=2), 1), (dict(qdq_flags=16), 1), (dict(qdq_flags=8 | 3), 2),
    (dict(io_dtype=0, dk=128, qdq_flags=3 | _lib.GDN_QDQ_W), 2),
    (dict(io_dtype=0, dk=128, gate_per_channel=1, qdq_flags=3 | _lib.GDN_QDQ_W), 2),
    (dict(gate_grid_log2=-1), 1), (dict(gate_grid_log2=25), 1),
])
def test_chunk_fwd_rejects_bad_shape(kw, status):
    assert _chunk(_shape(**kw)) == status
    assert _lib.last_error()


def test_chunk_fwd_rejects_null_and_misaligned():
    assert _chunk(None) == 1
    assert _chunk(_shape(), q=0) == 1
    assert _chunk(_shape(), cu=0) == 1
    assert _chunk(_shape(), fin=0) == 1
    assert _chunk(_shape(), q=FAKE + 8) == 1
    assert _chunk(_shape(), beta=FAKE + 2) == 1
    dbg = GdnDebug(None, ctypes.c_void_p(FAKE), None, None)   # record without offsets
    assert _chunk(_shape(), dbg=ctypes.byref(dbg)) == 1
    for bad in (-1, 4):                                        # unknown schedules
        dbg = GdnDebug(None, None, None, None, None, None, bad)
        assert _chunk(_shape(), dbg=ctypes.byref(dbg)) == 1
        assert "schedule" in _lib.last_error()


def test_workspace_size_and_checks():
    """Workspace: for the worst-case chunk count ceil(T/64) + N, two records
    per chunk and head (T in an 18 KiB slot: three bf16 planes; P: 12 KiB),
    one ready flag per chunk and head, the chunk offsets and the status word,
    each region padded to 256 bytes; too small, NULL or misaligned is
    rejected."""
    s = _shape(n_seqs=3, n_heads=2, total_tokens=130)
    n = _ws(s)
    assert n == 256 + 256 + 256 + (3 + 3) * 2 * (18432 + 12288)   # status, offsets, flags, records
    big = _shape(n_seqs=70, n_heads=3, total_tokens=64 * 100)   # 72 offsets, 510 flags
    assert _ws(big) == 256 + 512 + 2048 + 170 * 3 * (18432 + 12288)
    assert _ws(_shape(n_seqs=3, n_heads=2, total_tokens=130, gate_per_channel=1)) == n
    assert _ws(_shape(dv=96)) == 0 and _lib.last_error()
    assert _chunk(s, ws_bytes=n - 1) == 1
    assert _chunk(s, ws=0) == 1
    assert _chunk(s, ws=FAKE + 64) == 1


def test_w_qdq_flag():
    """GDN_QDQ_W adds one W record per chunk and head (the codes of 64 rows x
    dk as bf16 and a 1 KiB block for the row scales), for either gate;
    unknown flag bits stay rejected."""
    base = _ws(_shape(n_seqs=3, n_heads=2, total_tokens=130))
    for dk in (64, 128):
        w = _ws(_shape(n_seqs=3, n_heads=2, total_tokens=130, dk=dk, qdq_flags=3 | _lib.GDN_QDQ_W))
        assert w == base + (3 + 3) * 2 * (dk * 128 + 1024)
    assert _ws(_shape(n_seqs=3, n_heads=2, total_tokens=130, gate_per_channel=1, qdq_flags=7)) == \
        _ws(_shape(n_seqs=3, n_heads=2, total_tokens=130, qdq_flags=7))
    assert _chunk(_shape(qdq_flags=16)) == 1
    dbg = GdnDebug(None, None, None, None, None, None, 0, ctypes.c_void_p(FAKE), None)  # W record without offsets
    assert _chunk(_shape(qdq_flags=7), dbg=ctypes.byref(dbg)) == 1


def test_state_qdq_rejects_bad_args():
    L = _lib.lib()
    p = ctypes.c_void_p
    assert L.gdn_state_qdq(p(FAKE), p(FAKE), None, -1, 64, 128, None) == 1
    assert L.gdn_state_qdq(p(FAKE), p(FAKE), None, 4, 96, 128, None) == 1
    assert L.gdn_state_qdq(p(FAKE), p(FAKE), None, 4, 64, 6, None) == 1
    assert L.gdn_state_qdq(p(FAKE), p(FAKE), None, 4, 64, 512, None) == 2
    assert L.gdn_state_qdq(None, p(FAKE), None, 4, 64, 128, None) == 1
    assert L.gdn_state_qdq(p(FAKE + 4), p(FAKE), None, 4, 64, 128, None) == 1


def test_state_qdq_int8_rejects_bad_args():
    L = _lib.lib()
    p = ctypes.c_void_p
    assert L.gdn_state_qdq_int8(p(FAKE), p(FAKE), None, -1, 64, 128, None) == 1
    assert L.gdn_state_qdq_int8(p(FAKE), p(FAKE), None, 4, 96, 128, None) == 1
    assert L.gdn_state_qdq_int8(p(FAKE), p(FAKE), None, 4, 64, 48, None) == 1
    assert L.gdn_state_qdq_int8(p(FAKE), p(FAKE), None, 4, 64, 512, None) == 2
    assert L.gdn_state_qdq_int8(None, p(FAKE), None, 4, 64, 128, None) == 1
    assert L.gdn_state_qdq_int8(p(FAKE + 4), p(FAKE), None, 4, 64, 128, None) == 1
    assert L.gdn_state_qdq_int8(None, None, None, 0, 64, 128, None) in (0, 3)  # nothing to do


def test_decode_rejects_bad_args():
    L = _lib.lib()
    p = ctypes.c_void_p
    # q, k, v, beta, g, active, state, o, state_pre, scales, stream
    s = _shape(total_tokens=3)     # decode needs total_tokens == n_seqs
    args = [p(FAKE)] * 5 + [None, p(FAKE), p(FAKE), None, None, None]
    assert L.gdn_decode_step(ctypes.byref(s), *args) == 1
    s = _shape(total_tokens=2)
    bad = [p(FAKE)] * 5 + [None, None, p(FAKE), None, None, None]   # state NULL
    assert L.gdn_decode_step(ctypes.byref(s), *bad) == 1
    bad = [p(FAKE)] * 5 + [p(FAKE + 2), p(FAKE), p(FAKE), None, None, None]   # misaligned active
    assert L.gdn_decode_step(ctypes.byref(s), *bad) == 1
    assert "misaligned" in _lib.last_error()


def test_suffix_record_and_debug_alignment():
    """The recurrent suffix's per-token record needs its offsets; every state
    record must be 16-byte aligned."""
    f = ctypes.c_void_p(FAKE)
    # bound_offsets, bound_pre, bound_post, scales, kernel_start, kernel_end, schedule,
    # w_pre, w_post, suffix_offsets, suffix_pre, suffix_post
    dbg = GdnDebug(None, None, None, None, None, None, 0, None, None, None, f, None)
    assert _chunk(_shape(), dbg=ctypes.byref(dbg)) == 1
    assert "suffix_offsets" in _lib.last_error()
    dbg = GdnDebug(None, None, None, None, None, None, 0, None, None, f, None, ctypes.c_void_p(FAKE + 4))
    assert _chunk(_shape(), dbg=ctypes.byref(dbg)) == 1
    dbg = GdnDebug(f, ctypes.c_void_p(FAKE + 8), None, None, None, None, 0, None, None, None, None, None)
    assert _chunk(_shape(), dbg=ctypes.byref(dbg)) == 1


def test_workspace_status_checks():
    """gdn_workspace_status takes the call's workspace: NULL or misaligned is
    rejected on the host; without a GPU the read reports a device error."""
    L = _lib.lib()
    assert L.gdn_workspace_status(None, None) == 1
    assert L.gdn_workspace_status(ctypes.c_void_p(FAKE + 16), None) == 1
    if not HAS_GPU:
        assert L.gdn_workspace_status(ctypes.c_void_p(FAKE), None) == 3


@pytest.mark.skipif(HAS_GPU, reason="would launch with stand-in pointers on a GPU")
def test_valid_call_without_gpu_reports_device_error():
    assert _chunk(_shape()) == 3
    assert "device" in _lib.last_error().lower()


def test_fp32_dk128_takes_no_w_qdq():
    """fp32 inputs with dk = 128 (the token-recurrence path) refuse W QDQ on
    the host (UNSUPPORTED); without it the call passes the host checks."""
    assert _chunk(_shape(io_dtype=0, o_dtype=0, qdq_flags=3 | _lib.GDN_QDQ_W)) == 2
    assert "W QDQ" in _lib.last_error()
    if not HAS_GPU:
        assert _chunk(_shape(io_dtype=0, o_dtype=0, qdq_flags=3)) == 3   # no device here
        assert _chunk(_shape(io_dtype=0, o_dtype=0, gate_per_channel=1, qdq_flags=3)) == 3


def _bwd(shape, q=FAKE, do=FAKE, dh=FAKE, d0=FAKE, ws=FAKE, ws_bytes=None):
    p = ctypes.c_void_p
    L = _lib.lib()
    if ws_bytes is None:
        ws_bytes = L.gdn_chunk_bwd_workspace_bytes(ctypes.byref(shape))
    return L.gdn_chunk_bwd_dh(ctypes.byref(shape), p(q), p(FAKE), p(FAKE), p(FAKE), p(FAKE), None, p(do), None,
                              p(dh) if dh else None, p(d0) if d0 else None, None, p(ws), ws_bytes, None)


def test_chunk_bwd_dh_checks():
    """Workspace: the status word and chunk offsets plus two 16 KiB records
    (T^T, P^T) per chunk and head of the worst-case count, and for the
    backward of a W-QDQ forward also the forward's T (18 KiB), P (12 KiB)
    and W (dk * 128 + 1 KiB) records (the per-channel gate's token
    recurrence needs none, and has no W-QDQ backward); bf16 only; the INT8
    decode codec refused; at least one output; buffers aligned."""
    L = _lib.lib()
    s = _shape(n_seqs=3, n_heads=2, total_tokens=130)
    assert L.gdn_chunk_bwd_workspace_bytes(ctypes.byref(s)) == 256 + 256 + (3 + 3) * 2 * 2 * 16384
    sw = _shape(n_seqs=3, n_heads=2, total_tokens=130, qdq_flags=3 | _lib.GDN_QDQ_W)
    assert L.gdn_chunk_bwd_workspace_bytes(ctypes.byref(sw)) == \
        256 + 256 + (3 + 3) * 2 * (2 * 16384 + 18432 + 12288 + 128 * 128 + 1024)
    assert _bwd(_shape(io_dtype=0, dk=64)) == 2
    sp = _shape(n_seqs=3, n_heads=2, total_tokens=130, gate_per_channel=1)
    assert L.gdn_chunk_bwd_workspace_bytes(ctypes.byref(sp)) == 256 + 256   # the token recurrence: no records
    assert _bwd(_shape(gate_per_channel=1, qdq_flags=3 | _lib.GDN_QDQ_W)) == 2
    assert _bwd(_shape(gate_per_channel=1)) == 3   # accepted on the host; no device here
    assert _bwd(_shape(qdq_flags=3 | _lib.GDN_QDQ_INT8)) == 2
    assert _bwd(_shape(gate_grid_log2=8)) == 1   # no recurrent writes in a fully chunked backward
    assert "gate_grid_log2" in _lib.last_error()
    assert _bwd(_shape(), dh=0, d0=0) == 1
    assert _bwd(_shape(), q=FAKE + 8) == 1
    assert _bwd(_shape(), ws_bytes=100) == 1


def test_noalloc_rejects_shapes_beyond_its_scratch():
    """gdn_chunk_fwd_noalloc runs in the library's static 64 MiB scratch: a
    shape whose workspace is larger is refused on the host (UNSUPPORTED,
    nothing launched); argument checks are those of gdn_chunk_fwd."""
    L = _lib.lib()
    p = ctypes.c_void_p
    big = _shape(n_seqs=4, n_heads=16, total_tokens=4 * 4096)   # about 124 MiB of records
    assert _ws(big) > _lib.NOALLOC_SCRATCH_BYTES
    args = [p(FAKE)] * 6 + [None, None, None, p(FAKE), p(FAKE), None, None]
    assert L.gdn_chunk_fwd_noalloc(ctypes.byref(big), *args) == 2
    assert "scratch" in _lib.last_error()
    small = _shape(n_seqs=2, n_heads=4, total_tokens=1000)
    assert _ws(small) <= _lib.NOALLOC_SCRATCH_BYTES
    assert L.gdn_chunk_fwd_noalloc(ctypes.byref(_shape(dv=96)), *args) == 1
    bad = [p(FAKE + 8)] + [p(FAKE)] * 5 + [None, None, None, p(FAKE), p(FAKE), None, None]   # misaligned q
    assert L.gdn_chunk_fwd_noalloc(ctypes.byref(small), *bad) == 1
    assert "misaligned" in _lib.last_error()
    if not HAS_GPU:
        assert L.gdn_chunk_fwd_noalloc(ctypes.byref(small), *args) == 3   # no device here
