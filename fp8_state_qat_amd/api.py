"""torch-facing binding of the C ABI: argument marshalling only.

Every function takes device tensors (torch is used for device memory and the
current stream), turns them into pointers and sizes, and calls one entry
point of libgdn.so on torch's current stream.  All arithmetic runs in the
HIP kernels.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import GDN_BF16, GDN_F32, GDN_QDQ_CHUNK, GDN_QDQ_WRITE, GdnDebug, GdnShape

_DT = {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, name, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _shape(N, H, dk, dv, T, io_dt, o_dt, per_channel, flags):
    return GdnShape(N, H, dk, dv, T, _DT[io_dt], _DT[o_dt], 1 if per_channel else 0, int(flags))


def chunk_workspace_bytes(N, H, dk, dv, T, io_dtype=torch.bfloat16, qdq_flags=0):
    """Device workspace gdn_chunk_fwd needs for this shape (bytes)."""
    shape = _shape(N, H, dk, dv, T, io_dtype, io_dtype, False, qdq_flags)
    n = _lib.lib().gdn_chunk_fwd_workspace_bytes(ctypes.byref(shape))
    if n == 0:
        _lib.check(_lib.GDN_ERR_INVALID_ARG)
    return n


def chunk_fwd(q, k, v, beta, g, cu_seqlens, *, seq_lens=None, prefix_lens=None,
              initial_state=None, qdq_flags=GDN_QDQ_CHUNK | GDN_QDQ_WRITE, o_dtype=None,
              out=None, final_state=None, workspace=None, debug=None):
    """gdn_chunk_fwd.  q, k: [T, H, dk]; v: [T, H, dv] (fp32 or bf16); beta:
    [T, H] fp32; g: [T, H] or [T, H, dk] fp32; cu_seqlens: [N+1] int32.
    workspace: optional uint8 device tensor of chunk_workspace_bytes(...)
    bytes (allocated here when None).  debug: optional dict with device
    tensors bound_offsets, bound_pre, bound_post, scales, w_pre, w_post
    ([n_bounds, H, 64, dk] fp32, W of each chunk before and after its QDQ,
    with GDN_QDQ_W in qdq_flags), torch.cuda.Event
    objects kernel_start, kernel_end (recorded around the sequential state
    kernel) and/or schedule (GDN_SCHEDULE_AUTO, _SPLIT or _FUSED: the
    per-chunk solve as its own kernel or inside the state kernel's launch;
    _FUSED_NO_PRODUCERS, a test hook whose bounded waits all run out).
    Returns (o, final_state)."""
    T, H, dk = k.shape
    dv = v.shape[2]
    N = cu_seqlens.numel() - 1
    if q.dtype != k.dtype or v.dtype != k.dtype or k.dtype not in _DT:
        raise ValueError("q, k, v must share one dtype: float32 or bfloat16")
    o_dtype = k.dtype if o_dtype is None else o_dtype
    for name, t, dt in (("q", q, None), ("k", k, None), ("v", v, None), ("beta", beta, torch.float32),
                        ("g", g, torch.float32), ("cu_seqlens", cu_seqlens, torch.int32),
                        ("seq_lens", seq_lens, torch.int32), ("prefix_lens", prefix_lens, torch.int32),
                        ("initial_state", initial_state, torch.float32)):
        _dev(t, name, dt)
    if out is None:
        out = torch.empty((T, H, dv), dtype=o_dtype, device=k.device)
    if final_state is None:
        final_state = torch.empty((N, H, dv, dk), dtype=torch.float32, device=k.device)
    _dev(out, "out", o_dtype)
    _dev(final_state, "final_state", torch.float32)
    shape = _shape(N, H, dk, dv, T, k.dtype, o_dtype, g.dim() == 3, qdq_flags)
    ws_bytes = _lib.lib().gdn_chunk_fwd_workspace_bytes(ctypes.byref(shape))
    if ws_bytes == 0:
        _lib.check(_lib.GDN_ERR_INVALID_ARG)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=k.device)
    _dev(workspace, "workspace", torch.uint8)
    dbg = None
    if debug is not None:
        evs = []
        for key in ("kernel_start", "kernel_end"):
            ev = debug.get(key)
            if ev is not None and not ev.cuda_event:
                ev.record()  # torch creates its HIP event on first record
            evs.append(None if ev is None else ctypes.c_void_p(ev.cuda_event))
        dbg = GdnDebug(*(_ptr(debug.get(key)) for key in ("bound_offsets", "bound_pre",
                                                          "bound_post", "scales")), *evs,
                       int(debug.get("schedule", _lib.GDN_SCHEDULE_AUTO)),
                       _ptr(debug.get("w_pre")), _ptr(debug.get("w_post")))
    st = _lib.lib().gdn_chunk_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                  _ptr(g), _ptr(cu_seqlens), _ptr(seq_lens), _ptr(prefix_lens),
                                  _ptr(initial_state), _ptr(out), _ptr(final_state),
                                  _ptr(workspace), workspace.numel(),
                                  ctypes.byref(dbg) if dbg is not None else None, _stream())
    _lib.check(st)
    return out, final_state


def chunk_bwd_dh(q, k, beta, g, cu_seqlens, d_o, *, seq_lens=None, d_final_state=None, dh=None,
                 d_initial_state=None, d_v=None, want_dv=False, workspace=None):
    """gdn_chunk_bwd_dh: gradients of the state entering every 64-token chunk
    (dh [n_bounds, H, dv, dk]) and of the initial state ([N, H, dv, dk]) for
    L = sum o . d_o + <S_L, d_final_state>, identity straight-through QDQ;
    with want_dv (or a d_v tensor) also the gradient of v ([T, H, dv] fp32).
    q, k: [T, H, dk] bf16; d_o: [T, H, dv] bf16; beta, g: [T, H] fp32.
    Returns (dh, d_initial_state) or (dh, d_initial_state, d_v)."""
    T, H, dk = k.shape
    dv = d_o.shape[2]
    N = cu_seqlens.numel() - 1
    for name, t, dt in (("q", q, torch.bfloat16), ("k", k, torch.bfloat16), ("d_o", d_o, torch.bfloat16),
                        ("beta", beta, torch.float32), ("g", g, torch.float32),
                        ("cu_seqlens", cu_seqlens, torch.int32), ("seq_lens", seq_lens, torch.int32),
                        ("d_final_state", d_final_state, torch.float32), ("d_v", d_v, torch.float32)):
        _dev(t, name, dt)
    lens = seq_lens if seq_lens is not None else (cu_seqlens[1:] - cu_seqlens[:-1])
    n_bounds = int(((lens.to(torch.int64) + 63) // 64).sum().item()) if N else 0
    if dh is None:
        dh = torch.empty((n_bounds, H, dv, dk), dtype=torch.float32, device=k.device)
    if d_initial_state is None:
        d_initial_state = torch.empty((N, H, dv, dk), dtype=torch.float32, device=k.device)
    if want_dv and d_v is None:
        d_v = torch.empty((T, H, dv), dtype=torch.float32, device=k.device)
    shape = _shape(N, H, dk, dv, T, k.dtype, k.dtype, g.dim() == 3, 0)
    ws_bytes = _lib.lib().gdn_chunk_bwd_workspace_bytes(ctypes.byref(shape))
    if ws_bytes == 0:
        _lib.check(_lib.GDN_ERR_INVALID_ARG)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=k.device)
    st = _lib.lib().gdn_chunk_bwd_dh(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(beta), _ptr(g),
                                     _ptr(cu_seqlens), _ptr(seq_lens), _ptr(d_o), _ptr(d_final_state),
                                     _ptr(dh) if dh.numel() else None, _ptr(d_initial_state), _ptr(d_v),
                                     _ptr(workspace), workspace.numel(), _stream())
    _lib.check(st)
    if d_v is not None:
        return dh, d_initial_state, d_v
    return dh, d_initial_state


def state_qdq(x, out=None, scales=None, want_scales=True):
    """gdn_state_qdq on x [..., dv, dk] fp32.  Returns (out, scales [..., dv/64])."""
    _dev(x, "x", torch.float32)
    dv, dk = x.shape[-2], x.shape[-1]
    n = x.numel() // (dv * dk) if x.numel() else 0
    if out is None:
        out = torch.empty_like(x)
    if scales is None and want_scales:
        scales = torch.empty(x.shape[:-2] + (dv // 64,), dtype=torch.float32, device=x.device)
    _dev(out, "out", torch.float32)
    st = _lib.lib().gdn_state_qdq(_ptr(x), _ptr(out), _ptr(scales), n, dv, dk, _stream())
    _lib.check(st)
    return out, scales


def state_qdq_int8(x, out=None, scales=None, want_scales=True):
    """gdn_state_qdq_int8 on x [..., dv, dk] fp32 (blocks of 32 key columns).
    Returns (out, scales [..., dv, dk/32])."""
    _dev(x, "x", torch.float32)
    dv, dk = x.shape[-2], x.shape[-1]
    n = x.numel() // (dv * dk) if x.numel() else 0
    if out is None:
        out = torch.empty_like(x)
    if scales is None and want_scales:
        scales = torch.empty(x.shape[:-1] + (dk // 32,), dtype=torch.float32, device=x.device)
    _dev(out, "out", torch.float32)
    st = _lib.lib().gdn_state_qdq_int8(_ptr(x), _ptr(out), _ptr(scales), n, dv, dk, _stream())
    _lib.check(st)
    return out, scales


def decode_step(q, k, v, beta, g, state, *, qdq=True, o=None, o_dtype=None, state_pre=None,
                scales=None, int8=False):
    """gdn_decode_step.  q, k: [N, H, dk]; v: [N, H, dv]; beta: [N, H]; g: [N, H]
    or [N, H, dk]; state [N, H, dv, dk] fp32 updated in place.  int8: the
    per-write QDQ is INT8 block-32 (scales [N, H, dv, dk/32]) instead of FP8
    per tile.  Returns o."""
    N, H, dk = k.shape
    dv = v.shape[2]
    o_dtype = k.dtype if o_dtype is None else o_dtype
    for name, t, dt in (("q", q, None), ("k", k, None), ("v", v, None), ("beta", beta, torch.float32),
                        ("g", g, torch.float32), ("state", state, torch.float32),
                        ("state_pre", state_pre, torch.float32), ("scales", scales, torch.float32)):
        _dev(t, name, dt)
    if o is None:
        o = torch.empty((N, H, dv), dtype=o_dtype, device=k.device)
    shape = GdnShape(N, H, dk, dv, N, _DT[k.dtype], _DT[o_dtype], 1 if g.dim() == 3 else 0,
                     (GDN_QDQ_WRITE if qdq else 0) | (_lib.GDN_QDQ_INT8 if int8 else 0))
    st = _lib.lib().gdn_decode_step(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                    _ptr(g), _ptr(state), _ptr(o), _ptr(state_pre), _ptr(scales),
                                    _stream())
    _lib.check(st)
    return o
