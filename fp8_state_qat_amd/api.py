"""torch-facing binding of the C ABI: argument marshalling only.

Every function takes device tensors (torch is used for device memory and the
current stream), checks their dtypes, shapes and contiguity against the
call's contract, turns them into pointers and sizes, and calls one entry
point of libgdn.so on torch's current stream.  All arithmetic runs in the
HIP kernels.  A tensor of the wrong shape raises ValueError before anything
is launched: the kernels trust the sizes they are given.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import GDN_BF16, GDN_F32, GDN_QDQ_CHUNK, GDN_QDQ_WRITE, GdnDebug, GdnShape

_DT = {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, name, dtype=None, shape=None):
    """Check that t (if given) is a contiguous tensor of this dtype and exact
    shape.  Whether it lives on the device is checked by _on_device, after
    every tensor of the call has passed these checks."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_device(**tensors):
    """Every given tensor lives on the current device."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _shape(N, H, dk, dv, T, io_dt, o_dt, per_channel, flags, grid=0):
    return GdnShape(N, H, dk, dv, T, _DT[io_dt], _DT[o_dt], 1 if per_channel else 0, int(flags), int(grid))


def _offsets_total(offs, N, name):
    """Host copy of a device [N + 1] offsets tensor (debug records only);
    returns its last entry, the record's first dimension."""
    _dev(offs, name, torch.int32, (N + 1,))
    _on_device(**{name: offs})
    return int(offs[-1].item())


def chunk_workspace_bytes(N, H, dk, dv, T, io_dtype=torch.bfloat16, qdq_flags=0):
    """Device workspace gdn_chunk_fwd needs for this shape (bytes)."""
    shape = _shape(N, H, dk, dv, T, io_dtype, io_dtype, False, qdq_flags)
    n = _lib.lib().gdn_chunk_fwd_workspace_bytes(ctypes.byref(shape))
    if n == 0:
        _lib.check(_lib.GDN_ERR_INVALID_ARG)
    return n


def workspace_status(workspace):
    """gdn_workspace_status: synchronizes torch's current stream and raises
    GdnError when the call that last used this workspace found its index
    arrays out of contract (GDN_ERR_INVALID_ARG) or had a bounded wait run out
    (GDN_ERR_DEVICE)."""
    _dev(workspace, "workspace", torch.uint8)
    _on_device(workspace=workspace)
    _lib.check(_lib.lib().gdn_workspace_status(_ptr(workspace), _stream()))


def chunk_fwd(q, k, v, beta, g, cu_seqlens, *, seq_lens=None, prefix_lens=None,
              initial_state=None, qdq_flags=GDN_QDQ_CHUNK | GDN_QDQ_WRITE, o_dtype=None,
              out=None, final_state=None, workspace=None, debug=None, check_status=False, noalloc=False,
              gate_grid_log2=0):
    """gdn_chunk_fwd.  q, k: [T, H, dk]; v: [T, H, dv] (fp32 or bf16); beta:
    [T, H] fp32; g: [T, H] or [T, H, dk] fp32; cu_seqlens: [N+1] int32;
    seq_lens, prefix_lens: [N] int32 or None; initial_state: [N, H, dv, dk]
    fp32 or None.
    workspace: optional uint8 device tensor of at least
    chunk_workspace_bytes(...) bytes (allocated here when None).
    debug: optional dict with device tensors bound_offsets ([N+1] int32),
    bound_pre, bound_post ([n_bounds, H, dv, dk] fp32), scales ([n_bounds, H,
    dv/64]), w_pre, w_post ([n_bounds, H, 64, dk] fp32, W of each chunk before
    and after its QDQ, with GDN_QDQ_W in qdq_flags), suffix_offsets ([N+1]
    int32), suffix_pre, suffix_post ([n_suffix, H, dv, dk] fp32, the state
    after each recurrent suffix token before and after its QDQ),
    status ([1] int32: receives the call's status word on the stream),
    torch.cuda.Event objects kernel_start, kernel_end (recorded around the
    sequential state kernel) and/or schedule (GDN_SCHEDULE_AUTO, _SPLIT or
    _FUSED: the per-chunk solve as its own kernel or inside the state
    kernel's launch; _FUSED_NO_PRODUCERS, a test hook whose bounded waits all
    run out).  check_status: read the workspace's status word after the call
    (synchronizes; raises GdnError on a device-side failure).
    noalloc: call gdn_chunk_fwd_noalloc instead, whose workspace is the
    library's static per-GPU scratch (out and final_state must be given, no
    workspace; the status word comes back through debug["status"]).
    gate_grid_log2: 0, or k in 1..24: the log-gates of the recurrent suffix
    rounded to multiples of 2^-k (the log-retention grid).
    Returns (o, final_state)."""
    if noalloc:
        if workspace is not None or check_status:
            raise ValueError("noalloc takes no workspace (pass debug['status'] for the status word)")
        if out is None or final_state is None:
            raise ValueError("noalloc needs out and final_state")
    _dev(k, "k")
    if k.dim() != 3:
        raise ValueError(f"k must be [T, H, dk], got shape {tuple(k.shape)}")
    T, H, dk = k.shape
    _dev(v, "v")
    if v.dim() != 3 or tuple(v.shape[:2]) != (T, H):
        raise ValueError(f"v must be [{T}, {H}, dv], got shape {tuple(v.shape)}")
    dv = v.shape[2]
    _dev(cu_seqlens, "cu_seqlens", torch.int32)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be [N + 1] with N >= 1")
    N = cu_seqlens.numel() - 1
    if q.dtype != k.dtype or v.dtype != k.dtype or k.dtype not in _DT:
        raise ValueError("q, k, v must share one dtype: float32 or bfloat16")
    if o_dtype is None:
        o_dtype = out.dtype if isinstance(out, torch.Tensor) else k.dtype
    if o_dtype not in _DT:
        raise ValueError("o_dtype must be float32 or bfloat16")
    per_channel = g.dim() == 3
    for name, t, dt, shp in (("q", q, None, (T, H, dk)), ("beta", beta, torch.float32, (T, H)),
                             ("g", g, torch.float32, (T, H, dk) if per_channel else (T, H)),
                             ("seq_lens", seq_lens, torch.int32, (N,)),
                             ("prefix_lens", prefix_lens, torch.int32, (N,)),
                             ("initial_state", initial_state, torch.float32, (N, H, dv, dk))):
        _dev(t, name, dt, shp)
    _dev(out, "out", o_dtype, (T, H, dv))
    _dev(final_state, "final_state", torch.float32, (N, H, dv, dk))
    _dev(q, "q", k.dtype, (T, H, dk))
    _on_device(q=q, k=k, v=v, beta=beta, g=g, cu_seqlens=cu_seqlens, seq_lens=seq_lens,
               prefix_lens=prefix_lens, initial_state=initial_state, out=out, final_state=final_state)
    if out is None:
        out = torch.empty((T, H, dv), dtype=o_dtype, device=k.device)
    if final_state is None:
        final_state = torch.empty((N, H, dv, dk), dtype=torch.float32, device=k.device)
    shape = _shape(N, H, dk, dv, T, k.dtype, o_dtype, per_channel, qdq_flags, gate_grid_log2)
    if not noalloc:
        ws_bytes = _lib.lib().gdn_chunk_fwd_workspace_bytes(ctypes.byref(shape))
        if ws_bytes == 0:
            _lib.check(_lib.GDN_ERR_INVALID_ARG)
        if workspace is None:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=k.device)
        _dev(workspace, "workspace", torch.uint8)
        _on_device(k=k, workspace=workspace)
        if workspace.dim() != 1:
            raise ValueError("workspace must be a 1-D uint8 tensor")
    dbg = None
    if debug is not None:
        unknown = set(debug) - {"bound_offsets", "bound_pre", "bound_post", "scales", "kernel_start",
                                "kernel_end", "schedule", "w_pre", "w_post", "suffix_offsets",
                                "suffix_pre", "suffix_post", "status"}
        if unknown:
            raise ValueError(f"unknown debug keys {sorted(unknown)}")
        if any(debug.get(key) is not None for key in ("bound_pre", "bound_post", "scales", "w_pre", "w_post")):
            if debug.get("bound_offsets") is None:
                raise ValueError("the per-boundary record needs bound_offsets")
            nb = _offsets_total(debug["bound_offsets"], N, "bound_offsets")
            for key, shp in (("bound_pre", (nb, H, dv, dk)), ("bound_post", (nb, H, dv, dk)),
                             ("scales", (nb, H, dv // 64)), ("w_pre", (nb, H, 64, dk)),
                             ("w_post", (nb, H, 64, dk))):
                _dev(debug.get(key), key, torch.float32, shp)
                _on_device(k=k, **{key: debug.get(key)})
        if debug.get("suffix_pre") is not None or debug.get("suffix_post") is not None:
            if debug.get("suffix_offsets") is None:
                raise ValueError("the suffix record needs suffix_offsets")
            ns = _offsets_total(debug["suffix_offsets"], N, "suffix_offsets")
            for key in ("suffix_pre", "suffix_post"):
                _dev(debug.get(key), key, torch.float32, (ns, H, dv, dk))
                _on_device(k=k, **{key: debug.get(key)})
        _dev(debug.get("status"), "status", torch.int32, (1,))
        _on_device(k=k, status=debug.get("status"))
        evs = []
        for key in ("kernel_start", "kernel_end"):
            ev = debug.get(key)
            if ev is not None and not ev.cuda_event:
                ev.record()  # torch creates its HIP event on first record
            evs.append(None if ev is None else ctypes.c_void_p(ev.cuda_event))
        dbg = GdnDebug(*(_ptr(debug.get(key)) for key in ("bound_offsets", "bound_pre",
                                                          "bound_post", "scales")), *evs,
                       int(debug.get("schedule", _lib.GDN_SCHEDULE_AUTO)),
                       _ptr(debug.get("w_pre")), _ptr(debug.get("w_post")),
                       _ptr(debug.get("suffix_offsets")), _ptr(debug.get("suffix_pre")),
                       _ptr(debug.get("suffix_post")), _ptr(debug.get("status")))
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(cu_seqlens), _ptr(seq_lens), _ptr(prefix_lens),
            _ptr(initial_state), _ptr(out), _ptr(final_state))
    dbg_p = ctypes.byref(dbg) if dbg is not None else None
    if noalloc:
        st = _lib.lib().gdn_chunk_fwd_noalloc(ctypes.byref(shape), *args, dbg_p, _stream())
    else:
        st = _lib.lib().gdn_chunk_fwd(ctypes.byref(shape), *args, _ptr(workspace), workspace.numel(), dbg_p,
                                      _stream())
    _lib.check(st)
    if check_status:
        workspace_status(workspace)
    return out, final_state


def chunk_bwd_dh(q, k, beta, g, cu_seqlens, d_o, *, seq_lens=None, d_final_state=None, dh=None,
                 d_initial_state=None, d_v=None, want_dv=False, workspace=None, qdq_flags=0,
                 check_status=False):
    """gdn_chunk_bwd_dh: gradients of the state entering every 64-token chunk
    (dh [n_bounds, H, dv, dk]) and of the initial state ([N, H, dv, dk]) for
    L = sum o . d_o + <S_L, d_final_state>, identity straight-through QDQ;
    with want_dv (or a d_v tensor) also the gradient of v ([T, H, dv] fp32).
    q, k: [T, H, dk] bf16; d_o: [T, H, dv] bf16; beta, g: [T, H] fp32.
    qdq_flags: those of the forward (with GDN_QDQ_W, the backward of the W-QDQ
    forward: its quantized W enters the state gradient).
    dh: an empty tensor asks for no per-chunk gradient.
    Returns (dh, d_initial_state) or (dh, d_initial_state, d_v)."""
    _dev(k, "k", torch.bfloat16)
    if k.dim() != 3:
        raise ValueError(f"k must be [T, H, dk], got shape {tuple(k.shape)}")
    T, H, dk = k.shape
    _dev(d_o, "d_o", torch.bfloat16)
    if d_o.dim() != 3 or tuple(d_o.shape[:2]) != (T, H):
        raise ValueError(f"d_o must be [{T}, {H}, dv], got shape {tuple(d_o.shape)}")
    dv = d_o.shape[2]
    _dev(cu_seqlens, "cu_seqlens", torch.int32)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be [N + 1] with N >= 1")
    N = cu_seqlens.numel() - 1
    gshape = (T, H, dk) if g.dim() == 3 else (T, H)
    for name, t, dt, shp in (("q", q, torch.bfloat16, (T, H, dk)), ("beta", beta, torch.float32, (T, H)),
                             ("g", g, torch.float32, gshape), ("seq_lens", seq_lens, torch.int32, (N,)),
                             ("d_final_state", d_final_state, torch.float32, (N, H, dv, dk)),
                             ("d_v", d_v, torch.float32, (T, H, dv))):
        _dev(t, name, dt, shp)
    _on_device(q=q, k=k, beta=beta, g=g, cu_seqlens=cu_seqlens, d_o=d_o, seq_lens=seq_lens,
               d_final_state=d_final_state, d_v=d_v)
    lens = seq_lens if seq_lens is not None else (cu_seqlens[1:] - cu_seqlens[:-1])
    n_bounds = int(((lens.to(torch.int64) + 63) // 64).clamp(min=0).sum().item()) if N else 0
    if dh is None:
        dh = torch.empty((n_bounds, H, dv, dk), dtype=torch.float32, device=k.device)
    if d_initial_state is None:
        d_initial_state = torch.empty((N, H, dv, dk), dtype=torch.float32, device=k.device)
    if want_dv and d_v is None:
        d_v = torch.empty((T, H, dv), dtype=torch.float32, device=k.device)
    if dh.numel():   # an empty tensor asks for no dh output
        _dev(dh, "dh", torch.float32, (n_bounds, H, dv, dk))
    _dev(d_initial_state, "d_initial_state", torch.float32, (N, H, dv, dk))
    _on_device(k=k, dh=dh, d_initial_state=d_initial_state, d_v=d_v)
    shape = _shape(N, H, dk, dv, T, k.dtype, k.dtype, g.dim() == 3, qdq_flags)
    ws_bytes = _lib.lib().gdn_chunk_bwd_workspace_bytes(ctypes.byref(shape))
    if ws_bytes == 0:
        _lib.check(_lib.GDN_ERR_INVALID_ARG)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=k.device)
    _dev(workspace, "workspace", torch.uint8)
    _on_device(k=k, workspace=workspace)
    st = _lib.lib().gdn_chunk_bwd_dh(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(beta), _ptr(g),
                                     _ptr(cu_seqlens), _ptr(seq_lens), _ptr(d_o), _ptr(d_final_state),
                                     _ptr(dh) if dh.numel() else None, _ptr(d_initial_state), _ptr(d_v),
                                     _ptr(workspace), workspace.numel(), _stream())
    _lib.check(st)
    if check_status:
        workspace_status(workspace)
    if d_v is not None:
        return dh, d_initial_state, d_v
    return dh, d_initial_state


def _states_shape(x, name):
    _dev(x, name, torch.float32)
    if x.dim() < 2:
        raise ValueError(f"{name} must be [..., dv, dk]")
    dv, dk = x.shape[-2], x.shape[-1]
    return dv, dk, (x.numel() // (dv * dk) if x.numel() else 0)


def state_qdq(x, out=None, scales=None, want_scales=True):
    """gdn_state_qdq on x [..., dv, dk] fp32.  Returns (out, scales [..., dv/64])."""
    dv, dk, n = _states_shape(x, "x")
    if out is None:
        out = torch.empty_like(x)
    if scales is None and want_scales:
        scales = torch.empty(x.shape[:-2] + (dv // 64,), dtype=torch.float32, device=x.device)
    _dev(out, "out", torch.float32, tuple(x.shape))
    _dev(scales, "scales", torch.float32, tuple(x.shape[:-2]) + (dv // 64,))
    _on_device(x=x, out=out, scales=scales)
    st = _lib.lib().gdn_state_qdq(_ptr(x), _ptr(out), _ptr(scales), n, dv, dk, _stream())
    _lib.check(st)
    return out, scales


def state_qdq_int8(x, out=None, scales=None, want_scales=True):
    """gdn_state_qdq_int8 on x [..., dv, dk] fp32 (blocks of 32 key columns).
    Returns (out, scales [..., dv, dk/32])."""
    dv, dk, n = _states_shape(x, "x")
    if out is None:
        out = torch.empty_like(x)
    if scales is None and want_scales:
        scales = torch.empty(x.shape[:-1] + (dk // 32,), dtype=torch.float32, device=x.device)
    _dev(out, "out", torch.float32, tuple(x.shape))
    _dev(scales, "scales", torch.float32, tuple(x.shape[:-1]) + (dk // 32,))
    _on_device(x=x, out=out, scales=scales)
    st = _lib.lib().gdn_state_qdq_int8(_ptr(x), _ptr(out), _ptr(scales), n, dv, dk, _stream())
    _lib.check(st)
    return out, scales


def decode_step(q, k, v, beta, g, state, *, qdq=True, o=None, o_dtype=None, state_pre=None,
                scales=None, int8=False, active=None, gate_grid_log2=0):
    """gdn_decode_step.  q, k: [N, H, dk]; v: [N, H, dv]; beta: [N, H]; g: [N, H]
    or [N, H, dk]; state [N, H, dv, dk] fp32 updated in place.  int8: the
    per-write QDQ is INT8 block-32 (scales [N, H, dv, dk/32]) instead of FP8
    per tile (scales [N, H, dv/64]).  active: optional [N] int32; sequences
    with active[n] == 0 are left untouched (state, o and the records).
    gate_grid_log2: 0, or k in 1..24: the log-gates rounded to multiples of
    2^-k (the log-retention grid).
    Returns o."""
    _dev(k, "k")
    if k.dim() != 3:
        raise ValueError(f"k must be [N, H, dk], got shape {tuple(k.shape)}")
    N, H, dk = k.shape
    _dev(v, "v")
    if v.dim() != 3 or tuple(v.shape[:2]) != (N, H):
        raise ValueError(f"v must be [{N}, {H}, dv], got shape {tuple(v.shape)}")
    dv = v.shape[2]
    if q.dtype != k.dtype or v.dtype != k.dtype or k.dtype not in _DT:
        raise ValueError("q, k, v must share one dtype: float32 or bfloat16")
    if o_dtype is None:
        o_dtype = o.dtype if isinstance(o, torch.Tensor) else k.dtype
    if o_dtype not in _DT:
        raise ValueError("o_dtype must be float32 or bfloat16")
    per_channel = g.dim() == 3
    sc_shape = (N, H, dv, dk // 32) if (int8 and qdq) else (N, H, dv // 64)
    for name, t, dt, shp in (("q", q, None, (N, H, dk)), ("beta", beta, torch.float32, (N, H)),
                             ("g", g, torch.float32, (N, H, dk) if per_channel else (N, H)),
                             ("state", state, torch.float32, (N, H, dv, dk)),
                             ("state_pre", state_pre, torch.float32, (N, H, dv, dk)),
                             ("scales", scales, torch.float32, sc_shape),
                             ("active", active, torch.int32, (N,))):
        _dev(t, name, dt, shp)
    if state is None:
        raise ValueError("state is required")
    _dev(o, "o", o_dtype, (N, H, dv))
    _on_device(q=q, k=k, v=v, beta=beta, g=g, state=state, state_pre=state_pre, scales=scales,
               active=active, o=o)
    if o is None:
        o = torch.empty((N, H, dv), dtype=o_dtype, device=k.device)
    shape = GdnShape(N, H, dk, dv, N, _DT[k.dtype], _DT[o_dtype], 1 if per_channel else 0,
                     (GDN_QDQ_WRITE if qdq else 0) | (_lib.GDN_QDQ_INT8 if int8 else 0), int(gate_grid_log2))
    st = _lib.lib().gdn_decode_step(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                    _ptr(g), _ptr(active), _ptr(state), _ptr(o), _ptr(state_pre),
                                    _ptr(scales), _stream())
    _lib.check(st)
    return o
