"""ctypes wrapper around the CPU oracle in gdn_oracle.c.

TEST INFRASTRUCTURE ONLY -- used by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py.  The HIP library never imports this module.

All floating-point inputs are taken as numpy float64 arrays holding the exact
values the kernel sees (bf16 or fp32 inputs widened without rounding).
"""
from __future__ import annotations

import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

QDQ_CHUNK = 1
QDQ_WRITE = 2
QDQ_INT8 = 8          # INT8 block-32 codec for every state QDQ of a sequence
INT8_BLOCK = 32
CHUNK = 64
TILE_ROWS = 64

_HERE = os.path.dirname(os.path.abspath(__file__))
# GDN_ORACLE_LIB: another build of the same source (the sanitized one)
_LIB_PATH = os.environ.get("GDN_ORACLE_LIB") or os.path.join(_HERE, "libgdn_oracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)
_u8p = ctypes.POINTER(ctypes.c_uint8)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.orc_e4m3_decode.argtypes = [ctypes.c_int]
    lib.orc_e4m3_decode.restype = ctypes.c_double
    lib.orc_e4m3_encode.argtypes = [ctypes.c_float]
    lib.orc_e4m3_encode.restype = ctypes.c_int
    lib.orc_e4m3_encode_bruteforce.argtypes = [ctypes.c_float]
    lib.orc_e4m3_encode_bruteforce.restype = ctypes.c_int
    lib.orc_e4m3_encode_array.argtypes = [_fp, ctypes.c_int64, _u8p]
    lib.orc_e4m3_encode_array.restype = None
    lib.orc_qdq_tile_f32.argtypes = [_fp, ctypes.c_int64, _fp, _fp, _u8p]
    lib.orc_qdq_tile_f32.restype = None
    lib.orc_qdq_int8_blocks_f32.argtypes = [_fp, ctypes.c_int64, ctypes.c_int, _fp, _fp,
                                            ctypes.POINTER(ctypes.c_int8)]
    lib.orc_qdq_int8_blocks_f32.restype = None
    lib.orc_qdq_rows_f32.argtypes = [_fp, ctypes.c_int64, ctypes.c_int, _fp, _fp, _u8p]
    lib.orc_qdq_rows_f32.restype = None
    lib.orc_qdq_states_f32.argtypes = [_fp, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                       _fp, _fp, _u8p]
    lib.orc_qdq_states_f32.restype = None
    lib.orc_gdn_sequence.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint,
        _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp,
        ctypes.c_int, _dp, _dp, _fp, ctypes.c_int]
    lib.orc_gdn_sequence.restype = ctypes.c_int
    lib.orc_grid_gate.argtypes = [ctypes.c_double, ctypes.c_int]
    lib.orc_grid_gate.restype = ctypes.c_double
    _lib = lib
    return lib


def _ptr(a, typ):
    if a is None:
        return ctypes.cast(None, typ)
    return a.ctypes.data_as(typ)


# --------------------------------------------------------------------------
# E4M3
# --------------------------------------------------------------------------
def e4m3_decode(codes) -> np.ndarray:
    """Values of E4M3FN codes (uint8 array) as float64."""
    lib = _load()
    table = np.array([lib.orc_e4m3_decode(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(y) -> np.ndarray:
    """Round fp32 values to E4M3FN codes (nearest, ties to even, saturating)."""
    lib = _load()
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, dtype=np.uint8)
    lib.orc_e4m3_encode_array(_ptr(y, _fp), y.size, _ptr(out, _u8p))
    return out


def e4m3_encode_bruteforce(y) -> np.ndarray:
    lib = _load()
    y = np.ascontiguousarray(y, dtype=np.float32).ravel()
    return np.array([lib.orc_e4m3_encode_bruteforce(float(v)) for v in y], dtype=np.uint8)


# --------------------------------------------------------------------------
# QDQ
# --------------------------------------------------------------------------
def qdq_states(x):
    """QDQ of fp32 states [..., dv, dk]; one tile per 64 value rows.

    Returns (out fp32 same shape, scales [..., dv/64] fp32, codes uint8)."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    dv, dk = x.shape[-2], x.shape[-1]
    assert dv % TILE_ROWS == 0
    n = x.size // (dv * dk)
    out = np.empty_like(x)
    scales = np.empty(x.shape[:-2] + (dv // TILE_ROWS,), dtype=np.float32)
    codes = np.empty(x.shape, dtype=np.uint8)
    lib.orc_qdq_states_f32(_ptr(x, _fp), n, dv, dk, _ptr(out, _fp), _ptr(scales, _fp),
                           _ptr(codes, _u8p))
    return out, scales, codes


def qdq_rows(x):
    """QDQ of fp32 rows [..., n]: every row (last axis) is one group with its
    own scale amax / 448 (zero guard), the grouping of the W quantizer.

    Returns (out fp32 same shape, scales [...] fp32, codes uint8)."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    n = x.shape[-1]
    rows = x.size // n if n else 0
    out = np.empty_like(x)
    scales = np.empty(x.shape[:-1], dtype=np.float32)
    codes = np.empty(x.shape, dtype=np.uint8)
    if rows:
        lib.orc_qdq_rows_f32(_ptr(x, _fp), rows, n, _ptr(out, _fp), _ptr(scales, _fp), _ptr(codes, _u8p))
    return out, scales, codes


def qdq_int8_blocks(x, block=INT8_BLOCK):
    """INT8 QDQ of fp32 values [..., n] (n a multiple of block): every block
    of `block` consecutive values along the last axis is one group with
    scale amax / 127 (zero guard), codes rounded half to even.

    Returns (out fp32 same shape, scales [..., n / block] fp32, codes int8)."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.shape[-1] % block == 0
    nb = x.size // block
    out = np.empty_like(x)
    scales = np.empty(x.shape[:-1] + (x.shape[-1] // block,), dtype=np.float32)
    codes = np.empty(x.shape, dtype=np.int8)
    if nb:
        lib.orc_qdq_int8_blocks_f32(_ptr(x, _fp), nb, block, _ptr(out, _fp), _ptr(scales, _fp),
                                    codes.ctypes.data_as(ctypes.POINTER(ctypes.c_int8)))
    return out, scales, codes


# --------------------------------------------------------------------------
# Recurrence
# --------------------------------------------------------------------------
def grid_gate(g, k):
    """Log-gate on the log-retention grid 2^-k (the oracle's orc_grid_gate)."""
    return _load().orc_grid_gate(float(g), int(k))


def gdn_sequence(q, k, v, beta, g, *, prefix_len=None, flags=QDQ_CHUNK | QDQ_WRITE,
                 S0=None, record=False, grid_log2=0):
    """Run one (sequence, head).

    q, k: [L, dk]; v: [L, dv]; beta: [L]; g: [L] (scalar gate) or [L, dk]
    (per-key-channel gate); S0: [dv, dk] or None.  float64 everywhere.
    Returns dict(o [L, dv], S [dv, dk]) plus, when record, the per-boundary
    pre/post-QDQ states [nb, dv, dk] and scales [nb, dv/64]."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    beta = np.ascontiguousarray(beta, dtype=np.float64)
    g = np.ascontiguousarray(g, dtype=np.float64)
    L, dk = k.shape
    dv = v.shape[1]
    P = L if prefix_len is None else int(prefix_len)
    per_channel = 1 if g.ndim == 2 else 0
    S0a = None if S0 is None else np.ascontiguousarray(S0, dtype=np.float64)
    o = np.zeros((L, dv), dtype=np.float64)
    S = np.zeros((dv, dk), dtype=np.float64)
    nb_max = (P + CHUNK - 1) // CHUNK if record else 0
    pre = np.zeros((nb_max, dv, dk), dtype=np.float64) if record else None
    post = np.zeros((nb_max, dv, dk), dtype=np.float64) if record else None
    sc = np.zeros((nb_max, max(1, dv // TILE_ROWS)), dtype=np.float32) if record else None
    nb = lib.orc_gdn_sequence(L, P, dk, dv, per_channel, flags,
                              _ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp), _ptr(beta, _dp),
                              _ptr(g, _dp), _ptr(S0a, _dp), _ptr(o, _dp), _ptr(S, _dp),
                              nb_max, _ptr(pre, _dp), _ptr(post, _dp), _ptr(sc, _fp), int(grid_log2))
    if nb < 0:
        raise ValueError("oracle rejected arguments")
    res = {"o": o, "S": S}
    if record:
        res.update(bound_pre=pre, bound_post=post, scales=sc, n_bounds=nb)
    return res


def gdn_packed(q, k, v, beta, g, cu_seqlens, *, seq_lens=None, prefix_lens=None,
               flags=QDQ_CHUNK | QDQ_WRITE, S0=None, pairs=None, threads=1, record=False,
               grid_log2=0):
    """Packed varlen layout, as the library takes it.

    q, k: [T, H, dk]; v: [T, H, dv]; beta: [T, H]; g: [T, H] or [T, H, dk];
    cu_seqlens: [N+1] storage boundaries; seq_lens / prefix_lens: [N] or None;
    S0: [N, H, dv, dk] or None.  pairs: optional list of (n, h) to run (others
    are left zero).  Returns dict(o [T, H, dv] with zero padding rows,
    S [N, H, dv, dk]) and, when record, {(n, h): per-boundary record}."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    N = cu.size - 1
    T, H, dk = k.shape
    dv = v.shape[2]
    lens = (cu[1:] - cu[:-1]) if seq_lens is None else np.asarray(seq_lens, dtype=np.int64)
    pref = lens if prefix_lens is None else np.asarray(prefix_lens, dtype=np.int64)
    o = np.zeros((T, H, dv), dtype=np.float64)
    S = np.zeros((N, H, dv, dk), dtype=np.float64)
    if pairs is None:
        pairs = [(n, h) for n in range(N) for h in range(H)]
    recs = {}

    def run(nh):
        n, h = nh
        s0, L = int(cu[n]), int(lens[n])
        sl = slice(s0, s0 + L)
        gg = g[sl, h] if g.ndim == 2 else g[sl, h, :]
        r = gdn_sequence(q[sl, h, :], k[sl, h, :], v[sl, h, :], beta[sl, h], gg,
                         prefix_len=int(pref[n]), flags=flags,
                         S0=None if S0 is None else S0[n, h], record=record, grid_log2=grid_log2)
        return nh, sl, r

    if threads > 1:
        with ThreadPoolExecutor(threads) as ex:
            results = list(ex.map(run, pairs))
    else:
        results = [run(p) for p in pairs]
    for (n, h), sl, r in results:
        o[sl, h, :] = r["o"]
        S[n, h] = r["S"]
        if record:
            recs[(n, h)] = r
    out = {"o": o, "S": S}
    if record:
        out["records"] = recs
    return out
