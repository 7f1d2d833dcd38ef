"""Seeded synthetic inputs for the gated delta rule workloads.

This module holds none of the method's arithmetic.  It draws random numbers
with numpy's PCG64, applies the input recipe of each workload (L2
normalisation of q and k per token and head, beta = sigmoid, log-gate =
-softplus * scale), rounds to the I/O dtype, and packs sequences.  Both the
HIP library's callers and the CPU oracle's callers take their inputs from
here; the random numbers are inputs, never drawn inside the method.

Rounding recipe: values are drawn and transformed in fp64, rounded to fp32
(round to nearest even), and for bf16 I/O rounded again from fp32 to bf16
(round to nearest even).  bf16 arrays are held as their uint16 bit patterns.
Draw order per workload: sequence lengths, padding counts, q, k, v, beta, g.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

F32 = "f32"
BF16 = "bf16"


def f32_to_bf16_bits(x) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _softplus(x):
    return np.logaddexp(0.0, x)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


@dataclass
class Workload:
    """Packed varlen inputs.  q, k: [T, H, dk]; v: [T, H, dv] (float32, or
    uint16 bf16 bits); beta: [T, H] fp32; g: [T, H] or [T, H, dk] fp32;
    cu_seqlens: [N+1] storage boundaries; seq_lens / prefix_lens: [N]."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    beta: np.ndarray
    g: np.ndarray
    cu_seqlens: np.ndarray
    seq_lens: np.ndarray
    prefix_lens: np.ndarray
    io_dtype: str
    n_heads: int
    dk: int
    dv: int
    meta: dict = field(default_factory=dict)

    @property
    def n_seqs(self) -> int:
        return int(self.cu_seqlens.size - 1)

    @property
    def total_tokens(self) -> int:
        return int(self.k.shape[0])

    @property
    def per_channel(self) -> bool:
        return self.g.ndim == 3

    def f64(self, name: str) -> np.ndarray:
        """Exact values of an input array as float64."""
        a = getattr(self, name)
        if a.dtype == np.uint16:
            return bf16_bits_to_f32(a).astype(np.float64)
        return a.astype(np.float64)


def _round_io(x64: np.ndarray, io_dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    if io_dtype == BF16:
        return f32_to_bf16_bits(x32)
    if io_dtype == F32:
        return x32
    raise ValueError(io_dtype)


def _l2n(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def make_packed(seq_lens, n_heads, dk, dv, *, io_dtype=BF16, per_channel=False,
                g_scale=0.1, pads=None, prefix_lens=None, seed=0, rng=None,
                pad_fill=None) -> Workload:
    """Pack sequences of the given valid lengths, each followed by pads[i]
    padding rows, into one buffer.  pad_fill=None draws padding rows like the
    rest; a float (e.g. nan) fills them with that value instead."""
    rng = np.random.Generator(np.random.PCG64(seed)) if rng is None else rng
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    N = seq_lens.size
    pads = np.zeros(N, dtype=np.int64) if pads is None else np.asarray(pads, dtype=np.int64)
    seg = seq_lens + pads
    cu = np.zeros(N + 1, dtype=np.int64)
    cu[1:] = np.cumsum(seg)
    T = int(cu[-1])
    H = n_heads
    q = _l2n(rng.standard_normal((T, H, dk)))
    k = _l2n(rng.standard_normal((T, H, dk)))
    v = rng.standard_normal((T, H, dv))
    beta = _sigmoid(rng.standard_normal((T, H)))
    gshape = (T, H, dk) if per_channel else (T, H)
    g = -_softplus(rng.standard_normal(gshape)) * g_scale
    if pad_fill is not None:
        for n in range(N):
            sl = slice(int(cu[n] + seq_lens[n]), int(cu[n + 1]))
            for a in (q, k, v, beta, g):
                a[sl] = pad_fill
    pl = seq_lens.copy() if prefix_lens is None else np.asarray(prefix_lens, dtype=np.int64)
    return Workload(q=_round_io(q, io_dtype), k=_round_io(k, io_dtype), v=_round_io(v, io_dtype),
                    beta=beta.astype(np.float32), g=g.astype(np.float32),
                    cu_seqlens=cu.astype(np.int32), seq_lens=seq_lens.astype(np.int32),
                    prefix_lens=pl.astype(np.int32), io_dtype=io_dtype, n_heads=H,
                    dk=dk, dv=dv)


# ---------------------------------------------------------------------------
# The five workloads of the measurement plan.
# ---------------------------------------------------------------------------
def tiny(seed=0) -> Workload:
    """B=1, T=256, H=2, dk=dv=64, fp32 I/O, scalar gate (scale 0.1)."""
    w = make_packed([256], 2, 64, 64, io_dtype=F32, seed=seed)
    w.meta["name"] = "tiny gdn prefill B=1 T=256 H=2 d=64 fp32"
    return w


def gdn_prefill(B=4, T=4096, H=16, d=128, io_dtype=BF16, seed=0) -> Workload:
    """B=4, T=4096, H=16, dk=dv=128, bf16 I/O (Qwen3-Next-like head shape)."""
    w = make_packed([T] * B, H, d, d, io_dtype=io_dtype, seed=seed)
    w.meta["name"] = f"gdn prefill B={B} T={T} H={H} d={d} {io_dtype}"
    return w


def varlen(n_seqs=16, max_len=8192, H=16, d=128, io_dtype=BF16, seed=0, pad_fill=None) -> Workload:
    """16 sequences, valid lengths uniform in [1, max_len], each followed by
    0..63 padding rows (uniform), H=16, dk=dv=128, bf16."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(1, max_len + 1, size=n_seqs)
    pads = rng.integers(0, 64, size=n_seqs)
    w = make_packed(lens, H, d, d, io_dtype=io_dtype, pads=pads, rng=rng, pad_fill=pad_fill)
    w.meta["name"] = f"packed varlen gdn prefill {n_seqs} seqs L~U[1,{max_len}] H={H} d={d} {io_dtype}"
    return w


def kda_prefill(B=4, T=4096, H=16, d=128, io_dtype=BF16, seed=0) -> Workload:
    """As gdn_prefill but with a per-key-channel log-gate (scale 0.05)."""
    w = make_packed([T] * B, H, d, d, io_dtype=io_dtype, per_channel=True, g_scale=0.05,
                    seed=seed)
    w.meta["name"] = f"kda prefill B={B} T={T} H={H} d={d} {io_dtype}"
    return w


def decode_tokens(n_seqs, H, dk, dv, steps, *, io_dtype=BF16, per_channel=False,
                  g_scale=0.1, rng=None, seed=0):
    """Fresh decode tokens from the same distributions: list of per-step
    dicts with q, k [N, H, dk], v [N, H, dv], beta [N, H], g [N, H](, dk)."""
    rng = np.random.Generator(np.random.PCG64(seed)) if rng is None else rng
    out = []
    for _ in range(steps):
        q = _l2n(rng.standard_normal((n_seqs, H, dk)))
        k = _l2n(rng.standard_normal((n_seqs, H, dk)))
        v = rng.standard_normal((n_seqs, H, dv))
        beta = _sigmoid(rng.standard_normal((n_seqs, H)))
        g = -_softplus(rng.standard_normal((n_seqs, H, dk) if per_channel else (n_seqs, H))) * g_scale
        out.append(dict(q=_round_io(q, io_dtype), k=_round_io(k, io_dtype),
                        v=_round_io(v, io_dtype), beta=beta.astype(np.float32),
                        g=g.astype(np.float32)))
    return out


def to_torch(a, device):
    """numpy input array -> torch tensor on device (uint16 bf16 bits become
    torch.bfloat16 without any rounding)."""
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def device_tensors(w: Workload, device="cuda"):
    """All inputs of a workload as device tensors (dict)."""
    return {name: to_torch(getattr(w, name), device)
            for name in ("q", "k", "v", "beta", "g", "cu_seqlens", "seq_lens", "prefix_lens")}


def device_packed(seq_lens, n_heads, dk, dv, *, io_dtype=BF16, per_channel=False, g_scale=0.1,
                  seed=0, device="cuda"):
    """Same distributions as make_packed, drawn on the device with torch's
    seeded Philox generator (for workloads too large to draw on the host).
    Transforms run in fp32 on the device, then round to the I/O dtype.
    Returns a dict of device tensors (q, k, v, beta, g, cu_seqlens)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    lens = torch.as_tensor(np.asarray(seq_lens, np.int64))
    T = int(lens.sum())
    H = n_heads
    dt = torch.bfloat16 if io_dtype == BF16 else torch.float32

    def unit(d):
        x = torch.randn((T, H, d), generator=gen, device=device, dtype=torch.float32)
        x /= torch.linalg.vector_norm(x, dim=-1, keepdim=True)
        return x.to(dt)

    q = unit(dk)
    k = unit(dk)
    v = torch.randn((T, H, dv), generator=gen, device=device, dtype=torch.float32).to(dt)
    beta = torch.sigmoid(torch.randn((T, H), generator=gen, device=device))
    gshape = (T, H, dk) if per_channel else (T, H)
    g = -torch.nn.functional.softplus(torch.randn(gshape, generator=gen, device=device)) * g_scale
    cu = torch.zeros(lens.numel() + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(lens, 0).to(torch.int32)
    return dict(q=q, k=k, v=v, beta=beta.contiguous(), g=g.contiguous(), cu_seqlens=cu.to(device))


def device_decode_tokens(n_seqs, n_heads, dk, dv, steps, *, io_dtype=BF16, per_channel=False,
                         g_scale=0.1, seed=1, device="cuda"):
    """Decode tokens for `steps` steps drawn on the device: dict of tensors
    with a leading step axis (q, k [steps, N, H, dk], v, beta, g)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    dt = torch.bfloat16 if io_dtype == BF16 else torch.float32
    shp = (steps, n_seqs, n_heads)

    def unit(d):
        x = torch.randn(shp + (d,), generator=gen, device=device)
        x /= torch.linalg.vector_norm(x, dim=-1, keepdim=True)
        return x.to(dt)

    q = unit(dk)
    k = unit(dk)
    v = torch.randn(shp + (dv,), generator=gen, device=device).to(dt)
    beta = torch.sigmoid(torch.randn(shp, generator=gen, device=device))
    g = -torch.nn.functional.softplus(
        torch.randn(shp + ((dk,) if per_channel else ()), generator=gen, device=device)) * g_scale
    return dict(q=q, k=k, v=v, beta=beta, g=g)
