"""Regression test for a fixed GPU memory fault: the kernels' direct
global->LDS loads take a 64-bit scalar base that is broadcast from one lane
in two 32-bit halves, and a half widened with sign extension turned every
buffer whose address had bit 31 set into a wild address.  Whether a buffer
gets such an address depends on the allocator, so this test places every
buffer of the call there on purpose: q, k, v, o, the states, the workspace
(whose records are read by the same loads) and the backward's inputs, all
carved out of one allocation at addresses with bit 31 set.  The results are
compared bit for bit with the same calls on ordinary buffers."""
import numpy as np
import pytest
import torch

from fp8_state_qat_amd import api
from fp8_state_qat_amd import inputs as gi

pytestmark = pytest.mark.gpu

BIT31 = 1 << 31
WINDOW = 1 << 32


class Carver:
    """Sub-buffers of one device allocation, each 256-byte aligned, all at
    addresses whose bit 31 is set (checked)."""

    def __init__(self, need):
        self.buf = torch.empty(BIT31 + 2 * need + 4096, dtype=torch.uint8, device="cuda")
        base = self.buf.data_ptr()
        off = base % WINDOW
        if off >= BIT31 and off + need <= WINDOW:
            start = base
        elif off < BIT31:
            start = base + (BIT31 - off)
        else:
            start = base + (WINDOW - off) + BIT31
        self.pos = start - base
        self.end = self.pos + need
        assert self.end <= self.buf.numel()

    def take(self, shape, dtype):
        n = int(np.prod(shape)) * torch.empty(0, dtype=dtype).element_size()
        self.pos = (self.pos + 255) // 256 * 256
        assert self.pos + n <= self.end
        t = self.buf[self.pos:self.pos + n].view(dtype).view(shape)
        self.pos += n
        assert t.data_ptr() & BIT31 and (t.data_ptr() + n - 1) & BIT31
        return t

    def copy(self, src):
        t = self.take(tuple(src.shape), src.dtype)
        t.copy_(src)
        return t


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


@pytest.mark.parametrize("per_channel", [False, True])
def test_buffers_with_address_bit31_set(per_channel):
    w = gi.make_packed([300, 129, 64], 2, 128, 128, io_dtype=gi.BF16, per_channel=per_channel,
                       g_scale=0.05 if per_channel else 0.1, seed=101)
    d = gi.device_tensors(w)
    T, H, dk, dv, N = w.total_tokens, 2, 128, 128, 3
    ws_bytes = api.chunk_workspace_bytes(N, H, dk, dv, T, qdq_flags=3)
    c = Carver(ws_bytes + 64 * T * H * dk + 4 * 8 * N * H * dv * dk + (1 << 20))
    hi = {k: c.copy(d[k]) for k in ("q", "k", "v", "beta", "g", "cu_seqlens")}
    o_hi = c.take((T, H, dv), torch.bfloat16)
    S_hi = c.take((N, H, dv, dk), torch.float32)
    ws_hi = c.take((ws_bytes,), torch.uint8)
    print(f"q at {hi['q'].data_ptr():#x}, workspace at {ws_hi.data_ptr():#x}", flush=True)
    for flags in (0, 3):
        ref_o, ref_S = api.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["cu_seqlens"],
                                     qdq_flags=flags, check_status=True)
        api.chunk_fwd(hi["q"], hi["k"], hi["v"], hi["beta"], hi["g"], hi["cu_seqlens"], qdq_flags=flags,
                      out=o_hi, final_state=S_hi, workspace=ws_hi, check_status=True)
        torch.cuda.synchronize()
        assert torch.equal(_bits(o_hi), _bits(ref_o)) and torch.equal(_bits(S_hi), _bits(ref_S))
    if not per_channel:   # the backward's direct loads (q, k, dO and its records)
        d_o = c.copy(torch.randn((T, H, dv), device="cuda").to(torch.bfloat16))
        bws = c.take((api_bwd_bytes(N, H, dk, dv, T),), torch.uint8)
        d0_hi = c.take((N, H, dv, dk), torch.float32)
        dv_hi = c.take((T, H, dv), torch.float32)
        ref_d0, ref_dv = api.chunk_bwd_dh(d["q"], d["k"], d["beta"], d["g"], d["cu_seqlens"], d_o.clone(),
                                          want_dv=True)[1:]
        api.chunk_bwd_dh(hi["q"], hi["k"], hi["beta"], hi["g"], hi["cu_seqlens"], d_o, d_initial_state=d0_hi,
                         d_v=dv_hi, workspace=bws, check_status=True)
        torch.cuda.synchronize()
        assert torch.equal(_bits(d0_hi), _bits(ref_d0)) and torch.equal(_bits(dv_hi), _bits(ref_dv))


def api_bwd_bytes(N, H, dk, dv, T):
    import ctypes
    from fp8_state_qat_amd import _lib
    shape = _lib.GdnShape(N, H, dk, dv, T, _lib.GDN_BF16, _lib.GDN_BF16, 0, 0)
    return _lib.lib().gdn_chunk_bwd_workspace_bytes(ctypes.byref(shape))
