"""gdn_chunk_fwd_noalloc (the variant for callers that cannot allocate: its
workspace is the library's static per-GPU scratch) against gdn_chunk_fwd
with a caller workspace, through the C ABI: two calls in a row, the second
with a smaller input (the scratch keeps the first call's contents), then a
W-QDQ call; outputs and final states bit for bit, the status word clean.
A shape beyond the scratch is refused."""
import numpy as np
import pytest
import torch

from fp8_state_qat_amd import _lib, api
from fp8_state_qat_amd import inputs as gi

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _pair(w, flags, o_dtype):
    d = gi.device_tensors(w)
    T, H, dv, dk, N = w.total_tokens, w.n_heads, w.dv, w.dk, w.n_seqs
    ref_o, ref_S = api.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["cu_seqlens"],
                                 seq_lens=d["seq_lens"], prefix_lens=d["prefix_lens"], qdq_flags=flags,
                                 o_dtype=o_dtype, check_status=True)
    o = torch.full((T, H, dv), 3.0, dtype=o_dtype, device="cuda")
    S = torch.full((N, H, dv, dk), 3.0, device="cuda")
    st = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    api.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["cu_seqlens"], seq_lens=d["seq_lens"],
                  prefix_lens=d["prefix_lens"], qdq_flags=flags, out=o, final_state=S, noalloc=True,
                  debug={"status": st})
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.isfinite(S).all()
    assert torch.equal(_bits(o), _bits(ref_o)), "o differs from gdn_chunk_fwd"
    assert torch.equal(_bits(S), _bits(ref_S)), "final state differs from gdn_chunk_fwd"


def test_noalloc_matches_chunk_fwd_two_calls():
    big = gi.make_packed([700, 300, 513], 4, 128, 128, io_dtype=gi.BF16, pads=[5, 0, 17], seed=211,
                         prefix_lens=[700, 257, 500])
    small = gi.make_packed([150, 64], 2, 128, 128, io_dtype=gi.BF16, seed=212)
    assert api.chunk_workspace_bytes(3, 4, 128, 128, big.total_tokens, qdq_flags=3) <= _lib.NOALLOC_SCRATCH_BYTES
    _pair(big, 3, torch.bfloat16)
    _pair(small, 3, torch.float32)
    _pair(gi.make_packed([200, 90], 2, 128, 128, io_dtype=gi.BF16, seed=213), 7, torch.bfloat16)


def test_noalloc_refuses_shapes_beyond_the_scratch():
    w = gi.gdn_prefill()
    d = gi.device_tensors(w)
    o = torch.empty((w.total_tokens, 16, 128), dtype=torch.bfloat16, device="cuda")
    S = torch.empty((4, 16, 128, 128), device="cuda")
    with pytest.raises(_lib.GdnError) as e:
        api.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["cu_seqlens"], out=o, final_state=S,
                      noalloc=True)
    assert e.value.status == _lib.GDN_ERR_UNSUPPORTED
