"""The torch binding checks every tensor's dtype and exact shape against the
call's contract before anything reaches the library (the kernels trust the
sizes they are given, so a wrong size would become an out-of-bounds device
access).  These run on CPU tensors: the shape checks come before the check
that the tensors live on the device."""
import pytest
import torch

from fp8_state_qat_amd import api

T, H, DK, DV, N = 100, 2, 64, 128, 2


def _chunk_args(**over):
    a = dict(q=torch.zeros(T, H, DK, dtype=torch.bfloat16), k=torch.zeros(T, H, DK, dtype=torch.bfloat16),
             v=torch.zeros(T, H, DV, dtype=torch.bfloat16), beta=torch.zeros(T, H), g=torch.zeros(T, H),
             cu_seqlens=torch.tensor([0, 40, 100], dtype=torch.int32))
    a.update(over)
    return a


def _chunk(kw=None, **over):
    a = _chunk_args(**over)
    return api.chunk_fwd(a.pop("q"), a.pop("k"), a.pop("v"), a.pop("beta"), a.pop("g"), a.pop("cu_seqlens"),
                         **(kw or {}))


def test_chunk_fwd_valid_shapes_reach_the_device_check():
    with pytest.raises(ValueError, match="device tensor"):
        _chunk()
    with pytest.raises(ValueError, match="device tensor"):
        _chunk(g=torch.zeros(T, H, DK))   # per-key-channel gate


@pytest.mark.parametrize("over,kw,what", [
    (dict(q=torch.zeros(T, H, DK + 1, dtype=torch.bfloat16)), {}, "q"),
    (dict(v=torch.zeros(T + 1, H, DV, dtype=torch.bfloat16)), {}, "v"),
    (dict(beta=torch.zeros(T, H + 1)), {}, "beta"),
    (dict(beta=torch.zeros(T, H, dtype=torch.float64)), {}, "beta"),
    (dict(g=torch.zeros(T, H, DK + 2)), {}, "g"),
    (dict(cu_seqlens=torch.tensor([0, 40, 100], dtype=torch.int64)), {}, "cu_seqlens"),
    ({}, dict(seq_lens=torch.zeros(N + 1, dtype=torch.int32)), "seq_lens"),
    ({}, dict(prefix_lens=torch.zeros(N, dtype=torch.int64)), "prefix_lens"),
    ({}, dict(initial_state=torch.zeros(N, H, DK, DV)), "initial_state"),
    ({}, dict(out=torch.zeros(T, H, DV, dtype=torch.float32), o_dtype=torch.bfloat16), "out"),
    ({}, dict(out=torch.zeros(T, H, DV, dtype=torch.float64)), "o_dtype"),
    ({}, dict(out=torch.zeros(T, H, DV - 64, dtype=torch.bfloat16)), "out"),
    ({}, dict(final_state=torch.zeros(N, H, DV, DK + 1)), "final_state"),
    ({}, dict(final_state=torch.zeros(N + 1, H, DV, DK)), "final_state"),
])
def test_chunk_fwd_rejects_wrong_shapes(over, kw, what):
    with pytest.raises(ValueError, match=what):
        _chunk(kw, **over)


def test_chunk_fwd_rejects_non_contiguous():
    q = torch.zeros(T, DK, H, dtype=torch.bfloat16).transpose(1, 2)
    with pytest.raises(ValueError, match="contiguous"):
        _chunk(q=q)


def _dec_args(**over):
    a = dict(q=torch.zeros(N, H, DK), k=torch.zeros(N, H, DK), v=torch.zeros(N, H, DV),
             beta=torch.zeros(N, H), g=torch.zeros(N, H), state=torch.zeros(N, H, DV, DK))
    a.update(over)
    return a


def _dec(kw=None, **over):
    a = _dec_args(**over)
    return api.decode_step(a.pop("q"), a.pop("k"), a.pop("v"), a.pop("beta"), a.pop("g"), a.pop("state"),
                           **(kw or {}))


def test_decode_valid_shapes_reach_the_device_check():
    with pytest.raises(ValueError, match="device tensor"):
        _dec()
    with pytest.raises(ValueError, match="device tensor"):
        _dec(dict(int8=True, scales=torch.zeros(N, H, DV, DK // 32)))
    with pytest.raises(ValueError, match="device tensor"):
        _dec(dict(scales=torch.zeros(N, H, DV // 64), active=torch.ones(N, dtype=torch.int32)))


@pytest.mark.parametrize("over,kw,what", [
    (dict(state=torch.zeros(N, H, DV, DK + 4)), {}, "state"),
    (dict(q=torch.zeros(N, H, DK - 1)), {}, "q"),
    (dict(g=torch.zeros(N, H, DK - 1)), {}, "g"),
    ({}, dict(state_pre=torch.zeros(N, H, DV // 2, DK)), "state_pre"),
    # FP8 per-tile scales handed to the INT8 codec (128x too few elements)
    ({}, dict(int8=True, scales=torch.zeros(N, H, DV // 64)), "scales"),
    ({}, dict(scales=torch.zeros(N, H, DV, DK // 32)), "scales"),
    ({}, dict(active=torch.ones(N + 1, dtype=torch.int32)), "active"),
    ({}, dict(active=torch.ones(N, dtype=torch.int64)), "active"),
    ({}, dict(o=torch.zeros(N, H, DV + 1)), "o"),
])
def test_decode_rejects_wrong_shapes(over, kw, what):
    with pytest.raises(ValueError, match=what):
        _dec(kw, **over)


def test_state_qdq_rejects_wrong_shapes():
    x = torch.zeros(3, 128, 64)
    with pytest.raises(ValueError, match="out"):
        api.state_qdq(x, out=torch.zeros(3, 128, 32))
    with pytest.raises(ValueError, match="scales"):
        api.state_qdq(x, scales=torch.zeros(3, 1))
    with pytest.raises(ValueError, match="scales"):
        api.state_qdq_int8(x, scales=torch.zeros(3, 2))
    with pytest.raises(ValueError, match="device tensor"):
        api.state_qdq(x)


def test_bwd_rejects_wrong_shapes():
    q = torch.zeros(T, H, DK, dtype=torch.bfloat16)
    d_o = torch.zeros(T, H, DV, dtype=torch.bfloat16)
    cu = torch.tensor([0, 40, 100], dtype=torch.int32)
    with pytest.raises(ValueError, match="beta"):
        api.chunk_bwd_dh(q, q, torch.zeros(T, H + 1), torch.zeros(T, H), cu, d_o)
    with pytest.raises(ValueError, match="d_final_state"):
        api.chunk_bwd_dh(q, q, torch.zeros(T, H), torch.zeros(T, H), cu, d_o,
                         d_final_state=torch.zeros(N, H, DK, DV))
    with pytest.raises(ValueError, match="d_v"):
        api.chunk_bwd_dh(q, q, torch.zeros(T, H), torch.zeros(T, H), cu, d_o, d_v=torch.zeros(T, H, DK))
    with pytest.raises(ValueError, match="device tensor"):
        api.chunk_bwd_dh(q, q, torch.zeros(T, H), torch.zeros(T, H), cu, d_o)
