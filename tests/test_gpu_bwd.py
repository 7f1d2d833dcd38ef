"""GPU parity of the backward state recurrence (gdn_chunk_bwd_dh) against the
oracle's reverse token recurrence (oracle/backward.py, pinned against exact
differences of the forward oracle), through the C ABI.

Gate: the gradient of every chunk's entering state, of the initial state
and of v within the bf16-input tolerance of G1 (rel-L2 <= 2e-3) of the fp64
oracle on the same (bf16-valued) inputs; measured errors are reported.
Padding rows filled with NaN change nothing; the value gradient's padding
rows are zero.
"""
import numpy as np
import pytest
import torch

from fp8_state_qat_amd import api
from fp8_state_qat_amd import inputs as gi
from fp8_state_qat_amd import _lib
from oracle.backward import chunked_state_grads, packed_state_grads, state_grads

from helpers import rel_l2

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _case(lens, H, dk, dv, seed, pads=None, pad_fill=None, per_channel=False):
    w = gi.make_packed(lens, H, dk, dv, io_dtype=gi.BF16, seed=seed, pads=pads, pad_fill=pad_fill,
                       per_channel=per_channel, g_scale=0.05 if per_channel else 0.1)
    rng = np.random.default_rng(seed + 1)
    do = gi._round_io(rng.standard_normal((w.total_tokens, H, dv)), gi.BF16)
    dS = rng.standard_normal((len(lens), H, dv, dk)).astype(np.float32)
    return w, do, dS


def _run(w, do, dS, want_dv=False, flags=0):
    d = gi.device_tensors(w)
    out = api.chunk_bwd_dh(d["q"], d["k"], d["beta"], d["g"], d["cu_seqlens"], gi.to_torch(do, "cuda"),
                           seq_lens=d["seq_lens"], d_final_state=torch.from_numpy(dS).cuda(), want_dv=want_dv,
                           qdq_flags=flags)
    torch.cuda.synchronize()
    return tuple(x.cpu().numpy() for x in out)


def _do_f64(do):
    return (gi.bf16_bits_to_f32(do) if do.dtype == np.uint16 else do).astype(np.float64)


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 256)])
def test_bwd_dh_against_oracle(dk, dv):
    """Ragged lengths: an empty sequence (its initial-state gradient is the
    final-state gradient), one token, chunk multiples and tails."""
    w, do, dS = _case([300, 0, 1, 64, 129], 2, dk, dv, seed=91 + dk + dv)
    dh, d0, dval = _run(w, do, dS, want_dv=True)
    ref_dh, ref_d0, ref_dv = packed_state_grads(w.f64("q"), w.f64("k"), w.f64("beta"), w.f64("g"), _do_f64(do),
                                                w.cu_seqlens, seq_lens=w.seq_lens, dS_L=dS)
    r1, r0, rv = rel_l2(dh, ref_dh), rel_l2(d0, ref_d0), rel_l2(dval, ref_dv)
    print(f"dk={dk} dv={dv}: dh rel={r1:.3e} d_initial rel={r0:.3e} d_v rel={rv:.3e}", flush=True)
    assert dh.shape == ref_dh.shape and dval.shape == ref_dv.shape
    assert r1 <= TOL and r0 <= TOL and rv <= TOL
    np.testing.assert_array_equal(d0[1], dS[1])


def test_bwd_dh_nan_padding_changes_nothing():
    lens, pads = [130, 5, 64], [3, 61, 0]
    w, do, dS = _case(lens, 2, 128, 128, seed=95, pads=pads, pad_fill=np.nan)
    valid = np.zeros(w.total_tokens, bool)
    for n in range(3):
        valid[w.cu_seqlens[n]:w.cu_seqlens[n] + w.seq_lens[n]] = True
    do_nan = do.copy()
    do_nan[~valid] = 0x7FC0  # bf16 NaN
    dh, d0, dval = _run(w, do_nan, dS, want_dv=True)
    assert np.all(np.isfinite(dh)) and np.all(np.isfinite(d0)) and np.all(np.isfinite(dval))
    ref_dh, ref_d0, ref_dv = packed_state_grads(np.nan_to_num(w.f64("q")), np.nan_to_num(w.f64("k")),
                                                np.nan_to_num(w.f64("beta")), np.nan_to_num(w.f64("g")),
                                                np.nan_to_num(_do_f64(do_nan)), w.cu_seqlens, seq_lens=w.seq_lens,
                                                dS_L=dS)
    assert rel_l2(dh, ref_dh) <= TOL and rel_l2(d0, ref_d0) <= TOL and rel_l2(dval, ref_dv) <= TOL
    assert np.all(dval[~valid] == 0)


def test_bwd_dh_full_size_sampled():
    """The GDN prefill shape (B=4, T=4096, H=16, d=128): the oracle on sampled
    (sequence, head) pairs, every chunk of each."""
    w, do, dS = _case([4096] * 4, 16, 128, 128, seed=97)
    dh, d0, dval = _run(w, do, dS, want_dv=True)
    q, k, b, g, dof = w.f64("q"), w.f64("k"), w.f64("beta"), w.f64("g"), _do_f64(do)
    for (n, h) in [(0, 0), (1, 7), (3, 15)]:
        sl = slice(4096 * n, 4096 * (n + 1))
        r_dh, r_0, r_v = state_grads(q[sl, h], k[sl, h], b[sl, h], g[sl, h], dof[sl, h], dS[n, h], want_dv=True)
        r1, r0, rv = rel_l2(dh[64 * n:64 * (n + 1), h], r_dh), rel_l2(d0[n, h], r_0), rel_l2(dval[sl, h], r_v)
        print(f"(n, h)=({n}, {h}): dh rel={r1:.3e} d_initial rel={r0:.3e} d_v rel={rv:.3e}", flush=True)
        assert r1 <= TOL and r0 <= TOL and rv <= TOL


def test_bwd_dh_many_workgroups_against_oracle():
    """192 dh workgroups (24 heads, 2 value tiles, uneven lengths): sampled
    pairs against the oracle."""
    w, do, dS = _case([300, 200, 64, 130], 24, 128, 128, seed=99)
    dh, d0 = _run(w, do, dS)
    q, k, b, g, dof = w.f64("q"), w.f64("k"), w.f64("beta"), w.f64("g"), _do_f64(do)
    offs = np.concatenate([[0], np.cumsum([(int(L) + 63) // 64 for L in w.seq_lens])])
    for (n, h) in [(0, 0), (1, 13), (3, 23)]:
        sl = slice(int(w.cu_seqlens[n]), int(w.cu_seqlens[n]) + int(w.seq_lens[n]))
        r_dh, r_0 = state_grads(q[sl, h], k[sl, h], b[sl, h], g[sl, h], dof[sl, h], dS[n, h])
        r1, r0 = rel_l2(dh[offs[n]:offs[n + 1], h], r_dh), rel_l2(d0[n, h], r_0)
        print(f"(n, h)=({n}, {h}): dh rel={r1:.3e} d_initial rel={r0:.3e}", flush=True)
        assert r1 <= TOL and r0 <= TOL


def test_bwd_without_dh_output_same_results():
    """dh NULL (no per-chunk state gradients stored): the initial state's
    gradient and d_v are bit-identical to the call that stores dh."""
    w, do, dS = _case([200, 64, 1], 2, 128, 128, seed=101)
    dh, d0, dval = _run(w, do, dS, want_dv=True)
    d = gi.device_tensors(w)
    _, d0_b, dv_b = api.chunk_bwd_dh(d["q"], d["k"], d["beta"], d["g"], d["cu_seqlens"], gi.to_torch(do, "cuda"),
                                     seq_lens=d["seq_lens"], d_final_state=torch.from_numpy(dS).cuda(),
                                     dh=torch.empty(0, device="cuda"), want_dv=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(d0_b.cpu().numpy(), d0)
    np.testing.assert_array_equal(dv_b.cpu().numpy(), dval)


def _forward_wq(w):
    """The W-QDQ forward's quantized W of every chunk ([n_bounds, H, 64, dk]
    fp32, debug w_post) and the chunk offsets."""
    d = gi.device_tensors(w)
    nb = [(int(L) + 63) // 64 for L in w.seq_lens]
    offs = np.concatenate([[0], np.cumsum(nb)]).astype(np.int32)
    wpost = torch.zeros((int(offs[-1]), w.n_heads, 64, w.dk), device="cuda")
    api.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["cu_seqlens"], seq_lens=d["seq_lens"],
                  qdq_flags=3 | _lib.GDN_QDQ_W,
                  debug=dict(bound_offsets=torch.from_numpy(offs).cuda(), w_post=wpost))
    torch.cuda.synchronize()
    return wpost.cpu().numpy(), offs


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 256)])
def test_bwd_dh_w_qdq_against_oracle(dk, dv):
    """The backward of a W-QDQ forward (identity straight-through rule on the
    W quantizer): the state term takes the forward's quantized W.  The
    oracle's chunk-level backward (pinned by exact differences of the W-QDQ
    forward oracle) runs with the GPU forward's own quantized W (teacher
    forcing, so a W code that rounds the other way at a tie does not count):
    dh, the initial-state gradient and d_v within 1e-4 (the measured error
    is about 1e-6; W QDQ itself moves the gradient by about 3e-3, so a
    backward that used the unquantized W fails).  Free-running (the oracle
    quantizes its own W) within the bf16 gate.  Ragged lengths, an empty
    sequence, one token."""
    w, do, dS = _case([300, 0, 1, 64, 129], 2, dk, dv, seed=131 + dk + dv)
    dh, d0, dval = _run(w, do, dS, want_dv=True, flags=3 | _lib.GDN_QDQ_W)
    wq, offs = _forward_wq(w)
    q, k, b, g, dof = w.f64("q"), w.f64("k"), w.f64("beta"), w.f64("g"), _do_f64(do)
    ref_dh, ref_d0, ref_dv = np.zeros_like(dh), np.zeros_like(d0), np.zeros_like(dval)
    own_dh = np.zeros_like(dh)
    for n in range(len(w.seq_lens)):
        s0, L = int(w.cu_seqlens[n]), int(w.seq_lens[n])
        sl = slice(s0, s0 + L)
        for h in range(w.n_heads):
            r_dh, r_0, r_v = chunked_state_grads(q[sl, h], k[sl, h], b[sl, h], g[sl, h], dof[sl, h], dS[n, h],
                                                 w_qdq=True, want_dv=True, Wq=wq[offs[n]:offs[n + 1], h])
            ref_dh[offs[n]:offs[n + 1], h], ref_d0[n, h], ref_dv[sl, h] = r_dh, r_0, r_v
            own_dh[offs[n]:offs[n + 1], h] = chunked_state_grads(q[sl, h], k[sl, h], b[sl, h], g[sl, h],
                                                                 dof[sl, h], dS[n, h], w_qdq=True)[0]
    r1, r0, rv = rel_l2(dh, ref_dh), rel_l2(d0, ref_d0), rel_l2(dval, ref_dv)
    plain, _ = packed_state_grads(q, k, b, g, dof, w.cu_seqlens, seq_lens=w.seq_lens, dS_L=dS)[:2]
    print(f"dk={dk} dv={dv} W QDQ: teacher-forced dh rel={r1:.3e} d_initial rel={r0:.3e} d_v rel={rv:.3e}; "
          f"free-running dh rel={rel_l2(dh, own_dh):.3e}; against the plain backward {rel_l2(dh, plain):.3e}",
          flush=True)
    assert r1 <= 1e-4 and r0 <= 1e-4 and rv <= 1e-4
    assert rel_l2(dh, own_dh) <= TOL
    assert rel_l2(dh, plain) > 10 * r1
    np.testing.assert_array_equal(d0[1], dS[1])


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 256)])
def test_bwd_per_channel_gate_against_oracle(dk, dv):
    """The per-key-channel gate's backward (the reverse token recurrence on
    the GPU): dh of every chunk, the initial-state gradient and d_v against
    the oracle's token backward (pinned by exact differences of the forward
    oracle with the per-channel gate).  fp32 arithmetic on bf16-valued
    inputs, so within the fp32 gate of 1e-5 (measured: about 1e-7); ragged lengths,
    an empty sequence, one token; padding rows of d_v zero."""
    w, do, dS = _case([300, 0, 1, 64, 129], 2, dk, dv, seed=151 + dk + dv, per_channel=True)
    dh, d0, dval = _run(w, do, dS, want_dv=True)
    ref_dh, ref_d0, ref_dv = packed_state_grads(w.f64("q"), w.f64("k"), w.f64("beta"), w.f64("g"), _do_f64(do),
                                                w.cu_seqlens, seq_lens=w.seq_lens, dS_L=dS)
    r1, r0, rv = rel_l2(dh, ref_dh), rel_l2(d0, ref_d0), rel_l2(dval, ref_dv)
    print(f"per-channel dk={dk} dv={dv}: dh rel={r1:.3e} d_initial rel={r0:.3e} d_v rel={rv:.3e}", flush=True)
    assert dh.shape == ref_dh.shape and dval.shape == ref_dv.shape
    assert r1 <= 1e-5 and r0 <= 1e-5 and rv <= 1e-5
    np.testing.assert_array_equal(d0[1], dS[1])


def test_bwd_per_channel_gate_nan_padding_changes_nothing():
    """Per-channel gate: NaN in every padding row of q, k, v, beta, g and d_o
    changes no gradient, and d_v's padding rows are zero."""
    lens, pads = [130, 5, 64], [3, 61, 0]
    w, do, dS = _case(lens, 2, 128, 128, seed=157, pads=pads, per_channel=True)
    wn, _, _ = _case(lens, 2, 128, 128, seed=157, pads=pads, pad_fill=np.nan, per_channel=True)
    valid = np.zeros(w.total_tokens, bool)
    for n in range(3):
        valid[w.cu_seqlens[n]:w.cu_seqlens[n] + w.seq_lens[n]] = True
    don = do.copy()
    don[~valid] = gi._round_io(np.full(don[~valid].shape, np.nan), gi.BF16)
    a = _run(w, do, dS, want_dv=True)
    b = _run(wn, don, dS, want_dv=True)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    assert np.all(b[2][~valid] == 0)
