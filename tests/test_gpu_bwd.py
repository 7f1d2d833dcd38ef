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
from oracle.backward import packed_state_grads, state_grads

from helpers import rel_l2

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _case(lens, H, dk, dv, seed, pads=None, pad_fill=None):
    w = gi.make_packed(lens, H, dk, dv, io_dtype=gi.BF16, seed=seed, pads=pads, pad_fill=pad_fill)
    rng = np.random.default_rng(seed + 1)
    do = gi._round_io(rng.standard_normal((w.total_tokens, H, dv)), gi.BF16)
    dS = rng.standard_normal((len(lens), H, dv, dk)).astype(np.float32)
    return w, do, dS


def _run(w, do, dS, want_dv=False):
    d = gi.device_tensors(w)
    out = api.chunk_bwd_dh(d["q"], d["k"], d["beta"], d["g"], d["cu_seqlens"], gi.to_torch(do, "cuda"),
                           seq_lens=d["seq_lens"], d_final_state=torch.from_numpy(dS).cuda(), want_dv=want_dv)
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
