"""GPU parity of gdn_chunk_fwd with a per-key-channel gate (g [T, H, dk]:
KDA-style retention, decay on the key side of the state) against the
oracle, through the C ABI.  Same gates as the scalar-gate tests:

  G1  QDQ off, free-running: o and final state within 1e-5 (fp32 inputs) or
      2e-3 (bf16 inputs) rel-L2 of the oracle.
  G2  QDQ on, teacher-forced per boundary (the oracle restarts every chunk
      from the GPU's post-QDQ state; the GPU's post-QDQ state is the
      oracle's QDQ of the GPU's pre-QDQ state bit for bit).
"""
import numpy as np
import pytest

from fp8_state_qat_amd import inputs as gi

from helpers import (KDA_CODES, TOL, check_codes, check_g1, check_g2, check_prefix_suffix, rel_l2, run_chunk_gpu,
                     run_chunk_oracle, teacher_forced)

pytestmark = pytest.mark.gpu


def _kda(lens, H, dk, dv, io, seed, g_scale=0.05, **kw):
    return gi.make_packed(lens, H, dk, dv, io_dtype=io, per_channel=True, g_scale=g_scale,
                          seed=seed, **kw)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("lens", [[256], [200, 1, 64, 65, 130]])
def test_kda_fp32_qdq_off(lens, d):
    """fp32 inputs; at d = 128 the token-recurrence kernel (gdn_token.hip)."""
    w = _kda(lens, 2, d, d, gi.F32, seed=31 + len(lens) + d)
    check_g1(w, run_chunk_gpu(w, 0), run_chunk_oracle(w, 0), TOL[gi.F32])


@pytest.mark.parametrize("d", [64, 128])
def test_kda_fp32_qdq_on(d):
    """Teacher-forced per boundary, and free-running (fp32 compute keeps
    the code decisions of the oracle here)."""
    w = _kda([256, 100], 2, d, d, gi.F32, seed=37 + d)
    gpu = run_chunk_gpu(w, 3, record=True)
    check_g2(w, gpu, 3, TOL[gi.F32])
    ref = run_chunk_oracle(w, 3)
    o_rel, s_rel = rel_l2(gpu["o"], ref["o"]), rel_l2(gpu["S"], ref["S"])
    print(f"free-running QDQ on: o_rel={o_rel:.3e} S_rel={s_rel:.3e}", flush=True)
    assert o_rel <= 1e-5 and s_rel <= 1e-5


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("o_dtype", ["f32", "bf16"])
def test_kda_bf16_qdq_off(d, o_dtype):
    w = _kda([300, 129, 64], 2, d, d, gi.BF16, seed=41 + d)
    check_g1(w, run_chunk_gpu(w, 0, o_dtype=o_dtype), run_chunk_oracle(w, 0), TOL[gi.BF16])


@pytest.mark.parametrize("d,dv", [(128, 128), (64, 64), (128, 256), (64, 192)])
def test_kda_bf16_qdq_on_teacher_forced(d, dv):
    w = _kda([300, 129, 1], 2, d, dv, gi.BF16, seed=43 + d + dv)
    gpu = run_chunk_gpu(w, 3, o_dtype="f32", record=True)
    check_g2(w, gpu, 3, TOL[gi.BF16], codes=KDA_CODES)
    ref = run_chunk_oracle(w, 3)
    print(f"free-running QDQ on (reported): o_rel={rel_l2(gpu['o'], ref['o']):.3e} "
          f"S_rel={rel_l2(gpu['S'], ref['S']):.3e}", flush=True)


def test_kda_strong_gates_fp32():
    """Gates up to several units per token (decay factors down to ~1e-5 per
    token, cumulative products far below the fp32 range inside a chunk): no
    overflow, no NaN, and G1 still holds, since every exponential is taken of
    a non-positive difference."""
    w = _kda([200, 64], 2, 64, 64, gi.F32, seed=47, g_scale=4.0)
    gpu = run_chunk_gpu(w, 0)
    assert np.all(np.isfinite(gpu["o"])) and np.all(np.isfinite(gpu["S"]))
    check_g1(w, gpu, run_chunk_oracle(w, 0), TOL[gi.F32])


def test_kda_in_block_decay_beyond_guard_fp32():
    """Gates of ~-6 per token: the decay across one 16-token block passes the
    prep kernel's guard band, so its diagonal tiles take the per-channel path
    (exponentials of differences only) while the off-diagonal tiles stay on
    the scaled-operand MFMA path."""
    w = _kda([192, 77], 2, 64, 64, gi.F32, seed=71, g_scale=8.0)
    gpu = run_chunk_gpu(w, 0)
    assert np.all(np.isfinite(gpu["o"])) and np.all(np.isfinite(gpu["S"]))
    check_g1(w, gpu, run_chunk_oracle(w, 0), TOL[gi.F32])
    wb = _kda([192, 77], 2, 128, 128, gi.BF16, seed=73, g_scale=8.0)
    check_g1(wb, run_chunk_gpu(wb, 0, o_dtype="f32"), run_chunk_oracle(wb, 0), TOL[gi.BF16])


def test_kda_varlen_padding_is_isolated():
    w = _kda([70, 0, 5, 130, 64], 2, 128, 128, gi.BF16, seed=53, pads=[3, 4, 0, 61, 1],
             pad_fill=np.nan)
    gpu = run_chunk_gpu(w, 0, o_dtype="f32")
    assert np.all(np.isfinite(gpu["o"])) and np.all(np.isfinite(gpu["S"]))
    check_g1(w, gpu, run_chunk_oracle(w, 0), TOL[gi.BF16])
    assert np.all(gpu["S"][1] == 0)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("flags", [1, 2, 3])
def test_kda_prefix_suffix_fp32(flags, d):
    """Chunked prefix P, then the recurrent suffix up to L with the
    per-channel decay, under the three QDQ placements."""
    w = _kda([150, 70, 9], 2, d, d, gi.F32, seed=59 + flags + d, prefix_lens=[128, 33, 0])
    gpu = run_chunk_gpu(w, flags, record=True, suffix_record=True)
    check_prefix_suffix(w, gpu, flags, TOL[gi.F32])


@pytest.mark.parametrize("flags", [2, 3])
def test_kda_prefix_suffix_bf16(flags):
    """bf16, d=128: the per-channel decay through the prefix/suffix split,
    both teacher-forced (per boundary, per suffix token)."""
    w = _kda([200, 100, 45], 2, 128, 128, gi.BF16, seed=67 + flags, prefix_lens=[130, 64, 0])
    gpu = run_chunk_gpu(w, flags, o_dtype="f32", record=True, suffix_record=True)
    check_prefix_suffix(w, gpu, flags, TOL[gi.BF16], codes=KDA_CODES)


def test_kda_prefix_suffix_log_grid_fp32():
    """Log-retention grid (#2509) with the per-channel gate: every key
    channel's log-gate of a recurrent suffix token rounded to a multiple of
    2^-3; prefix and suffix teacher-forced against the oracle's grid reading."""
    w = _kda([150, 70, 9], 2, 64, 64, gi.F32, seed=71, prefix_lens=[128, 33, 0])
    gpu = run_chunk_gpu(w, 3, record=True, suffix_record=True, grid_log2=3)
    check_prefix_suffix(w, gpu, 3, TOL[gi.F32], grid_log2=3)


def test_kda_initial_state_fp32():
    w = _kda([130, 64], 2, 64, 64, gi.F32, seed=61)
    rng = np.random.default_rng(61)
    S0 = (rng.standard_normal((2, 2, 64, 64)) * 0.5).astype(np.float32)
    gpu = run_chunk_gpu(w, 3, record=True, initial_state=S0)
    check_g2(w, gpu, 3, TOL[gi.F32], initial_state=S0)
    gpu0 = run_chunk_gpu(w, 0, initial_state=S0)
    check_g1(w, gpu0, run_chunk_oracle(w, 0, initial_state=S0), TOL[gi.F32])


def test_kda_deterministic():
    w = _kda([257, 64], 3, 128, 128, gi.BF16, seed=67)
    r1 = run_chunk_gpu(w, 3)
    r2 = run_chunk_gpu(w, 3)
    np.testing.assert_array_equal(r1["o"], r2["o"])
    np.testing.assert_array_equal(r1["S"], r2["S"])


@pytest.mark.parametrize("flags", [0, 3])
def test_full_size_kda_prefill_sampled(flags):
    """The full per-channel-gate workload (B=4, T=4096, H=16, d=128, bf16, g
    [T, H, dk]) in the launch configuration the benchmark times; sampled
    (sequence, head) pairs against the oracle."""
    w = gi.kda_prefill()
    gpu = run_chunk_gpu(w, flags, o_dtype="bf16", record=(flags != 0))
    pairs = [(0, 0), (2, 9), (3, 15)]
    if flags == 0:
        ref = run_chunk_oracle(w, 0, pairs=pairs)
        for (n, h) in pairs:
            sl = slice(int(w.cu_seqlens[n]), int(w.cu_seqlens[n + 1]))
            o_rel = rel_l2(gpu["o"][sl, h], ref["o"][sl, h])
            s_rel = rel_l2(gpu["S"][n, h], ref["S"][n, h])
            print(f"pair {(n, h)} o_rel={o_rel:.3e} S_rel={s_rel:.3e}", flush=True)
            assert o_rel <= TOL[gi.BF16] and s_rel <= TOL[gi.BF16]
    else:
        r = teacher_forced(w, gpu, flags, pairs)
        print("G2 sampled", r, flush=True)
        assert r["o_rel"] <= TOL[gi.BF16] and r["pre_rel"] <= TOL[gi.BF16]
        assert r["gpu_code_mismatch"] == 0 and r["scale_mismatch"] == 0
        check_codes(r, **KDA_CODES)
