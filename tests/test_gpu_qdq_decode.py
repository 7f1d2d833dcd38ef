"""GPU parity of the standalone state QDQ and the decode step against the
oracle, through the C ABI."""
import numpy as np
import pytest
import torch

from fp8_state_qat_amd import api
from fp8_state_qat_amd import inputs as gi
from oracle import oracle as orc

from helpers import _code_fields, check_codes, code_mismatch_stats, np64, rel_l2

pytestmark = pytest.mark.gpu


def _states(rng, n, dv, dk, scale_spread=True):
    x = rng.standard_normal((n, dv, dk)).astype(np.float32)
    if scale_spread:
        x *= np.exp2(rng.uniform(-30, 30, (n, 1, 1))).astype(np.float32)
    return x


@pytest.mark.parametrize("dv,dk", [(64, 64), (128, 128), (192, 32), (64, 256), (256, 4)])
def test_state_qdq_bit_exact(dv, dk):
    """Every value and every scale equals the oracle's (same fp32 decision)."""
    rng = np.random.default_rng(dv * 1000 + dk)
    x = _states(rng, 37, dv, dk)
    x[3] = 0.0                       # zero tile -> scale 1
    x[5, :64] *= 0                   # one zero tile among non-zero tiles
    want, sc, _ = orc.qdq_states(x)
    xt = torch.from_numpy(x).cuda()
    out, scales = api.state_qdq(xt)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), want.view(np.uint32))
    np.testing.assert_array_equal(scales.cpu().numpy(), sc)


def test_state_qdq_many_scales_bit_exact():
    """4096 tiles, each with its own scale (random amax mantissa and
    exponent) and elements with random fp32 bit patterns below amax: the
    device QDQ (quotient by reciprocal plus correction steps, hardware E4M3
    rounding) equals the oracle's IEEE x / s decision bit for bit."""
    rng = np.random.default_rng(123)
    n = 4096
    amax = (rng.uniform(1.0, 2.0, n) * np.exp2(rng.integers(-40, 40, n))).astype(np.float32)
    mant = rng.integers(0, 1 << 23, size=(n, 64 * 128), dtype=np.uint32)
    expo = rng.integers(0, 40, size=(n, 64 * 128), dtype=np.uint32)
    top = amax.view(np.uint32) >> 23
    e = np.clip(top[:, None].astype(np.int64) - expo.astype(np.int64), 1, 254).astype(np.uint32)
    x = ((e << 23) | mant).view(np.float32)
    x = np.where(np.abs(x) > amax[:, None], amax[:, None], x)
    sign = rng.integers(0, 2, size=x.shape).astype(bool)
    x = np.where(sign, -x, x).astype(np.float32)
    x[:, 0] = amax
    x = x.reshape(n, 64, 128)
    want, sc, _ = orc.qdq_states(x)
    out, scales = api.state_qdq(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    bad = np.flatnonzero(got.view(np.uint32).ravel() != want.view(np.uint32).ravel())
    assert bad.size == 0, (bad.size, x.ravel()[bad[:4]], got.ravel()[bad[:4]], want.ravel()[bad[:4]])
    np.testing.assert_array_equal(scales.cpu().numpy().ravel(), sc.ravel())


def test_state_qdq_subnormal_scale_ties_bit_exact():
    """Tiles whose amax / 448 is a subnormal fp32 number lying exactly on a
    rounding tie (amax = 7 (2k + 1) 2^-144, so amax / 448 = (k + 1/2) 2^-149):
    the device's scale and codes equal the oracle's IEEE division (ties to
    even) bit for bit."""
    rng = np.random.default_rng(77)
    n = 256
    k = rng.integers(0, 1 << 20, n)
    amax = (7.0 * (2 * k + 1) * 2.0 ** -144).astype(np.float32)
    assert np.all(amax.astype(np.float64) == 7.0 * (2 * k + 1) * 2.0 ** -144)
    x = (rng.uniform(-1.0, 1.0, size=(n, 64 * 128)) * amax[:, None].astype(np.float64)).astype(np.float32)
    x[:, 0] = amax
    x = x.reshape(n, 64, 128)
    want, sc, _ = orc.qdq_states(x)
    assert np.all(sc.ravel() == (amax / np.float32(448.0)))
    out, scales = api.state_qdq(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(scales.cpu().numpy().ravel().view(np.uint32), sc.ravel().view(np.uint32))
    got = out.cpu().numpy()
    bad = np.flatnonzero(got.view(np.uint32).ravel() != want.view(np.uint32).ravel())
    assert bad.size == 0, (bad.size, x.ravel()[bad[:4]], got.ravel()[bad[:4]], want.ravel()[bad[:4]])


def test_state_qdq_in_place_and_already_e4m3():
    rng = np.random.default_rng(1)
    grid = orc.e4m3_decode(np.arange(127, dtype=np.uint8))
    C = rng.choice(grid, size=(4, 128, 128)) * rng.choice([-1.0, 1.0], size=(4, 128, 128))
    C[:, 0, 0] = 448.0
    C[:, 64, 0] = -448.0
    X = (C * 2.0 ** -7).astype(np.float32)
    xt = torch.from_numpy(X).cuda()
    api.state_qdq(xt, out=xt, want_scales=False)   # in place
    torch.cuda.synchronize()
    np.testing.assert_array_equal(xt.cpu().numpy().view(np.uint32), X.view(np.uint32))


def _encode_threaded(vals, parts=8):
    from concurrent.futures import ThreadPoolExecutor
    chunks = np.array_split(vals, parts)
    with ThreadPoolExecutor(parts) as ex:
        return np.concatenate(list(ex.map(orc.e4m3_encode, chunks)))


def test_e4m3_rounding_exhaustive_on_device():
    """Every non-negative fp32 value up to 448 (and a strided sample of the
    negatives) goes through the device QDQ with scale exactly 1 (each tile
    holds 448 in its first slot); the result equals the oracle's E4M3
    rounding of that value."""
    table = orc.e4m3_decode(np.arange(256, dtype=np.uint8)).astype(np.float32)
    top = int(np.float32(448.0).view(np.uint32))
    per = 1 << 26
    dk = 128
    tile = 64 * dk
    for start in range(0, top + 1, per):
        n = min(per, top + 1 - start)
        vals = np.arange(start, start + n, dtype=np.uint32).view(np.float32)
        vals = np.concatenate([vals, -vals[::1021]])
        m = vals.size
        ntiles = -(-m // (tile - 1))
        buf = np.empty((ntiles, tile), np.float32)
        buf[:, 0] = 448.0
        padded = np.zeros(ntiles * (tile - 1), np.float32)
        padded[:m] = vals
        buf[:, 1:] = padded.reshape(ntiles, tile - 1)
        xt = torch.from_numpy(buf.reshape(ntiles, 64, dk)).cuda()
        out, scales = api.state_qdq(xt)
        torch.cuda.synchronize()
        assert torch.all(scales == 1.0)
        got = out.cpu().numpy().reshape(ntiles, tile)[:, 1:].reshape(-1)[:m]
        want = table[_encode_threaded(vals)]
        bad = np.flatnonzero(got.view(np.uint32) != want.view(np.uint32))
        assert bad.size == 0, (vals[bad[:5]], got[bad[:5]], want[bad[:5]])


def _decode_case(N, H, dk, dv, io, per_channel, steps, o_dtype, qdq, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    S0 = (rng.standard_normal((N, H, dv, dk)) * 0.3).astype(np.float32)
    if qdq:
        S0, _, _ = orc.qdq_states(S0)
    toks = gi.decode_tokens(N, H, dk, dv, steps, io_dtype=io, per_channel=per_channel,
                            g_scale=0.05 if per_channel else 0.1, rng=rng)
    return S0, toks


@pytest.mark.parametrize("dk,dv,io,pc,o_dt", [
    (128, 128, gi.BF16, False, torch.float32),
    (128, 128, gi.F32, False, torch.float32),
    (64, 192, gi.BF16, False, torch.float32),
    (128, 128, gi.BF16, True, torch.float32),
    (128, 128, gi.BF16, False, torch.bfloat16),
])
@pytest.mark.parametrize("qdq", [True, False])
def test_decode_step_teacher_forced(dk, dv, io, pc, o_dt, qdq):
    """Per step: o and the pre-QDQ state match the oracle's step from the
    same stored state; the stored state is the oracle's QDQ of the GPU's
    pre-QDQ state, bit for bit."""
    N, H, steps = 5, 3, 4
    S0, toks = _decode_case(N, H, dk, dv, io, pc, steps, o_dt, qdq, seed=dk + dv + pc)
    state = torch.from_numpy(S0).cuda()
    pre = torch.empty_like(state)
    scales = torch.empty((N, H, dv // 64), device="cuda")
    o_tol = 2e-3 if o_dt == torch.bfloat16 else 1e-5
    for t in range(steps):
        tk = toks[t]
        dev = {k_: gi.to_torch(a, "cuda") for k_, a in tk.items()}
        S_before = state.cpu().numpy().astype(np.float64)
        o = api.decode_step(dev["q"], dev["k"], dev["v"], dev["beta"], dev["g"], state, qdq=qdq,
                            o_dtype=o_dt, state_pre=pre, scales=scales)
        torch.cuda.synchronize()
        f64 = {k_: (gi.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)
               for k_, a in tk.items()}
        o_ref = np.zeros((N, H, dv))
        pre_ref = np.zeros((N, H, dv, dk))
        for n in range(N):
            for h in range(H):
                g = f64["g"][n, h] if not pc else f64["g"][n, h][None, :]
                r = orc.gdn_sequence(f64["q"][n, h][None], f64["k"][n, h][None],
                                     f64["v"][n, h][None], f64["beta"][n, h][None],
                                     np.atleast_1d(g) if not pc else g, prefix_len=0, flags=0,
                                     S0=S_before[n, h])
                o_ref[n, h] = r["o"][0]
                pre_ref[n, h] = r["S"]
        assert rel_l2(np64(o), o_ref) <= o_tol
        pre_np = pre.cpu().numpy()
        assert rel_l2(pre_np, pre_ref) <= 1e-6
        if qdq:
            want, sc, codes_gpu = orc.qdq_states(pre_np)
            np.testing.assert_array_equal(state.cpu().numpy().view(np.uint32), want.view(np.uint32))
            np.testing.assert_array_equal(scales.cpu().numpy(), sc)
            # the oracle's own codes on its own pre-QDQ state (G3)
            _, sc_o, codes_orc = orc.qdq_states(pre_ref.astype(np.float32))
            r = _code_fields()
            y = pre_ref / np.repeat(sc_o.astype(np.float64), 64, axis=-1)[..., None]
            code_mismatch_stats(r, codes_orc, codes_gpu, y)
            check_codes(r)
        else:
            np.testing.assert_array_equal(state.cpu().numpy(), pre_np)


@pytest.mark.parametrize("int8", [False, True])
def test_decode_active_mask(int8):
    """Sequences whose active flag is 0 are skipped: their state, o row and
    records keep their contents bit for bit; the active ones take the step
    exactly as in a call without a mask (bit-identical)."""
    N, H, dk, dv = 6, 3, 128, 128
    S0, toks = _decode_case(N, H, dk, dv, gi.BF16, False, 1, torch.float32, True, seed=97)
    dev = {k_: gi.to_torch(a, "cuda") for k_, a in toks[0].items()}
    active_np = np.array([1, 0, 1, 1, 0, 0], np.int32)
    sc_shape = (N, H, dv, dk // 32) if int8 else (N, H, dv // 64)
    ref_state = torch.from_numpy(S0).cuda()
    ref_pre = torch.full_like(ref_state, 3.0)
    ref_sc = torch.full(sc_shape, 3.0, device="cuda")
    ref_o = api.decode_step(dev["q"], dev["k"], dev["v"], dev["beta"], dev["g"], ref_state, qdq=True,
                            o_dtype=torch.float32, state_pre=ref_pre, scales=ref_sc, int8=int8)
    state = torch.from_numpy(S0).cuda()
    pre = torch.full_like(state, 3.0)
    sc = torch.full(sc_shape, 3.0, device="cuda")
    o = torch.full((N, H, dv), 5.0, device="cuda")
    api.decode_step(dev["q"], dev["k"], dev["v"], dev["beta"], dev["g"], state, qdq=True, o=o,
                    state_pre=pre, scales=sc, int8=int8, active=torch.from_numpy(active_np).cuda())
    torch.cuda.synchronize()
    on = torch.from_numpy(active_np.astype(bool)).cuda()
    bits = lambda t: t.view(torch.int32)  # noqa: E731
    assert torch.equal(bits(state[on]), bits(ref_state[on])) and torch.equal(bits(pre[on]), bits(ref_pre[on]))
    assert torch.equal(bits(o[on]), bits(ref_o[on])) and torch.equal(bits(sc[on]), bits(ref_sc[on]))
    off = ~on
    assert torch.equal(bits(state[off]), bits(torch.from_numpy(S0).cuda()[off]))
    assert bool((pre[off] == 3.0).all()) and bool((sc[off] == 3.0).all()) and bool((o[off] == 5.0).all())


@pytest.mark.parametrize("pc", [False, True])
@pytest.mark.parametrize("grid", [3, 8])
def test_decode_step_log_grid(pc, grid):
    """Log-retention grid (#2509): each decode token decays with its
    log-gate rounded to a multiple of 2^-grid.  Teacher-forced per step
    against the oracle's grid reading (o and the pre-QDQ state, the stored
    state bit for bit as the oracle's QDQ of the GPU's pre-QDQ state); grid 3
    is coarse enough that a kernel ignoring the grid fails the pre-QDQ gate."""
    N, H, dk, dv, steps = 4, 3, 128, 128, 3
    S0, toks = _decode_case(N, H, dk, dv, gi.BF16, pc, steps, torch.float32, True, seed=211 + grid + pc)
    state = torch.from_numpy(S0).cuda()
    pre = torch.empty_like(state)
    scales = torch.empty((N, H, dv // 64), device="cuda")
    for t in range(steps):
        tk = toks[t]
        dev = {k_: gi.to_torch(a, "cuda") for k_, a in tk.items()}
        S_before = state.cpu().numpy().astype(np.float64)
        o = api.decode_step(dev["q"], dev["k"], dev["v"], dev["beta"], dev["g"], state, qdq=True,
                            o_dtype=torch.float32, state_pre=pre, scales=scales, gate_grid_log2=grid)
        torch.cuda.synchronize()
        f64 = {k_: (gi.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)
               for k_, a in tk.items()}
        o_ref = np.zeros((N, H, dv))
        pre_ref = np.zeros((N, H, dv, dk))
        for n in range(N):
            for h in range(H):
                g = f64["g"][n, h] if not pc else f64["g"][n, h][None, :]
                r = orc.gdn_sequence(f64["q"][n, h][None], f64["k"][n, h][None],
                                     f64["v"][n, h][None], f64["beta"][n, h][None],
                                     np.atleast_1d(g) if not pc else g, prefix_len=0, flags=0,
                                     S0=S_before[n, h], grid_log2=grid)
                o_ref[n, h] = r["o"][0]
                pre_ref[n, h] = r["S"]
        assert rel_l2(np64(o), o_ref) <= 1e-5
        pre_np = pre.cpu().numpy()
        assert rel_l2(pre_np, pre_ref) <= 1e-6
        want, sc, _ = orc.qdq_states(pre_np)
        np.testing.assert_array_equal(state.cpu().numpy().view(np.uint32), want.view(np.uint32))
        np.testing.assert_array_equal(scales.cpu().numpy(), sc)
