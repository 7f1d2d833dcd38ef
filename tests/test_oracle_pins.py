"""Pins of the CPU oracle against what the format, the mathematics and the
pages fix -- never against the oracle itself.  No GPU needed.

Each test names the plausible oracle mistake it would catch.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import oracle as orc
from oracle.chunked import gdn_chunked
from fp8_state_qat_amd import inputs as gi


# ---------------------------------------------------------------------------
# E4M3 rounding
# ---------------------------------------------------------------------------
def _golden_e4m3(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "e4m3_cases.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            y, code, val = line.split()
            rows.append((float(y), int(code, 16), float(val)))
    return rows


def test_e4m3_golden_cases(golden_dir):
    """Hand-derived cases: ties to even code, saturation at 448, subnormals,
    the sign bit.  Catches ties-away rounding or a wrong maximum."""
    rows = _golden_e4m3(golden_dir)
    y = np.array([r[0] for r in rows], dtype=np.float32)
    codes = orc.e4m3_encode(y)
    for (yy, c, val), got in zip(rows, codes):
        assert got == c, (yy, hex(c), hex(got))
        dec = orc.e4m3_decode(np.array([got], np.uint8))[0]
        assert dec == val and np.signbit(dec) == np.signbit(val), (yy, dec, val)


def _grid_f64():
    """E4M3FN non-negative finite values from the format definition."""
    vals = []
    for c in range(127):
        e, m = c >> 3, c & 7
        vals.append((m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals)


def _numpy_bruteforce(y):
    grid = _grid_f64()
    a = np.minimum(np.abs(y.astype(np.float64)), 448.0)
    d = np.abs(a[:, None] - grid[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among equally near codes prefer the even one
    even = cand & ((np.arange(127) & 1) == 0)[None, :]
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    return (pick | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def _e4m3_probe_values():
    grid = _grid_f64()
    mids = (grid[1:] + grid[:-1]) / 2
    pts = np.concatenate([grid, mids, [464.0, 470.0, 2 ** -10, 1e-30, 0.0]]).astype(np.float32)
    nb = [pts]
    for k in (1, 2, 3):
        nb.append(np.nextafter(pts, np.float32(np.inf)))
        nb.append(np.nextafter(pts, np.float32(0)))
        pts = nb[-2]
    rng = np.random.default_rng(7)
    rnd = (np.exp2(rng.uniform(-14, np.log2(460), 200_000))).astype(np.float32)
    allv = np.concatenate(nb + [rnd])
    return np.concatenate([allv, -allv])


def test_e4m3_bisection_matches_bruteforce():
    """The oracle's bisection equals an exhaustive nearest search (written
    here independently in numpy) at every grid point, every midpoint, their
    fp32 neighbours, and 400k random values."""
    y = _e4m3_probe_values()
    np.testing.assert_array_equal(orc.e4m3_encode(y), _numpy_bruteforce(y))


def test_e4m3_c_bruteforce_subset():
    y = _e4m3_probe_values()[::97]
    np.testing.assert_array_equal(orc.e4m3_encode(y), orc.e4m3_encode_bruteforce(y))


def test_e4m3_matches_torch_cast():
    """torch's float8_e4m3fn cast (round to nearest even) agrees wherever it
    is finite (|y| <= 464)."""
    y = _e4m3_probe_values()
    y = y[np.abs(y) <= 464]
    t = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(orc.e4m3_encode(y), t)


# ---------------------------------------------------------------------------
# Tile QDQ
# ---------------------------------------------------------------------------
def test_qdq_zero_tile():
    x = np.zeros((1, 64, 32), np.float32)
    out, sc, codes = orc.qdq_states(x)
    assert np.all(out == 0) and sc[0, 0] == 1.0 and np.all(codes == 0)


def test_qdq_scale_is_amax_over_448_per_tile():
    """One fp32 scale per 64 value rows x all key columns, amax/448 (fp32
    division).  Catches a per-tensor scale, a per-row scale, or 240."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 128, 64)).astype(np.float32)
    x[1, 64:] *= 1000.0
    out, sc, codes = orc.qdq_states(x)
    for s in range(3):
        for j in range(2):
            tile = x[s, 64 * j:64 * (j + 1)]
            amax = np.float32(np.abs(tile).max())
            assert sc[s, j] == np.float32(amax / np.float32(448.0))
            # the largest element lands exactly on the largest code
            i = np.unravel_index(np.abs(tile).argmax(), tile.shape)
            assert codes[s, 64 * j + i[0], i[1]] & 0x7F == 0x7E


def test_qdq_already_e4m3_tile_is_unchanged():
    """A tile X = C * 2^e with every C on the E4M3 grid and max |C| = 448 is
    returned bitwise unchanged (scale 2^e)."""
    rng = np.random.default_rng(2)
    grid = _grid_f64()
    C = rng.choice(grid, size=(2, 64, 128)) * rng.choice([-1.0, 1.0], size=(2, 64, 128))
    C[:, 0, 0] = 448.0
    for e in (-20, -3, 0, 5):
        X = (C * 2.0 ** e).astype(np.float32)
        out, sc, _ = orc.qdq_states(X)
        assert np.all(sc == np.float32(2.0 ** e))
        np.testing.assert_array_equal(out.view(np.uint32), X.view(np.uint32))


def test_qdq_idempotent_codes():
    """QDQ(QDQ(x)) keeps the same codes and its values move by at most one
    fp32 ulp (only the rounding of code * scale can differ)."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((4, 64, 128)) * rng.uniform(0.01, 100, (4, 1, 1))).astype(np.float32)
    y, s1, c1 = orc.qdq_states(x)
    z, s2, c2 = orc.qdq_states(y)
    np.testing.assert_array_equal(c1, c2)
    ulp = np.spacing(np.abs(y).astype(np.float32))
    assert np.all(np.abs(z - y) <= ulp)


def test_qdq_power_of_two_and_sign():
    """QDQ(2^e x) = 2^e QDQ(x) and QDQ(-x) = -QDQ(x), bitwise."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2, 64, 64)).astype(np.float32)
    y, _, _ = orc.qdq_states(x)
    y8, _, _ = orc.qdq_states(x * np.float32(8.0))
    yn, _, _ = orc.qdq_states(-x)
    np.testing.assert_array_equal(y8, y * np.float32(8.0))
    np.testing.assert_array_equal(yn, -y)


def test_qdq_relative_error_bound():
    """Every element moves by at most half an E4M3 step of its binade times
    the scale (relative 2^-4 for normals, absolute 2^-10 * scale below)."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((8, 64, 128)).astype(np.float32)
    y, sc, _ = orc.qdq_states(x)
    s = np.repeat(sc, 64, axis=1)[..., None]
    bound = np.maximum(np.abs(x) * 2.0 ** -4, s * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(np.abs(y - x) <= bound)


# ---------------------------------------------------------------------------
# Recurrence
# ---------------------------------------------------------------------------
def test_recurrence_hand_worked_two_tokens(golden_dir):
    """Hand-worked two-token examples (scalar and per-key-channel gate).
    Catches a transposed state, a wrong sign in the delta correction, decay
    after instead of before the correction, or the output taken before the
    update."""
    with open(os.path.join(golden_dir, "gdn_two_token.json")) as f:
        gold = json.load(f)
    for key in ("scalar", "per_channel"):
        c = gold[key]
        a = np.array(c["a"], dtype=np.float64)
        r = orc.gdn_sequence(np.array(c["q"]), np.array(c["k"]), np.array(c["v"]),
                             np.array(c["beta"]), np.log(a), flags=0)
        np.testing.assert_allclose(r["o"], np.array(c["o"]), rtol=1e-14, atol=1e-14)
        np.testing.assert_allclose(r["S"], np.array(c["S"]), rtol=1e-14, atol=1e-14)


def _seq(L, dk, dv, per_channel=False, seed=0, g_scale=0.1, io=gi.F32):
    w = gi.make_packed([L], 1, dk, dv, io_dtype=io, per_channel=per_channel,
                       g_scale=g_scale, seed=seed)
    g = w.f64("g")[:, 0]
    return (w.f64("q")[:, 0], w.f64("k")[:, 0], w.f64("v")[:, 0], w.f64("beta")[:, 0], g)


def test_one_token_closed_form():
    """From the zero state, o_1 = beta (k.q) v and S_1 = beta v k^T."""
    q, k, v, b, g = _seq(1, 64, 64, seed=11)
    r = orc.gdn_sequence(q, k, v, b, g, flags=0)
    np.testing.assert_allclose(r["o"][0], b[0] * (k[0] @ q[0]) * v[0], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(r["S"], b[0] * np.outer(v[0], k[0]), rtol=1e-13, atol=1e-15)


def test_one_chunk_qdq_only_touches_final_state():
    """Within one chunk (L <= 64) the outputs are the same with QDQ on or
    off, and the final state with QDQ is QDQ of the final state without."""
    q, k, v, b, g = _seq(50, 64, 128, seed=12)
    off = orc.gdn_sequence(q, k, v, b, g, flags=0)
    on = orc.gdn_sequence(q, k, v, b, g, flags=orc.QDQ_CHUNK)
    np.testing.assert_array_equal(off["o"], on["o"])
    want, _, _ = orc.qdq_states(off["S"].astype(np.float32))
    np.testing.assert_array_equal(on["S"], want.astype(np.float64))


def test_beta_zero_keeps_zero_state():
    q, k, v, b, g = _seq(130, 64, 64, seed=13)
    r = orc.gdn_sequence(q, k, v, np.zeros_like(b), g)
    assert np.all(r["o"] == 0) and np.all(r["S"] == 0)


def test_full_forgetting_gate():
    """a_t = 0 (g = -inf): each token sees only itself, o_t = beta_t (k_t.q_t) v_t."""
    q, k, v, b, g = _seq(70, 64, 64, seed=14)
    r = orc.gdn_sequence(q, k, v, b, np.full_like(g, -np.inf), flags=0)
    want = (b * np.einsum("tc,tc->t", k, q))[:, None] * v
    np.testing.assert_allclose(r["o"], want, rtol=1e-13, atol=1e-15)


def test_delta_rule_overwrite():
    """beta = 1, a = 1, unit basis keys: S k_t = v_t after the write, so with
    q_t = k_t the output is v_t (the delta rule replaces the value stored
    under a key).  Catches a missing delta correction (o would accumulate)."""
    rng = np.random.default_rng(15)
    L, d = 40, 64
    idx = rng.integers(0, d, L)
    k = np.eye(d)[idx]
    v = rng.standard_normal((L, d))
    r = orc.gdn_sequence(k, k, v, np.ones(L), np.zeros(L), flags=0)
    # exact in real arithmetic; old + (new - old) rounds by at most an ulp
    np.testing.assert_allclose(r["o"], v, rtol=0, atol=4 * np.spacing(np.abs(v).max()))


def test_orthogonal_keys_sum():
    """Distinct basis keys, a = 1: S_{t-1} k_t = 0, so S_L = sum beta v k^T."""
    rng = np.random.default_rng(16)
    L, d = 64, 64
    k = np.eye(d)[rng.permutation(d)[:L]]
    v = rng.standard_normal((L, d))
    b = rng.uniform(0.1, 0.9, L)
    r = orc.gdn_sequence(rng.standard_normal((L, d)), k, v, b, np.zeros(L), flags=0)
    np.testing.assert_allclose(r["S"], (b[:, None] * v).T @ k, rtol=1e-15, atol=1e-15)


@pytest.mark.parametrize("per_channel", [False, True])
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_chunked_form_equals_recurrence_qdq_off(per_channel, chunk):
    """The chunk-parallel form (exact solve, WY/UT W and U) is an identity of
    the recurrence: agreement to fp64 rounding, ragged last chunk included."""
    q, k, v, b, g = _seq(203, 64, 64, per_channel=per_channel, seed=17,
                         g_scale=0.05 if per_channel else 0.1)
    rec = orc.gdn_sequence(q, k, v, b, g, flags=0)
    chk = gdn_chunked(q, k, v, b, g, chunk=chunk, qdq=False)
    for key in ("o", "S"):
        rel = np.linalg.norm(chk[key] - rec[key]) / np.linalg.norm(rec[key])
        assert rel < 1e-12, (key, rel)


@pytest.mark.parametrize("per_channel", [False, True])
def test_chunked_form_equals_recurrence_qdq_on(per_channel):
    """With state QDQ at every 64-token boundary (and at t = L) both forms
    place the QDQ at the same points: outputs and final state agree."""
    q, k, v, b, g = _seq(203, 64, 128, per_channel=per_channel, seed=18,
                         g_scale=0.05 if per_channel else 0.1)
    rec = orc.gdn_sequence(q, k, v, b, g, flags=orc.QDQ_CHUNK)
    chk = gdn_chunked(q, k, v, b, g, chunk=64, qdq=True)
    for key in ("o", "S"):
        rel = np.linalg.norm(chk[key] - rec[key]) / np.linalg.norm(rec[key])
        assert rel < 1e-10, (key, rel)
    # and QDQ really happened: off differs
    off = orc.gdn_sequence(q, k, v, b, g, flags=0)
    assert np.linalg.norm(off["o"] - rec["o"]) / np.linalg.norm(rec["o"]) > 1e-4


def test_power_of_two_and_sign_invariance_with_qdq():
    """S is linear in v and QDQ commutes with power-of-two scaling and
    negation, so o(2^e v) = 2^e o(v) and o(-v) = -o(v) bitwise."""
    q, k, v, b, g = _seq(150, 64, 64, seed=19)
    r = orc.gdn_sequence(q, k, v, b, g)
    r4 = orc.gdn_sequence(q, k, 4.0 * v, b, g)
    rn = orc.gdn_sequence(q, k, -v, b, g)
    np.testing.assert_array_equal(r4["o"], 4.0 * r["o"])
    np.testing.assert_array_equal(rn["o"], -r["o"])


def test_handoff_and_per_write_qdq_composition():
    """Write QDQ with a prefix P < L equals: prefix without internal QDQ,
    QDQ at the handoff, then one recurrent step per token, each quantizing
    the state it stores, each output taken before that QDQ."""
    q, k, v, b, g = _seq(100, 64, 64, seed=20)
    P = 70
    full = orc.gdn_sequence(q, k, v, b, g, prefix_len=P, flags=orc.QDQ_WRITE)
    pre = orc.gdn_sequence(q[:P], k[:P], v[:P], b[:P], g[:P], flags=0)
    S, _, _ = orc.qdq_states(pre["S"].astype(np.float32))
    S = S.astype(np.float64)
    np.testing.assert_array_equal(full["o"][:P], pre["o"])
    for t in range(P, 100):
        step = orc.gdn_sequence(q[t:t + 1], k[t:t + 1], v[t:t + 1], b[t:t + 1], g[t:t + 1],
                                prefix_len=0, flags=orc.QDQ_WRITE, S0=S)
        np.testing.assert_array_equal(full["o"][t], step["o"][0])
        S = step["S"]
    np.testing.assert_array_equal(full["S"], S)


def test_split_resume_matches_single_call():
    """Running [0, P) then [P, L) from the returned state (P a multiple of 64,
    boundary QDQ on) equals one call over [0, L)."""
    q, k, v, b, g = _seq(300, 64, 64, seed=21)
    whole = orc.gdn_sequence(q, k, v, b, g, flags=orc.QDQ_CHUNK)
    a = orc.gdn_sequence(q[:128], k[:128], v[:128], b[:128], g[:128], flags=orc.QDQ_CHUNK)
    c = orc.gdn_sequence(q[128:], k[128:], v[128:], b[128:], g[128:], flags=orc.QDQ_CHUNK,
                         S0=a["S"])
    np.testing.assert_array_equal(whole["o"], np.concatenate([a["o"], c["o"]]))
    np.testing.assert_array_equal(whole["S"], c["S"])


def test_boundary_record():
    """Recorded boundaries: one per 64 tokens plus the ragged end; post is the
    QDQ of pre; the final post is the returned state."""
    q, k, v, b, g = _seq(200, 64, 64, seed=22)
    r = orc.gdn_sequence(q, k, v, b, g, flags=orc.QDQ_CHUNK, record=True)
    assert r["n_bounds"] == 4
    for i in range(4):
        want, sc, _ = orc.qdq_states(r["bound_pre"][i].astype(np.float32))
        np.testing.assert_array_equal(r["bound_post"][i], want.astype(np.float64))
        np.testing.assert_array_equal(r["scales"][i], sc)
    np.testing.assert_array_equal(r["bound_post"][-1], r["S"])


def test_packed_matches_per_sequence():
    """Packed varlen with padding: each sequence's rows equal a standalone
    run; padding rows are zero."""
    w = gi.make_packed([70, 5, 130], 2, 64, 64, io_dtype=gi.F32, pads=[3, 0, 10], seed=23)
    res = orc.gdn_packed(w.f64("q"), w.f64("k"), w.f64("v"), w.f64("beta"), w.f64("g"),
                         w.cu_seqlens, seq_lens=w.seq_lens)
    cu = w.cu_seqlens
    for n in range(3):
        for h in range(2):
            s, L = cu[n], w.seq_lens[n]
            r = orc.gdn_sequence(w.f64("q")[s:s + L, h], w.f64("k")[s:s + L, h],
                                 w.f64("v")[s:s + L, h], w.f64("beta")[s:s + L, h],
                                 w.f64("g")[s:s + L, h])
            np.testing.assert_array_equal(res["o"][s:s + L, h], r["o"])
            np.testing.assert_array_equal(res["S"][n, h], r["S"])
            assert np.all(res["o"][s + L:cu[n + 1], h] == 0)


# ---------------------------------------------------------------------------
# W QDQ (chunked form only; #2497 page: independent dynamic FP8 fake QDQ of
# the WY-transformed W, grouping per token and head over the key axis)
# ---------------------------------------------------------------------------
from oracle.chunked import chunk_step, qdq_w  # noqa: E402


def test_w_rows_grouping_and_error_bound():
    """Each row of W is its own group: a row quantized inside a tile where
    it is alone (the state QDQ's grouping, pinned above) gives the same bits;
    every element is within half an E4M3 step of its row's scale, the row
    maximum survives, a zero row stays zero with scale 1.  Catches a
    per-column or per-matrix grouping (small rows would flush to zero) and a
    wrong largest code."""
    rng = np.random.default_rng(31)
    W = rng.standard_normal((9, 128)) * (10.0 ** rng.uniform(-6, 3, 9))[:, None]
    W[4] = 0.0
    Wq, sc = qdq_w(W)
    W32 = W.astype(np.float32)
    for r in range(9):
        tile = np.zeros((64, 128), np.float32)
        tile[0] = W32[r]
        alone, s_alone, _ = orc.qdq_states(tile)
        np.testing.assert_array_equal(Wq[r].astype(np.float32), alone[0])
        assert sc[r] == s_alone[0]
        amax = np.abs(W32[r]).max()
        if amax == 0:
            assert sc[r] == 1.0 and np.all(Wq[r] == 0)
            continue
        assert np.all(np.abs(Wq[r] - W32[r]) <= 2.0 ** -4 * amax * (1 + 1e-6))
        i = np.abs(W32[r]).argmax()
        assert abs(abs(Wq[r, i]) - amax) <= 2.0 ** -22 * amax


@pytest.mark.parametrize("per_channel", [False, True])
def test_w_qdq_has_no_effect_from_zero_state(per_channel):
    """W only enters U' through W S^T: from the zero state one chunk gives the
    same outputs and state with W QDQ on or off (bitwise), and from a nonzero
    state it changes them.  Catches QDQ'd W leaking into U = T V or the
    state update."""
    q, k, v, b, g = _seq(64, 64, 64, per_channel=per_channel, seed=32,
                         g_scale=0.05 if per_channel else 0.1)
    z = np.zeros((64, 64))
    on = chunk_step(q, k, v, b, g, z, w_qdq=True)
    off = chunk_step(q, k, v, b, g, z, w_qdq=False)
    np.testing.assert_array_equal(on["o"], off["o"])
    np.testing.assert_array_equal(on["S"], off["S"])
    assert np.linalg.norm(on["Wq"] - on["W"]) > 0
    S = np.random.default_rng(33).standard_normal((64, 64))
    on = chunk_step(q, k, v, b, g, S, w_qdq=True)
    off = chunk_step(q, k, v, b, g, S, w_qdq=False)
    assert np.linalg.norm(on["o"] - off["o"]) > 1e-6 * np.linalg.norm(off["o"])


@pytest.mark.parametrize("per_channel", [False, True])
def test_w_qdq_one_token_chunks_token_form(per_channel):
    """With one-token chunks, T = beta and W = beta (k * exp(g)): the chunked
    form with W QDQ is the token recurrence in which the term beta a S k of the
    delta correction uses the row-quantized beta (a * k) -- written out here
    token by token, with no solve and no WY algebra.  Catches a W without its
    gate factor or beta, or quantized along the wrong axis."""
    L, d = 40, 64
    q, k, v, b, g = _seq(L, d, d, per_channel=per_channel, seed=34,
                         g_scale=0.05 if per_channel else 0.1)
    g = g * 3.0  # gate factors far from 1
    chk = gdn_chunked(q, k, v, b, g, chunk=1, qdq=False, w_qdq=True)
    S = np.zeros((d, d))
    o = np.zeros((L, d))
    for t in range(L):
        a = np.exp(g[t])                       # scalar or [dk]
        w, _ = qdq_w((b[t] * (a * k[t]))[None, :])
        u = b[t] * v[t] - S @ w[0]
        o[t] = S @ (a * q[t]) + (q[t] @ k[t]) * u
        S = S * a + np.outer(u, k[t])
    np.testing.assert_allclose(chk["o"], o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(chk["S"], S, rtol=1e-12, atol=1e-14)


def test_w_qdq_power_of_two_and_sign_invariance():
    """W does not depend on v, so with W QDQ and state QDQ on, o(4 v) = 4 o(v)
    and o(-v) = -o(v) bitwise over several chunks."""
    q, k, v, b, g = _seq(150, 64, 64, seed=35)
    r = gdn_chunked(q, k, v, b, g, w_qdq=True)
    r4 = gdn_chunked(q, k, 4.0 * v, b, g, w_qdq=True)
    rn = gdn_chunked(q, k, -v, b, g, w_qdq=True)
    np.testing.assert_array_equal(r4["o"], 4.0 * r["o"])
    np.testing.assert_array_equal(rn["o"], -r["o"])


def test_w_qdq_record():
    """Per-chunk record: Wq is the row QDQ of W, rows past a chunk's end are
    zero, the boundary states follow the QDQ flags."""
    q, k, v, b, g = _seq(150, 64, 64, seed=36)
    r = gdn_chunked(q, k, v, b, g, w_qdq=True, record=True)
    assert r["W"].shape == (3, 64, 64)
    for i, n in enumerate((64, 64, 22)):
        want, sc = qdq_w(r["W"][i, :n])
        np.testing.assert_array_equal(r["Wq"][i, :n], want)
        np.testing.assert_array_equal(r["w_scales"][i, :n], sc)
        assert np.all(r["W"][i, n:] == 0) and np.all(r["Wq"][i, n:] == 0)
        post, _, _ = orc.qdq_states(r["bound_pre"][i].astype(np.float32))
        np.testing.assert_array_equal(r["bound_post"][i], post.astype(np.float64))
    np.testing.assert_array_equal(r["bound_post"][-1], r["S"])


@pytest.mark.parametrize("flags", [0, 1, 2, 3])
def test_chunked_prefix_and_suffix_equal_recurrence(flags):
    """Chunked prefix of P tokens, then token-by-token writes: with W QDQ off
    the chunked oracle places every QDQ where the recurrence does (chunk
    boundaries, the handoff t = P, each later write)."""
    q, k, v, b, g = _seq(230, 64, 64, seed=37)
    for P in (0, 1, 64, 100, 230):
        rec = orc.gdn_sequence(q, k, v, b, g, prefix_len=P, flags=flags)
        chk = gdn_chunked(q, k, v, b, g, prefix_len=P, flags=flags)
        for key in ("o", "S"):
            rel = np.linalg.norm(chk[key] - rec[key]) / np.linalg.norm(rec[key])
            assert rel < 1e-10, (P, key, rel)


# ---------------------------------------------------------------------------
# INT8 block-32 state QDQ (#2519 page: dynamic INT8 state recipes with
# 32-element blocks; the formula is the oracle's reading: signed symmetric,
# scale amax / 127 per block of 32 key columns, round half to even)
# ---------------------------------------------------------------------------
def test_int8_hand_cases():
    """Scale 1 (block amax 127): ties go to the even integer in both signs,
    everything else to the nearest; -0.5 gives a zero code."""
    x = np.zeros((1, 32), np.float32)
    x[0, :10] = [127, 2.5, -2.5, 3.5, 0.5, 1.5, 126.5, -0.5, 0.49999997, -1.5000001]
    out, sc, codes = orc.qdq_int8_blocks(x)
    assert sc[0, 0] == 1.0
    assert list(codes[0, :10]) == [127, 2, -2, 4, 0, 2, 126, 0, 0, -2]
    np.testing.assert_array_equal(out[0, :10], codes[0, :10].astype(np.float32))
    # a value that rounds to zero keeps its sign, as IEEE rounding to integral does
    assert np.signbit(out[0, 7]) and not np.signbit(out[0, 4])


def test_int8_rounding_against_brute_force():
    """Codes at scale 1 against a nearest-integer search over every code in
    [-127, 127] with ties to the even one; values drawn at and around every
    half-integer.  Catches ties-away rounding or truncation."""
    rng = np.random.default_rng(61)
    halves = np.arange(-127, 127) + 0.5
    y = np.concatenate([halves, np.nextafter(halves, 0, dtype=np.float64),
                        np.nextafter(halves, 200, dtype=np.float64), rng.uniform(-127, 127, 4000)])
    y = y.astype(np.float32)
    n = (y.size + 30) // 31 * 31
    y = np.pad(y, (0, n - y.size))
    blocks = np.zeros((n // 31, 32), np.float32)
    blocks[:, 0] = 127.0                       # fixes the scale at 1
    blocks[:, 1:] = y.reshape(-1, 31)
    _, sc, codes = orc.qdq_int8_blocks(blocks)
    assert np.all(sc == 1.0)
    cand = np.arange(-127, 128, dtype=np.float64)
    d = np.abs(blocks[:, 1:, None].astype(np.float64) - cand[None, None, :])
    best = d.min(axis=2, keepdims=True)
    tie_even = np.where(d == best, np.where(cand % 2 == 0, 0, 1), 2)   # prefer the even one on a tie
    want = cand[np.argmin(tie_even, axis=2)]
    np.testing.assert_array_equal(codes[:, 1:].astype(np.float64), want)


def test_int8_blocks_grouping_and_bounds():
    """Each run of 32 consecutive key columns is its own group: a block
    quantized alone gives the same bits; every element is within half a step
    of its block's scale; the block maximum maps to +-127; a zero block stays
    zero with scale 1.  Catches a per-row or per-tile grouping."""
    rng = np.random.default_rng(62)
    S = (rng.standard_normal((64, 128)) * (10.0 ** rng.uniform(-5, 3, (64, 4))).repeat(32, axis=1))
    S = S.astype(np.float32)
    S[3, 32:64] = 0.0
    out, sc, codes = orc.qdq_int8_blocks(S)
    assert sc.shape == (64, 4)
    for r in (0, 3, 17, 63):
        for b in range(4):
            blk = S[r, 32 * b:32 * b + 32]
            o1, s1, c1 = orc.qdq_int8_blocks(blk[None, :])
            np.testing.assert_array_equal(o1[0], out[r, 32 * b:32 * b + 32])
            assert s1[0, 0] == sc[r, b]
            amax = np.abs(blk).max()
            if amax == 0:
                assert sc[r, b] == 1.0 and np.all(out[r, 32 * b:32 * b + 32] == 0)
                continue
            assert np.all(np.abs(out[r, 32 * b:32 * b + 32] - blk) <= 0.5 * sc[r, b] * (1 + 1e-6))
            assert np.abs(c1[0]).max() == 127


def test_int8_decode_one_token_closed_form():
    """From the zero state one token with a per-write INT8 QDQ: the output is
    taken before the QDQ (o_1 = beta (k.q) v) and the stored state is the
    INT8 QDQ of beta v k^T."""
    q, k, v, b, g = _seq(1, 128, 64, seed=63)
    r = orc.gdn_sequence(q, k, v, b, g, prefix_len=0, flags=orc.QDQ_WRITE | orc.QDQ_INT8)
    np.testing.assert_allclose(r["o"][0], b[0] * (k[0] @ q[0]) * v[0], rtol=1e-13, atol=1e-15)
    want, _, _ = orc.qdq_int8_blocks((b[0] * np.outer(v[0], k[0])).astype(np.float32))
    np.testing.assert_array_equal(r["S"], want.astype(np.float64))
    fp8 = orc.gdn_sequence(q, k, v, b, g, prefix_len=0, flags=orc.QDQ_WRITE)
    assert not np.array_equal(fp8["S"], r["S"])


def test_int8_power_of_two_and_sign_invariance():
    """INT8 QDQ commutes with power-of-two scaling and negation, so over a
    run of per-write QDQs o(4 v) = 4 o(v) and o(-v) = -o(v) bitwise."""
    q, k, v, b, g = _seq(40, 64, 64, seed=64)
    f = orc.QDQ_WRITE | orc.QDQ_INT8
    r = orc.gdn_sequence(q, k, v, b, g, prefix_len=0, flags=f)
    r4 = orc.gdn_sequence(q, k, 4.0 * v, b, g, prefix_len=0, flags=f)
    rn = orc.gdn_sequence(q, k, -v, b, g, prefix_len=0, flags=f)
    np.testing.assert_array_equal(r4["o"], 4.0 * r["o"])
    np.testing.assert_array_equal(rn["o"], -r["o"])


# ---------------------------------------------------------------------------
# State gradients (reverse recurrence; identity straight-through QDQ)
# ---------------------------------------------------------------------------
from oracle.backward import state_grads  # noqa: E402


def _loss(q, k, v, b, g, do, dS, S0):
    """L = sum_t o_t . do_t + <S_L, dS> by the forward oracle (QDQ off)."""
    r = orc.gdn_sequence(q, k, v, b, g, flags=0, S0=S0)
    return float(np.sum(r["o"] * do) + np.sum(r["S"] * dS))


@pytest.mark.parametrize("per_channel", [False, True])
def test_state_grads_against_forward_differences(per_channel):
    """L is affine in any state, so <dh_c, S> = L_c(S) - L_c(0), where L_c
    runs the forward oracle from chunk c's first token with entering state S
    -- for every chunk and the initial state, on random directions S and on
    single entries.  Catches a missing decay, a transposed k k^T term, a
    dropped output term or an off-by-one chunk boundary."""
    L, dk, dv = 150, 64, 64
    q, k, v, b, g = _seq(L, dk, dv, per_channel=per_channel, seed=81,
                         g_scale=0.05 if per_channel else 0.1)
    rng = np.random.default_rng(82)
    do = rng.standard_normal((L, dv))
    dS = rng.standard_normal((dv, dk))
    dh, dS0 = state_grads(q, k, b, g, do, dS)
    assert dh.shape == (3, dv, dk)
    np.testing.assert_array_equal(dh[0], dS0)
    for c in range(3):
        sl = slice(64 * c, L)
        base = _loss(q[sl], k[sl], v[sl], b[sl], g[sl], do[sl], dS, None)
        S = rng.standard_normal((dv, dk))
        lin = _loss(q[sl], k[sl], v[sl], b[sl], g[sl], do[sl], dS, S) - base
        assert abs(lin - np.sum(dh[c] * S)) <= 1e-9 * max(1.0, abs(lin)), (c, lin)
        for (i, j) in ((0, 0), (5, 17), (63, 63)):
            E = np.zeros((dv, dk))
            E[i, j] = 1.0
            d = _loss(q[sl], k[sl], v[sl], b[sl], g[sl], do[sl], dS, E) - base
            assert abs(d - dh[c, i, j]) <= 1e-10 * max(1.0, abs(d)), (c, i, j)


@pytest.mark.parametrize("per_channel", [False, True])
def test_value_grads_against_forward_differences(per_channel):
    """L is affine in every value vector, so <dv_t, u> = L(v + u e_t) - L(v)
    for a random direction u at sampled tokens t (chunk ends and middles).
    Catches a missing beta or a gradient taken before the output term."""
    L, dk, dv = 150, 64, 64
    q, k, v, b, g = _seq(L, dk, dv, per_channel=per_channel, seed=85,
                         g_scale=0.05 if per_channel else 0.1)
    rng = np.random.default_rng(86)
    do = rng.standard_normal((L, dv))
    dS = rng.standard_normal((dv, dk))
    _, _, dvals = state_grads(q, k, b, g, do, dS, want_dv=True)
    base = _loss(q, k, v, b, g, do, dS, None)
    for t in (0, 63, 64, 100, 149):
        u = rng.standard_normal(dv)
        v2 = v.copy()
        v2[t] += u
        d = _loss(q, k, v2, b, g, do, dS, None) - base
        assert abs(d - dvals[t] @ u) <= 1e-9 * max(1.0, abs(d)), (t, d, dvals[t] @ u)


def test_state_grads_one_token_closed_form():
    """One token from S_0: o = S_1 q with S_1 = a S_0 (I - b k k^T) + b v k^T,
    so dL/dS_0 = a (do q^T + dS) (I - b k k^T)."""
    q, k, v, b, g = _seq(1, 64, 64, seed=83)
    rng = np.random.default_rng(84)
    do = rng.standard_normal((1, 64))
    dS = rng.standard_normal((64, 64))
    _, dS0 = state_grads(q, k, b, g, do, dS)
    a = np.exp(g[0])
    want = a * (np.outer(do[0], q[0]) + dS) @ (np.eye(64) - b[0] * np.outer(k[0], k[0]))
    np.testing.assert_allclose(dS0, want, rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# Log-retention grid of the recurrent writes (the decode/replay page #2509:
# an optional rounding of the log-retention; its pilot selected 1/256).
# Reading (parity unpinned against the pages, which give no formula): each
# recurrent write t > P decays with g rounded to the nearest multiple of
# 2^-k, ties to even.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("g_units,k,want_units", [
    (-1.5, 8, -2.0), (-2.5, 8, -2.0), (-0.5, 8, -0.0), (0.5, 8, 0.0), (-0.896, 8, -1.0),
    (-77.49, 8, -77.0), (-77.5, 8, -78.0), (-76.5, 8, -76.0), (3.5, 1, 4.0), (-1.0, 24, -1.0),
])
def test_grid_gate_rounding_table(g_units, k, want_units):
    """Hand-derived: g = g_units * 2^-k goes to want_units * 2^-k (nearest
    multiple of the step, ties to the even multiple)."""
    got = orc.grid_gate(g_units * 2.0 ** -k, k)
    assert got == want_units * 2.0 ** -k
    assert orc.grid_gate(g_units * 2.0 ** -k, 0) == g_units * 2.0 ** -k   # k = 0: off


def _two_token(q, k, v, b, a2):
    """Zero state, two tokens, no QDQ, decay a2 at token 2 (the decay of
    token 1 meets the zero state): S_1 = b1 v1 k1^T, o_1 = S_1 q1;
    S~ = a2 S_1, u = b2 (v2 - S~ k2), S_2 = S~ + u k2^T, o_2 = S_2 q2."""
    S1 = b[0] * np.outer(v[0], k[0])
    St = a2 * S1
    u = b[1] * (v[1] - St @ k[1])
    S2 = St + np.outer(u, k[1])
    return np.stack([S1 @ q[0], S2 @ q[1]]), S2


@pytest.mark.parametrize("per_channel", [False, True])
def test_grid_two_token_closed_form(per_channel):
    """From the zero state with P = 0, token 2's decay is exp of its gate on
    the grid: g = -0.3 at k = 8 is -77/256 (scalar); per channel each key
    channel's gate is rounded on its own.  The expected values retype the
    closed form, not the oracle's code."""
    q, k, v, b, _ = _seq(2, 64, 64, seed=91)
    if per_channel:
        g = np.full((2, 64), -0.3)
        g[1, ::2] = -0.1                          # 25.6 -> 26 units
        a2 = np.where(np.arange(64) % 2 == 0, np.exp(-26 / 256), np.exp(-77 / 256))
        r = orc.gdn_sequence(q, k, v, b, g, prefix_len=0, flags=0, grid_log2=8)
        S1 = b[0] * np.outer(v[0], k[0])
        St = S1 * a2[None, :]
        u = b[1] * (v[1] - St @ k[1])
        S2 = St + np.outer(u, k[1])
        o = np.stack([S1 @ q[0], S2 @ q[1]])
    else:
        g = np.array([-0.3, -0.3])
        r = orc.gdn_sequence(q, k, v, b, g, prefix_len=0, flags=0, grid_log2=8)
        o, S2 = _two_token(q, k, v, b, np.exp(-77 / 256))
    np.testing.assert_allclose(r["o"], o, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(r["S"], S2, rtol=1e-13, atol=1e-15)


def test_grid_leaves_the_chunked_prefix_and_on_grid_gates_alone():
    """The grid only touches recurrent writes: with P = L (no suffix) the
    result is bitwise the one without the grid; with gates already on the
    grid it is bitwise unchanged for any P; with off-grid gates and a suffix
    it changes, and only from the first suffix token on."""
    q, k, v, b, g = _seq(150, 64, 64, seed=92)
    base = orc.gdn_sequence(q, k, v, b, g, prefix_len=150, flags=3)
    grid = orc.gdn_sequence(q, k, v, b, g, prefix_len=150, flags=3, grid_log2=8)
    assert np.array_equal(base["o"], grid["o"]) and np.array_equal(base["S"], grid["S"])
    g_on = np.round(g * 256) / 256
    base = orc.gdn_sequence(q, k, v, b, g_on, prefix_len=70, flags=3)
    grid = orc.gdn_sequence(q, k, v, b, g_on, prefix_len=70, flags=3, grid_log2=8)
    assert np.array_equal(base["o"], grid["o"]) and np.array_equal(base["S"], grid["S"])
    base = orc.gdn_sequence(q, k, v, b, g, prefix_len=70, flags=3)
    grid = orc.gdn_sequence(q, k, v, b, g, prefix_len=70, flags=3, grid_log2=3)
    assert np.array_equal(base["o"][:70], grid["o"][:70])
    assert not np.array_equal(base["o"][70], grid["o"][70])


def test_grid_fine_step_approaches_no_grid():
    """At k = 24 each gate moves by at most 2^-25, so the whole suffix moves
    by about that relative amount (QDQ off)."""
    q, k, v, b, g = _seq(100, 64, 64, seed=93)
    base = orc.gdn_sequence(q, k, v, b, g, prefix_len=10, flags=0)
    fine = orc.gdn_sequence(q, k, v, b, g, prefix_len=10, flags=0, grid_log2=24)
    rel = np.linalg.norm(fine["S"] - base["S"]) / np.linalg.norm(base["S"])
    assert 0 < rel < 1e-6


# --------------------------------------------------------------------------
# The backward of the W-QDQ forward (identity straight-through rule on the
# W quantizer): the chunk-level reverse recurrence.
# --------------------------------------------------------------------------
from oracle.backward import chunked_state_grads  # noqa: E402


@pytest.mark.parametrize("per_channel", [False, True])
def test_chunked_grads_equal_token_grads_without_w_qdq(per_channel):
    """Without W QDQ the chunk-level backward is the token backward
    regrouped (an algebraic identity): dh per chunk, dS0 and dv agree to
    1e-12 relative."""
    L, dk, dv = 150, 64, 64
    q, k, v, b, g = _seq(L, dk, dv, per_channel=per_channel, seed=101,
                         g_scale=0.05 if per_channel else 0.1)
    rng = np.random.default_rng(102)
    do = rng.standard_normal((L, dv))
    dS = rng.standard_normal((dv, dk))
    t_dh, t_0, t_v = state_grads(q, k, b, g, do, dS, want_dv=True)
    c_dh, c_0, c_v = chunked_state_grads(q, k, b, g, do, dS, want_dv=True)
    for x, y in ((c_dh, t_dh), (c_0, t_0), (c_v, t_v)):
        assert np.linalg.norm(x - y) <= 1e-12 * np.linalg.norm(y)


def _wq_loss(q, k, v, b, g, do, dS, S0):
    """L = sum_t o_t . do_t + <S_L, dS> by the chunked forward oracle with W
    QDQ and no state QDQ: affine in S0 and in v, since the quantized W
    depends on k, beta and g alone."""
    r = gdn_chunked(q, k, v, b, g, qdq=False, w_qdq=True, S0=S0)
    return float(np.sum(r["o"] * do) + np.sum(r["S"] * dS))


@pytest.mark.parametrize("per_channel", [False, True])
def test_w_qdq_grads_against_forward_differences(per_channel):
    """The W-QDQ forward is affine in the initial state and the values, so
    <dS0, U> = L(S0 + U) - L(S0) and <dv_t, u> = L(v + u e_t) - L(v) hold
    exactly (to fp64 rounding) for the gradient of that forward.  Catches a
    backward that uses the unquantized W (the difference is the W
    quantization error, far above the bound) or drops a term."""
    L, dk, dv = 150, 64, 64
    q, k, v, b, g = _seq(L, dk, dv, per_channel=per_channel, seed=103,
                         g_scale=0.05 if per_channel else 0.1)
    rng = np.random.default_rng(104)
    do = rng.standard_normal((L, dv))
    dS = rng.standard_normal((dv, dk))
    S0 = rng.standard_normal((dv, dk)) * 0.3
    _, dS0, dvals = chunked_state_grads(q, k, b, g, do, dS, w_qdq=True, want_dv=True)
    base = _wq_loss(q, k, v, b, g, do, dS, S0)
    for _ in range(3):
        U = rng.standard_normal((dv, dk))
        d = _wq_loss(q, k, v, b, g, do, dS, S0 + U) - base
        assert abs(d - np.sum(dS0 * U)) <= 1e-9 * max(1.0, abs(d))
    for t in (0, 63, 64, 149):
        u = rng.standard_normal(dv)
        v2 = v.copy()
        v2[t] += u
        d = _wq_loss(q, k, v2, b, g, do, dS, S0) - base
        assert abs(d - dvals[t] @ u) <= 1e-9 * max(1.0, abs(d))
    # the plain backward is not the gradient of this forward
    _, dS0_plain = state_grads(q, k, b, g, do, dS)
    assert np.linalg.norm(dS0_plain - dS0) > 1e-4 * np.linalg.norm(dS0)
