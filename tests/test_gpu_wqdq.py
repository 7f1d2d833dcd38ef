"""GPU parity of W QDQ (GDN_QDQ_W: dynamic FP8 E4M3 QDQ of each row of the
WY-transformed W = T (K exp(gamma)) before W S^T) against the chunked oracle,
through the C ABI.  The token recurrence has no W, so the reference is the
chunked fp64 form (oracle/chunked.py), pinned against the recurrence and a
token-form one-token-chunk case.

Gates, per chunk of every (sequence, head), over valid rows:
  GW1  the GPU's W before QDQ (debug record) is the oracle's W of the same
       chunk (it depends on k, beta and g alone) within G1's tolerance
       (1e-5 fp32 inputs, 2e-3 bf16 inputs);
  GW2  the GPU's W after QDQ is the oracle's row QDQ of the GPU's own W bit
       for bit (the same fp32 decision, scales included); the oracle's codes
       on its own W differ from the GPU's on at most 1e-4 of the elements,
       each within 1e-6 (of the row's range) of a rounding midpoint;
  GW3  teacher-forced: the oracle restarts each chunk from the GPU's post-QDQ
       boundary state and takes the GPU's quantized W; that chunk's o and
       pre-QDQ state meet G1's tolerances, and the GPU's state QDQ is the
       oracle's QDQ of the GPU's pre-QDQ state bit for bit.
Free-running differences are reported: one flipped W code moves a row of U'.
"""
import numpy as np
import pytest
import torch

from fp8_state_qat_amd import api
from fp8_state_qat_amd import inputs as gi
from fp8_state_qat_amd._lib import GDN_QDQ_W, GDN_SCHEDULE_AUTO, GDN_SCHEDULE_FUSED, GDN_SCHEDULE_SPLIT
from oracle import oracle as orc
from oracle.chunked import chunk_step, gdn_chunked

from helpers import (CHUNK, TOL, canon_codes, midpoint_distance, midpoint_distance_range, n_bounds, np64,
                     rel_l2, valid_rows)

pytestmark = pytest.mark.gpu


def run_w_gpu(w, flags, *, o_dtype="f32", schedule=GDN_SCHEDULE_AUTO, initial_state=None, record=True):
    d = gi.device_tensors(w)
    H, dk, dv = w.n_heads, w.dk, w.dv
    nb = n_bounds(w.prefix_lens)
    offs = np.zeros(len(nb) + 1, np.int32)
    offs[1:] = np.cumsum(nb)
    tot = int(offs[-1])
    dbg = {"schedule": schedule}
    if record:
        nan = float("nan")
        dbg.update(bound_offsets=torch.from_numpy(offs).cuda(),
                   bound_pre=torch.full((tot, H, dv, dk), nan, device="cuda"),
                   bound_post=torch.full((tot, H, dv, dk), nan, device="cuda"),
                   scales=torch.full((tot, H, dv // 64), nan, device="cuda"),
                   w_pre=torch.full((tot, H, 64, dk), nan, device="cuda"),
                   w_post=torch.full((tot, H, 64, dk), nan, device="cuda"))
    init = None if initial_state is None else torch.from_numpy(
        np.ascontiguousarray(initial_state, np.float32)).cuda()
    o_dt = {"f32": torch.float32, "bf16": torch.bfloat16}[o_dtype]
    o, S = api.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["cu_seqlens"],
                         seq_lens=d["seq_lens"], prefix_lens=d["prefix_lens"], initial_state=init,
                         qdq_flags=flags, o_dtype=o_dt, debug=dbg)
    torch.cuda.synchronize()
    res = {"o": np64(o), "S": S.cpu().numpy(), "offsets": offs}
    if record:
        for key in ("bound_pre", "bound_post", "scales", "w_pre", "w_post"):
            res[key] = dbg[key].cpu().numpy()
    return res


def check_w(w, gpu, flags, tol, *, initial_state=None, pairs=None):
    """GW1-GW3 over every chunk of the given (n, h) pairs; returns the stats."""
    q, k, v, b, g = (w.f64(x) for x in ("q", "k", "v", "beta", "g"))
    cu, offs = w.cu_seqlens, gpu["offsets"]
    if pairs is None:
        pairs = [(n, h) for n in range(w.n_seqs) for h in range(w.n_heads)]
    st = dict(w_bits=0, w_codes=0, w_mism=0, w_far=0, w_far_rel=0, w_max_dist=0.0, s_bits=0, s_scale=0, pad=0)
    acc = np.zeros(6)   # W err, W ref, o err, o ref, pre err, pre ref (squared sums)
    for (n, h) in pairs:
        P, s0 = int(w.prefix_lens[n]), int(cu[n])
        nch = (P + CHUNK - 1) // CHUNK
        for c in range(nch):
            bidx = int(offs[n]) + c
            t0, t1 = c * CHUNK, min(P, (c + 1) * CHUNK)
            nv = t1 - t0
            sl = slice(s0 + t0, s0 + t1)
            if c == 0:
                S_in = (np.zeros((w.dv, w.dk)) if initial_state is None
                        else np.asarray(initial_state[n, h], np.float64))
            else:
                S_in = gpu["bound_post"][bidx - 1, h].astype(np.float64)
            Wg = gpu["w_pre"][bidx, h, :nv]
            Wqg = gpu["w_post"][bidx, h, :nv]
            st["pad"] += int(np.sum(gpu["w_pre"][bidx, h, nv:] != 0) + np.sum(gpu["w_post"][bidx, h, nv:] != 0))
            r = chunk_step(q[sl, h], k[sl, h], v[sl, h], b[sl, h], g[sl, h], S_in,
                           Wq=Wqg.astype(np.float64))
            acc[:2] += [np.sum((Wg - r["W"]) ** 2), np.sum(r["W"] ** 2)]
            # GW2: the GPU's decision on its own W, then the oracle's on its own
            want, _, codes_g = orc.qdq_rows(Wg)
            st["w_bits"] += int(np.sum(want.view(np.uint32) != Wqg.view(np.uint32)))
            _, sc_o, codes_o = orc.qdq_rows(r["W"].astype(np.float32))
            mism = canon_codes(codes_o) != canon_codes(codes_g)
            st["w_codes"] += codes_o.size
            st["w_mism"] += int(mism.sum())
            if mism.any():
                y = r["W"] / sc_o.astype(np.float64)[:, None]
                st["w_far"] += int(np.sum(midpoint_distance_range(y[mism]) > 1e-6))
                dist = midpoint_distance(y[mism])
                st["w_far_rel"] += int(np.sum(dist > 1e-6))
                st["w_max_dist"] = max(st["w_max_dist"], float(dist.max()))
            # GW3
            pre_g = gpu["bound_pre"][bidx, h]
            acc[2:] += [np.sum((gpu["o"][sl, h] - r["o"]) ** 2), np.sum(r["o"] ** 2),
                        np.sum((pre_g - r["S"]) ** 2), np.sum(r["S"] ** 2)]
            last = c == nch - 1
            if (flags & orc.QDQ_CHUNK) or ((flags & orc.QDQ_WRITE) and last):
                want_s, sc_s, _ = orc.qdq_states(pre_g)
                st["s_bits"] += int(np.sum(want_s.view(np.uint32) != gpu["bound_post"][bidx, h].view(np.uint32)))
                st["s_scale"] += int(np.sum(sc_s != gpu["scales"][bidx, h]))
    den = lambda x: max(x, 1e-300)  # noqa: E731
    st.update(w_rel=float(np.sqrt(acc[0] / den(acc[1]))), o_rel=float(np.sqrt(acc[2] / den(acc[3]))),
              pre_rel=float(np.sqrt(acc[4] / den(acc[5]))))
    print("GW", st, flush=True)
    assert st["w_rel"] <= tol and st["o_rel"] <= tol and st["pre_rel"] <= tol
    assert st["w_bits"] == 0 and st["pad"] == 0
    assert st["s_bits"] == 0 and st["s_scale"] == 0
    assert st["w_mism"] <= max(1, 1e-4 * st["w_codes"]) and st["w_far"] == 0
    return st


def free_running(w, gpu, flags, *, initial_state=None):
    """Whole-sequence oracle (chunked prefix with W QDQ, then the suffix);
    the rel-L2 of o and of the final states."""
    q, k, v, b, g = (w.f64(x) for x in ("q", "k", "v", "beta", "g"))
    o = np.zeros_like(gpu["o"])
    S = np.zeros_like(gpu["S"], dtype=np.float64)
    for n in range(w.n_seqs):
        s0, L = int(w.cu_seqlens[n]), int(w.seq_lens[n])
        for h in range(w.n_heads):
            sl = slice(s0, s0 + L)
            r = gdn_chunked(q[sl, h], k[sl, h], v[sl, h], b[sl, h], g[sl, h],
                            S0=None if initial_state is None else initial_state[n, h],
                            prefix_len=int(w.prefix_lens[n]), flags=flags & 3, w_qdq=True)
            o[sl, h] = r["o"]
            S[n, h] = r["S"]
    m = valid_rows(w)
    return rel_l2(gpu["o"][m], o[m]), rel_l2(gpu["S"], S)


@pytest.mark.parametrize("flags", [GDN_QDQ_W, 3 | GDN_QDQ_W])
def test_w_qdq_fp32(flags):
    """fp32 inputs, d = 64, ragged lengths (an empty sequence, one token,
    chunk multiples and tails)."""
    w = gi.make_packed([256, 0, 1, 64, 129, 200], 2, 64, 64, io_dtype=gi.F32, seed=41)
    gpu = run_w_gpu(w, flags)
    check_w(w, gpu, flags, TOL[gi.F32])
    o_rel, s_rel = free_running(w, gpu, flags)
    print(f"free-running (reported): o_rel={o_rel:.3e} S_rel={s_rel:.3e}", flush=True)
    assert np.all(gpu["S"][1] == 0)


@pytest.mark.parametrize("d,dv", [(128, 128), (64, 64), (128, 256)])
def test_w_qdq_bf16(d, dv):
    w = gi.make_packed([300, 129, 1, 64], 2, d, dv, io_dtype=gi.BF16, seed=43 + d + dv)
    gpu = run_w_gpu(w, 3 | GDN_QDQ_W)
    check_w(w, gpu, 3, TOL[gi.BF16])
    o_rel, s_rel = free_running(w, gpu, 3)
    print(f"free-running (reported): o_rel={o_rel:.3e} S_rel={s_rel:.3e}", flush=True)


@pytest.mark.parametrize("io,d", [(gi.F32, 64), (gi.BF16, 64), (gi.BF16, 128)])
def test_w_qdq_per_channel_gate(io, d):
    """A per-key-channel gate (KDA): W = T (K o exp(gamma)) with gamma per
    channel, formed on the fp32 MFMA by the per-channel prep."""
    w = gi.make_packed([300, 129, 1, 64], 2, d, d, io_dtype=io, per_channel=True, g_scale=0.05,
                       seed=57 + d)
    gpu = run_w_gpu(w, 3 | GDN_QDQ_W)
    check_w(w, gpu, 3, TOL[io])
    o_rel, s_rel = free_running(w, gpu, 3)
    print(f"free-running (reported): o_rel={o_rel:.3e} S_rel={s_rel:.3e}", flush=True)


@pytest.mark.parametrize("io", [gi.F32, gi.BF16])
def test_w_qdq_initial_state(io):
    """A supplied initial state enters the first chunk unquantized (as an
    fp32 pair on the bf16 engine) and meets W S^T there."""
    d = 64 if io == gi.F32 else 128
    w = gi.make_packed([130, 64, 20], 2, d, d, io_dtype=io, seed=47)
    S0 = (np.random.default_rng(47).standard_normal((3, 2, d, d)) * 0.5).astype(np.float32)
    gpu = run_w_gpu(w, 3 | GDN_QDQ_W, initial_state=S0)
    check_w(w, gpu, 3, TOL[io], initial_state=S0)


@pytest.mark.parametrize("flags", [1 | GDN_QDQ_W, 3 | GDN_QDQ_W])
def test_w_qdq_prefix_suffix(flags):
    """W QDQ in the chunked prefix only; the recurrent suffix (no W) starts
    from the GPU's handoff state and follows the token recurrence: the whole
    suffix within G1's tolerance when it does not quantize; with a QDQ after
    every write an fp32-versus-fp64 difference flips a code now and then and
    the flip carries on, so there the first suffix token (taken from the
    handoff state before its own QDQ) is held to G1's tolerance and the rest
    is reported (the per-write rule is pinned by the decode-step tests)."""
    w = gi.make_packed([150, 70, 9], 2, 64, 64, io_dtype=gi.F32, seed=49, prefix_lens=[128, 33, 0])
    gpu = run_w_gpu(w, flags)
    check_w(w, gpu, flags, TOL[gi.F32], pairs=[(n, h) for n in range(2) for h in range(2)])
    q, k, v, b, g = (w.f64(x) for x in ("q", "k", "v", "beta", "g"))
    acc = np.zeros(4)
    first = np.zeros(2)
    for n in range(3):
        P, L, s0 = int(w.prefix_lens[n]), int(w.seq_lens[n]), int(w.cu_seqlens[n])
        for h in range(2):
            S0 = None
            if P > 0:
                S0 = gpu["bound_post"][int(gpu["offsets"][n]) + (P + CHUNK - 1) // CHUNK - 1, h].astype(np.float64)
            sl = slice(s0 + P, s0 + L)
            r = orc.gdn_sequence(q[sl, h], k[sl, h], v[sl, h], b[sl, h], g[sl, h], prefix_len=0,
                                 flags=orc.QDQ_WRITE if flags & orc.QDQ_WRITE else 0, S0=S0)
            acc += [np.sum((gpu["o"][sl, h] - r["o"]) ** 2), np.sum(r["o"] ** 2),
                    np.sum((gpu["S"][n, h] - r["S"]) ** 2), np.sum(r["S"] ** 2)]
            first += [np.sum((gpu["o"][s0 + P, h] - r["o"][0]) ** 2), np.sum(r["o"][0] ** 2)]
    o_rel, s_rel = np.sqrt(acc[0] / acc[1]), np.sqrt(acc[2] / acc[3])
    first_rel = np.sqrt(first[0] / first[1])
    print(f"suffix from the handoff state: first token o_rel={first_rel:.3e}; whole suffix "
          f"o_rel={o_rel:.3e} S_rel={s_rel:.3e}", flush=True)
    assert first_rel <= TOL[gi.F32]
    if not flags & orc.QDQ_WRITE:
        assert o_rel <= TOL[gi.F32] and s_rel <= TOL[gi.F32]


@pytest.mark.parametrize("pc", [False, True])
@pytest.mark.parametrize("io", [gi.F32, gi.BF16])
def test_w_qdq_single_chunk_from_zero_state_changes_nothing(io, pc):
    """From the zero state a one-chunk sequence never meets W S^T: with W QDQ
    on the GPU gives the bits it gives with W QDQ off."""
    d = 64 if io == gi.F32 else 128
    w = gi.make_packed([64, 1, 40], 2, d, d, io_dtype=io, seed=51, per_channel=pc, g_scale=0.05)
    a = run_w_gpu(w, 3, record=False)
    b = run_w_gpu(w, 3 | GDN_QDQ_W, record=False)
    np.testing.assert_array_equal(a["o"], b["o"])
    np.testing.assert_array_equal(a["S"], b["S"])


@pytest.mark.parametrize("pc", [False, True])
def test_w_qdq_fused_equals_split(pc):
    """B=4, T=4096, H=16, d=128, bf16, state and W QDQ, scalar and
    per-channel gate: the fused launch (W formed on its producer workgroups)
    and the split one give the same bits, W records included."""
    w_dev = gi.device_packed([4096] * 4, 16, 128, 128, seed=53, per_channel=pc, g_scale=0.05)
    outs = []
    for sched in (GDN_SCHEDULE_SPLIT, GDN_SCHEDULE_FUSED):
        nan = float("nan")
        offs = torch.arange(0, 4 * 64 + 1, 64, dtype=torch.int32, device="cuda")
        dbg = dict(schedule=sched, bound_offsets=offs,
                   w_pre=torch.full((256, 16, 64, 128), nan, device="cuda"),
                   w_post=torch.full((256, 16, 64, 128), nan, device="cuda"))
        o, S = api.chunk_fwd(w_dev["q"], w_dev["k"], w_dev["v"], w_dev["beta"], w_dev["g"],
                             w_dev["cu_seqlens"], qdq_flags=3 | GDN_QDQ_W, o_dtype=torch.bfloat16,
                             debug=dbg)
        torch.cuda.synchronize()
        outs.append((o.clone(), S.clone(), dbg["w_pre"], dbg["w_post"]))
    assert torch.isfinite(outs[1][1]).all()
    for x, y, name in zip(outs[0], outs[1], ("o", "S", "w_pre", "w_post")):
        bx = x.view(torch.int16) if x.element_size() == 2 else x.view(torch.int32)
        by = y.view(torch.int16) if y.element_size() == 2 else y.view(torch.int32)
        diff = int((bx != by).sum())
        print(f"{name}: {diff} differing elements of {x.numel()}", flush=True)
        assert diff == 0


def test_w_qdq_full_size_sampled():
    """The GDN prefill workload at full size (B=4, T=4096, H=16, d=128, bf16,
    state and W QDQ) in the launch configuration the benchmark times: GW1-GW3
    on sampled chunks, read back from the device one at a time."""
    w = gi.make_packed([4096] * 4, 16, 128, 128, io_dtype=gi.BF16, seed=55)
    gpu = run_w_gpu_sampled(w, samples=[(0, 0, 0), (1, 5, 17), (2, 9, 40), (3, 15, 63), (3, 3, 62)])
    for (n, h, c), rec in gpu.items():
        q, k, v, b, g = (w.f64(x)[4096 * n + 64 * c: 4096 * n + 64 * c + 64, h]
                         for x in ("q", "k", "v", "beta", "g"))
        r = chunk_step(q, k, v, b, g, rec["S_in"], Wq=rec["w_post"].astype(np.float64))
        w_rel = rel_l2(rec["w_pre"], r["W"])
        want, _, _ = orc.qdq_rows(rec["w_pre"])
        w_bits = int(np.sum(want.view(np.uint32) != rec["w_post"].view(np.uint32)))
        o_rel, pre_rel = rel_l2(rec["o"], r["o"]), rel_l2(rec["pre"], r["S"])
        print(f"(n, h, c)=({n}, {h}, {c}): w_rel={w_rel:.3e} w_bits={w_bits} o_rel={o_rel:.3e} "
              f"pre_rel={pre_rel:.3e}", flush=True)
        assert w_rel <= TOL[gi.BF16] and w_bits == 0
        assert o_rel <= TOL[gi.BF16] and pre_rel <= TOL[gi.BF16]


def run_w_gpu_sampled(w, samples):
    d = gi.device_tensors(w)
    H, dk, dv = w.n_heads, w.dk, w.dv
    tot = 4 * 64
    nan = float("nan")
    dbg = dict(bound_offsets=torch.arange(0, tot + 1, 64, dtype=torch.int32, device="cuda"),
               bound_pre=torch.full((tot, H, dv, dk), nan, device="cuda"),
               bound_post=torch.full((tot, H, dv, dk), nan, device="cuda"),
               w_pre=torch.full((tot, H, 64, dk), nan, device="cuda"),
               w_post=torch.full((tot, H, 64, dk), nan, device="cuda"))
    o, S = api.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["cu_seqlens"],
                         qdq_flags=3 | GDN_QDQ_W, o_dtype=torch.bfloat16, debug=dbg)
    torch.cuda.synchronize()
    out = {}
    for (n, h, c) in samples:
        b = 64 * n + c
        out[(n, h, c)] = dict(
            S_in=(np.zeros((dv, dk)) if c == 0 else dbg["bound_post"][b - 1, h].cpu().numpy().astype(np.float64)),
            pre=dbg["bound_pre"][b, h].cpu().numpy(), w_pre=dbg["w_pre"][b, h].cpu().numpy(),
            w_post=dbg["w_post"][b, h].cpu().numpy(),
            o=np64(o[4096 * n + 64 * c: 4096 * n + 64 * c + 64, h]))
    return out
