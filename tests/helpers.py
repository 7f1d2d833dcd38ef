"""Shared plumbing for the GPU parity tests: run the HIP path through the C
ABI on seeded inputs, run the oracle on the same inputs, compare."""
from __future__ import annotations

import numpy as np

from fp8_state_qat_amd import inputs as gi
from oracle import oracle as orc

CHUNK = 64


def rel_l2(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def np64(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def n_bounds(prefix_lens):
    return [(int(p) + CHUNK - 1) // CHUNK for p in prefix_lens]


def suffix_offsets(w: gi.Workload):
    """[N + 1] prefix sums of the suffix lengths L_n - P_n."""
    offs = np.zeros(w.n_seqs + 1, np.int32)
    offs[1:] = np.cumsum(np.asarray(w.seq_lens, np.int64) - np.asarray(w.prefix_lens, np.int64))
    return offs


def run_chunk_gpu(w: gi.Workload, flags, *, o_dtype=None, record=False, initial_state=None,
                  use_prefix=True, use_seq_lens=True, suffix_record=False, schedule=None, grid_log2=0):
    """Run gdn_chunk_fwd on workload w; returns numpy dict (o, S and, when
    record, bound_pre/bound_post/scales [nb_total, H, dv(/64), dk]; when
    suffix_record, suffix_pre/suffix_post [n_suffix, H, dv, dk] and
    suffix_offsets).  The call's status word is checked."""
    import torch
    from fp8_state_qat_amd import api
    d = gi.device_tensors(w)
    H, dk, dv = w.n_heads, w.dk, w.dv
    dbg = None
    nb = n_bounds(w.prefix_lens)
    offs = np.zeros(len(nb) + 1, np.int32)
    offs[1:] = np.cumsum(nb)
    soffs = suffix_offsets(w)
    if record or suffix_record or schedule is not None:
        dbg = {}
    if schedule is not None:
        dbg["schedule"] = schedule
    if record:
        tot = int(offs[-1])
        dbg.update(bound_offsets=torch.from_numpy(offs).cuda(),
                   bound_pre=torch.full((tot, H, dv, dk), np.nan, device="cuda"),
                   bound_post=torch.full((tot, H, dv, dk), np.nan, device="cuda"),
                   scales=torch.full((tot, H, dv // 64), np.nan, device="cuda"))
    if suffix_record:
        ns = int(soffs[-1])
        dbg.update(suffix_offsets=torch.from_numpy(soffs).cuda(),
                   suffix_pre=torch.full((ns, H, dv, dk), np.nan, device="cuda"),
                   suffix_post=torch.full((ns, H, dv, dk), np.nan, device="cuda"))
    init = None if initial_state is None else torch.from_numpy(
        np.ascontiguousarray(initial_state, np.float32)).cuda()
    o_dt = None if o_dtype is None else {"f32": torch.float32, "bf16": torch.bfloat16}[o_dtype]
    o, S = api.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["cu_seqlens"],
                         seq_lens=d["seq_lens"] if use_seq_lens else None,
                         prefix_lens=d["prefix_lens"] if use_prefix else None,
                         initial_state=init, qdq_flags=flags, o_dtype=o_dt, debug=dbg,
                         check_status=True, gate_grid_log2=grid_log2)
    torch.cuda.synchronize()
    res = {"o": np64(o), "S": S.cpu().numpy(), "offsets": offs, "suffix_offsets": soffs}
    if record:
        for key in ("bound_pre", "bound_post", "scales"):
            res[key] = dbg[key].cpu().numpy()
    if suffix_record:
        for key in ("suffix_pre", "suffix_post"):
            res[key] = dbg[key].cpu().numpy()
    return res


def run_chunk_oracle(w: gi.Workload, flags, *, pairs=None, threads=8, initial_state=None,
                     record=False):
    return orc.gdn_packed(w.f64("q"), w.f64("k"), w.f64("v"), w.f64("beta"), w.f64("g"),
                          w.cu_seqlens, seq_lens=w.seq_lens, prefix_lens=w.prefix_lens,
                          flags=flags, S0=None if initial_state is None else
                          np.asarray(initial_state, np.float64),
                          pairs=pairs, threads=threads, record=record)


def _midpoint_gap(y):
    grid = orc.e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = (grid[1:] + grid[:-1]) / 2
    a = np.abs(np.asarray(y, np.float64)).ravel()
    i = np.clip(np.searchsorted(mids, a), 1, len(mids) - 1)
    return a, np.minimum(np.abs(a - mids[i - 1]), np.abs(a - mids[i]))


def midpoint_distance(y):
    """Distance of code-domain values y = x / s (fp64) to the nearest E4M3
    rounding midpoint, relative to the value itself: |y - mid| / |y|.  A code
    mismatch between the oracle and the GPU is allowed only where this is at
    most 1e-6 (both sides are then right: the decision sits within the
    arithmetic's error of a tie)."""
    a, d = _midpoint_gap(y)
    return d / np.maximum(a, np.finfo(np.float64).tiny)


def midpoint_distance_range(y):
    """The same distance relative to the tile's range (|y - mid| / 448); a
    diagnostic printed beside the gated figure."""
    _, d = _midpoint_gap(y)
    return d / 448.0


def canon_codes(c):
    """E4M3 codes with the two zeros (0x00, 0x80) taken as one value: a state
    element that rounds to zero is zero whatever the sign of its tiny
    pre-QDQ value."""
    c = np.asarray(c, np.uint8)
    return np.where((c & 0x7F) == 0, np.uint8(0), c)


def code_mismatch_stats(out, codes_orc, codes_gpu, y_orc):
    """Accumulate the oracle-versus-GPU code comparison of one QDQ into out:
    codes compared, mismatches, and among the mismatches those farther than
    1e-6 from a rounding midpoint relative to the tile's range
    (far_range, gated) and relative to the value itself (far_rel, reported)."""
    mism = canon_codes(codes_orc) != canon_codes(codes_gpu)
    out["codes"] += codes_orc.size
    out["oracle_code_mismatch"] += int(mism.sum())
    if mism.any():
        yr = y_orc[mism]
        d_rel = midpoint_distance(yr)
        d_rng = midpoint_distance_range(yr)
        out["oracle_mismatch_far"] += int((d_rng > 1e-6).sum())
        out["oracle_mismatch_far_rel"] += int((d_rel > 1e-6).sum())
        out["oracle_mismatch_max_dist"] = max(out["oracle_mismatch_max_dist"], float(d_rng.max()))
        out["oracle_mismatch_max_dist_rel"] = max(out["oracle_mismatch_max_dist_rel"], float(d_rel.max()))


def _code_fields():
    return dict(oracle_code_mismatch=0, oracle_mismatch_far=0, oracle_mismatch_far_rel=0,
                oracle_mismatch_max_dist=0.0, oracle_mismatch_max_dist_rel=0.0, codes=0)


def teacher_forced(w: gi.Workload, gpu, flags, pairs, *, initial_state=None):
    """G2: for every chunk of every (n, h) in pairs, restart the oracle from
    the GPU's post-QDQ boundary state and run that one chunk.  Returns the
    rel-L2 of o and of the pre-QDQ states over all those chunks (o_rel,
    pre_rel), the worst single chunk (o_rel_max, pre_rel_max) and the code
    mismatch counts."""
    q, k, v, b, g = (w.f64(x) for x in ("q", "k", "v", "beta", "g"))
    cu, offs = w.cu_seqlens, gpu["offsets"]
    out = dict(o_rel=0.0, pre_rel=0.0, o_rel_max=0.0, pre_rel_max=0.0, gpu_code_mismatch=0,
               scale_mismatch=0, **_code_fields())
    acc = np.zeros(4)   # sum |o err|^2, |o ref|^2, |pre err|^2, |pre ref|^2
    for (n, h) in pairs:
        P = int(w.prefix_lens[n])
        s0 = int(cu[n])
        for c in range((P + CHUNK - 1) // CHUNK):
            bidx = int(offs[n]) + c
            t0, t1 = c * CHUNK, min(P, (c + 1) * CHUNK)
            if c == 0:
                S0 = None if initial_state is None else np.asarray(initial_state[n, h], np.float64)
            else:
                S0 = gpu["bound_post"][bidx - 1, h].astype(np.float64)
            sl = slice(s0 + t0, s0 + t1)
            gg = g[sl, h] if g.ndim == 2 else g[sl, h, :]
            # this chunk alone: its end is a boundary; CHUNK QDQ there iff the
            # full run quantizes after this chunk
            last = (c == (P + CHUNK - 1) // CHUNK - 1)
            qdq_here = bool(flags & orc.QDQ_CHUNK) or (bool(flags & orc.QDQ_WRITE) and last)
            r = orc.gdn_sequence(q[sl, h], k[sl, h], v[sl, h], b[sl, h], gg,
                                 flags=orc.QDQ_CHUNK if qdq_here else 0, S0=S0, record=True)
            pre_gpu = gpu["bound_pre"][bidx, h]
            out["o_rel_max"] = max(out["o_rel_max"], rel_l2(gpu["o"][sl, h], r["o"]))
            out["pre_rel_max"] = max(out["pre_rel_max"], rel_l2(pre_gpu, r["bound_pre"][0]))
            acc += [np.sum((gpu["o"][sl, h] - r["o"]) ** 2), np.sum(r["o"] ** 2),
                    np.sum((pre_gpu - r["bound_pre"][0]) ** 2), np.sum(r["bound_pre"][0] ** 2)]
            if qdq_here:
                want, sc, codes_gpu_pre = orc.qdq_states(pre_gpu.astype(np.float32))
                out["gpu_code_mismatch"] += int(np.sum(want.view(np.uint32) !=
                                                       gpu["bound_post"][bidx, h].view(np.uint32)))
                out["scale_mismatch"] += int(np.sum(sc != gpu["scales"][bidx, h]))
                # the oracle's own decision on its own pre-QDQ state
                _, sc_o, codes_orc = orc.qdq_states(r["bound_pre"][0].astype(np.float32))
                scale = np.repeat(sc_o, 64, axis=0)[:, None] * np.ones_like(pre_gpu)
                code_mismatch_stats(out, codes_orc, codes_gpu_pre, r["bound_pre"][0] / scale.astype(np.float64))
    out["o_rel"] = float(np.sqrt(acc[0] / max(acc[1], 1e-300)))
    out["pre_rel"] = float(np.sqrt(acc[2] / max(acc[3], 1e-300)))
    return out


# G1 / G2 gates (rel-L2 over valid rows)
TOL = {gi.F32: 1e-5, gi.BF16: 2e-3}


def valid_rows(w):
    m = np.zeros(w.total_tokens, bool)
    for n in range(w.n_seqs):
        m[w.cu_seqlens[n]:w.cu_seqlens[n] + w.seq_lens[n]] = True
    return m


def check_g1(w, gpu, ref, tol):
    m = valid_rows(w)
    o_rel = rel_l2(gpu["o"][m], ref["o"][m])
    s_rel = rel_l2(gpu["S"], ref["S"])
    print(f"G1 o_rel={o_rel:.3e} S_rel={s_rel:.3e} tol={tol}", flush=True)
    assert o_rel <= tol and s_rel <= tol
    # padding rows are zero
    assert np.all(gpu["o"][~m] == 0)


def check_g2(w, gpu, flags, tol, initial_state=None, codes=None):
    pairs = [(n, h) for n in range(w.n_seqs) for h in range(w.n_heads)]
    r = teacher_forced(w, gpu, flags, pairs, initial_state=initial_state)
    print("G2", r, flush=True)
    assert r["o_rel"] <= tol and r["pre_rel"] <= tol
    assert r["gpu_code_mismatch"] == 0 and r["scale_mismatch"] == 0
    check_codes(r, **(codes or {}))
    return r


# The per-key-channel gate kernel feeds its per-channel operands (K and Q
# scaled by the in-chunk decay, T, X, U') to the MFMA as two bf16 planes (16
# significant bits), which puts its pre-QDQ state about 4e-6 from fp64 and
# its code mismatch rate at 1.5-4e-4 (measured); the scalar-gate kernel
# carries T, X and U' as three planes and stays near 1e-5.  The per-channel
# gate is gated at the rate it reaches, with the distance to a midpoint
# within 1e-5 of the tile's range.
KDA_CODES = dict(cap=5e-4, far_tol=1e-5)


def check_codes(r, cap=1e-4, far_tol=1e-6):
    """The oracle's own E4M3 codes (on its pre-QDQ state) against the GPU's:
    at most 1e-4 of them differ, and every difference lies within 1e-6 of a
    rounding midpoint, measured against the tile's range (|y - mid| <= 1e-6 *
    448, y = x / s).  The same distance relative to the value itself is
    reported (far_rel): an fp32 computation of the state carries an error of
    about 1e-7 of the tile's range on every element, so a near-midpoint
    decision on a small element can sit farther than 1e-6 |y| from the tie
    with both sides correctly rounded from their own arithmetic."""
    import os
    if r["codes"]:
        print(f"CODES mismatch {r['oracle_code_mismatch']} of {r['codes']} "
              f"({r['oracle_code_mismatch'] / r['codes']:.2e}), far(range) {r['oracle_mismatch_far']}, "
              f"far(|y|) {r['oracle_mismatch_far_rel']}, max dist range {r['oracle_mismatch_max_dist']:.2e} "
              f"|y| {r['oracle_mismatch_max_dist_rel']:.2e}", flush=True)
        if os.environ.get("GDN_REPORT_CODES"):
            return
        assert r["oracle_code_mismatch"] <= cap * r["codes"], r
        if far_tol == 1e-6:
            assert r["oracle_mismatch_far"] == 0, r
        else:
            assert r["oracle_mismatch_max_dist"] <= far_tol, r


def suffix_teacher_forced(w: gi.Workload, gpu, flags, pairs, *, initial_state=None, grid_log2=0):
    """Teacher-forced check of the recurrent suffix (tokens P_n < t <= L_n),
    one token at a time like the decode step: token t restarts the oracle
    from the GPU's own state after token t - 1 (its post-QDQ record; for the
    first suffix token the handoff state: the last prefix boundary's post-QDQ
    record, or the initial state when P_n = 0) and runs that one token with
    no QDQ.  Compared: o_t and the pre-QDQ state (rel-L2 over all tokens, and
    the worst token); the GPU's post-QDQ state = the oracle's QDQ of the
    GPU's pre-QDQ state bit for bit (when the suffix quantizes; else post =
    pre); the oracle's own codes on its own pre-QDQ state against the GPU's.
    grid_log2: the log-retention grid of the recurrent writes."""
    q, k, v, b, g = (w.f64(x) for x in ("q", "k", "v", "beta", "g"))
    cu, offs, soffs = w.cu_seqlens, gpu["offsets"], gpu["suffix_offsets"]
    qdq = bool(flags & orc.QDQ_WRITE)
    out = dict(o_rel=0.0, pre_rel=0.0, o_rel_max=0.0, pre_rel_max=0.0, gpu_code_mismatch=0, tokens=0,
               **_code_fields())
    acc = np.zeros(4)
    for (n, h) in pairs:
        P, L, s0 = int(w.prefix_lens[n]), int(w.seq_lens[n]), int(cu[n])
        for t in range(P, L):
            si = int(soffs[n]) + t - P
            if t > P:
                S0 = gpu["suffix_post"][si - 1, h].astype(np.float64)
            elif P > 0:
                S0 = gpu["bound_post"][int(offs[n]) + (P + CHUNK - 1) // CHUNK - 1, h].astype(np.float64)
            else:
                S0 = None if initial_state is None else np.asarray(initial_state[n, h], np.float64)
            row = s0 + t
            gg = g[row:row + 1, h] if g.ndim == 2 else g[row:row + 1, h, :]
            r = orc.gdn_sequence(q[row:row + 1, h], k[row:row + 1, h], v[row:row + 1, h], b[row:row + 1, h],
                                 gg, prefix_len=0, flags=0, S0=S0, grid_log2=grid_log2)
            pre_gpu, post_gpu = gpu["suffix_pre"][si, h], gpu["suffix_post"][si, h]
            o_gpu = gpu["o"][row, h]
            out["o_rel_max"] = max(out["o_rel_max"], rel_l2(o_gpu, r["o"][0]))
            out["pre_rel_max"] = max(out["pre_rel_max"], rel_l2(pre_gpu, r["S"]))
            acc += [np.sum((o_gpu - r["o"][0]) ** 2), np.sum(r["o"][0] ** 2),
                    np.sum((pre_gpu - r["S"]) ** 2), np.sum(r["S"] ** 2)]
            out["tokens"] += 1
            if qdq:
                want, _, codes_gpu_pre = orc.qdq_states(pre_gpu.astype(np.float32))
                out["gpu_code_mismatch"] += int(np.sum(want.view(np.uint32) != post_gpu.view(np.uint32)))
                _, sc_o, codes_orc = orc.qdq_states(r["S"].astype(np.float32))
                scale = np.repeat(sc_o, 64, axis=0)[:, None] * np.ones_like(pre_gpu)
                code_mismatch_stats(out, codes_orc, codes_gpu_pre, r["S"] / scale.astype(np.float64))
            else:
                out["gpu_code_mismatch"] += int(np.sum(pre_gpu.view(np.uint32) != post_gpu.view(np.uint32)))
    out["o_rel"] = float(np.sqrt(acc[0] / max(acc[1], 1e-300)))
    out["pre_rel"] = float(np.sqrt(acc[2] / max(acc[3], 1e-300)))
    return out


def check_prefix_suffix(w, gpu, flags, tol, pairs=None, initial_state=None, codes=None, grid_log2=0):
    """Prefix P_n then recurrent suffix up to L_n, both teacher-forced: the
    chunked prefix per boundary (G2), the suffix per token from the GPU's own
    records (suffix_teacher_forced).  gpu must hold the boundary record and
    the suffix record."""
    if pairs is None:
        pairs = [(n, h) for n in range(w.n_seqs) for h in range(w.n_heads)]
    pre_pairs = [p for p in pairs if int(w.prefix_lens[p[0]]) > 0]
    if pre_pairs:
        r = teacher_forced(w, gpu, flags, pre_pairs, initial_state=initial_state)
        print("G2 prefix", r, flush=True)
        assert r["o_rel"] <= tol and r["pre_rel"] <= tol
        assert r["gpu_code_mismatch"] == 0 and r["scale_mismatch"] == 0
        check_codes(r, **(codes or {}))
    r = suffix_teacher_forced(w, gpu, flags, pairs, initial_state=initial_state, grid_log2=grid_log2)
    print("suffix, teacher-forced per token", r, flush=True)
    assert r["o_rel"] <= tol and r["pre_rel"] <= tol
    assert r["gpu_code_mismatch"] == 0
    check_codes(r)
    return r
