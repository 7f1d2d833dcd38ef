"""The prefill->decode handoff workload at full size (256 sequences, H=32,
dk=dv=128, bf16, 2048-token chunked prefix with QDQ, then decode steps with
a QDQ on every write), drawn on the device as the benchmark draws it.

The prefill is checked through a slice (sequences 0..15 and 255 packed on
their own): outputs and final states of the slice are bit-identical to the
full call (per-sequence independence), and the slice is checked against the
oracle teacher-forced per boundary on sampled (sequence, head) pairs.  Each
decode step is checked teacher-forced on sampled pairs: from the GPU's state
before the step, the oracle's output and pre-QDQ state (2e-3) and the
GPU's post-QDQ state = the oracle's QDQ of the GPU's pre-QDQ state, bit for
bit."""
import numpy as np
import pytest

from fp8_state_qat_amd import inputs as gi
from oracle import oracle as orc

from helpers import TOL, np64, rel_l2, teacher_forced

pytestmark = pytest.mark.gpu

N, H, PL, D = 256, 32, 2048, 128


def _bits(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def test_full_size_handoff_sampled():
    import torch
    from fp8_state_qat_amd import api
    dev = torch.device("cuda:0")
    pd = gi.device_packed([PL] * N, H, D, D, seed=4, device=dev)
    o = torch.empty((N * PL, H, D), dtype=torch.bfloat16, device=dev)
    state = torch.empty((N, H, D, D), dtype=torch.float32, device=dev)
    api.chunk_fwd(pd["q"], pd["k"], pd["v"], pd["beta"], pd["g"], pd["cu_seqlens"], qdq_flags=3,
                  out=o, final_state=state)
    torch.cuda.synchronize()

    # ---- the slice: sequences 0..15 and 255 on their own, with the per-boundary record
    seqs = list(range(16)) + [N - 1]
    rows = torch.cat([torch.arange(n * PL, (n + 1) * PL, device=dev) for n in seqs])
    sl = {k: pd[k][rows].contiguous() for k in ("q", "k", "v", "beta", "g")}
    ns = len(seqs)
    cu = torch.arange(0, (ns + 1) * PL, PL, dtype=torch.int32, device=dev)
    nb = PL // 64
    dbg = dict(bound_offsets=torch.arange(0, (ns + 1) * nb, nb, dtype=torch.int32, device=dev),
               bound_pre=torch.empty((ns * nb, H, D, D), device=dev),
               bound_post=torch.empty((ns * nb, H, D, D), device=dev),
               scales=torch.empty((ns * nb, H, D // 64), device=dev))
    o_s, S_s = api.chunk_fwd(sl["q"], sl["k"], sl["v"], sl["beta"], sl["g"], cu, qdq_flags=3,
                             o_dtype=torch.bfloat16, debug=dbg)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o[rows]), "slice outputs differ from the full call"
    assert torch.equal(S_s, state[seqs]), "slice final states differ from the full call"

    w = gi.Workload(q=_bits(sl["q"]), k=_bits(sl["k"]), v=_bits(sl["v"]),
                    beta=sl["beta"].cpu().numpy(), g=sl["g"].cpu().numpy(),
                    cu_seqlens=cu.cpu().numpy(), seq_lens=np.full(ns, PL, np.int32),
                    prefix_lens=np.full(ns, PL, np.int32), io_dtype=gi.BF16, n_heads=H, dk=D, dv=D)
    pairs = [(0, 0), (7, 13), (15, 31), (ns - 1, 20)]
    gpu = {"o": np64(o_s), "offsets": dbg["bound_offsets"].cpu().numpy()}
    for key in ("bound_pre", "bound_post", "scales"):
        gpu[key] = np.zeros((ns * nb, H) + tuple(dbg[key].shape[2:]), np.float32)
        for (n, h) in pairs:  # copy only the sampled pairs' records
            gpu[key][n * nb:(n + 1) * nb, h] = dbg[key][n * nb:(n + 1) * nb, h].cpu().numpy()
    r = teacher_forced(w, gpu, 3, pairs)
    print("prefill G2 sampled", r, flush=True)
    assert r["o_rel"] <= TOL[gi.BF16] and r["pre_rel"] <= TOL[gi.BF16]
    assert r["gpu_code_mismatch"] == 0 and r["scale_mismatch"] == 0
    del dbg, sl, o_s, pd, o
    torch.cuda.empty_cache()

    # ---- decode steps at full size, teacher-forced per step on sampled pairs
    tok = gi.device_decode_tokens(N, H, D, D, 3, seed=5, device=dev)
    dpairs = [(0, 0), (100, 7), (255, 31)]
    pre = torch.empty_like(state)
    sc = torch.empty((N, H, D // 64), device=dev)
    for i in range(3):
        before = {p: state[p[0], p[1]].double().cpu().numpy() for p in dpairs}
        od = api.decode_step(tok["q"][i], tok["k"][i], tok["v"][i], tok["beta"][i], tok["g"][i], state,
                             qdq=True, state_pre=pre, scales=sc)
        torch.cuda.synchronize()
        for (n, h) in dpairs:
            f = lambda x: x[i, n, h].float().cpu().numpy().astype(np.float64)[None]
            ref = orc.gdn_sequence(f(tok["q"]), f(tok["k"]), f(tok["v"]), f(tok["beta"]), f(tok["g"]),
                                   prefix_len=0, flags=orc.QDQ_WRITE, S0=before[(n, h)], record=False)
            o_rel = rel_l2(np64(od[n, h]), ref["o"][0])
            pre_gpu = pre[n, h].cpu().numpy()
            # the oracle's pre-QDQ state of this step is its recurrence before the QDQ
            ref_pre = orc.gdn_sequence(f(tok["q"]), f(tok["k"]), f(tok["v"]), f(tok["beta"]), f(tok["g"]),
                                       prefix_len=0, flags=0, S0=before[(n, h)])["S"]
            pre_rel = rel_l2(pre_gpu, ref_pre)
            want, wsc, _ = orc.qdq_states(pre_gpu)
            print(f"decode step {i} pair {(n, h)} o_rel={o_rel:.3e} pre_rel={pre_rel:.3e}", flush=True)
            assert o_rel <= TOL[gi.BF16] and pre_rel <= TOL[gi.BF16]
            assert np.array_equal(want.view(np.uint32), state[n, h].cpu().numpy().view(np.uint32))
            assert np.array_equal(wsc, sc[n, h].cpu().numpy())
