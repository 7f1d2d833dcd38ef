"""The two schedules of the per-chunk solve give bit-identical results, for
the scalar gate and for a per-key-channel gate:
SPLIT runs it as its own kernel before the sequential state kernel, FUSED
inside the state kernel's launch on compute units the state workgroups leave
idle, each (chunk, head) record handed over through a ready flag.  The
parity tests of the other files run with the automatic choice (fused for
every workload whose state workgroups fill at most half of the GPU), so this
equality carries their oracle comparisons over to the split schedule, and
back for the workloads that split automatically."""
import time

import numpy as np
import pytest
import torch

from fp8_state_qat_amd import api
from fp8_state_qat_amd import inputs as gi
from fp8_state_qat_amd._lib import (GDN_ERR_DEVICE, GDN_ERR_INVALID_ARG, GDN_SCHEDULE_AUTO, GDN_SCHEDULE_FUSED,
                                    GDN_SCHEDULE_FUSED_NO_PRODUCERS, GDN_SCHEDULE_SPLIT, GdnError)

pytestmark = pytest.mark.gpu


def _run(d, flags, sched, *, o_dtype=None, seq_lens=None, prefix_lens=None, workspace=None):
    o, S = api.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["cu_seqlens"],
                         seq_lens=seq_lens, prefix_lens=prefix_lens, qdq_flags=flags,
                         o_dtype=o_dtype, workspace=workspace, debug={"schedule": sched})
    torch.cuda.synchronize()
    return o.clone(), S.clone()


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _same(a, b, what):
    for x, y, name in ((a[0], b[0], "o"), (a[1], b[1], "S")):
        diff = int((_bits(x) != _bits(y)).sum())
        print(f"{what} {name}: {diff} differing elements of {x.numel()}", flush=True)
        assert diff == 0


@pytest.mark.parametrize("flags", [0, 3])
def test_full_prefill_fused_equals_split(flags):
    """B=4, T=4096, H=16, d=128, bf16: 128 state workgroups, fused by default."""
    d = gi.device_packed([4096] * 4, 16, 128, 128, seed=11)
    split = _run(d, flags, GDN_SCHEDULE_SPLIT, o_dtype=torch.bfloat16)
    auto = _run(d, flags, GDN_SCHEDULE_AUTO, o_dtype=torch.bfloat16)
    assert torch.isfinite(auto[1]).all()
    _same(split, auto, f"full prefill flags={flags}")


@pytest.mark.parametrize("io,d", [(gi.F32, 64), (gi.BF16, 64), (gi.BF16, 128)])
def test_ragged_prefix_fused_equals_split(io, d):
    """Ragged lengths (empty, one token, chunk multiples and tails), padding
    rows and chunked prefixes shorter than the sequences."""
    w = gi.make_packed([300, 0, 1, 64, 129, 77], 3, d, d, io_dtype=io, seed=5 + d,
                       pads=[2, 0, 5, 0, 63, 1], prefix_lens=[256, 0, 1, 64, 100, 0])
    dt = gi.device_tensors(w)
    for flags in (0, 1, 2, 3):
        a = _run(dt, flags, GDN_SCHEDULE_SPLIT, o_dtype=torch.float32, seq_lens=dt["seq_lens"],
                 prefix_lens=dt["prefix_lens"])
        b = _run(dt, flags, GDN_SCHEDULE_FUSED, o_dtype=torch.float32, seq_lens=dt["seq_lens"],
                 prefix_lens=dt["prefix_lens"])
        _same(a, b, f"ragged {io} d={d} flags={flags}")


def test_forced_fusion_where_auto_splits():
    """192 state workgroups (more than half of the GPU): automatic splits,
    FUSED still fuses with the 64 compute units left; same bits."""
    d = gi.device_packed([1024, 700, 1024, 333], 24, 128, 128, seed=13)
    a = _run(d, 3, GDN_SCHEDULE_AUTO, o_dtype=torch.bfloat16)
    b = _run(d, 3, GDN_SCHEDULE_FUSED, o_dtype=torch.bfloat16)
    _same(a, b, "192 state workgroups")


def test_workspace_reuse_and_garbage():
    """Ready flags are cleared on every call: a workspace full of nonzero
    bytes, and one reused right after another fused call on other inputs,
    give the bits of a fresh split run."""
    d1 = gi.device_packed([2048, 1500], 8, 128, 128, seed=17)
    d2 = gi.device_packed([2048, 1500], 8, 128, 128, seed=19)
    ref = _run(d2, 3, GDN_SCHEDULE_SPLIT, o_dtype=torch.bfloat16)
    n = api.chunk_workspace_bytes(2, 8, 128, 128, 3548)
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")
    _same(ref, _run(d2, 3, GDN_SCHEDULE_FUSED, o_dtype=torch.bfloat16, workspace=ws), "garbage workspace")
    _run(d1, 3, GDN_SCHEDULE_FUSED, o_dtype=torch.bfloat16, workspace=ws)
    _same(ref, _run(d2, 3, GDN_SCHEDULE_FUSED, o_dtype=torch.bfloat16, workspace=ws), "reused workspace")
    # every (chunk, head) of the call after a sequence's first chunk was
    # produced and flagged: bit 0 ready, bits 4:1 the producer's XCD, bit 8 a
    # device-wide release (producer off its XCD, expected never); the first
    # chunk of each sequence is formed by its state workgroups and never
    # flagged (its flags stay as the call's offsets kernel cleared them)
    hdr = 256 + ((2 + 2) * 4 + 255) // 256 * 256   # status word; chunk offsets and the largest chunk count
    n_items = (32 + 24) * 8                    # (chunk, head) pairs of the call
    flags = ws[hdr:hdr + 4 * n_items].view(torch.int32).cpu().numpy()
    first = np.zeros((56, 8), dtype=bool)
    first[[0, 32], :] = True
    flags2 = flags.reshape(56, 8)
    assert np.all(flags2[first] == 0)
    assert np.all(flags2[~first] & 1 == 1) and np.all(flags >> 9 == 0)
    nh = np.concatenate([np.repeat(0, 32), np.repeat(1, 24)])[:, None] * 8 + np.arange(8)[None, :]
    home = (((flags2 >> 1) & 15) == nh % 8)[~first]
    print(f"producers on the XCD of their consumers: {int(home.sum())} of {home.size}; "
          f"released device-wide: {int((flags >> 8 & 1).sum())}", flush=True)


@pytest.mark.parametrize("flags", [0, 3])
def test_kda_full_prefill_fused_equals_split(flags):
    """Per-key-channel gate, B=4, T=4096, H=16, d=128, bf16: the per-channel
    prep items run on the producer workgroups of the fused launch."""
    d = gi.device_packed([4096] * 4, 16, 128, 128, per_channel=True, g_scale=0.05, seed=23)
    split = _run(d, flags, GDN_SCHEDULE_SPLIT, o_dtype=torch.bfloat16)
    auto = _run(d, flags, GDN_SCHEDULE_AUTO, o_dtype=torch.bfloat16)
    assert torch.isfinite(auto[1]).all()
    _same(split, auto, f"KDA full prefill flags={flags}")


@pytest.mark.parametrize("io,d", [(gi.F32, 64), (gi.BF16, 128)])
def test_kda_ragged_prefix_fused_equals_split(io, d):
    w = gi.make_packed([300, 0, 1, 64, 129, 77], 3, d, d, io_dtype=io, per_channel=True, g_scale=0.05,
                       seed=29 + d, pads=[2, 0, 5, 0, 63, 1], prefix_lens=[256, 0, 1, 64, 100, 0])
    dt = gi.device_tensors(w)
    for flags in (0, 3):
        a = _run(dt, flags, GDN_SCHEDULE_SPLIT, o_dtype=torch.float32, seq_lens=dt["seq_lens"],
                 prefix_lens=dt["prefix_lens"])
        b = _run(dt, flags, GDN_SCHEDULE_FUSED, o_dtype=torch.float32, seq_lens=dt["seq_lens"],
                 prefix_lens=dt["prefix_lens"])
        _same(a, b, f"KDA ragged {io} d={d} flags={flags}")


@pytest.mark.parametrize("per_channel", [False, True])
def test_fused_wait_runs_out_and_poisons(per_channel):
    """Failure path of the handoff, forced from the host: the fused launch
    with no producer workgroups, so no ready flag is ever set.  Each state
    workgroup's wait is bounded by the device's real-time clock (200 ms);
    when it runs out the workgroup carries on with NaN in its decay, so the
    launch ends and the final state of every (sequence, head) that waited is
    NaN instead of a silently wrong value.  With the scalar gate the state
    workgroups form each sequence's first chunk themselves, so the one-chunk
    sequence (64 tokens) waits for nothing and comes out finite.  A normal
    call afterwards is unaffected."""
    kw = dict(per_channel=True, g_scale=0.05) if per_channel else {}
    d = gi.device_packed([200, 64, 130], 2, 64, 64, seed=31, **kw)
    ws = torch.empty(api.chunk_workspace_bytes(3, 2, 64, 64, 394), dtype=torch.uint8, device="cuda")
    st = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    t0 = time.perf_counter()
    o, S = api.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["cu_seqlens"], qdq_flags=3,
                         o_dtype=torch.float32, workspace=ws,
                         debug={"schedule": GDN_SCHEDULE_FUSED_NO_PRODUCERS, "status": st})
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    assert int(st.item()) == 1   # the status word, copied out on the stream
    print(f"per_channel={per_channel}: call with no producers took {dt:.3f} s; "
          f"NaN state elements {int(torch.isnan(S).sum())} of {S.numel()}", flush=True)
    if per_channel:
        assert torch.isnan(S).all()
    else:
        assert torch.isnan(S[[0, 2]]).all() and torch.isfinite(S[1]).all()
    assert torch.isnan(o).any()
    assert dt < 30.0
    # the call returned GDN_OK (it was enqueued); its status word says what happened
    with pytest.raises(GdnError) as e:
        api.workspace_status(ws)
    assert e.value.status == GDN_ERR_DEVICE and "wait" in str(e.value)
    a = _run(d, 3, GDN_SCHEDULE_SPLIT, o_dtype=torch.float32, workspace=ws)
    api.workspace_status(ws)
    b = _run(d, 3, GDN_SCHEDULE_FUSED, o_dtype=torch.float32, workspace=ws)
    api.workspace_status(ws)   # cleared by the next call
    assert torch.isfinite(a[1]).all() and torch.isfinite(a[0]).all()
    _same(a, b, f"after the failed waits, per_channel={per_channel}")


BAD_INDEX_CASES = {
    "cu_seqlens decreasing": dict(cu=[0, 150, 80, 200]),
    "cu_seqlens beyond total_tokens": dict(cu=[0, 80, 150, 260]),
    "cu_seqlens negative": dict(cu=[-5, 80, 150, 200]),
    "length above its segment": dict(seq=[81, 70, 50]),
    "negative length": dict(seq=[-1, 70, 50]),
    "prefix above the length": dict(pre=[80, 71, 50]),
    "negative prefix": dict(pre=[80, -64, 50]),
}


@pytest.mark.parametrize("case", sorted(BAD_INDEX_CASES))
@pytest.mark.parametrize("sched", [GDN_SCHEDULE_SPLIT, GDN_SCHEDULE_AUTO])
def test_out_of_contract_index_arrays_run_nothing(case, sched):
    """Index arrays whose contents break the contract (checked on the device
    by the offsets kernel, before any other kernel reads them): every kernel
    of the call returns at once, o and the final state keep their contents,
    and the workspace's status word reports GDN_ERR_INVALID_ARG.  The next
    valid call on the same workspace runs normally."""
    c = BAD_INDEX_CASES[case]
    w = gi.make_packed([80, 70, 50], 2, 64, 64, io_dtype=gi.BF16, seed=37)
    d = gi.device_tensors(w)
    cu = torch.tensor(c.get("cu", [0, 80, 150, 200]), dtype=torch.int32, device="cuda")
    seq = torch.tensor(c["seq"], dtype=torch.int32, device="cuda") if "seq" in c else None
    pre = torch.tensor(c["pre"], dtype=torch.int32, device="cuda") if "pre" in c else None
    ws = torch.empty(api.chunk_workspace_bytes(3, 2, 64, 64, 200), dtype=torch.uint8, device="cuda")
    o = torch.full((200, 2, 64), 7.0, dtype=torch.float32, device="cuda")
    S = torch.full((3, 2, 64, 64), -3.0, dtype=torch.float32, device="cuda")
    for per_channel in (False, True):
        g = d["g"] if not per_channel else torch.full((200, 2, 64), -0.05, device="cuda")
        st = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        api.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], g, cu, seq_lens=seq, prefix_lens=pre, qdq_flags=3,
                      out=o, final_state=S, workspace=ws, debug={"schedule": sched, "status": st})
        with pytest.raises(GdnError) as e:
            api.workspace_status(ws)
        assert e.value.status == GDN_ERR_INVALID_ARG
        assert int(st.item()) == 2   # the same word, copied out on the stream
        assert bool((o == 7.0).all()) and bool((S == -3.0).all()), f"{case}: outputs were written"
    api.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["cu_seqlens"], qdq_flags=3, out=o,
                  final_state=S, workspace=ws, debug={"schedule": sched})
    api.workspace_status(ws)
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(S).all())


@pytest.mark.parametrize("case", sorted(k for k in BAD_INDEX_CASES if "pre" not in BAD_INDEX_CASES[k]))
def test_bwd_out_of_contract_index_arrays_run_nothing(case):
    """The same device-side index check guards the backward: nothing is
    written and the status word reports GDN_ERR_INVALID_ARG."""
    c = BAD_INDEX_CASES[case]
    w = gi.make_packed([80, 70, 50], 2, 64, 64, io_dtype=gi.BF16, seed=41)
    d = gi.device_tensors(w)
    cu = torch.tensor(c.get("cu", [0, 80, 150, 200]), dtype=torch.int32, device="cuda")
    seq = torch.tensor(c["seq"], dtype=torch.int32, device="cuda") if "seq" in c else None
    d_o = torch.ones((200, 2, 64), dtype=torch.bfloat16, device="cuda")
    d0 = torch.full((3, 2, 64, 64), 5.0, device="cuda")
    dv = torch.full((200, 2, 64), 9.0, device="cuda")
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    api.chunk_bwd_dh(d["q"], d["k"], d["beta"], d["g"], cu, d_o, seq_lens=seq, d_initial_state=d0, d_v=dv,
                     workspace=ws)
    with pytest.raises(GdnError) as e:
        api.workspace_status(ws)
    assert e.value.status == GDN_ERR_INVALID_ARG
    assert bool((d0 == 5.0).all()) and bool((dv == 9.0).all())
    api.chunk_bwd_dh(d["q"], d["k"], d["beta"], d["g"], d["cu_seqlens"], d_o, d_initial_state=d0, d_v=dv,
                     workspace=ws, check_status=True)
    assert bool(torch.isfinite(d0).all()) and not bool((d0 == 5.0).all())
