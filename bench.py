#!/usr/bin/env python3
"""Benchmark of the gated delta rule hot path on one MI355X.

One step = one gdn_chunk_fwd call over the GDN prefill workload (B=4,
T=4096, H=16, dk=dv=128, bf16 q/k/v and o, fp32 state, FP8-E4M3 state QDQ
at every 64-token boundary and at the end): a small chunk-offsets kernel,
then one launch in which 128 producer workgroups form the per-chunk records
(gates, K K^T, the exact solve, P) while the 128 state workgroups run the
sequential part (U', O, the state update and the boundary QDQ) and consume
them.  Inputs are resident in HBM before the timed region.  The roofline
object covers that launch, timed with HIP events recorded around it by the
library; the split schedule (prep kernel, then the state kernel alone) is
timed too and reported beside it.

Timing: warmup steps, then exactly --steps steps between synchronizations
(the headline value); per-launch HIP events give the mean (the roofline's
average launch) and the median; a MALL-flushed median writes 512 MiB before
each trial.  After every timed loop the workspace status word must be clean
and the outputs finite.

Also reported: the same prefill with W QDQ on top (each row of the
WY-transformed W quantized to FP8 E4M3 before W S^T); the packed varlen
workload at full size (16 sequences, lengths U{1..8192} plus padding); the
backward state recurrence on the prefill shape; the same prefill with a
per-key-channel gate (KDA-style g [T, H, dk]) as tokens/s and its launch's
time; the prefill->decode handoff workload (256 sequences, H=32, d=128:
2048-token chunked prefix with QDQ, then 512 single-token decode steps each
writing the state through per-tile QDQ) as decode-step HBM GB/s (and the
same steps with the INT8 block-32 codec), and the CPU oracle's throughput
on the prefill workload (all 64 (sequence, head) pairs by default) on the
cores this process may use (at most 16) and on one thread, with the host's
CPU model.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
T_RECORD_BYTES = 18432         # per (chunk, head): T = (I + A)^-1 diag(beta) as hi, mid, lo bf16 planes
P_RECORD_BYTES = 12288         # per (chunk, head): the decayed, masked P = Q K^T as hi + lo bf16 planes
BF16_MFMA_PEAK_TFLOPS = 2516.6 # MI355X dense bf16 MFMA, TFLOP/s
# MI355X fp32 vector ALU: 256 CUs x 4 SIMDs x 16 lanes x 2 (FMA) x 2 (packed fp32) x 2.4 GHz;
# without packed fp32 instructions (not used here) the ceiling is half of it
FP32_VALU_PEAK_TFLOPS = 157.3
METRIC = "GDN chunked-prefill tokens/s + MFMA %peak; decode step HBM GB/s, 1×MI355X"


def flops_per_token_head(C, dk, dv):
    """Algorithmic flops of the chunked forward per token and head (dense
    64x64 tiles): K K^T, W, Q K^T (2C dk each), U, P U' (2C dv each), W S^T,
    Q S^T, U'^T K (2 dk dv each) and the solve (C^2 / 3)."""
    return 2 * C * (3 * dk + 2 * dv) + 6 * dk * dv + C * C / 3


def state_kernel_flops_per_token_head(C, dk, dv):
    """The part of flops_per_token_head done by the sequential state kernel:
    everything but K K^T and the solve, which the parallel prep kernel does."""
    return flops_per_token_head(C, dk, dv) - 2 * C * dk - C * C / 3


def prefill_bytes(T_heads, n_states, dk, dv, io_bytes, o_bytes, gate_floats=1):
    """Algorithmic HBM bytes of one prefill call: q, k, v read once, beta
    and g read once, o written once, the final state written once."""
    per = io_bytes * (2 * dk + dv) + 4 * (1 + gate_floats) + o_bytes * dv
    return T_heads * per + n_states * dv * dk * 4


def split_state_kernel_bytes(T_heads, n_chunk_heads, n_states, dk, dv, io_bytes, o_bytes):
    """Algorithmic HBM bytes of the sequential state kernel: the prefill bytes
    plus one read of the two per-chunk records the prep kernel writes (T,
    18 KiB, and P, 12 KiB, per chunk and head)."""
    return (prefill_bytes(T_heads, n_states, dk, dv, io_bytes, o_bytes)
            + n_chunk_heads * (T_RECORD_BYTES + P_RECORD_BYTES))


def bwd_flops_per_token_head(C, dk, dv):
    """Algorithmic flops of the backward state recurrence per token and head
    (dense 64x64 tiles): K K^T and Q K^T for A and P (2C dk each), the solve
    (C^2 / 3), K dh^T (2 dk dv), P^T dO and T^T dU' (2C dv each), and the two
    update products Q^T (e dO), K^T (e Y) (2 dk dv each)."""
    return 2 * C * (2 * dk + 2 * dv) + 6 * dk * dv + C * C / 3


def bwd_bytes(T_heads, n_chunk_heads, n_states, dk, dv, io_bytes):
    """Algorithmic HBM bytes of the backward state recurrence: q, k, dO
    read once, beta and g read once, the fp32 value gradient written once,
    dh written once per chunk, the final state's gradient read and the
    initial state's written."""
    return (T_heads * (io_bytes * (2 * dk + dv) + 8 + 4 * dv) + n_chunk_heads * dv * dk * 4
            + 2 * n_states * dv * dk * 4)


def decode_bytes(n_heads_seqs, dk, dv, io_bytes, o_bytes):
    """Per decode step: the fp32 state read and written once, q, k, v read,
    beta and g read, o written."""
    return n_heads_seqs * (2 * 4 * dv * dk + io_bytes * (2 * dk + dv) + 8 + o_bytes * dv)


# the sources of the headline launch (its traffic summary is keyed by their hash)
PREFILL_SOURCES = ("gdn_chunk_bf16.hip", "gdn_chunk.hip", "gdn_chunk_common.hpp", "gdn_device.hpp",
                   "gdn_prep_item.hpp")


def copy_calibration(dev, mib):
    """One plain device copy of mib MiB (the PMC byte counters read for it
    calibrate those of the kernels).  Returns the bytes copied."""
    import torch
    n = mib * (1 << 20) // 4
    a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    return n * 4


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def med(xs):
    return float(np.median(np.asarray(xs, np.float64)))


def time_flushed(fn, events, trials, flush):
    """MALL-flushed timing: before each trial a 512 MiB buffer is written
    (more than the 256 MB MALL), so the call finds none of its inputs in the
    last-level cache; returns the per-trial durations (ms) of the launch
    bracketed by the (start, end) event pairs the call records."""
    import torch
    out = []
    for i in range(trials):
        flush.zero_()
        torch.cuda.synchronize()
        fn(events[i])
        torch.cuda.synchronize()
        out.append(events[i][0].elapsed_time(events[i][1]))
    return out


def check_outputs(api, ws, *tensors):
    """After a timed loop: the workspace's status word is clean and every
    output is finite (a run that went wrong must not yield a number)."""
    import torch
    if ws is not None:
        api.workspace_status(ws)
    for t in tensors:
        if not bool(torch.isfinite(t).all()):
            raise RuntimeError("non-finite output after the timed loop")


def host_info():
    """Cores this process may use, the machine's logical CPUs, and the CPU model."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return {"nproc": os.cpu_count(), "usable": usable, "model": model}


def time_launches(fn, steps, warmup):
    """Warm up, then time exactly `steps` calls between synchronizations with
    HIP events on torch's current stream (the stream the library launches
    on).  Returns (total ms, per-call ms list)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for i in range(steps):
        fn()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    total = evs[0].elapsed_time(evs[-1])
    print(f"timed {steps} calls of {getattr(fn, '__name__', 'step')}: {total / max(steps, 1):.4f} ms each",
          file=sys.stderr, flush=True)
    return total, per


def cpu_baseline(w, flags, n_pairs, threads, repeats):
    """The oracle (plain fp64 recurrence with QDQ) over `n_pairs` (sequence,
    head) pairs of the prefill workload, run `repeats` times."""
    from oracle import oracle as orc
    pairs = [(n, h) for n in range(w.n_seqs) for h in range(w.n_heads)][:n_pairs]
    q, k, v, b, g = (w.f64(x) for x in ("q", "k", "v", "beta", "g"))
    t0 = time.perf_counter()
    for _ in range(repeats):
        orc.gdn_packed(q, k, v, b, g, w.cu_seqlens, seq_lens=w.seq_lens,
                       prefix_lens=w.prefix_lens, flags=flags, pairs=pairs, threads=threads)
    dt = time.perf_counter() - t0
    token_heads = repeats * sum(int(w.seq_lens[n]) for n, _ in pairs)
    return {"value": token_heads / w.n_heads / dt, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{len(pairs)} of {w.n_seqs * w.n_heads} (sequence, head) pairs x "
                      f"{int(w.seq_lens[0])} tokens of the prefill workload, run {repeats} times, "
                      f"QDQ on, fp64 recurrence; token-heads/s divided by H={w.n_heads}; "
                      f"{dt:.1f} s wall on {threads} threads"}


def launch_stats(pairs):
    """Mean and median (ms) of the durations between (start, end) event pairs."""
    xs = [e0.elapsed_time(e1) for e0, e1 in pairs]
    return float(np.mean(xs)), med(xs)


def load_traffic(kernel_key, src_hash):
    """HBM traffic per launch from a committed rocprofv3 PMC summary, if the
    kernel source has not changed since the counters were taken."""
    p = os.path.join(ROOT, "profiles", f"{kernel_key}_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("source_hash") != src_hash:
        return None
    return d.get("traffic_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-kda", action="store_true")
    ap.add_argument("--no-varlen", action="store_true")
    ap.add_argument("--only-prefill", action="store_true",
                    help="the headline prefill step alone (for profiler runs): no other workloads, no CPU baseline")
    ap.add_argument("--cpu-pairs", type=int, default=64,
                    help="(sequence, head) pairs the oracle runs (64 = the whole workload)")
    ap.add_argument("--cpu-repeats", type=int, default=20,
                    help="repeats of the oracle sample (about 10 s on 16 cores of the GPU box)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also launch one plain device copy of this many MiB (PMC calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark measures one GPU; the path shards by "
                                   "(sequence, head) with no exchange, and multi-GPU runs are "
                                   "not part of it", "n_gpus": args.gpus}))
        sys.exit(2)

    if args.only_prefill:
        args.no_decode = args.no_kda = args.no_varlen = args.no_cpu_baseline = True
    import torch
    from fp8_state_qat_amd import api, inputs as gi
    from fp8_state_qat_amd._lib import GDN_QDQ_CHUNK, GDN_QDQ_W, GDN_QDQ_WRITE, GDN_SCHEDULE_SPLIT

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    flags = GDN_QDQ_CHUNK | GDN_QDQ_WRITE

    # ---------------- prefill workload (headline) ----------------
    w = gi.gdn_prefill()
    d = gi.device_tensors(w, dev)
    B, T, H, dk, dv = w.n_seqs, int(w.seq_lens[0]), w.n_heads, w.dk, w.dv
    o = torch.empty((w.total_tokens, H, dv), dtype=torch.bfloat16, device=dev)
    fin = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps + args.warmup)]
    it = {"i": 0}

    ws = torch.empty(api.chunk_workspace_bytes(B, H, dk, dv, w.total_tokens, qdq_flags=flags),
                     dtype=torch.uint8, device=dev)

    def step():
        api.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["cu_seqlens"], qdq_flags=flags,
                      out=o, final_state=fin, workspace=ws)

    def step_ev():  # the same call with the library's events around the fused launch
        e0, e1 = ev[it["i"]]
        it["i"] += 1
        api.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["cu_seqlens"], qdq_flags=flags,
                      out=o, final_state=fin, workspace=ws, debug={"kernel_start": e0, "kernel_end": e1})

    for e0, e1 in ev:  # create the HIP events outside the timed region
        e0.record()
        e1.record()
    torch.cuda.synchronize()
    # the step (the headline) timed without per-launch events, then the launch
    # durations from a second pass with them
    total_ms, per = time_launches(step, args.steps, args.warmup)
    check_outputs(api, ws, o, fin)
    ms_step = total_ms / args.steps
    time_launches(step_ev, args.steps, args.warmup)
    check_outputs(api, ws, o, fin)
    kern_ms, kern_med = launch_stats(ev[args.warmup:])
    # MALL-flushed: a 512 MiB write before each trial, the launch timed alone
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    evf = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]

    def step_f(e):
        api.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["cu_seqlens"], qdq_flags=flags,
                      out=o, final_state=fin, workspace=ws, debug={"kernel_start": e[0], "kernel_end": e[1]})

    flushed = time_flushed(step_f, evf, args.steps, flush)
    check_outputs(api, ws, o, fin)
    del flush
    tokens = B * T
    token_heads = tokens * H
    n_chunk_heads = B * H * ((T + 63) // 64)
    fl_all = flops_per_token_head(64, dk, dv) * token_heads
    fl = state_kernel_flops_per_token_head(64, dk, dv) * token_heads
    # the fused launch does every flop of the step and moves the prefill's bytes
    # (the records stay inside it: written and read back through the L2)
    by = prefill_bytes(token_heads, B * H, dk, dv, 2, 2)
    src = source_hash([os.path.join(ROOT, "fp8_state_qat_amd", "csrc", f)
                       for f in PREFILL_SOURCES])
    traffic = load_traffic("chunk_fwd_gdn_prefill", src)
    tflops = fl_all / (kern_ms * 1e-3) / 1e12
    hbm_gbs = by / (kern_ms * 1e-3) / 1e9
    roofline = {"bound": "mfma", "achieved": round(tflops, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                "traffic": traffic,
                "kernel": "chunk_bf16_kernel<128, bf16 out, fused> (128 producer + 128 state workgroups)",
                "algorithmic_flops_per_launch": fl_all,
                "flops_per_token_head": flops_per_token_head(64, dk, dv),
                "avg_launch_ms": round(kern_ms, 5),
                "median_launch_ms": round(kern_med, 5),
                "mall_flushed_median_launch_ms": round(med(flushed), 5),
                "mall_flushed_frac": round(fl_all / (med(flushed) * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                "hbm": {"achieved": round(hbm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(hbm_gbs / HBM_PEAK_GBS, 4),
                        "algorithmic_bytes_per_launch": by}}
    step_tflops = fl_all / (ms_step * 1e-3) / 1e12
    mfma = {"scope": "whole step (prep + state kernels)", "achieved": round(step_tflops, 2),
            "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(step_tflops / BF16_MFMA_PEAK_TFLOPS, 4),
            "algorithmic_flops_per_step": fl_all,
            "flops_per_token_head": flops_per_token_head(64, dk, dv)}

    if args.only_prefill:
        line = {"metric": METRIC, "value": round(tokens / (ms_step * 1e-3), 1), "unit": "tokens/s",
                "ms_per_step": round(ms_step, 5), "roofline": roofline}
        if args.copy_calibration_mib:
            line["copy_calibration_bytes"] = copy_calibration(dev, args.copy_calibration_mib)
        print(json.dumps(line), flush=True)
        return

    # QDQ off, same workload (reported)
    def step_off():
        api.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["cu_seqlens"], qdq_flags=0,
                      out=o, final_state=fin)
    off_ms, _ = time_launches(step_off, args.steps, args.warmup)

    # split schedule, same workload (reported): prep kernel, then the state kernel alone
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps + args.warmup)]
    its = {"i": 0}

    def step_split():
        e0, e1 = evs[its["i"]]
        its["i"] += 1
        api.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["cu_seqlens"], qdq_flags=flags,
                      out=o, final_state=fin,
                      debug={"kernel_start": e0, "kernel_end": e1, "schedule": GDN_SCHEDULE_SPLIT})

    for e0, e1 in evs:
        e0.record()
        e1.record()
    torch.cuda.synchronize()
    split_ms, _ = time_launches(step_split, args.steps, args.warmup)
    split_kern = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs[args.warmup:]]))
    split_by = split_state_kernel_bytes(token_heads, n_chunk_heads, B * H, dk, dv, 2, 2)

    # W QDQ on top, same workload (reported): W formed and row-quantized by the producers
    evw = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps + args.warmup)]
    itw = {"i": 0}

    def step_w():
        e0, e1 = evw[itw["i"]]
        itw["i"] += 1
        api.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["cu_seqlens"],
                      qdq_flags=flags | GDN_QDQ_W, out=o, final_state=fin,
                      debug={"kernel_start": e0, "kernel_end": e1})

    for e0, e1 in evw:
        e0.record()
        e1.record()
    torch.cuda.synchronize()
    w_ms, _ = time_launches(step_w, args.steps, args.warmup)
    check_outputs(api, None, o, fin)
    w_kern = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evw[args.warmup:]]))
    w_tflops = fl_all / (w_kern * 1e-3) / 1e12

    out = {"metric": METRIC, "value": round(tokens / (ms_step * 1e-3), 1), "unit": "tokens/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "GDN chunked prefill, B=4 T=4096 H=16 dk=dv=128, bf16 q/k/v "
                                  "and o, fp32 state, chunk 64, FP8-E4M3 state QDQ at every "
                                  "boundary (tiles 128x64 per head)",
                      "global_batch": B, "seq_len": T, "heads": H, "dk": dk, "dv": dv,
                      "qdq_flags": flags},
           "roofline": roofline, "mfma": mfma,
           "qdq_off": {"ms_per_step": round(off_ms / args.steps, 5),
                       "tokens_per_s": round(tokens / (off_ms / args.steps * 1e-3), 1)},
           "split_schedule": {"ms_per_step": round(split_ms / args.steps, 5),
                              "tokens_per_s": round(tokens / (split_ms / args.steps * 1e-3), 1),
                              "state_kernel": "chunk_bf16_kernel<128, bf16 out>",
                              "state_kernel_avg_launch_ms": round(split_kern, 5),
                              "state_kernel_mfma_tflops": round(fl / (split_kern * 1e-3) / 1e12, 2),
                              "state_kernel_hbm_gbs": round(split_by / (split_kern * 1e-3) / 1e9, 1),
                              "state_kernel_algorithmic_bytes": split_by},
           "w_qdq": {"qdq_flags": flags | GDN_QDQ_W,
                     "ms_per_step": round(w_ms / args.steps, 5),
                     "tokens_per_s": round(tokens / (w_ms / args.steps * 1e-3), 1),
                     "kernel": "chunk_fwd_kernel<128, EngBF16, bf16, bf16, fused, W QDQ>",
                     "avg_launch_ms": round(w_kern, 5),
                     "mfma_tflops": round(w_tflops, 2),
                     "mfma_frac": round(w_tflops / BF16_MFMA_PEAK_TFLOPS, 4)}}

    # ---------------- backward state recurrence, same shape (reported) ----------------
    gen = torch.Generator(device=dev)
    gen.manual_seed(6)
    d_o = torch.randn((w.total_tokens, H, dv), generator=gen, device=dev).to(torch.bfloat16)
    dS_L = torch.randn((B, H, dv, dk), generator=gen, device=dev)
    n_bounds = B * ((T + 63) // 64)
    dh_out = torch.empty((n_bounds, H, dv, dk), device=dev)
    d0_out = torch.empty((B, H, dv, dk), device=dev)
    dv_out = torch.empty((w.total_tokens, H, dv), device=dev)

    def step_bwd():
        api.chunk_bwd_dh(d["q"], d["k"], d["beta"], d["g"], d["cu_seqlens"], d_o, d_final_state=dS_L,
                         dh=dh_out, d_initial_state=d0_out, d_v=dv_out)

    bwd_ms, _ = time_launches(step_bwd, args.steps, args.warmup)
    check_outputs(api, None, dh_out, d0_out, dv_out)
    bwd_ms /= args.steps
    bfl = bwd_flops_per_token_head(64, dk, dv) * token_heads
    bby = bwd_bytes(token_heads, n_chunk_heads, B * H, dk, dv, 2)
    out["bwd_dh"] = {"workload": "the same prefill workload: gradients of every chunk's entering state, "
                                 "of the initial state and of v for L = sum o . dO + <S_L, dS_L>, identity "
                                 "straight-through QDQ",
                     "ms_per_step": round(bwd_ms, 5), "tokens_per_s": round(tokens / (bwd_ms * 1e-3), 1),
                     "kernels": "chunk_offsets_kernel + chunk_bwd_prep_kernel<128> + chunk_bwd_dh_kernel<128>",
                     "mfma_tflops": round(bfl / (bwd_ms * 1e-3) / 1e12, 2),
                     "mfma_frac": round(bfl / (bwd_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                     "hbm_gbs": round(bby / (bwd_ms * 1e-3) / 1e9, 1),
                     "algorithmic_flops_per_step": bfl, "algorithmic_bytes_per_step": bby}

    # the backward of the W-QDQ forward (the forward's quantized W in the state term)
    def step_bwd_w():
        api.chunk_bwd_dh(d["q"], d["k"], d["beta"], d["g"], d["cu_seqlens"], d_o, d_final_state=dS_L,
                         dh=dh_out, d_initial_state=d0_out, d_v=dv_out, qdq_flags=flags | GDN_QDQ_W)

    bwdw_ms, _ = time_launches(step_bwd_w, args.steps, args.warmup)
    check_outputs(api, None, dh_out, d0_out, dv_out)
    bwdw_ms /= args.steps
    out["bwd_dh"]["w_qdq"] = {"qdq_flags": flags | GDN_QDQ_W, "ms_per_step": round(bwdw_ms, 5),
                              "kernels": "chunk_offsets_kernel + chunk_prep_kernel<128, bf16, true> (the "
                                         "forward's W records) + chunk_bwd_prep_kernel<128> + "
                                         "chunk_bwd_dh_kernel<128, true>",
                              "mfma_frac": round(bfl / (bwdw_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)}
    del d_o, dS_L, dh_out, d0_out, dv_out

    # ---------------- packed varlen prefill at full size (reported) ----------------
    if not args.no_varlen:
        wv = gi.varlen()
        dvl = gi.device_tensors(wv, dev)
        Tv, Nv = wv.total_tokens, wv.n_seqs
        ov = torch.empty((Tv, H, dv), dtype=torch.bfloat16, device=dev)
        finv = torch.empty((Nv, H, dv, dk), dtype=torch.float32, device=dev)
        wsv = torch.empty(api.chunk_workspace_bytes(Nv, H, dk, dv, Tv, qdq_flags=flags), dtype=torch.uint8,
                          device=dev)
        evv = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps + args.warmup)]
        itv = {"i": 0}

        def vstep():
            e0, e1 = evv[itv["i"]]
            itv["i"] += 1
            api.chunk_fwd(dvl["q"], dvl["k"], dvl["v"], dvl["beta"], dvl["g"], dvl["cu_seqlens"],
                          seq_lens=dvl["seq_lens"], qdq_flags=flags, out=ov, final_state=finv, workspace=wsv,
                          debug={"kernel_start": e0, "kernel_end": e1})

        for e0, e1 in evv:
            e0.record()
            e1.record()
        torch.cuda.synchronize()
        vtot, _ = time_launches(vstep, args.steps, args.warmup)
        check_outputs(api, wsv, finv)
        vkern, vkern_med = launch_stats(evv[args.warmup:])
        valid = int(np.sum(wv.seq_lens))
        vfl = flops_per_token_head(64, dk, dv) * valid * H
        # q, k, v, beta, g of the valid rows read; every row of o written (padding rows as 0); final states
        vby = prefill_bytes(valid * H, Nv * H, dk, dv, 2, 2) + (Tv - valid) * H * dv * 2
        out["varlen"] = {"workload": f"packed varlen prefill: {Nv} sequences, lengths U{{1..8192}} "
                                     f"(longest {int(np.max(wv.seq_lens))}, {valid} valid tokens) plus "
                                     f"U{{0..63}} padding rows each ({Tv} rows), H=16, dk=dv=128, bf16, QDQ on",
                         "ms_per_step": round(vtot / args.steps, 5),
                         "tokens_per_s": round(valid / (vtot / args.steps * 1e-3), 1),
                         "roofline": {"bound": "mfma", "avg_launch_ms": round(vkern, 5),
                                      "median_launch_ms": round(vkern_med, 5),
                                      "achieved": round(vfl / (vkern * 1e-3) / 1e12, 2),
                                      "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                      "frac": round(vfl / (vkern * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                                      "algorithmic_flops_per_launch": vfl,
                                      "hbm_gbs": round(vby / (vkern * 1e-3) / 1e9, 1),
                                      "hbm_frac": round(vby / (vkern * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                      "algorithmic_bytes_per_launch": vby,
                                      "critical_path_chunks": int(-(-int(np.max(wv.seq_lens)) // 64))}}
        del dvl, ov, finv, wsv
        torch.cuda.empty_cache()

    # ---------------- per-key-channel gate (KDA) prefill, same shape (reported) ----------------
    if not args.no_kda:
        wk = gi.kda_prefill()
        dk_ = gi.device_tensors(wk, dev)
        evk = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps + args.warmup)]
        itk = {"i": 0}

        def kstep():
            e0, e1 = evk[itk["i"]]
            itk["i"] += 1
            api.chunk_fwd(dk_["q"], dk_["k"], dk_["v"], dk_["beta"], dk_["g"], dk_["cu_seqlens"],
                          qdq_flags=flags, out=o, final_state=fin,
                          debug={"kernel_start": e0, "kernel_end": e1})

        for e0, e1 in evk:
            e0.record()
            e1.record()
        torch.cuda.synchronize()
        ktot, _ = time_launches(kstep, args.steps, args.warmup)
        kms = ktot / args.steps
        check_outputs(api, None, o, fin)
        kkern, kkern_med = launch_stats(evk[args.warmup:])
        # the fused launch does every flop of the step and moves the prefill's bytes
        # (g is [T, H, dk]; the records stay inside the launch)
        kfl = flops_per_token_head(64, dk, dv) * token_heads
        kby = prefill_bytes(token_heads, B * H, dk, dv, 2, 2, gate_floats=dk)

        def kstep_w():
            api.chunk_fwd(dk_["q"], dk_["k"], dk_["v"], dk_["beta"], dk_["g"], dk_["cu_seqlens"],
                          qdq_flags=flags | GDN_QDQ_W, out=o, final_state=fin)

        kwtot, _ = time_launches(kstep_w, args.steps, args.warmup)
        out["kda"] = {"workload": "per-key-channel gate prefill, B=4 T=4096 H=16 dk=dv=128, bf16 "
                                  "q/k/v and o, fp32 g [T, H, dk] and state, FP8-E4M3 state QDQ "
                                  "at every boundary",
                      "ms_per_step": round(kms, 5), "tokens_per_s": round(tokens / (kms * 1e-3), 1),
                      "fused_launch": {"kernel": "kda_fwd_kernel<128, EngBF16, bf16, bf16, fused> "
                                                 "(128 producer + 128 state workgroups)",
                                       "avg_launch_ms": round(kkern, 5),
                                       "median_launch_ms": round(kkern_med, 5),
                                       "mfma_tflops": round(kfl / (kkern * 1e-3) / 1e12, 2),
                                       "mfma_frac": round(kfl / (kkern * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                                       "hbm_gbs": round(kby / (kkern * 1e-3) / 1e9, 1),
                                       "algorithmic_bytes_per_launch": kby},
                      "w_qdq": {"qdq_flags": flags | GDN_QDQ_W,
                                "ms_per_step": round(kwtot / args.steps, 5),
                                "tokens_per_s": round(tokens / (kwtot / args.steps * 1e-3), 1)}}

        # its backward: the reverse token recurrence (fp32 vector ALU)
        genk = torch.Generator(device=dev)
        genk.manual_seed(7)
        d_ok = torch.randn((wk.total_tokens, H, dv), generator=genk, device=dev).to(torch.bfloat16)
        dS_k = torch.randn((B, H, dv, dk), generator=genk, device=dev)
        dh_k = torch.empty((B * ((T + 63) // 64), H, dv, dk), device=dev)
        d0_k = torch.empty((B, H, dv, dk), device=dev)
        dv_k = torch.empty((wk.total_tokens, H, dv), device=dev)

        def kstep_bwd():
            api.chunk_bwd_dh(dk_["q"], dk_["k"], dk_["beta"], dk_["g"], dk_["cu_seqlens"], d_ok,
                             d_final_state=dS_k, dh=dh_k, d_initial_state=d0_k, d_v=dv_k)

        kb_ms, _ = time_launches(kstep_bwd, args.steps, args.warmup)
        check_outputs(api, None, dh_k, d0_k, dv_k)
        kb_ms /= args.steps
        # per token and head: G += do q^T, y = G k, G -= beta y k^T (2 dv dk flops each), G *= exp(g) (dv dk)
        kb_fl = 7 * dv * dk * token_heads
        out["kda"]["bwd_dh"] = {"ms_per_step": round(kb_ms, 5), "tokens_per_s": round(tokens / (kb_ms * 1e-3), 1),
                                "kernels": "chunk_offsets_kernel + kda_bwd_token_kernel<128>",
                                "roofline": {"bound": "alu", "achieved": round(kb_fl / (kb_ms * 1e-3) / 1e12, 2),
                                             "peak": FP32_VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                                             "frac": round(kb_fl / (kb_ms * 1e-3) / 1e12 / FP32_VALU_PEAK_TFLOPS, 4),
                                             "algorithmic_flops_per_step": kb_fl}}
        del d_ok, dS_k, dh_k, d0_k, dv_k
        del dk_
        torch.cuda.empty_cache()

    # ---------------- prefill -> decode handoff workload ----------------
    if not args.no_decode:
        del d
        torch.cuda.empty_cache()
        N4, H4, P4, steps4 = 256, 32, 2048, 512
        pd = gi.device_packed([P4] * N4, H4, 128, 128, seed=4, device=dev)
        o4 = torch.empty((N4 * P4, H4, 128), dtype=torch.bfloat16, device=dev)
        state = torch.empty((N4, H4, 128, 128), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        api.chunk_fwd(pd["q"], pd["k"], pd["v"], pd["beta"], pd["g"], pd["cu_seqlens"],
                      qdq_flags=flags, out=o4, final_state=state)
        torch.cuda.synchronize()
        pre_ms = (time.perf_counter() - t0) * 1e3
        del pd, o4
        torch.cuda.empty_cache()
        tok = gi.device_decode_tokens(N4, H4, 128, 128, steps4, seed=5, device=dev)
        od = torch.empty((N4, H4, 128), dtype=torch.bfloat16, device=dev)
        it = {"i": 0}

        def dstep():
            i = it["i"] % steps4
            api.decode_step(tok["q"][i], tok["k"][i], tok["v"][i], tok["beta"][i], tok["g"][i],
                            state, qdq=True, o=od)
            it["i"] += 1

        dwarm = 8
        dtot, dper = time_launches(dstep, steps4 - dwarm, dwarm)
        check_outputs(api, None, od, state)
        dms = float(np.mean(dper))
        dmed = med(dper)
        dby = decode_bytes(N4 * H4, 128, 128, 2, 2)
        dsrc = source_hash([os.path.join(ROOT, "fp8_state_qat_amd", "csrc", f)
                            for f in ("gdn_decode.hip", "gdn_device.hpp")])
        out["decode"] = {"workload": "256 sequences, H=32, dk=dv=128, bf16 q/k/v/o, fp32 state; "
                                     "2048-token chunked prefix with QDQ, then 512 decode steps "
                                     "with per-write QDQ",
                         "prefill_ms": round(pre_ms, 3),
                         "prefill_tokens_per_s": round(N4 * P4 / (pre_ms * 1e-3), 1),
                         "decode_steps_timed": steps4 - dwarm,
                         "ms_per_step": round(dms, 5),
                         "median_ms_per_step": round(dmed, 5),
                         "tokens_per_s": round(N4 / (dms * 1e-3), 1),
                         "roofline": {"bound": "hbm", "achieved": round(dby / (dms * 1e-3) / 1e9, 1),
                                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": round(dby / (dms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                      "algorithmic_bytes_per_launch": dby,
                                      "traffic": load_traffic("decode_step_handoff", dsrc),
                                      "kernel": "decode_step_kernel<128, bf16, bf16>"}}

        # the same decode steps with the INT8 block-32 codec (reported)
        def dstep8():
            i = it["i"] % steps4
            api.decode_step(tok["q"][i], tok["k"][i], tok["v"][i], tok["beta"][i], tok["g"][i],
                            state, qdq=True, o=od, int8=True)
            it["i"] += 1

        _, dper8 = time_launches(dstep8, steps4 - dwarm, dwarm)
        check_outputs(api, None, od, state)
        dms8 = float(np.mean(dper8))
        out["decode_int8"] = {"codec": "INT8, one scale per 32 key columns of a state row",
                              "ms_per_step": round(dms8, 5),
                              "median_ms_per_step": round(med(dper8), 5),
                              "tokens_per_s": round(N4 / (dms8 * 1e-3), 1),
                              "hbm_gbs": round(dby / (dms8 * 1e-3) / 1e9, 1),
                              "hbm_frac": round(dby / (dms8 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                              "kernel": "decode_step_kernel<128, bf16, bf16, int8>"}

        # the standalone state QDQ calls, in place on the same states (reported)
        sc8 = torch.empty(state.shape[:-2] + (state.shape[-2] // 64,), dtype=torch.float32, device=dev)
        sci = torch.empty(state.shape[:-1] + (state.shape[-1] // 32,), dtype=torch.float32, device=dev)
        for name, fn, sc, kern in (("state_qdq", api.state_qdq, sc8, "state_qdq_kernel<8>"),
                                   ("state_qdq_int8", api.state_qdq_int8, sci, "state_qdq_int8_kernel")):
            qms, _ = time_launches(lambda: fn(state, out=state, scales=sc), args.steps, args.warmup)
            qms /= args.steps
            qby = 2 * state.numel() * 4 + sc.numel() * 4
            out[name] = {"workload": f"{tuple(state.shape)} fp32 states, in place",
                         "ms_per_call": round(qms, 5), "kernel": kern,
                         "hbm_gbs": round(qby / (qms * 1e-3) / 1e9, 1),
                         "hbm_frac": round(qby / (qms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes_per_call": qby}
        del tok, state, sc8, sci
        torch.cuda.empty_cache()

    if args.copy_calibration_mib:
        out["copy_calibration_bytes"] = copy_calibration(dev, args.copy_calibration_mib)

    if not args.no_cpu_baseline:
        # all the cores this process may use (the GPU's share of the host, at most 16), and one
        hi = host_info()
        threads = max(1, min(16, hi["usable"]))
        print(f"oracle on {threads} host threads", file=sys.stderr, flush=True)
        cb = cpu_baseline(w, flags, args.cpu_pairs, threads, args.cpu_repeats)
        one = cpu_baseline(w, flags, max(1, args.cpu_pairs // 16), 1, 1)
        cb["one_thread"] = {"value": one["value"], "unit": one["unit"], "cores": 1, "sample": one["sample"]}
        cb["host"] = hi
        out["cpu_baseline"] = cb

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
