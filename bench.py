#!/usr/bin/env python3
"""Benchmark of the KDA forward hot path on one MI355X; prints one JSON line.

A step is one chunk prefill of the mid workload (B=4, H=32, T=8192,
dk=dv=128, bf16 q/k/v, fp32 gates and state, C=64) through the C ABI
(kda_chunk_fwd), with every input already resident in HBM.  `value` is
prefill tokens/s (a token = one position of one sequence, all 32 heads).
Before the W warm-up steps, about 100 ms of untimed launches let the GPU
clocks settle (they ramp up over the first ~30 ms of load).

Extra fields measure the other entry points on their own workloads:
  decode        256 sequences x 32 heads, 1024 one-token steps (steps/s), one
                launch per step from the host and, as graph_steps_per_s, the
                same steps captured in one HIP graph
  decode_multi  the same sizes, 4 tokens per sequence and launch (tokens/s)
  fused_prep    mid sizes from raw q, k and bf16 gate pre-activations, against
                separate preparation passes feeding the plain kernel (ms)
  long_context  B=1, H=16, T=65536 with an initial state (tokens/s)
  varlen        8 packed sequences of U[2048, 16384] tokens x 16 heads (tokens/s), with
                the library's device-side split of the longest sequences
  small_configs the tiny fp32 and small bf16 prefills, bound by launch latency
                (microseconds per launch and tokens/s, no roofline)

roofline: the chunk kernel against HBM bandwidth.  `achieved` is the
algorithmic bytes of one launch (one read of every input, one write of
every output and final state) divided by the kernel's average duration,
measured with HIP events recorded around each launch on the stream the
kernel runs on.  `traffic` is the HBM bytes per launch from rocprofv3
FETCH_SIZE / WRITE_SIZE counters (scaled by the same counters on a plain
copy kernel), taken from profiles/traffic.json when that file was made from
the current kernel sources, else null.  `copy_peak_gbs` is the bandwidth
the library's streaming copy (kda_stream_copy: 16-byte nontemporal loads and
stores, the decode kernels' access pattern) reaches on 1 GiB on the same GPU
in the same run (bytes read plus bytes written, median of 10 timed copies),
and `frac_of_copy` the kernel's achieved bandwidth as a fraction of it; the
decode rooflines carry the same two fields.

cpu_baseline: the float64 CPU oracle on the same mid workload (all of it,
repeated until about ten seconds of CPU work are timed), OpenMP over the
(sequence, head) pairs.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s & decode steps/s on 1 MI355X; % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
KERNEL_SOURCES = ["kimi_delta_attention_fwd_amd/csrc/kda_chunk.h",
                  "kimi_delta_attention_fwd_amd/csrc/kda_device.h",
                  "kimi_delta_attention_fwd_amd/csrc/kda_decode.h",
                  "kimi_delta_attention_fwd_amd/build.py"]   # (its compiler flags shape the kernels too)


def kernel_source_hash() -> str:
    """Hash of the kernel sources with // comments and blank lines removed, so
    that counters taken from a kernel stay valid across comment edits only."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            for line in f:
                code = line.split("//", 1)[0].strip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def prefill_bytes(ntok_heads, dk, dv, nheads, in_bytes=2, s0=False, sfinal=True):
    """Algorithmic HBM bytes of one prefill launch: q, k (dk each) and v (dv) in
    the input type, log_alpha (dk) and beta in fp32, out (dv) in the input type,
    plus the fp32 states read / written."""
    per_tok = in_bytes * (2 * dk + dv) + 4 * dk + 4 + in_bytes * dv
    state = 4 * dk * dv * nheads
    return ntok_heads * per_tok + (state if s0 else 0) + (state if sfinal else 0)


def prefill_flops(ntok_heads, dk, dv, C):
    """Useful flops per token-head: the three state contractions (6 dk dv) and
    the four triangular C x C products (2 C (dk + dv))."""
    return ntok_heads * (6 * dk * dv + 2 * C * (dk + dv))


def decode_bytes(nheads, dk, dv, in_bytes=2):
    """One decode step: the fp32 state read and written once, plus q, k, v,
    log_alpha, beta and out."""
    return nheads * (8 * dk * dv + in_bytes * (2 * dk + dv) + 4 * dk + 4 + in_bytes * dv)


def load_traffic(kernel: str, workload: str):
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    if data.get("kernel_source_hash") != kernel_source_hash():
        return None
    entry = data.get("kernels", {}).get(kernel, {}).get(workload)
    return None if entry is None else entry.get("bytes_per_launch")


def settle_clocks(launch, torch, seconds=0.1):
    """Untimed launches for about `seconds` of wall time.  The GPU raises its
    clocks over the first ~30 ms of sustained load (a launch of the mid
    prefill takes ~0.9 ms cold and ~0.77 ms once settled), so a few warm-up
    steps alone would time the ramp rather than the kernel."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            launch()
        torch.cuda.synchronize()


def time_launches(launch, stream, steps, warmup, torch, settle=True):
    """Settle the clocks, run `warmup` untimed launches, then exactly `steps`
    timed ones.  Returns (wall seconds over the steps, mean kernel ms from HIP
    events)."""
    if settle:
        settle_clocks(launch, torch)
    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        launch()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kms = sum(s.elapsed_time(e) for s, e in zip(starts, ends)) / steps
    return wall, kms


def bench_prefill(args, torch, kda, kda_synth, stream):
    w = kda_synth.WORKLOADS["mid"]
    p = kda_synth.workload("mid", device="cuda")
    B, T, H, dk, dv, C = w["B"], w["T"], w["H"], w["dk"], w["dv"], w["C"]
    out = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device="cuda")
    sf = torch.empty((B, H, dv, dk), dtype=torch.float32, device="cuda")
    h = stream.cuda_stream

    def launch():
        kda.kda_chunk_fwd(p.q, p.k, p.v, p.log_alpha, p.beta, None, out, sf, B, T, H, dk, dv, C, h)

    wall, kms = time_launches(launch, stream, args.steps, args.warmup, torch)
    nth = B * T * H
    nbytes = prefill_bytes(nth, dk, dv, B * H, s0=False, sfinal=True)
    flops = prefill_flops(nth, dk, dv, C)
    res = dict(wall=wall, kernel_ms=kms, tokens=B * T, bytes=nbytes, flops=flops, inputs=p,
               config=dict(workload="mid prefill: B=4 H=32 T=8192 dk=dv=128 bf16 C=64, zero S0, S_final written",
                           global_batch=B, seq_len=T, heads=H, dk=dk, dv=dv, chunk=C))
    return res


def bench_decode(args, torch, kda, kda_synth, stream):
    w = kda_synth.WORKLOADS["decode"]
    N, H, dk, dv, steps = w["N"], w["H"], w["dk"], w["dv"], w["steps"]
    if args.decode_steps:
        steps = min(steps, args.decode_steps)
    d = kda_synth.decode(N, H, dk, dv, steps, device="cuda")
    S = d.S0.clone()
    out = torch.empty((N, H, dv), dtype=torch.bfloat16, device="cuda")
    h = stream.cuda_stream
    Sw = d.S0.clone()
    for t in range(min(8, steps)):   # warm-up on a scratch copy of the state
        kda.kda_recurrent_step(d.q[t], d.k[t], d.v[t], d.log_alpha[t], d.beta[t], Sw, out, N, H, dk, dv, h)
    del Sw
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for t in range(steps):
        starts[t].record(stream)
        kda.kda_recurrent_step(d.q[t], d.k[t], d.v[t], d.log_alpha[t], d.beta[t], S, out, N, H, dk, dv, h)
        ends[t].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    times = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    kms = sum(times) / steps
    nbytes = decode_bytes(N * H, dk, dv)
    # The same steps captured once in a HIP graph and replayed: no host work
    # between launches.  The capture records on torch's capture stream.
    g = torch.cuda.CUDAGraph()
    Sg = d.S0.clone()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        hs = torch.cuda.current_stream().cuda_stream
        for t in range(steps):
            kda.kda_recurrent_step(d.q[t], d.k[t], d.v[t], d.log_alpha[t], d.beta[t], Sg, out, N, H, dk, dv, hs)
    g.replay()   # untimed
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    gwall = time.perf_counter() - t0
    del g, Sg, d, S
    return dict(
        workload="decode: 256 sequences x H=32, dk=dv=128, bf16 q/k/v, fp32 state, 1024 steps",
        steps_per_s=steps / wall, tokens_per_s=N * steps / wall, ms_per_step=wall * 1e3 / steps,
        graph_steps_per_s=steps / gwall, graph_ms_per_step=gwall * 1e3 / steps,
        kernel_ms_mean=kms, kernel_ms_median=times[steps // 2],
        roofline=dict(bound="hbm", achieved=round(nbytes / (kms * 1e-3) / 1e9, 1), peak=HBM_PEAK_GBS,
                      unit="GB/s", frac=round(nbytes / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                      traffic=load_traffic("decode_step", "decode"), algorithmic_bytes=nbytes))


def bench_decode_multi(args, torch, kda, kda_synth, stream, T=4, launches=50):
    """T decode tokens per sequence and launch (kda_recurrent_fwd) on the decode
    workload's sizes: 256 sequences x 32 heads, dk = dv = 128."""
    w = kda_synth.WORKLOADS["decode"]
    N, H, dk, dv = w["N"], w["H"], w["dk"], w["dv"]
    p = kda_synth.prefill(N, T, H, dk, dv, dtype="bf16", g_mu=w["g_mu"], g_sigma=w["g_sigma"], beta=w["beta"],
                          s0_sigma=0.1, seed=kda_synth.SEEDS["decode"], device="cuda")
    S = p.S0.clone()
    out = torch.empty((N, T, H, dv), dtype=torch.bfloat16, device="cuda")
    h = stream.cuda_stream

    def launch():
        kda.kda_recurrent_fwd(p.q, p.k, p.v, p.log_alpha, p.beta, S, out, N, T, H, dk, dv, h)

    wall, kms = time_launches(launch, stream, launches, 3, torch)
    nbytes = N * H * 8 * dk * dv + N * T * H * (2 * (2 * dk + dv) + 4 * dk + 4 + 2 * dv)
    del p, S, out
    return dict(workload=f"multi-token decode: {N} sequences x H={H}, dk=dv={dk}, {T} tokens per launch",
                tokens_per_s=N * T * launches / wall, launches_per_s=launches / wall, kernel_ms=kms,
                roofline=dict(bound="hbm", achieved=round(nbytes / (kms * 1e-3) / 1e9, 1), peak=HBM_PEAK_GBS,
                              unit="GB/s", frac=round(nbytes / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                              traffic=load_traffic("decode_multi", "decode_multi"), algorithmic_bytes=nbytes))


def bench_prep(args, torch, kda, kda_synth, stream, steps=10):
    """Fused input preparation on the mid sizes: raw q, k and bf16 gate
    pre-activations into kda_chunk_fwd_ex (KDA_INPUT_RAW), against the plain
    kernel fed by separate preparation passes (torch ops: L2 normalisation of
    q and k, -softplus of g in fp32), timed the same way."""
    w = kda_synth.WORKLOADS["mid"]
    B, T, H, dk, dv, C = w["B"], w["T"], w["H"], w["dk"], w["dv"], w["C"]
    p = kda_synth.prefill_raw(B, T, H, dk, dv, dtype="bf16", g_mu=w["g_mu"], g_sigma=w["g_sigma"],
                              seed=kda_synth.SEEDS["mid"], device="cuda")
    out = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device="cuda")
    sf = torch.empty((B, H, dv, dk), dtype=torch.float32, device="cuda")
    h = stream.cuda_stream
    raw = kda.variant(raw=True)

    def fused():
        kda.kda_chunk_fwd_ex(p.q, p.k, p.v, p.log_alpha, p.beta, None, out, sf, B, T, H, dk, dv, C, raw, 1, None,
                             0, h)

    def separate():
        qf, kf = p.q.float(), p.k.float()
        qn = (qf / qf.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
        kn = (kf / kf.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
        la = -torch.nn.functional.softplus(p.log_alpha.float())
        kda.kda_chunk_fwd(qn, kn, p.v, la, p.beta, None, out, sf, B, T, H, dk, dv, C, h)

    _, kms_fused = time_launches(fused, stream, steps, 2, torch)
    _, kms_sep = time_launches(separate, stream, steps, 2, torch)
    ntok = B * T * H
    fused_bytes = ntok * (2 * (2 * dk + dv) + 2 * dk + 4 + 2 * dv) + 4 * dk * dv * B * H
    del p, out, sf
    return dict(workload="mid sizes (B=4 H=32 T=8192 d=128, C=64) with raw q, k and bf16 gate pre-activations",
                fused_kernel_ms=kms_fused, separate_prep_plus_kernel_ms=kms_sep,
                fused_algorithmic_bytes=fused_bytes,
                fused_hbm_frac=round(fused_bytes / (kms_fused * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))


def bench_long(args, torch, kda, kda_synth, stream, steps=3):
    w = kda_synth.WORKLOADS["long"]
    p = kda_synth.workload("long", device="cuda")
    B, T, H, dk, dv, C = w["B"], w["T"], w["H"], w["dk"], w["dv"], w["C"]
    out = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device="cuda")
    sf = torch.empty((B, H, dv, dk), dtype=torch.float32, device="cuda")
    h = stream.cuda_stream

    # the library's schedule and segment count (kda_chunk_auto_schedule,
    # kda_chunk_auto_segments_ex; workspace allocated before the timed region),
    # the other segmented schedule, and the single pass, for reference
    def seg_launcher(sched):
        nseg = kda.kda_chunk_auto_segments_ex(B, T, H, dk, dv, C, 0, sched)
        wsb = kda.kda_chunk_segmented_workspace_bytes_ex(B, B * T, H, dk, dv, nseg, sched, False)
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")

        def launch():
            kda.kda_chunk_fwd_ex(p.q, p.k, p.v, p.log_alpha, p.beta, p.S0, out, sf, B, T, H, dk, dv, C, sched, nseg,
                                 ws, wsb, h)
        return nseg, ws, launch

    def launch_single():
        kda.kda_chunk_fwd(p.q, p.k, p.v, p.log_alpha, p.beta, p.S0, out, sf, B, T, H, dk, dv, C, h)

    sched = kda.kda_chunk_auto_schedule(B, T, H, dk, dv, C, 0)
    nseg, ws, launch = seg_launcher(sched)
    wall, kms = time_launches(launch, stream, steps, 1, torch)
    del ws
    other = kda.SCHED_MAP_OUTPUTS - sched
    nseg2, ws, launch2 = seg_launcher(other)
    _, kms2 = time_launches(launch2, stream, steps, 1, torch)
    del ws
    _, kms1 = time_launches(launch_single, stream, 2, 1, torch)
    nbytes = prefill_bytes(B * T * H, dk, dv, B * H, s0=True, sfinal=True)
    del p, out, sf
    names = {0: "two-pass (map launch with the lead segment's whole pass, composition, second pass)",
             kda.SCHED_MAP_OUTPUTS: "one-pass (map launch with the lead segment's whole pass and every later "
                                    "segment's outputs from a zero state, composition, output epilogue)"}
    return dict(workload="long prefill: B=1 H=16 T=65536 dk=dv=128 bf16 C=64, S0 in, S_final out",
                schedule=f"segment-parallel, {nseg} segments per sequence, {names[sched]}",
                tokens_per_s=B * T * steps / wall, kernel_ms=kms,
                other_schedule=dict(schedule=names[other].split(" (")[0], segments=nseg2, kernel_ms=kms2),
                single_pass_kernel_ms=kms1,
                hbm_gbs=round(nbytes / (kms * 1e-3) / 1e9, 1),
                hbm_frac=round(nbytes / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))


def bench_varlen(args, torch, kda, kda_synth, stream, steps=3):
    w = kda_synth.WORKLOADS["varlen"]
    p = kda_synth.workload("varlen", device="cuda")
    Tt = p.cu_host[-1]
    N = len(p.cu_host) - 1
    H, dk, dv, C = w["H"], w["dk"], w["dv"], w["C"]
    out = torch.empty((1, Tt, H, dv), dtype=torch.bfloat16, device="cuda")
    sf = torch.empty((N, H, dv, dk), dtype=torch.float32, device="cuda")
    h = stream.cuda_stream

    # the library's schedule for packed sequences (the one-pass schedule with
    # the device-side split, nseg = 0; workspace allocated before the timed
    # region), and the single pass for reference
    sched = kda.SCHED_MAP_OUTPUTS
    wsb = kda.kda_chunk_segmented_workspace_bytes_ex(N, Tt, H, dk, dv, 0, sched, False)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")

    def launch():
        kda.kda_chunk_fwd_varlen_ex(p.q, p.k, p.v, p.log_alpha, p.beta, p.S0, out, sf, p.cu_seqlens, N, Tt, H, dk,
                                    dv, C, sched, 0, ws, wsb, h)

    def launch_single():
        kda.kda_chunk_fwd_varlen(p.q, p.k, p.v, p.log_alpha, p.beta, p.S0, out, sf, p.cu_seqlens, N, Tt, H, dk,
                                 dv, C, h)

    wall, kms = time_launches(launch, stream, steps, 1, torch)
    _, kms1 = time_launches(launch_single, stream, steps, 1, torch)
    nbytes = prefill_bytes(Tt * H, dk, dv, N * H, s0=True, sfinal=True)
    del p, out, sf, ws
    return dict(workload=f"varlen prefill: {N} packed sequences (T_total={Tt}) x H=16 dk=dv=128 bf16 C=64",
                schedule="one-pass with the device-side split (the sequences much longer than the rest run as a "
                         "lead segment and a mapped one)",
                tokens_per_s=Tt * steps / wall, kernel_ms=kms, single_pass_kernel_ms=kms1,
                hbm_gbs=round(nbytes / (kms * 1e-3) / 1e9, 1),
                hbm_frac=round(nbytes / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))


def measure_copy_peak(torch, kda, stream, nbytes=1 << 30, reps=10):
    """Achievable HBM bandwidth: the library's streaming copy of `nbytes`,
    counting the bytes read and written, median of `reps` copies timed with
    HIP events on `stream` after a few untimed ones."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(5):
        kda.kda_stream_copy(src, dst, nbytes, stream)
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        kda.kda_stream_copy(src, dst, nbytes, stream)
        b.record(stream)
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    del src, dst
    ms.sort()
    return 2 * nbytes / (ms[len(ms) // 2] * 1e-3) / 1e9


def bench_small(args, torch, kda, kda_synth, stream, launches=200):
    """The two small configurations, which are bound by launch latency and run
    from cache: tiny (fp32, B=1 H=1 T=64 d=16, C=16) as microseconds per launch,
    and small (bf16, B=2 H=4 T=1024 d=64, C=64, with S0) as tokens/s.  Kernel
    time from HIP events around each launch; host time per launch from the wall
    clock over back-to-back launches.  No roofline claim."""
    res = {}
    for name in ("tiny", "small"):
        w = kda_synth.WORKLOADS[name]
        p = kda_synth.workload(name, device="cuda")
        B, T, H, dk, dv, C = w["B"], w["T"], w["H"], w["dk"], w["dv"], w["C"]
        out = torch.empty_like(p.v)
        sf = torch.empty((B, H, dv, dk), dtype=torch.float32, device="cuda")
        fn = kda.kda_chunk_fwd_f32 if w["dtype"] == "f32" else kda.kda_chunk_fwd
        h = stream.cuda_stream

        def launch():
            fn(p.q, p.k, p.v, p.log_alpha, p.beta, p.S0, out, sf, B, T, H, dk, dv, C, h)

        wall, kms = time_launches(launch, stream, launches, 20, torch)
        res[name] = dict(workload=f"{name}: B={B} H={H} T={T} dk=dv={dk} {w['dtype']} C={C}",
                         kernel_us=round(kms * 1e3, 2), us_per_launch=round(wall * 1e6 / launches, 2),
                         tokens_per_s=round(B * T * launches / wall, 1))
        # the library's own schedule choice (kda_chunk_auto_schedule and
        # kda_chunk_auto_segments_ex), with a workspace allocated once
        f32 = w["dtype"] == "f32"
        sched = kda.kda_chunk_auto_schedule(B, T, H, dk, dv, C, f32)
        nseg = kda.kda_chunk_auto_segments_ex(B, T, H, dk, dv, C, f32, sched)
        if nseg > 1:
            wsb = kda.kda_chunk_segmented_workspace_bytes_ex(B, B * T, H, dk, dv, nseg, sched, f32)
            ws = torch.empty(wsb // 4 + 64, dtype=torch.float32, device="cuda")
            seg = kda.kda_chunk_fwd_ex_f32 if f32 else kda.kda_chunk_fwd_ex

            def launch_seg():
                seg(p.q, p.k, p.v, p.log_alpha, p.beta, p.S0, out, sf, B, T, H, dk, dv, C, sched, nseg, ws, wsb, h)

            wall, kms = time_launches(launch_seg, stream, launches, 20, torch)
            res[name]["auto_schedule"] = dict(segments=nseg, schedule="one-pass" if sched else "two-pass",
                                              kernel_us=round(kms * 1e3, 2),
                                              us_per_launch=round(wall * 1e6 / launches, 2),
                                              tokens_per_s=round(B * T * launches / wall, 1))
            del ws
        del p, out, sf
    return res


def host_cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo (empty where there is none)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def cpu_baseline(p, kda_synth, target_s=10.0, max_passes=24):
    """Float64 oracle on the whole mid workload (every sequence, head and token),
    repeated until about `target_s` seconds of CPU work have been timed."""
    import tempfile
    import oracle
    B, T, H, _ = p.q.shape
    build = "generic x86-64, -O2"
    try:   # compiled for this host's CPU, as a CPU implementation would be deployed
        oracle.use_library(oracle.build_native(tempfile.mkdtemp(prefix="kda_oracle_")))
        build = "-O3 -march=native on this host"
    except Exception as e:   # no compiler: the generic build of the same source
        print(f"note: native oracle build failed ({e}); timing the generic build", file=sys.stderr)
    args = [kda_synth.to_f64(x) for x in (p.q, p.k, p.v, p.log_alpha, p.beta)]
    threads = min(oracle.max_threads(), B * H)   # the oracle's OpenMP loop runs over (sequence, head)
    passes, dt = 0, 0.0
    while passes < max_passes and (passes == 0 or dt < target_s):
        t0 = time.perf_counter()
        oracle.forward(*args)
        dt += time.perf_counter() - t0
        passes += 1
    del args
    return dict(value=round(passes * B * T / dt, 2), unit="tokens/s", cores=threads, kind="oracle",
                host_cpu=host_cpu_model(), host_threads=os.cpu_count(),
                sample=f"the whole mid workload (B={B}, T={T}, H={H}, dk=dv=128, zero initial state) "
                       f"through the float64 token-by-token recurrence, {passes} pass(es) in {dt:.1f} s, "
                       f"OpenMP over the {B * H} (sequence, head) pairs; oracle built {build}")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extras", default="decode,multi,long,varlen,prep,small",
                    help="comma-separated extra workloads to run after the mid prefill "
                         "(decode, multi, long, varlen, prep, small; 'none' for the mid prefill only)")
    ap.add_argument("--no-extras", action="store_true", help="same as --extras none")
    ap.add_argument("--decode-steps", type=int, default=None,
                    help="fewer decode steps (profiling runs; the default is the workload's 1024)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 1 GiB device copy three times, so hardware counters can be "
                         "scaled by a kernel of known traffic")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the kernels run on a single MI355X; batches would shard by sequence or head, one long "
              "sequence by segments of its tokens)", file=sys.stderr)
        sys.exit(2)

    import torch

    import kda_synth
    import kimi_delta_attention_fwd_amd as kda
    if not os.path.exists(kda.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    kda.load()
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    pre = bench_prefill(args, torch, kda, kda_synth, stream)
    ach = pre["bytes"] / (pre["kernel_ms"] * 1e-3) / 1e9
    tfl = pre["flops"] / (pre["kernel_ms"] * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": round(pre["tokens"] * args.steps / pre["wall"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["wall"] * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": pre["config"],
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic("chunk_fwd", "mid"),
                     "kernel": "chunk_fwd_kernel<bf16,128,64,64>",
                     "kernel_ms": round(pre["kernel_ms"], 4), "algorithmic_bytes": pre["bytes"],
                     "mfma_tflops": round(tfl, 2), "mfma_frac": round(tfl / BF16_PEAK_TFLOPS, 4),
                     "kernel_source_hash": kernel_source_hash()},
    }
    p_mid = pre.pop("inputs")
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(p_mid, kda_synth)
    del p_mid
    torch.cuda.empty_cache()
    extras = set() if args.no_extras or args.extras == "none" else set(args.extras.split(","))
    unknown = extras - {"decode", "multi", "long", "varlen", "prep", "small"}
    if unknown:
        raise SystemExit(f"unknown --extras entries: {sorted(unknown)}")
    for name, key, fn in (("decode", "decode", bench_decode), ("multi", "decode_multi", bench_decode_multi),
                          ("long", "long_context", bench_long), ("varlen", "varlen", bench_varlen),
                          ("prep", "fused_prep", bench_prep), ("small", "small_configs", bench_small)):
        if name in extras:
            result[key] = fn(args, torch, kda, kda_synth, stream)
            torch.cuda.empty_cache()
    copy_gbs = measure_copy_peak(torch, kda, stream)
    for roof in [result["roofline"]] + [result[k]["roofline"] for k in ("decode", "decode_multi") if k in result]:
        roof["copy_peak_gbs"] = round(copy_gbs, 1)
        roof["frac_of_copy"] = round(roof["achieved"] / copy_gbs, 4)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
