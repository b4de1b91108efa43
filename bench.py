#!/usr/bin/env python3
"""Benchmark of the MI355X SSD scan: prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one ssd_prefill call over the batched long-context 2.7B-shaped
Mamba-2 layer (B=8, L=16384, H=80, P=64, N=128, G=1, Q=256, bf16 x/Bm/Cm,
fp32 dt/A/state), the largest of the stated workloads that fits one GPU:
every stage of the chunked scan (in-chunk cumsum and decay, intra-chunk
C*B^T (.) decay * X, chunk states, the chunk-to-chunk state hand-off,
C*h + D*x).  ``value`` is its prefill tokens/s.  In the same run, and
reported beside it:
  * the other prefill shapes: the 2.7B-shaped layer at B=1, L=4096 (in place,
    and over rotated inputs larger than the 256 MB Infinity Cache), the
    130M-shaped layer, 512-token chunks, fp32 activations, and the B=8 decode
    steps that follow the long-context prefill;
  * decode: 4096 consecutive fused decode steps (conv window + state update +
    readout) of the 2.7B-shaped layer at B=16 (conv C=5376, K=4), on one state
    and over rotated states, eager and as one HIP graph (the on-device decode
    loop); the step at B=1; the same-size in-place stream kernel and a 1 GiB
    copy as the box's measured bandwidth ceiling; cached decode against
    recomputing the prefix for the 130M- and 2.7B-shaped layers at B=1 and 16;
  * conv, the gated normalisation and the packed (varlen) serving mix;
  * cpu_baseline: the CPU oracle on a bounded sample of the same workload,
    and its decode step rate.
Inputs are seeded synthetic tensors (mamba_ssd_scan_chunk_amd.synth), resident
in device memory before timing starts.  GPU times come from HIP events on the
stream the kernels run on.  Host launch overhead is kept out of the timed
region: device-bound legs are timed right after about 50 ms of untimed calls
(so the GPU is busy and at its sustained clocks when timing starts), legs of
many tiny launches behind a GPU sleep sized to their host enqueue time.
"""
from __future__ import annotations

import argparse
import hashlib
import itertools
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")


def prefill_flops(B, L, H, P, G, N, Q):
    """Algorithmic flops of the causal chunked scan (C*B^T once per
    (batch, chunk, group); per (batch, chunk, head): masked M*X, chunk state,
    C*h and the state pass)."""
    total = 0
    for c0 in range(0, L, Q):
        q = min(Q, L - c0)
        total += G * N * q * (q + 1) + H * (P * q * (q + 1) + 4 * q * N * P + 2 * P * N)
    return B * total


def prefill_bytes(B, L, H, P, G, N, esize=2):
    return (2 * B * L * H * P * esize + 4 * B * L * H + 2 * B * L * G * N * esize
            + 4 * B * H * P * N + 8 * H)


def decode_bytes(B, H, P, G, N, K, esize=2):
    C = H * P + 2 * G * N
    return (8 * B * H * P * N + 2 * B * C * (K - 1) * esize + B * C * esize + 4 * B * H
            + C * K * esize + B * H * P * esize + 8 * H)


KERNEL_SOURCES = ["mamba_ssd_scan_chunk_amd/csrc/prefill_mfma.hip", "mamba_ssd_scan_chunk_amd/csrc/prefill_mfma.hpp",
                  "mamba_ssd_scan_chunk_amd/csrc/prefill_chain.hip", "mamba_ssd_scan_chunk_amd/csrc/ssd_device.hpp",
                  "mamba_ssd_scan_chunk_amd/csrc/ssd_internal.hpp"]
PREFILL_KERNELS = ("chunk_pack_mfma", "chunk_state_mfma", "state_pass_bf16", "chunk_out_mfma", "chunk_chain_mfma")


def stage_work(kernel, B, L, H, P, G, N, Q, esize=2, chained=False):
    """Own (bytes, flops) of one launch of a prefill kernel of the MFMA path:
    every input and output of that kernel moved once (workspace operands and
    hand-off slots included), and the flops of its stage of the chunked scan
    (causal, as in prefill_flops).  ``chained``: the single-pass form (its
    pack kernel also writes C in operand order)."""
    nch = -(-L // Q)
    items, groups = B * nch * H, B * nch * G
    tile_bytes = (Q // 32) * (Q // 32 + 1) // 2 * 32 * 32 * 2  # masked C B^T tiles, bf16
    qs = [min(Q, L - c * Q) for c in range(nch)]
    if kernel == "chunk_pack_mfma":
        nbytes = 2 * B * L * G * N * esize + groups * (tile_bytes + Q * N * 2 * (2 if chained else 1))
        flops = B * G * sum(N * q * (q + 1) for q in qs)
    elif kernel == "chunk_chain_mfma":
        # x, dt read and y written once; the packed G^T, B and C operands of
        # each (batch, chunk, group) read once; the carried state handed from
        # chunk to chunk (written and read back, fp32) and the final state
        nbytes = (B * L * H * (2 * P * esize + 4) + groups * (tile_bytes + 2 * Q * N * 2)
                  + 2 * B * H * (nch - 1) * P * N * 4 + B * H * P * N * 4)
        flops = B * H * sum(P * q * (q + 1) + 4 * q * N * P + 2 * P * N for q in qs)
    elif kernel == "chunk_state_mfma":
        nbytes = B * L * H * (P * esize + 4) + groups * Q * N * 2 + items * (P * N * 4 + 4)
        flops = B * H * sum(2 * q * N * P for q in qs)
    elif kernel == "state_pass_bf16":
        # plus C repacked into K3's operand order (read once, written once)
        nbytes = items * (P * N * 4 + 4 + P * N * 2) + B * H * P * N * 4 + B * L * G * N * esize + groups * Q * N * 2
        flops = items * 2 * P * N
    elif kernel == "chunk_out_mfma":
        nbytes = (B * L * H * (2 * P * esize + 4) + groups * Q * N * 2 + items * P * N * 2
                  + groups * tile_bytes)
        flops = B * H * sum(P * q * (q + 1) + 2 * q * N * P for q in qs)
    else:
        raise KeyError(kernel)
    return nbytes, flops


def section8d_bytes(kernel, B, L, H, P, G, N, esize=2):
    """Algorithmic bytes of one launch of a prefill kernel: the per-unit
    compulsory bytes of the scan (x and y at P*esize per token and head, dt
    4 B per token and head, B and C at 2*N*esize per token and group, the
    final state 4*P*N per (batch, head)) times the units that kernel
    processes; the whole call's total is prefill_bytes."""
    x = B * L * H * P * esize
    dt = 4 * B * L * H
    bc = 2 * B * L * G * N * esize
    st = 4 * B * H * P * N + 8 * H
    return {"chunk_chain_mfma": 2 * x + dt + st, "chunk_out_mfma": 2 * x + dt, "chunk_state_mfma": x + dt,
            "state_pass_bf16": st, "chunk_pack_mfma": bc}[kernel]


def measured_traffic(kernel, workload="mamba2-2.7b-longctx"):
    """HBM bytes per launch of `kernel` on `workload` from committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE runs
    (profiles/traffic_<kernel>_<workload>.json, written by
    mamba_ssd_scan_chunk_amd.profiling), or None if absent or taken on
    kernel sources that have changed since."""
    from mamba_ssd_scan_chunk_amd.profiling import source_hash

    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if not rec.get("sources") or rec.get("source_hash") != source_hash(rec["sources"]):
        return None
    return rec.get("bytes_per_launch")


def measured_mfma(workload):
    """Executed MFMA flops per launch of each prefill kernel, from a committed
    rocprofv3 SQ_INSTS_VALU_MFMA_MOPS_BF16 run on `workload`
    (profiles/mfma_prefill_<workload>.json, written by
    mamba_ssd_scan_chunk_amd.profiling), or {} if absent, taken on another
    workload or on kernel sources that have changed since."""
    from mamba_ssd_scan_chunk_amd.profiling import source_hash

    path = os.path.join(PROFILES, f"mfma_prefill_{workload.replace('-prefill', '')}.json")
    if not os.path.exists(path):
        return {}
    rec = json.load(open(path))
    if rec.get("workload") != workload or not rec.get("sources") or rec.get("source_hash") != source_hash(rec["sources"]):
        return {}
    return {k: v["flops"] for k, v in rec["kernels"].items()}


HOST_BOUND = []


HOT_MS = 50.0  # GPU work run right before a timed region, so that it starts at sustained clocks


def _timed(fn, steps, warmup, name):
    """GPU ms per call over ``steps`` back-to-back calls, none of which may
    wait for the host.

    A leg whose host enqueue per call is well below its GPU time gets a head
    start: about HOT_MS of untimed calls enqueued right before the timed ones,
    so the GPU is busy, and at the clocks it holds under sustained load, when
    timing starts (after an idle gap the first tens of milliseconds run a few
    percent slower).  A leg that is not (many tiny launches) instead waits
    behind a GPU sleep sized to the measured host enqueue time, so that the
    whole sequence is queued before the first timed call starts."""
    import torch

    for _ in range(warmup):
        fn(0)
    torch.cuda.synchronize()
    n0 = min(steps, 64)
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record()
    t0 = time.perf_counter()
    for i in range(n0):
        fn(i)
    per_call = (time.perf_counter() - t0) / n0
    p1.record()
    torch.cuda.synchronize()
    gpu_call_ms = p0.elapsed_time(p1) / n0
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if per_call * 1e3 < 0.7 * gpu_call_ms:
        n_pre = int(min(max(HOT_MS / gpu_call_ms, 16), 20000))
        for i in range(n_pre):
            fn(i)
        start.record()
        h0 = time.perf_counter()
        for i in range(steps):
            fn(i)
        host_ms = (time.perf_counter() - h0) * 1e3
        end.record()
        torch.cuda.synchronize()
        gpu_ms = start.elapsed_time(end)
        covered_ms = n_pre * gpu_call_ms + gpu_ms  # the queue ran dry only if the host took longer
    else:
        # calibrate the sleep kernel's clock
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        torch.cuda._sleep(1_000_000)
        s1.record()
        torch.cuda.synchronize()
        cyc_per_ms = 1_000_000 / max(s0.elapsed_time(s1), 1e-3)
        covered_ms = 1.5 * per_call * steps * 1e3 + 5.0
        torch.cuda._sleep(int(covered_ms * cyc_per_ms))
        start.record()
        h0 = time.perf_counter()
        for i in range(steps):
            fn(i)
        host_ms = (time.perf_counter() - h0) * 1e3
        end.record()
        torch.cuda.synchronize()
        gpu_ms = start.elapsed_time(end)
    if host_ms > covered_ms:
        if name not in HOST_BOUND:
            HOST_BOUND.append(name)
    return gpu_ms / steps


def bench_prefill(args, name, rotate=False, extras=True):
    """ssd_prefill on workload `name`: ms per call; with ``extras`` also the
    call captured in a HIP graph, the call with the step passed raw, and the
    per-kernel durations.  ``rotate``: distinct input/output/workspace sets
    whose total exceeds the 256 MB Infinity Cache, one per call in turn (the
    HBM-honest figure for a layer small enough to stay in that cache)."""
    import torch

    from mamba_ssd_scan_chunk_amd import binding as bd
    from mamba_ssd_scan_chunk_amd import synth

    w = synth.WORKLOADS[name]
    code = bd.SSD_BF16 if w.dtype == "bf16" else bd.SSD_F32
    need = bd.ssd_prefill_workspace_bytes(w.B, w.L, w.H, w.P, w.G, w.N, w.Q, code)
    d0 = {k: v.cuda() for k, v in synth.make_prefill(w.B, w.L, w.H, w.P, w.G, w.N, w.dtype, seed=2).items()}
    sets = [d0]
    if rotate:
        per_set = sum(t.numel() * t.element_size() for t in d0.values()) + d0["x"].numel() * d0["x"].element_size() + need
        nrot = max(2, -(-600 * 2**20 // per_set))
        sets = [d0] + [{k: v.clone() for k, v in d0.items()} for _ in range(nrot - 1)]
    bufs = [(torch.empty_like(d["x"]), torch.empty((w.B, w.H, w.P, w.N), dtype=torch.float32, device="cuda"),
             torch.empty(max(1, need), dtype=torch.uint8, device="cuda")) for d in sets]

    def step(i):
        d = sets[i % len(sets)]
        y, fs, ws = bufs[i % len(sets)]
        bd.ssd_prefill(d["x"], d["dt"], d["A_log"], d["Bm"], d["Cm"], d["D"], None, Q=w.Q, y=y,
                       final_state=fs, workspace=ws)

    steps = args.steps if w.B * w.L >= 65536 else max(args.steps, 50)
    ms = _timed(step, steps, args.warmup, f"prefill {name}{' rotated' if rotate else ''}")
    out = {"w": w, "ms": ms, "sets": len(sets)}
    if not extras:
        return out
    # the same calls captured in one HIP graph (as a serving loop would run
    # them): the kernels are the same, the dispatch gaps between them may not be
    out["graph_ms"] = _graph_timed(step, min(steps, 20))
    # the same calls with the step passed raw: softplus(dt + bias) clipped to
    # [1e-3, 0.1] inside the kernels
    raw, dt_bias = (t.cuda() for t in synth.make_dt_raw((w.B, w.L), w.H, seed=3))
    d, (y, fs, ws) = sets[0], bufs[0]

    def step_raw(_):
        bd.ssd_prefill(d["x"], raw, d["A_log"], d["Bm"], d["Cm"], d["D"], None, Q=w.Q, y=y, final_state=fs,
                       workspace=ws, dt_raw=True, dt_bias=dt_bias, dt_min=1e-3, dt_max=0.1)

    out["raw_ms"] = _timed(step_raw, steps, args.warmup, f"prefill_dt_raw {name}")
    del raw
    # per-kernel durations: HIP events the library records between its
    # kernels on the call's stream; each sample is the last of about HOT_MS
    # of back-to-back calls, so the GPU is busy as in the timed loop
    bd.stage_timing(True)
    stages = {}
    n_hot = int(min(max(HOT_MS / (ms if ms > 0 else 1.0), 4), 5000))
    try:
        for _ in range(args.stage_runs):
            for _ in range(n_hot):
                step(0)
            for kname, kms in bd.stage_times():
                stages.setdefault(kname, []).append(kms)
    finally:
        bd.stage_timing(False)
    out["stages"] = {k: sum(v) / len(v) for k, v in stages.items()}
    return out


def bench_decode(args, rotate, raw_dt=False):
    import torch

    from mamba_ssd_scan_chunk_amd import binding as bd
    from mamba_ssd_scan_chunk_amd import synth

    w = synth.WORKLOADS[args.decode_workload]
    B, H, P, G, N, K, C = w.B, w.H, w.P, w.G, w.N, w.K, w.conv_channels
    steps = args.decode_steps
    tdt = synth.torch_dtype(w.dtype)
    # the cache a 4096-token prefill leaves, produced by this library
    pre = {k: v.cuda() for k, v in synth.make_prefill(B, w.L, H, P, G, N, w.dtype, seed=3).items()}
    _, state = bd.ssd_prefill(pre["x"], pre["dt"], pre["A_log"], pre["Bm"], pre["Cm"], pre["D"], Q=w.Q)
    A_log, D = pre["A_log"], pre["D"]
    del pre
    xbc, dts = synth.make_decode_stream(steps, B, H, P, G, N, w.dtype, seed=4)
    xbc, dts = xbc.cuda(), dts.cuda()
    kw = {}
    if raw_dt:  # the step passed raw, preprocessed inside the kernel
        dts, dt_bias = (t.cuda() for t in synth.make_dt_raw((steps, B), H, seed=6))
        kw = dict(dt_raw=True, dt_bias=dt_bias, dt_min=1e-3, dt_max=0.1)
    cw, _ = synth.make_conv(C, K, w.dtype, seed=5)
    cw = cw.cuda()
    conv = [torch.zeros((B, C, K - 1), dtype=tdt, device="cuda") for _ in range(2)]
    y = torch.empty((B, H, P), dtype=tdt, device="cuda")
    nrot = 1
    states = [state]
    if rotate:
        # distinct states whose total exceeds the 256 MB Infinity Cache
        nrot = max(2, -(-600 * 2**20 // state.numel() // 4))
        states = [state.clone() for _ in range(nrot)]
    HP, GN = H * P, G * N

    def step(i):
        row = xbc[i % steps]
        bd.ssd_decode_step(row[:, :HP], dts[i % steps], A_log, row[:, HP:HP + GN], row[:, HP + GN:], D,
                           states[i % nrot], y_t=y, in_stride=C, G=G, conv_state_in=conv[i & 1],
                           conv_state_out=conv[(i + 1) & 1], conv_w=cw, K=K, activation=1, **kw)

    eager_ms = _timed(step, steps, min(args.warmup, 8), "decode")
    graph_ms = _graph_timed(step, steps)
    return w, eager_ms, graph_ms, decode_bytes(B, H, P, G, N, K, 2 if w.dtype == "bf16" else 4), nrot


def _graph_timed(fn, steps, reps=3):
    """GPU ms per step with all ``steps`` steps captured in one HIP graph
    (the on-device decode loop: no host work between steps); best of
    ``reps`` replays."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(0)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            fn(i)
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record()
    g.replay()
    p1.record()
    torch.cuda.synchronize()
    n_pre = int(min(max(HOT_MS / max(p0.elapsed_time(p1), 1e-3), 1), 1000))
    best = float("inf")
    for _ in range(reps):
        for _ in range(n_pre):  # untimed replays: the timed one starts on a busy GPU
            g.replay()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        g.replay()
        end.record()
        torch.cuda.synchronize()
        best = min(best, start.elapsed_time(end))
    del g
    return best / steps


def bench_conv(args):
    import torch

    from mamba_ssd_scan_chunk_amd import binding as bd
    from mamba_ssd_scan_chunk_amd import synth

    w = synth.WORKLOADS[args.layer_workload]
    C, K = w.conv_channels, w.K
    xbc = synth.make_tokens(w.B, w.L, C, w.dtype, seed=6).cuda()
    cw, _ = synth.make_conv(C, K, w.dtype, seed=7)
    cw = cw.cuda()
    st = torch.zeros((w.B, C, K - 1), dtype=xbc.dtype, device="cuda")
    out = torch.empty_like(xbc)

    def step(_):
        bd.conv_state_update(st, xbc, cw, activation=1, out=out)

    ms = _timed(step, args.steps, args.warmup, "conv")
    es = xbc.element_size()
    nbytes = 2 * w.B * w.L * C * es + 2 * w.B * C * (K - 1) * es + C * K * es
    return ms, nbytes


def bench_norm(args):
    """The layer's closing gated RMS normalisation over the prefill's output
    [B*L, H*P] (one group over all H*P channels, as in the 2.7B layer),
    eager back-to-back calls; and over a decode step's [B, H*P] in a HIP graph."""
    import torch

    from mamba_ssd_scan_chunk_amd import binding as bd
    from mamba_ssd_scan_chunk_amd import synth

    w = synth.WORKLOADS[args.layer_workload]
    D = w.H * w.P
    y = synth.make_tokens(1, w.B * w.L, D, w.dtype, seed=8)[0].cuda()
    z, nw = synth.make_gate((w.B * w.L,), D, w.dtype, seed=9)
    z, nw = z.cuda(), nw.cuda()
    out = torch.empty_like(y)

    def step(_):
        bd.ssd_gated_rmsnorm(y, z, nw, group=D, eps=1e-5, out=out)

    ms = _timed(step, args.steps, args.warmup, "norm")
    es = y.element_size()
    nbytes = 3 * w.B * w.L * D * es + D * 4

    dw = synth.WORKLOADS[args.decode_workload]
    yd, zd, od = y[:dw.B], z[:dw.B], out[:dw.B]

    def dstep(_):
        bd.ssd_gated_rmsnorm(yd, zd, nw, group=D, eps=1e-5, out=od)

    dms = _graph_timed(dstep, 100)
    return w, D, ms, nbytes, dw, dms


def norm_record(args):
    w, D, ms, nbytes, dw, dms = bench_norm(args)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"norm": {"workload": w.name, "rows": w.B * w.L, "channels": D, "group": D, "us": round(ms * 1e3, 2),
                     "algorithmic_mb": round(nbytes / 1e6, 2), "gbs": round(gbs, 1),
                     "hbm_peak_frac": round(gbs / PEAK_HBM_GBS, 4),
                     "decode_rows": {"workload": dw.name, "rows": dw.B, "graph_us": round(dms * 1e3, 2)}}}


def bench_varlen(args):
    """Prefill of 16 prompts of the workload's layer packed without padding,
    lengths log-uniform in [64, 4096], against the same prompts padded to the
    longest one in a uniform batch; 512 prompts of 16-512 tokens packed."""
    import torch

    from mamba_ssd_scan_chunk_amd import binding as bd
    from mamba_ssd_scan_chunk_amd import synth

    w = synth.WORKLOADS[args.layer_workload]
    lengths = synth.make_lengths(16, 64, 4096, seed=9)
    d = {k: v.cuda() for k, v in synth.make_varlen(lengths, w.H, w.P, w.G, w.N, w.dtype, seed=10).items()}
    T = sum(lengths)
    y = torch.empty_like(d["x"])
    fs = torch.empty((len(lengths), w.H, w.P, w.N), dtype=torch.float32, device="cuda")
    code = bd.SSD_BF16 if w.dtype == "bf16" else bd.SSD_F32
    ws = torch.empty(max(1, bd.lib().ssd_prefill_varlen_workspace_bytes(len(lengths), T, w.H, w.P, w.G, w.N, w.Q,
                                                                        code)), dtype=torch.uint8, device="cuda")

    def step(_):
        bd.ssd_prefill_varlen(d["x"], d["dt"], d["A_log"], d["Bm"], d["Cm"], d["D"], d["cu_seqlens"], None, Q=w.Q,
                              y=y, final_state=fs, workspace=ws)

    ms = _timed(step, args.steps, args.warmup, "varlen")
    del d, y, ws
    # many short prompts: 512 of 16-512 tokens (most chunks short)
    short = synth.make_lengths(512, 16, 512, seed=3)
    Ts = sum(short)
    d = {k: v.cuda() for k, v in synth.make_varlen(short, w.H, w.P, w.G, w.N, w.dtype, seed=10).items()}
    y = torch.empty_like(d["x"])
    fs2 = torch.empty((len(short), w.H, w.P, w.N), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, bd.lib().ssd_prefill_varlen_workspace_bytes(len(short), Ts, w.H, w.P, w.G, w.N, w.Q,
                                                                        code)), dtype=torch.uint8, device="cuda")

    def short_step(_):
        bd.ssd_prefill_varlen(d["x"], d["dt"], d["A_log"], d["Bm"], d["Cm"], d["D"], d["cu_seqlens"], None, Q=w.Q,
                              y=y, final_state=fs2, workspace=ws)

    sms = _timed(short_step, max(5, args.steps // 5), 2, "varlen_many_short")
    many_short = {"sequences": len(short), "tokens": Ts, "us": round(sms * 1e3, 2),
                  "tokens_per_s": round(Ts / (sms * 1e-3), 1)}
    del d, y, ws, fs2
    # the depthwise conv over the same packed prompts (x | B | C channels)
    C = w.conv_channels
    xbc = synth.make_tokens(1, T, C, w.dtype, seed=12)[0].cuda()
    cw, _ = synth.make_conv(C, w.K, w.dtype, seed=13)
    cw = cw.cuda()
    cst = torch.zeros((len(lengths), C, w.K - 1), dtype=xbc.dtype, device="cuda")
    cu = torch.tensor([0] + list(itertools.accumulate(lengths)), dtype=torch.int32, device="cuda")
    cout = torch.empty_like(xbc)
    cws = torch.empty(max(1, bd.lib().conv_state_update_varlen_workspace_bytes(len(lengths), T)), dtype=torch.uint8,
                      device="cuda")

    def conv_step(_):
        bd.conv_state_update_varlen(cst, xbc, cu, cw, activation=1, out=cout, workspace=cws)

    cms = _timed(conv_step, args.steps, args.warmup, "varlen_conv")
    cbytes = 2 * T * C * xbc.element_size()
    del xbc, cout
    Lmax = max(lengths)
    p = {k: v.cuda() for k, v in synth.make_prefill(len(lengths), Lmax, w.H, w.P, w.G, w.N, w.dtype, seed=11).items()}

    def padded(_):
        bd.ssd_prefill(p["x"], p["dt"], p["A_log"], p["Bm"], p["Cm"], p["D"], None, Q=w.Q, final_state=fs)

    pms = _timed(padded, max(5, args.steps // 5), 2, "varlen_padded")
    return lengths, T, ms, Lmax, pms, cms, cbytes, many_short


def varlen_record(args):
    lengths, T, ms, Lmax, pms, cms, cbytes, many_short = bench_varlen(args)
    return {"varlen": {"sequences": len(lengths), "tokens": T, "lengths": lengths, "us": round(ms * 1e3, 2),
                       "tokens_per_s": round(T / (ms * 1e-3), 1), "many_short": many_short,
                       "padded": {"batch": len(lengths), "seq_len": Lmax, "us": round(pms * 1e3, 2)},
                       "conv": {"us": round(cms * 1e3, 2), "gbs": round(cbytes / (cms * 1e-3) / 1e9, 1)}}}


def _prefill_rec(r):
    w, ms = r["w"], r["ms"]
    flops = prefill_flops(w.B, w.L, w.H, w.P, w.G, w.N, w.Q)
    nbytes = prefill_bytes(w.B, w.L, w.H, w.P, w.G, w.N, 2 if w.dtype == "bf16" else 4)
    return {"batch": w.B, "seq_len": w.L, "heads": w.H, "us": round(ms * 1e3, 2),
            "tokens_per_s": round(w.B * w.L / (ms * 1e-3), 1), "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "mfma_peak_frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "gbs_compulsory": round(nbytes / (ms * 1e-3) / 1e9, 1)}


def bench_other_prefills(args):
    """The other prefill workloads: the 2.7B-shaped layer at B=1, L=4096 in
    place and over rotated inputs, the 130M-shaped layer (B=1, L=4096, H=24),
    one 65536-token sequence of the 2.7B-shaped layer, the 2.7B-shaped layer
    with 512-token chunks and with fp32 activations, and
    the B=8 cached decode steps that follow the long-context prefill (a HIP
    graph of 256 steps)."""
    import torch

    from mamba_ssd_scan_chunk_amd import binding as bd
    from mamba_ssd_scan_chunk_amd import synth

    out = {}
    for name in ("mamba2-2.7b-prefill", "mamba2-130m-prefill", "mamba2-2.7b-longctx", "mamba2-2.7b-prefill-64k"):
        if name == args.workload:
            continue
        r = bench_prefill(args, name, extras=False)
        rec = _prefill_rec(r)
        if name == "mamba2-2.7b-prefill":
            rr = bench_prefill(args, name, rotate=True, extras=False)
            rec["rotated"] = {"sets": rr["sets"], **{k: v for k, v in _prefill_rec(rr).items()
                                                   if k in ("us", "tokens_per_s", "tflops", "mfma_peak_frac",
                                                            "gbs_compulsory")}}
        out[name] = rec
        torch.cuda.empty_cache()
    # the B=8 decode steps after the long-context prefill, in one HIP graph
    w = synth.WORKLOADS["mamba2-2.7b-longctx"]
    xbc, dts = synth.make_decode_stream(256, w.B, w.H, w.P, w.G, w.N, w.dtype, seed=15)
    xbc, dts = xbc.cuda(), dts.cuda()
    C, K = w.conv_channels, w.K
    cw, _ = synth.make_conv(C, K, w.dtype, seed=16)
    cw = cw.cuda()
    conv = [torch.zeros((w.B, C, K - 1), dtype=xbc.dtype, device="cuda") for _ in range(2)]
    yd = torch.empty((w.B, w.H, w.P), dtype=xbc.dtype, device="cuda")
    A_log = synth.make_prefill(1, 1, w.H, w.P, w.G, w.N, w.dtype, seed=14)["A_log"].cuda()
    fs = synth.make_state(w.B, w.H, w.P, w.N, seed=17, scale=0.3).cuda()
    HP, GN = w.H * w.P, w.G * w.N

    def dstep(i):
        row = xbc[i]
        bd.ssd_decode_step(row[:, :HP], dts[i], A_log, row[:, HP:HP + GN], row[:, HP + GN:], None, fs,
                           y_t=yd, in_stride=C, G=w.G, conv_state_in=conv[i & 1],
                           conv_state_out=conv[(i + 1) & 1], conv_w=cw, K=K, activation=1)

    gms = _graph_timed(dstep, 256)
    dbytes = decode_bytes(w.B, w.H, w.P, w.G, w.N, K, 2)
    out["mamba2-2.7b-longctx-decode"] = {"batch": w.B, "steps": 256, "graph_us_per_step": round(gms * 1e3, 3),
                                         "gbs": round(dbytes / (gms * 1e-3) / 1e9, 1)}
    del xbc, dts, fs
    # the 2.7B-shaped prefill with 512-token chunks (MFMA kernels, 256-token
    # sub-chunks) and with fp32 activations (vector path)
    w = synth.WORKLOADS["mamba2-2.7b-prefill"]
    for key, dtype, Q in (("mamba2-2.7b-prefill-q512", "bf16", 512), ("mamba2-2.7b-prefill-f32", "f32", 256)):
        d = {k: v.cuda() for k, v in synth.make_prefill(w.B, w.L, w.H, w.P, w.G, w.N, dtype, seed=17).items()}
        y = torch.empty_like(d["x"])
        fs = torch.empty((w.B, w.H, w.P, w.N), dtype=torch.float32, device="cuda")
        code = bd.SSD_BF16 if dtype == "bf16" else bd.SSD_F32
        ws = torch.empty(max(1, bd.ssd_prefill_workspace_bytes(w.B, w.L, w.H, w.P, w.G, w.N, Q, code)),
                         dtype=torch.uint8, device="cuda")

        def vstep(_):
            bd.ssd_prefill(d["x"], d["dt"], d["A_log"], d["Bm"], d["Cm"], d["D"], None, Q=Q, y=y, final_state=fs,
                           workspace=ws)

        ms = _timed(vstep, 5 if dtype == "f32" else 50, 1, key)
        path = "mfma, 256-token sub-chunks" if dtype == "bf16" and Q % 256 == 0 else "vector"
        # flops of the chunking the kernels evaluate (the MFMA path runs
        # 256-token sub-chunks, so its intra-chunk work is that of Q = 256)
        run_q = 256 if path.startswith("mfma") else Q
        flops = prefill_flops(w.B, w.L, w.H, w.P, w.G, w.N, run_q)
        out[key] = {"dtype": dtype, "chunk": Q, "path": path, "us": round(ms * 1e3, 1),
                    "tokens_per_s": round(w.B * w.L / (ms * 1e-3), 1),
                    "flop_chunk": run_q, "tflops": round(flops / (ms * 1e-3) / 1e12, 2)}
        del d, y, ws
    return {"other_workloads": out}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(args):
    """The oracle (fp64, token by token, threads over (batch, head) pairs) on
    the host cores.  The sample is bounded so that it takes about
    --cpu-seconds: batch element 0 of the workload, every head, its first
    min(L, 4096) tokens, repeated; the sequential scan costs the same per
    token at any length, so tokens/s of the sample is the oracle's rate on
    the whole workload.  Beside it, the decode step rate of the oracle on the
    decode workload (every batch element and head, conv included)."""
    import oracle
    from mamba_ssd_scan_chunk_amd import synth

    w = synth.WORKLOADS[args.workload]
    Ls = min(w.L, 4096)
    d = synth.make_prefill(1, Ls, w.H, w.P, w.G, w.N, w.dtype, seed=2)
    oracle.build()
    threads = oracle.default_threads()
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.ssd_scan(**d, nthreads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= args.cpu_seconds or reps >= 100:
            break
    dw = synth.WORKLOADS[args.decode_workload]
    H, P, G, N, K = dw.H, dw.P, dw.G, dw.N, dw.K
    xbc, dts = synth.make_decode_stream(8, dw.B, H, P, G, N, dw.dtype, seed=4)
    cw, _ = synth.make_conv(dw.conv_channels, K, dw.dtype, seed=5)
    pre = synth.make_prefill(1, 1, H, P, G, N, dw.dtype, seed=3)
    state = synth.make_state(dw.B, H, P, N, seed=6, scale=0.3).double().numpy()
    conv = synth.make_tokens(dw.B, K - 1, dw.conv_channels, dw.dtype, seed=7).transpose(1, 2).double().numpy()
    HP, GN = H * P, G * N
    dsteps, t1 = 0, time.perf_counter()
    while True:
        r = xbc[dsteps % 8]
        _, state, conv = oracle.decode_step(r[:, :HP], dts[dsteps % 8], pre["A_log"], r[:, HP:HP + GN],
                                            r[:, HP + GN:], pre["D"], state, conv_state=conv, conv_w=cw,
                                            activation=True, nthreads=threads)
        dsteps += 1
        dsec = time.perf_counter() - t1
        if dsec >= args.cpu_seconds / 3 or dsteps >= 2000:
            break
    return dict(value=round(reps * Ls / el, 2), unit="tokens/s", cores=threads, kind="oracle",
                cpu_model=_cpu_model(),
                sample=f"{w.name}: batch element 0, all {w.H} heads, first {Ls} tokens (P={w.P}, N={w.N}), "
                       f"run {reps} times in {el:.1f} s, fp64, one thread per (batch, head) share",
                decode={"workload": dw.name, "batch": dw.B, "steps": dsteps, "seconds": round(dsec, 2),
                        "steps_per_s": round(dsteps / dsec, 2),
                        "sample": "fused decode steps (conv window + state update + readout) of every batch "
                                  "element and head, fp64"})


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mamba2-2.7b-longctx", help="the prefill workload `value` measures")
    ap.add_argument("--layer-workload", default="mamba2-2.7b-prefill",
                    help="the one-prompt layer of the conv, norm and packed legs")
    ap.add_argument("--decode-workload", default="mamba2-2.7b-decode-b16")
    ap.add_argument("--decode-steps", type=int, default=4096)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-only", action="store_true", help="skip every leg but the prefill")
    ap.add_argument("--legs", default="prefill,decode,conv,norm,varlen,other",
                    help="comma-separated subset of prefill,decode,conv,norm,varlen,other, and the calibration "
                         "legs copy and gemm (for profiling runs)")
    ap.add_argument("--no-decode-extras", action="store_true",
                    help="decode leg: only the stated workload's one-state and rotated-state runs (no other batch, "
                         "raw-step, ceiling or recompute legs), so that every decode dispatch has the same size")
    ap.add_argument("--stage-runs", type=int, default=20, help="timed calls for the per-kernel durations")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: the benchmark measures one GPU; the scan "
              "shards over (batch, head) with no communication, so N GPUs run N independent copies",
              file=sys.stderr)
        return 2

    import torch

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)

    legs = set(args.legs.split(","))
    if args.prefill_only:
        legs = {"prefill"}
    out = {}
    steps = [("prefill", prefill_record), ("decode", decode_record), ("conv", conv_record), ("norm", norm_record),
             ("varlen", varlen_record), ("other", bench_other_prefills), ("copy", copy_record),
             ("gemm", gemm_record)]
    clocks = {}
    for leg, fn in steps:
        if leg in legs:
            print(f"[bench] {leg}", file=sys.stderr, flush=True)
            out.update(fn(args))
            if leg in ("prefill", "decode"):
                clocks[f"after_{leg}"] = gpu_clocks()
            torch.cuda.empty_cache()
    if clocks:
        out["clocks"] = clocks
    if HOST_BOUND:
        out["host_bound_legs"] = HOST_BOUND
    if not args.no_cpu_baseline:
        print("[bench] cpu_baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(args)
    print(json.dumps(out), flush=True)
    return 0


def gpu_clocks():
    """Shader (sclk) and memory (mclk) clock levels the GPU is at, in MHz, from
    the driver's sysfs DPM tables (the level marked '*'), or None where they
    cannot be read; sampled right after a timed leg, they show the clocks that
    leg ran at."""
    import glob

    out = {}
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        for key in ("sclk", "mclk"):
            try:
                with open(os.path.join(dev, f"pp_dpm_{key}")) as fh:
                    for line in fh:
                        if line.rstrip().endswith("*"):
                            out[f"{key}_mhz"] = int(line.split(":")[1].strip().lower().split("mhz")[0])
            except (OSError, ValueError, IndexError):
                pass
        if out:
            return out
    return None


def prefill_record(args):
    r = bench_prefill(args, args.workload)
    w, ms, stages = r["w"], r["ms"], r["stages"]
    esize = 2 if w.dtype == "bf16" else 4
    shape = (w.B, w.L, w.H, w.P, w.G, w.N)
    flops = prefill_flops(*shape, w.Q)
    nbytes = prefill_bytes(*shape, esize)
    tflops = flops / (ms * 1e-3) / 1e12
    chained = "chunk_chain_mfma" in stages
    stage_rec = {}
    counted = measured_mfma(w.name)
    for name, sms in stages.items():
        sb, sf = stage_work(name, *shape, w.Q, esize, chained)
        ab = section8d_bytes(name, *shape, esize)
        stage_rec[name] = {"us": round(sms * 1e3, 2), "algorithmic_mb": round(ab / 1e6, 2),
                           "gbs": round(ab / (sms * 1e-3) / 1e9, 1), "own_mb": round(sb / 1e6, 2),
                           "tflops": round(sf / (sms * 1e-3) / 1e12, 2),
                           "counted_traffic_mb": (lambda t: None if t is None else round(t / 1e6, 2))(
                               measured_traffic(name, w.name))}
        if name in counted:
            # flops the MFMA units executed (rocprofv3 counter, padding included) over this run's duration
            stage_rec[name]["mfma_counted_gflop"] = round(counted[name] / 1e9, 3)
            stage_rec[name]["mfma_counted_peak_frac"] = round(
                counted[name] / (sms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
    # dominant kernel: its algorithmic bytes (the compulsory bytes of the
    # units it processes) over its own average duration, against HBM: the
    # scan's arithmetic intensity (about 185 flop/B) is below the MI355X
    # ridge (2.5 PF / 8 TB/s = 312 flop/B)
    dom = max(stages, key=stages.get)
    db = section8d_bytes(dom, *shape, esize)
    own_b, dfl = stage_work(dom, *shape, w.Q, esize, chained)
    dt_s = stages[dom] * 1e-3
    call_traffic = [measured_traffic(k, w.name) for k in stages]
    roof = {"bound": "hbm", "achieved": round(db / dt_s / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(db / dt_s / 1e9 / PEAK_HBM_GBS, 4), "traffic": measured_traffic(dom, w.name),
            "kernel": dom, "algorithmic_bytes_per_launch": db, "algorithmic_flops_per_launch": dfl,
            "avg_launch_us": round(stages[dom] * 1e3, 2), "own_bytes_per_launch": own_b,
            "mfma_frac": round(dfl / dt_s / 1e12 / PEAK_BF16_TFLOPS, 4),
            "call": {"us": round(ms * 1e3, 2), "algorithmic_bytes": nbytes,
                     "achieved": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "counted_traffic": None if None in call_traffic else sum(call_traffic)}}
    return {
        "metric": "SSD prefill tokens/s + TFLOPS (% MFMA peak); decode step GB/s (% HBM peak)",
        "value": round(w.B * w.L / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "seq_len": w.L, "heads": w.H, "head_dim": w.P,
                   "state_dim": w.N, "groups": w.G, "chunk": w.Q, "parallelism": "single-gpu"},
        "prefill": {"tflops": round(tflops, 2), "mfma_peak_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                    "algorithmic_gflop": round(flops / 1e9, 3), "compulsory_mb": round(nbytes / 1e6, 2),
                    "gbs_compulsory": round(nbytes / (ms * 1e-3) / 1e9, 1),
                    "attainable_frac": round(tflops / min(PEAK_BF16_TFLOPS, flops / nbytes * PEAK_HBM_GBS / 1e3), 4),
                    "path": "chained single pass" if chained else ("four kernels" if "chunk_out_mfma" in stages
                                                                  else "vector"),
                    "graph": {"us_per_call": round(r["graph_ms"] * 1e3, 2),
                              "tokens_per_s": round(w.B * w.L / (r["graph_ms"] * 1e-3), 1)},
                    "dt_raw": {"us_per_call": round(r["raw_ms"] * 1e3, 2),
                               "tokens_per_s": round(w.B * w.L / (r["raw_ms"] * 1e-3), 1)},
                    "kernels": stage_rec},
        "roofline": roof,
    }


def copy_record(args):
    """A plain streaming kernel of known size, the reference for calibrating
    rocprofv3's FETCH_SIZE / WRITE_SIZE counters: torch.neg reading 256 MiB
    and writing 256 MiB (a kernel of its own name, unlike a memcpy)."""
    import torch

    n = 64 * 2**20
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    ms = _timed(lambda _: torch.neg(src, out=dst), max(3, min(args.steps, 20)), 2, "copy")
    return {"copy": {"bytes_read": 4 * n, "bytes_written": 4 * n, "us": round(ms * 1e3, 2),
                     "gbs": round(8 * n / (ms * 1e-3) / 1e9, 1)}}


def gemm_record(args):
    """A plain library GEMM of known flops, the reference for rocprofv3's MFMA
    counters: torch.matmul of two contiguous 8192 x 8192 bf16 matrices
    (2 * 8192^3 flops, no padding), timed like the other legs."""
    import torch

    n = 8192
    g = torch.Generator(device="cuda").manual_seed(7)
    a = torch.randn(n, n, dtype=torch.bfloat16, device="cuda", generator=g).contiguous()
    b = torch.randn(n, n, dtype=torch.bfloat16, device="cuda", generator=g).contiguous()
    c = torch.empty(n, n, dtype=torch.bfloat16, device="cuda")
    ms = _timed(lambda _: torch.matmul(a, b, out=c), max(3, min(args.steps, 10)), 2, "gemm")
    flops = 2 * n ** 3
    return {"gemm": {"m": n, "n": n, "k": n, "flops": flops, "us": round(ms * 1e3, 2),
                     "tflops": round(flops / (ms * 1e-3) / 1e12, 1)}}


def _decode_graph_step_ms(name, steps=512):
    """GPU ms per fused decode step (conv on) of workload `name`, 512 steps
    in one HIP graph, from a random state."""
    import torch

    from mamba_ssd_scan_chunk_amd import binding as bd
    from mamba_ssd_scan_chunk_amd import synth

    w = synth.WORKLOADS[name]
    B, H, P, G, N, K, C = w.B, w.H, w.P, w.G, w.N, w.K, w.conv_channels
    xbc, dts = synth.make_decode_stream(steps, B, H, P, G, N, w.dtype, seed=18)
    xbc, dts = xbc.cuda(), dts.cuda()
    cw, _ = synth.make_conv(C, K, w.dtype, seed=19)
    cw = cw.cuda()
    pre = synth.make_prefill(1, 1, H, P, G, N, w.dtype, seed=20)
    A_log, D = pre["A_log"].cuda(), pre["D"].cuda()
    state = synth.make_state(B, H, P, N, seed=21, scale=0.3).cuda()
    conv = [torch.zeros((B, C, K - 1), dtype=xbc.dtype, device="cuda") for _ in range(2)]
    y = torch.empty((B, H, P), dtype=xbc.dtype, device="cuda")
    HP, GN = H * P, G * N

    def step(i):
        row = xbc[i % steps]
        bd.ssd_decode_step(row[:, :HP], dts[i % steps], A_log, row[:, HP:HP + GN], row[:, HP + GN:], D, state,
                           y_t=y, in_stride=C, G=G, conv_state_in=conv[i & 1], conv_state_out=conv[(i + 1) & 1],
                           conv_w=cw, K=K, activation=1)

    return _graph_timed(step, steps)


def cached_vs_recompute(name, cached_step_ms=None):
    """The cached decode step against recomputing the sequence: conv over the
    L + 1 tokens plus the SSD prefill of L + 1 tokens, for the same layer and
    batch (the comparison behind the pages' cached-decode speedup at a
    4096-token context)."""
    import torch

    from mamba_ssd_scan_chunk_amd import binding as bd
    from mamba_ssd_scan_chunk_amd import synth

    w = synth.WORKLOADS[name]
    if cached_step_ms is None:
        cached_step_ms = _decode_graph_step_ms(name)
    L1 = w.L + 1
    C, K = w.conv_channels, w.K
    d = {k: v.cuda() for k, v in synth.make_prefill(w.B, L1, w.H, w.P, w.G, w.N, w.dtype, seed=8).items()}
    xbc = synth.make_tokens(w.B, L1, C, w.dtype, seed=9).cuda()
    cw, _ = synth.make_conv(C, K, w.dtype, seed=10)
    cw = cw.cuda()
    st = torch.zeros((w.B, C, K - 1), dtype=xbc.dtype, device="cuda")
    out = torch.empty_like(xbc)
    y = torch.empty_like(d["x"])
    code = bd.SSD_BF16 if w.dtype == "bf16" else bd.SSD_F32
    ws = torch.empty(bd.ssd_prefill_workspace_bytes(w.B, L1, w.H, w.P, w.G, w.N, w.Q, code),
                     dtype=torch.uint8, device="cuda")

    def recompute(_):
        st.zero_()
        bd.conv_state_update(st, xbc, cw, activation=1, out=out)
        bd.ssd_prefill(d["x"], d["dt"], d["A_log"], d["Bm"], d["Cm"], d["D"], None, Q=w.Q, y=y, workspace=ws)

    ms = _graph_timed(recompute, 10)
    return {"workload": w.name, "batch": w.B, "heads": w.H, "tokens": L1, "recompute_us": round(ms * 1e3, 2),
            "cached_step_us": round(cached_step_ms * 1e3, 3), "speedup": round(ms / cached_step_ms, 1)}


def stream_ceilings(args, state_elems, nrot, steps):
    """What a plain streaming kernel reaches on the box, for the decode
    fraction: an in-place scale h <- 0.9999 h (one torch kernel, reading and
    writing the decode state's bytes once) over the same rotated buffers as
    the decode leg and on one buffer, ``steps`` launches in one HIP graph;
    and a 1 GiB device copy, 20 launches in one graph."""
    import torch

    bufs = [torch.ones(state_elems, dtype=torch.float32, device="cuda") for _ in range(nrot)]
    nb = 8 * state_elems
    rot = _graph_timed(lambda i: bufs[i % nrot].mul_(0.9999), steps)
    one = _graph_timed(lambda i: bufs[0].mul_(0.9999), steps)
    del bufs
    n = 2**28  # 1 GiB of fp32
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    cp = _graph_timed(lambda i: dst.copy_(src), 20)
    del src, dst
    gbs = lambda b, ms: round(b / (ms * 1e-3) / 1e9, 1)  # noqa: E731
    return {"inplace_scale": {"bytes": nb, "buffers": nrot, "rotated_us": round(rot * 1e3, 3),
                              "rotated_gbs": gbs(nb, rot), "one_buffer_us": round(one * 1e3, 3),
                              "one_buffer_gbs": gbs(nb, one)},
            "copy_1gib": {"bytes": 2 * 4 * n, "us": round(cp * 1e3, 1), "gbs": gbs(2 * 4 * n, cp)}}


def decode_record(args):
    dw, dms, gms, dbytes, _ = bench_decode(args, rotate=False)
    _, rms, rgms, _, nrot = bench_decode(args, rotate=True)
    gbs = lambda ms: dbytes / (ms * 1e-3) / 1e9  # noqa: E731
    extra = {}
    b1_ms = gms if dw.B == 1 else None
    if not args.no_decode_extras:
        # the step passed raw and preprocessed in the kernel
        _, _, raw_gms, _, _ = bench_decode(args, rotate=False, raw_dt=True)
        extra["dt_raw"] = {"graph_us_per_step": round(raw_gms * 1e3, 3), "gbs": round(gbs(raw_gms), 1)}
        # the other batch size of the stated decode workload, in one HIP graph
        other = {"mamba2-2.7b-decode-b16": "mamba2-2.7b-decode-b1",
                 "mamba2-2.7b-decode-b1": "mamba2-2.7b-decode-b16"}.get(args.decode_workload)
        if other is not None:
            oargs = argparse.Namespace(**vars(args))
            oargs.decode_workload = other
            oargs.decode_steps = min(args.decode_steps, 1024)
            ow, _, ogms, obytes, _ = bench_decode(oargs, rotate=False)
            extra["other_batch"] = {"workload": ow.name, "batch": ow.B, "steps": oargs.decode_steps,
                                    "graph_us_per_step": round(ogms * 1e3, 3),
                                    "gbs": round(obytes / (ogms * 1e-3) / 1e9, 1)}
            if ow.B == 1:
                b1_ms = ogms
        # the box's streaming ceiling at the decode state's size
        ceil = stream_ceilings(args, dw.B * dw.H * dw.P * dw.N, nrot, min(args.decode_steps, 1024))
        ceil["decode_rotated_vs_inplace_scale"] = round(ceil["inplace_scale"]["rotated_us"] / (rgms * 1e3), 4)
        extra["ceilings"] = ceil
        # cached decode against recomputing the 4096-token prefix, per layer and batch
        cvr = []
        for name in ("mamba2-130m-decode-b1", "mamba2-130m-decode-b16", "mamba2-2.7b-decode-b1",
                     "mamba2-2.7b-decode-b16"):
            known = {dw.name: gms, "mamba2-2.7b-decode-b1": b1_ms}.get(name)
            cvr.append(cached_vs_recompute(name, known))
        extra["cached_vs_recompute"] = cvr
    return {
        "decode": {"workload": dw.name, "batch": dw.B, "steps": args.decode_steps, "bytes_per_step": dbytes,
                   "graph": {"us_per_step": round(gms * 1e3, 3), "steps_per_s": round(1e3 / gms, 1),
                             "gbs": round(gbs(gms), 1), "hbm_peak_frac": round(gbs(gms) / PEAK_HBM_GBS, 4)},
                   "eager": {"us_per_step": round(dms * 1e3, 3), "gbs": round(gbs(dms), 1)},
                   "rotated": {"states": nrot, "graph_us_per_step": round(rgms * 1e3, 3),
                               "graph_steps_per_s": round(1e3 / rgms, 1),
                               "graph_gbs": round(gbs(rgms), 1), "hbm_peak_frac": round(gbs(rgms) / PEAK_HBM_GBS, 4),
                               "eager_us_per_step": round(rms * 1e3, 3)},
                   **extra},
        "roofline_decode": {"bound": "hbm", "achieved": round(gbs(rgms), 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(gbs(rgms) / PEAK_HBM_GBS, 4),
                            # the committed counters were taken on the default (B = 16) workload
                            "traffic": measured_traffic("decode_step_kernel", dw.name),
                            "kernel": "ssd_decode_step, rotated states, 4096 steps in one HIP graph"},
    }


def conv_record(args):
    from mamba_ssd_scan_chunk_amd import synth

    w = synth.WORKLOADS[args.layer_workload]
    cms, cbytes = bench_conv(args)
    return {"conv": {"tokens": w.L, "channels": w.conv_channels, "us": round(cms * 1e3, 3),
                     "gbs": round(cbytes / (cms * 1e-3) / 1e9, 1)}}


if __name__ == "__main__":
    sys.exit(main())
