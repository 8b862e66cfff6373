#!/usr/bin/env python3
"""Throughput of the exact-attention hot path on one MI355X.

One step = the bf16 forward and backward of the long-context workload
B=1, H=32, N=16384, d=128 with the causal mask and without it: for each
mask, attn_fwd and the two backward stages that attn_bwd enqueues
(attn_bwd_dq, then attn_bwd_dkdv).  Inputs are seeded synthetic N(0,1)
values rounded to bf16, resident in HBM before timing starts; outputs are
preallocated.

value = credited FLOPs per step / step time, with the metric's convention:
forward 4*B*H*N^2*d (halved for causal), backward 2.5x the forward.  Each
kernel launch is bracketed by HIP events on the stream it runs on; the
dominant kernel (most GPU time per step) is reported against its roofline
(credited FLOPs per launch over its average launch time).  Launch labels
name the kernel each entry point runs, as the library reports it
(attn_kernel_name).  The fp64 CPU oracle is timed on a bounded sample of the
same workload as a reference point.

After the timed step, with their own HIP-event timing and outside `value`:
the fp8 forward (`fp8`, against the 16-bit MFMA peak that its products run
at, with the fp8 peak's fraction beside it), grouped-query attention
(`gqa`), decode (`decode`, against HBM), dropout (`dropout`, beside the same
calls without it) and every other workload of the metric (`configs`);
--no-extra-paths skips them.

The roofline's "traffic" (HBM bytes per launch of the dominant kernel) is
read from the rocprofv3 counter summary committed under profiles/, and only
while the kernel sources still hash to the value recorded there; otherwise
it is null.  --hbm-copy-mib M adds, after the timed region, one plain
device-to-device copy of M MiB whose known size calibrates those counters.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--no-extra-paths] [--hbm-copy-mib M]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "exact_attention_79_amd", "csrc")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "hbm_traffic_B1H32N16384.md")

METRIC = "attention fwd/bwd TFLOPS (bf16, causal & non-causal) and % of MFMA peak"
# MI355X dense peaks: 256 CUs x 2.4 GHz x (4096 bf16 | 8192 fp8) flop/clk/CU.
PEAK_BF16_TFLOPS = 2516.6
PEAK_FP8_TFLOPS = 5033.2
HBM_GBPS = 8000.0
# The timed workload: long-context, d = 128 (the targets are stated for
# N >= 4096, d = 128); seeds of the long-context workload (number 3).
STEP_B, STEP_H, STEP_N, STEP_D, STEP_SEEDS = 1, 32, 16384, 128, 3


def visible_pairs(N: int, causal: bool, window: int) -> int:
    """Number of (query, key) pairs that survive the mask, per head."""
    if window <= 0 or window >= N:
        return N * (N + 1) // 2 if causal else N * N
    W = window
    if causal:
        return W * (W + 1) // 2 + (N - W) * W
    # |i - j| < W
    return N * (2 * W - 1) - W * (W - 1)


def credited_fwd_flops(BH: int, N: int, d: int, causal: bool, window: int) -> float:
    """4*BH*N^2*d, halved for causal; exact visible pairs for a window."""
    if window > 0 and window < N:
        return 4.0 * d * BH * visible_pairs(N, causal, window)
    return 4.0 * BH * N * N * d * (0.5 if causal else 1.0)


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra-paths", action="store_true",
                    help="skip the fp8, grouped-query, decode, dropout and per-workload "
                         "measurements that follow the timed step (for profiler runs "
                         "that should see the step only)")
    ap.add_argument("--paths", default="fp8,gqa,decode,dropout,configs",
                    help="comma-separated extra measurements to run after the timed "
                         "step (a subset of the default; for profiler runs of one path)")
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="step",
                    help="time another workload in place of the step (for profiler runs: "
                         "bwd4096 = B4 H16 N4096 d128 causal forward + backward, fp8 = the "
                         "B2 H32 N8192 d128 fp8 forward); the result line then describes it")
    ap.add_argument("--hbm-copy-mib", type=int, default=0,
                    help="after timing, one fp32 -> bf16 copy of this many MiB of "
                         "fp32 (counter calibration for rocprofv3 --pmc runs)")
    return ap.parse_args()


def kernel_sources_sha256() -> str:
    """Hash of every kernel source file, in name order."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp")):
            h.update(name.encode())
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def recorded_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary,
    or None when there is none or the kernel sources changed since."""
    try:
        text = open(TRAFFIC_SUMMARY).read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, flags=re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel") != kernel or rec.get("sources_sha256") != kernel_sources_sha256():
        return None
    return rec.get("hbm_bytes_per_launch")


class Launch:
    """One kernel launch per step: its name, credited FLOPs, executed FLOPs
    and bound, plus the events around it."""

    def __init__(self, name, kernel, fn, credited, executed, peak):
        self.name, self.kernel, self.fn = name, kernel, fn
        self.credited, self.executed, self.peak = credited, executed, peak
        self.times_ms = []


# Workloads a profiler run can time in place of the step (--workload): the
# causal backward workload B4 H16 N4096 and the fp8 forward B2 H32 N8192.
# Each keeps the seeds of its workload number.
WORKLOADS = {
    "step": dict(B=STEP_B, H=STEP_H, N=STEP_N, d=STEP_D, masks=(False, True), seeds=STEP_SEEDS),
    "bwd4096": dict(B=4, H=16, N=4096, d=128, masks=(True,), seeds=4),
    "fp8": dict(B=2, H=32, N=8192, d=128, masks=(False,), seeds=5),
}


def build_fp8_step(ea, torch, attn_synth, w):
    """The fp8 forward as a step: inputs with one x10 outlier channel,
    quantised per tensor to e4m3 on the host (attn_synth).  The kernel runs
    both products on the 16-bit matrix cores (the e4m3 tiles widened in
    LDS), so its roofline is the bf16/fp16 peak."""
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    f8 = attn_synth.fp8_attention_inputs(w["seeds"], B, H, N, d)
    q8, k8, v8 = (torch.from_numpy(f8[n]).cuda() for n in ("q", "k", "v"))
    o = torch.empty((B, H, N, d), device="cuda", dtype=torch.bfloat16)
    lse = torch.empty((B, H, N), device="cuda", dtype=torch.float32)
    f = credited_fwd_flops(B * H, N, d, False, 0)
    fn = lambda: ea.attn_fwd_fp8(q8, k8, v8, f8["q_descale"], f8["k_descale"],
                                 f8["v_descale"], out=o, lse=lse)
    return [Launch("attn_fwd_fp8 non-causal", ea.kernel_name(ea.STAGE_FWD_FP8, B, H, N, d), fn,
                   f, f, PEAK_BF16_TFLOPS)]


def build_step(ea, torch, attn_synth, workload="step"):
    """All launches of one step, with inputs resident on the device."""
    import numpy as np
    w = WORKLOADS[workload]
    if workload == "fp8":
        return build_fp8_step(ea, torch, attn_synth, w)
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    BH = B * H
    launches = []

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.bfloat16).cuda()

    bits = attn_synth.bf16_attention_inputs(w["seeds"], B, H, N, d, with_dout=True)
    q, k, v, do = (dev_bf16(bits[n]) for n in ("q", "k", "v", "do"))
    del bits
    ws = torch.empty(ea.attn_bwd_workspace_bytes(B, H, N, d), device="cuda", dtype=torch.uint8)
    dq = torch.empty(q.shape, device="cuda", dtype=torch.float32)
    dk = torch.empty(q.shape, device="cuda", dtype=torch.float32)
    dv = torch.empty(q.shape, device="cuda", dtype=torch.float32)
    for causal in w["masks"]:
        tag = "causal" if causal else "non-causal"
        t = dict(q=q, k=k, v=v, do=do, causal=causal, o=torch.empty_like(q),
                 lse=torch.empty((B, H, N), device="cuda", dtype=torch.float32),
                 dq=dq, dk=dk, dv=dv, ws=ws)

        # Every launch reads the tensors bound in its own dict `t`; the
        # binding derives the descriptor from their shapes.
        def fwd(t=t):
            ea.attn_fwd(t["q"], t["k"], t["v"], causal=t["causal"], out=t["o"], lse=t["lse"])

        def bwd_dq(t=t):
            ea.attn_bwd_dq(t["q"], t["k"], t["v"], t["o"], t["do"], t["lse"], t["ws"], t["dq"],
                           causal=t["causal"])

        def bwd_dkdv(t=t):
            ea.attn_bwd_dkdv(t["q"], t["k"], t["v"], t["do"], t["ws"], t["dk"], t["dv"],
                             causal=t["causal"])

        fwd()  # O and L for the backward launches
        f = credited_fwd_flops(BH, N, d, causal, 0)
        # Backward credit (2.5x fwd) is split over the five products: the
        # dK/dV pass computes S, dP, dV, dK (4/5 of it), the dQ pass dQ
        # (1/5) and also recomputes S and dP (executed, not credited).
        bwd = 2.5 * f
        name = lambda stage: ea.kernel_name(stage, B, H, N, d, causal)
        launches.append(Launch(f"attn_fwd {tag}", name(ea.STAGE_FWD), fwd, f, f,
                               PEAK_BF16_TFLOPS))
        # The dQ pass runs first: it also forms D = rowsum(dO * O) and leaves
        # D and L log2(e) in the workspace for the dK/dV pass.
        launches.append(Launch(f"attn_bwd_dq {tag}", name(ea.STAGE_BWD_DQ), bwd_dq, 0.2 * bwd,
                               0.6 * bwd, PEAK_BF16_TFLOPS))
        launches.append(Launch(f"attn_bwd_dkdv {tag}", name(ea.STAGE_BWD_DKDV), bwd_dkdv,
                               0.8 * bwd, 0.8 * bwd, PEAK_BF16_TFLOPS))
    return launches


def run_step(launches, torch, record):
    evs = []
    for L in launches:
        if record:
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            evs.append(e)
        L.fn()
    if record:
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        evs.append(e)
    return evs


def measure_gqa(ea, torch, attn_synth, reps=10):
    """Grouped-query attention at B4 H16 N2048 d128 with 4 key/value heads
    (4 query heads per group), causal and non-causal: forward, dQ pass and
    dK/dV pass, each timed with HIP events over `reps` launches.  Measured
    after the timed step and reported beside it; it does not enter `value`.
    Credited FLOPs as for ordinary attention (the query heads decide them)."""
    import numpy as np
    B, H, Hkv, N, d = 4, 16, 4, 2048, 128
    bits = attn_synth.bf16_attention_inputs(2, B, H, N, d, with_dout=True)

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(
            torch.bfloat16).cuda()
    q, do = dev(bits["q"]), dev(bits["do"])
    k, v = dev(bits["k"][:, :Hkv]), dev(bits["v"][:, :Hkv])
    out = {"workload": f"B{B} H{H} H_kv{Hkv} N{N} d{d}, bf16"}
    for causal in (False, True):
        o, lse = ea.attn_fwd(q, k, v, causal=causal)
        ws = torch.empty(ea.attn_bwd_workspace_bytes(B, H, N, d, Hkv, causal), device="cuda",
                         dtype=torch.uint8)
        dq = torch.empty(q.shape, device="cuda", dtype=torch.float32)
        dk, dv = (torch.empty(k.shape, device="cuda", dtype=torch.float32)
                  for _ in range(2))
        runs = {
            "fwd": lambda: ea.attn_fwd(q, k, v, causal=causal, out=o, lse=lse),
            "bwd_dq": lambda: ea.attn_bwd_dq(q, k, v, o, do, lse, ws, dq, causal=causal),
            "bwd_dkdv": lambda: ea.attn_bwd_dkdv(q, k, v, do, ws, dk, dv, causal=causal),
        }
        f = credited_fwd_flops(B * H, N, d, causal, 0)
        credit = {"fwd": f, "bwd_dq": 0.5 * f, "bwd_dkdv": 2.0 * f}
        row = {}
        for name, fn in runs.items():
            fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            row[name] = {"ms": round(ms, 4),
                         "tflops": round(credit[name] / (ms * 1e-3) / 1e12, 1)}
        tot = sum(r["ms"] for r in row.values())
        row["fwd_bwd_tflops"] = round(3.5 * f / (tot * 1e-3) / 1e12, 1)
        out["causal" if causal else "non_causal"] = row
    return out


def measure_dropout(ea, torch, attn_synth, reps=10, p=0.1):
    """Dropout on P (p = 0.1) at B4 H16 N2048 d128, causal and non-causal: the
    forward and the whole backward (dQ pass + dK/dV pass), each timed with
    HIP events over `reps` calls, beside the same calls without dropout.
    Measured after the timed step; it does not enter `value`.  Credited FLOPs
    as without dropout."""
    import numpy as np
    B, H, N, d = 4, 16, 2048, 128
    bits = attn_synth.bf16_attention_inputs(2, B, H, N, d, with_dout=True)

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(
            torch.bfloat16).cuda()
    q, k, v, do = (dev(bits[n]) for n in ("q", "k", "v", "do"))
    out = {"workload": f"B{B} H{H} N{N} d{d}, bf16, p={p}"}
    ws = torch.empty(ea.attn_bwd_workspace_bytes(B, H, N, d), device="cuda",
                     dtype=torch.uint8)
    grads = tuple(torch.empty(q.shape, device="cuda", dtype=torch.float32) for _ in range(3))
    for causal in (False, True):
        o, lse = ea.attn_fwd_dropout(q, k, v, p, 1, 0, causal=causal)
        o0, lse0 = ea.attn_fwd(q, k, v, causal=causal)
        runs = {
            "fwd": lambda: ea.attn_fwd_dropout(q, k, v, p, 1, 0, causal=causal, out=o,
                                               lse=lse),
            "bwd": lambda: ea.attn_bwd_dropout(q, k, v, o, do, lse, p, 1, 0, causal=causal,
                                               workspace=ws, grads=grads),
            "fwd_plain": lambda: ea.attn_fwd(q, k, v, causal=causal, out=o0, lse=lse0),
            "bwd_plain": lambda: ea.attn_bwd(q, k, v, o0, do, lse0, causal=causal,
                                             workspace=ws, grads=grads),
        }
        f = credited_fwd_flops(B * H, N, d, causal, 0)
        credit = {"fwd": f, "bwd": 2.5 * f, "fwd_plain": f, "bwd_plain": 2.5 * f}
        row = {}
        for name, fn in runs.items():
            fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            row[name] = {"ms": round(ms, 4),
                         "tflops": round(credit[name] / (ms * 1e-3) / 1e12, 1)}
        row["fwd_bwd_tflops"] = round(3.5 * f / ((row["fwd"]["ms"] + row["bwd"]["ms"])
                                                 * 1e-3) / 1e12, 1)
        out["causal" if causal else "non_causal"] = row
    return out


def _time_ms(torch, fn, reps):
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _time_each_us(torch, fn, reps, flush=None):
    """GPU time of single calls, in microseconds: each call is enqueued behind
    a ~1 ms device-side spin (torch.cuda._sleep), so the events around it
    measure the device's work for the call and not the host's time to issue
    it; `flush`, when given, runs before the spin (untimed).  Returns
    (median, min) over `reps` calls after one untimed call."""
    fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        if flush is not None:
            flush()
        torch.cuda._sleep(2_000_000)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3)
    ts.sort()
    return ts[len(ts) // 2], ts[0]


def measure_configs(ea, torch, reps=10):
    """Every other workload of the metric beside the timed step: the
    single-head forward (latency and HBM rate), the B4 H16 N2048 sweep
    (d 64 and 128, both masks), the long-context causal window, the
    B4 H16 N4096 causal backward and the other N >= 4096, d = 128 points at
    which the forward and backward targets are stated.  Inputs are N(0,1)
    draws of torch's seeded device generator (the same distributions as the
    tests' inputs, drawn on the device because the host generator needs tens
    of seconds at these sizes).  Measured after the timed step; none of it
    enters `value`."""
    gen = torch.Generator(device="cuda").manual_seed(79)

    def randn(*shape):
        return torch.randn(shape, device="cuda", generator=gen).bfloat16()

    def pct(tf, peak=PEAK_BF16_TFLOPS):
        return round(100.0 * tf / peak, 1)

    out = {}
    # Single head, fp32 output: launch-latency bound, reported as time and GB/s.
    q, k, v = randn(1, 1, 256, 64), randn(1, 1, 256, 64), randn(1, 1, 256, 64)
    o = torch.empty(q.shape, device="cuda", dtype=torch.float32)
    lse = torch.empty((1, 1, 256), device="cuda", dtype=torch.float32)
    call = lambda: ea.attn_fwd(q, k, v, out_dtype=torch.float32, out=o, lse=lse)
    ms = _time_ms(torch, call, 50)
    nbytes = 3 * 256 * 64 * 2 + 256 * 64 * 4 + 256 * 4
    # Device time of one call with warm caches, and after 512 MiB have been
    # written (more than the L2s and the 256 MB MALL hold): median and min.
    flush_buf = torch.empty(512 << 20, device="cuda", dtype=torch.uint8)
    warm = _time_each_us(torch, call, 50)
    cold = _time_each_us(torch, call, 50, flush=lambda: flush_buf.zero_())
    del flush_buf
    gbps = lambda us: round(nbytes / (us * 1e-6) / 1e9, 1)
    out["fwd B1 H1 N256 d64 fp32-out"] = {
        "us": round(ms * 1e3, 2), "gbps": gbps(ms * 1e3),
        "device_us_warm_median": round(warm[0], 2), "device_us_warm_min": round(warm[1], 2),
        "device_us_cold_median": round(cold[0], 2), "device_us_cold_min": round(cold[1], 2),
        "gbps_warm": gbps(warm[0]), "gbps_cold": gbps(cold[0])}
    # Long context, causal window 4096 (exact visible-pair FLOPs).
    B, H, N, d = 1, 32, 16384, 128
    q, k, v = randn(B, H, N, d), randn(B, H, N, d), randn(B, H, N, d)
    o, lse = ea.attn_fwd(q, k, v, causal=True)
    f = credited_fwd_flops(B * H, N, d, True, 4096)
    ms = _time_ms(torch, lambda: ea.attn_fwd(q, k, v, causal=True, window=4096, out=o,
                                             lse=lse), reps)
    tf = f / (ms * 1e-3) / 1e12
    out["fwd B1 H32 N16384 d128 causal window=4096"] = {
        "ms": round(ms, 4), "tflops": round(tf, 1), "pct_peak": pct(tf)}
    del q, k, v, o, lse
    # The B4 H16 N2048 sweep, the N >= 4096, d = 128 points and the causal backward.
    shapes = [(4, 16, 2048, 64, False), (4, 16, 2048, 64, True), (4, 16, 2048, 128, False),
              (4, 16, 2048, 128, True), (4, 16, 4096, 128, True), (4, 16, 4096, 128, False),
              (2, 32, 8192, 128, False), (2, 32, 8192, 128, True)]
    for B, H, N, d, causal in shapes:
        q, k, v, do = (randn(B, H, N, d) for _ in range(4))
        o, lse = ea.attn_fwd(q, k, v, causal=causal)
        ws = torch.empty(ea.attn_bwd_workspace_bytes(B, H, N, d), device="cuda",
                         dtype=torch.uint8)
        grads = tuple(torch.empty(q.shape, device="cuda", dtype=torch.float32)
                      for _ in range(3))
        f = credited_fwd_flops(B * H, N, d, causal, 0)
        ms_f = _time_ms(torch, lambda: ea.attn_fwd(q, k, v, causal=causal, out=o, lse=lse),
                        reps)
        ms_b = _time_ms(torch, lambda: ea.attn_bwd(q, k, v, o, do, lse, causal=causal,
                                                   workspace=ws, grads=grads), reps)
        tf_f, tf_b = f / (ms_f * 1e-3) / 1e12, 2.5 * f / (ms_b * 1e-3) / 1e12
        out[f"B{B} H{H} N{N} d{d} {'causal' if causal else 'non-causal'}"] = {
            "fwd": {"ms": round(ms_f, 4), "tflops": round(tf_f, 1), "pct_peak": pct(tf_f)},
            "bwd": {"ms": round(ms_b, 4), "tflops": round(tf_b, 1), "pct_peak": pct(tf_b)}}
        del q, k, v, do, o, lse, ws, grads
    return out


def measure_fp8(ea, torch, reps=10):
    """The fp8 forward at B2 H32 N8192 d128, non-causal: N(0,1) inputs of
    torch's seeded device generator with one x10 outlier channel, quantised
    per tensor to e4m3 on the device.  Credited FLOPs 4*B*H*N^2*d; the kernel
    executes exactly those on the 16-bit matrix cores (e4m3 widened in LDS),
    so the fraction is of the bf16/fp16 peak; the fp8 peak's fraction is
    given beside it.  Measured after the timed step; it does not enter
    `value`."""
    gen = torch.Generator(device="cuda").manual_seed(80)
    B, H, N, d = 2, 32, 8192, 128
    codes, descales = [], []
    for _ in range(3):
        x = torch.randn((B, H, N, d), device="cuda", generator=gen)
        x[..., 17] *= 10.0
        ds = float(x.abs().max()) / 448.0
        codes.append((x / ds).to(torch.float8_e4m3fn).view(torch.uint8).contiguous())
        descales.append(ds)
        del x
    o = torch.empty((B, H, N, d), device="cuda", dtype=torch.bfloat16)
    lse = torch.empty((B, H, N), device="cuda", dtype=torch.float32)
    f = credited_fwd_flops(B * H, N, d, False, 0)
    ms = _time_ms(torch, lambda: ea.attn_fwd_fp8(*codes, *descales, out=o, lse=lse), reps)
    ms_bf16 = None
    qb, kb, vb = (torch.randn((B, H, N, d), device="cuda", generator=gen).bfloat16()
                  for _ in range(3))
    ob = torch.empty_like(qb)
    ms_bf16 = _time_ms(torch, lambda: ea.attn_fwd(qb, kb, vb, out=ob, lse=lse), reps)
    tf = f / (ms * 1e-3) / 1e12
    return {"workload": f"B{B} H{H} N{N} d{d} non-causal, e4m3 per-tensor, bf16 O",
            "kernel": ea.kernel_name(ea.STAGE_FWD_FP8, B, H, N, d),
            "ms": round(ms, 4), "tflops": round(tf, 1),
            "pct_16bit_mfma_peak": round(100.0 * tf / PEAK_BF16_TFLOPS, 1),
            "pct_fp8_peak": round(100.0 * tf / PEAK_FP8_TFLOPS, 1),
            "bf16_fwd_same_shape_ms": round(ms_bf16, 4),
            "speedup_vs_bf16": round(ms_bf16 / ms, 3)}


def measure_decode(ea, torch, attn_synth, reps=20):
    """Decode: one query per head at the end of a 32768-key sequence, B4 H32
    with 8 key/value heads, d128 (attn_fwd_decode: key-split pass + merge).
    HBM-bound: algorithmic bytes = K and V read once + Q read + O written.
    Measured after the timed step; it does not enter `value`."""
    import numpy as np
    B, H, Hkv, Nq, Nk, d = 4, 32, 8, 1, 32768, 128
    qb = attn_synth.bf16_attention_inputs(7, B, H, Nq, d)["q"]
    kv = attn_synth.bf16_attention_inputs(8, B, Hkv, Nk, d)

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(
            torch.bfloat16).cuda()
    q, k, v = dev(qb), dev(kv["k"]), dev(kv["v"])
    o, lse = ea.attn_fwd_decode(q, k, v)
    ws = torch.empty(ea.attn_decode_workspace_bytes(B, H, Hkv, Nq, Nk, d), device="cuda",
                     dtype=torch.uint8)
    fn = lambda: ea.attn_fwd_decode(q, k, v, out=o, lse=lse, workspace=ws)
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = 2 * B * Hkv * Nk * d * 2 + 2 * B * H * Nq * d * 2
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"workload": f"B{B} H{H} H_kv{Hkv} N_q{Nq} N_k{Nk} d{d}, bf16, non-causal",
            "us": round(ms * 1e3, 1), "algorithmic_bytes": nbytes,
            "gbps": round(gbps, 1), "frac_of_hbm": round(gbps / HBM_GBPS, 4)}


def cpu_model() -> str:
    """The host CPU from /proc/cpuinfo: model name, family and model numbers
    (a virtual machine may report only a generic name), the nominal clock
    implied by BogoMIPS (twice the TSC rate on x86) and whether a hypervisor
    is present; empty if unreadable."""
    info = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                k, v = (x.strip() for x in line.split(":", 1))
                info.setdefault(k, v)
    except OSError:
        return ""
    out = info.get("model name", "")
    if "cpu family" in info and "model" in info:
        out += f" (cpu family {info['cpu family']}, model {info['model']})"
    try:
        out += f", {float(info['bogomips']) / 2000:.2f} GHz nominal"
    except (KeyError, ValueError):
        pass
    if "hypervisor" in info.get("flags", "").split():
        out += ", virtual machine"
    return out


def cpu_baseline(attn_synth, seconds_budget=20.0):
    """The fp64 oracle, as it stands, on a bounded sample of the timed
    workload: forward + backward of whole heads (0, 0), (0, 1), ... of the
    causal and then the non-causal variant, until that variant's share of
    the budget is spent (at least one head each); credited FLOPs as for the
    GPU."""
    import oracle
    import numpy as np
    B, H, N, d = STEP_B, STEP_H, STEP_N, STEP_D
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count()
    s = 1.0 / math.sqrt(d)
    done_flops, t_total, parts = 0.0, 0.0, []
    for causal in (True, False):
        t_var, heads = 0.0, 0
        while heads == 0 or (t_var < seconds_budget / 2 and heads < B * H):
            b, h = divmod(heads, H)
            # Head (b, h) of the step's inputs: the generator's draws for one
            # head are the slice [b, h] of the full tensor, so draw the full
            # tensors' first heads only.
            bits = attn_synth.bf16_attention_inputs(STEP_SEEDS, 1, b * H + h + 1, N, d,
                                                    with_dout=True)
            ref = {k: oracle.decode_bf16(np.ascontiguousarray(v[0, -1])) for k, v in bits.items()}
            t0 = time.perf_counter()
            oracle.fwd(ref["q"], ref["k"], ref["v"], s, causal, 0, nthreads=threads)
            oracle.bwd(ref["q"], ref["k"], ref["v"], ref["do"], s, causal, 0, nthreads=threads)
            t_var += time.perf_counter() - t0
            heads += 1
            done_flops += 3.5 * credited_fwd_flops(1, N, d, causal, 0)
        t_total += t_var
        parts.append(f"{'causal' if causal else 'non-causal'}: {heads} of {B * H} heads")
    return {
        "value": done_flops / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"fp64 oracle forward + backward of whole heads of the B{B} H{H} N{N} "
                   f"d{d} step ({'; '.join(parts)}), {t_total:.1f} s of oracle time; "
                   f"credited FLOPs as for the GPU"),
    }


def workload_config(name: str) -> dict:
    w = WORKLOADS[name]
    shape = f"B{w['B']} H{w['H']} N{w['N']} d{w['d']}"
    masks = " and ".join("causal" if m else "non-causal" for m in w["masks"])
    what = ("fp8 (e4m3) forward (attn_fwd_fp8), " if name == "fp8" else
            "bf16 forward + backward (attn_fwd, attn_bwd_dq, attn_bwd_dkdv), ")
    return {"workload": f"{shape} {what}{masks}", "global_batch": w["B"], "heads": w["H"],
            "seq_len": w["N"], "head_dim": w["d"], "parallelism": "none (1 GPU)"}


def progress(msg: str):
    """A progress line on stderr (stdout carries only the result line)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the "
              "kernels are independent per (batch, head), so more GPUs would each "
              "run this same single-GPU workload.", file=sys.stderr)
        return 2
    import torch
    import attn_synth
    import exact_attention_79_amd as ea

    launches = build_step(ea, torch, attn_synth, args.workload)
    progress("inputs resident")
    for _ in range(args.warmup):
        run_step(launches, torch, record=False)
    torch.cuda.synchronize()

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    all_evs = []
    start.record()
    for _ in range(args.steps):
        all_evs.append(run_step(launches, torch, record=True))
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    for evs in all_evs:
        for i, L in enumerate(launches):
            L.times_ms.append(evs[i].elapsed_time(evs[i + 1]))

    ms_per_step = total_ms / args.steps
    credited = sum(L.credited for L in launches)
    value = credited / (ms_per_step * 1e-3) / 1e12

    breakdown = []
    for L in launches:
        t = sum(L.times_ms) / len(L.times_ms)
        row = {"launch": L.name, "kernel": L.kernel, "ms": round(t, 4)}
        if L.peak:
            tf = L.credited / (t * 1e-3) / 1e12
            row.update({"tflops": round(tf, 1), "pct_peak": round(100 * tf / L.peak, 1)})
            if L.executed != L.credited:
                row["executed_tflops"] = round(L.executed / (t * 1e-3) / 1e12, 1)
        else:
            row["gbps"] = round(L.bytes / (t * 1e-3) / 1e9, 1)
        breakdown.append(row)

    # The forward and the backward (both passes) of each mask, as fractions
    # of the bf16 peak: the targets are stated for them separately.
    phases = {}
    for L in launches:
        mask = L.name.split()[-1]
        ph = "fwd" if L.name.startswith("attn_fwd") else "bwd"
        row = phases.setdefault(f"{ph} {mask}", {"ms": 0.0, "credited": 0.0, "peak": L.peak})
        row["ms"] += sum(L.times_ms) / len(L.times_ms)
        row["credited"] += L.credited
    phases = {k: {"ms": round(v["ms"], 4),
                  "tflops": round(v["credited"] / (v["ms"] * 1e-3) / 1e12, 1),
                  "pct_peak": round(100 * v["credited"] / (v["ms"] * 1e-3) / 1e12
                                    / v["peak"], 1)}
              for k, v in phases.items()}

    # Dominant kernel: the kernel symbol with the most GPU time per step.
    per_kernel = {}
    for L in launches:
        k = per_kernel.setdefault(L.kernel, {"ms": 0.0, "n": 0, "credited": 0.0,
                                             "peak": L.peak})
        k["ms"] += sum(L.times_ms) / len(L.times_ms)
        k["n"] += 1
        k["credited"] += L.credited
    # (Only kernels priced against an MFMA peak are candidates.)
    dom_name, dom = max(((k, v) for k, v in per_kernel.items() if v["peak"]),
                        key=lambda kv: kv[1]["ms"])
    avg_ms = dom["ms"] / dom["n"]
    achieved = (dom["credited"] / dom["n"]) / (avg_ms * 1e-3) / 1e12
    roofline = {"kernel": dom_name, "bound": "mfma", "achieved": round(achieved, 1),
                "peak": dom["peak"], "unit": "TFLOP/s",
                "frac": round(achieved / dom["peak"], 4),
                "traffic": recorded_traffic(dom_name),
                "avg_launch_ms": round(avg_ms, 4)}

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if args.workload == "fp8" else "bf16",
        "data": "synthetic",
        "config": workload_config(args.workload),
        "roofline": roofline,
        "phases": phases,
        "breakdown": breakdown,
    }
    progress(f"timed step: {ms_per_step:.3f} ms, {value:.1f} TFLOP/s")
    if not args.no_extra_paths:
        wanted = set(args.paths.split(","))
        for key, fn in (("fp8", lambda: measure_fp8(ea, torch)),
                        ("gqa", lambda: measure_gqa(ea, torch, attn_synth)),
                        ("decode", lambda: measure_decode(ea, torch, attn_synth)),
                        ("dropout", lambda: measure_dropout(ea, torch, attn_synth)),
                        ("configs", lambda: measure_configs(ea, torch))):
            if key not in wanted:
                continue
            out[key] = fn()
            progress(f"measured {key}")
    if args.hbm_copy_mib > 0:
        # fp32 -> bf16, so that the copy runs as an elementwise kernel (a
        # same-dtype copy may go to a DMA engine that the counters miss).
        n = args.hbm_copy_mib << 18  # fp32 elements
        src = torch.ones(n, device="cuda", dtype=torch.float32)
        dst = torch.empty(n, device="cuda", dtype=torch.bfloat16)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        out["hbm_copy_bytes"] = {"read": 4 * n, "write": 2 * n}
        del src, dst
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(attn_synth)
        progress("timed the CPU oracle")
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
