#!/usr/bin/env python3
"""Benchmark of one Ulysses attention-front-end step on one MI355X.

A step is the whole hot path over one batch of synthetic inputs already
resident in HBM:
  1. Q/K RMSNorm + RoPE fused into their scatter, with V scattered in the
     same launch (one grid moves all of Q, K and V to head-sharded targets),
  2. the grouped wait,
  3. the attention output gathered back from head-sharded to
     sequence-sharded.
The two-stream form of step 1 (V on the library's comm stream overlapping
the fused Q/K kernel on the caller's stream) is timed alongside and reported
under "two_stream".

Workload: the video-DiT block with P=4 emulated ranks, B=1, S_local=4096
(S=16384), H=24, D=128, bf16, V strided from the fused QKV projection.  The
metric is algorithmic bytes per step (each input element read once and each
output element written once: 805,306,368 B) over wall time, in GB/s, and as
a fraction of the 8 TB/s HBM peak.

Prints one JSON line.  --gpus N with N > 1 exits: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Ulysses QKV scatter+gather GB/s and % HBM peak, P=4 bf16, 1 MI355X"
HBM_PEAK_GBS = 8000.0
PROFILE_EVERY = 8
KERNEL_SOURCES = [os.path.join(ROOT, "sequence_attention_ulysses_amd", "csrc", f)
                  for f in ("uly_kernels.hip", "uly_internal.h", "fastdiv.h")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str):
    """HBM bytes per launch of the dominant kernel from committed counter runs,
    or None when the counters were taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(args, inputs, min_seconds: float = 10.0):
    """The CPU oracle, as it stands, on whole steps of the same workload,
    repeated until about `min_seconds` of CPU work."""
    import numpy as np

    from oracle import oracle
    from sequence_attention_ulysses_amd import synth

    qkv, w_q, w_k, o = (synth.bits(t) for t in inputs)
    w = synth.VIDEO_DIT
    cos, sin = oracle.rope_table_1d(w.S, w.D, theta=w.theta)
    q_src, k_src, v_src = (np.ascontiguousarray(qkv[:, :, :, c]) for c in range(3))
    steps, dt = 0, 0.0
    while dt < min_seconds:
        t0 = time.perf_counter()
        yv = oracle.scatter(v_src)
        yq = oracle.fused_norm_rope_scatter(q_src, "bf16", w_q, w.eps, cos, sin)
        yk = oracle.fused_norm_rope_scatter(k_src, "bf16", w_k, w.eps, cos, sin)
        z = oracle.gather(o)
        dt += time.perf_counter() - t0
        steps += 1
        del yv, yq, yk, z
    return {"value": round(steps * args.bytes_per_step / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": "%d full steps of the workload (V scatter, Q/K norm+RoPE scatter, output gather; "
                      "%d algorithmic bytes each) in %.1f s, single-threaded C oracle in double"
                      % (steps, args.bytes_per_step, dt)}


def calibrate_copy(args, torch, UlyssesContext):
    """A plain copy of a known size through the library's relayout kernel
    (one rank, so the map is the identity): the reference that scales the
    FETCH_SIZE / WRITE_SIZE counters of the step's kernels."""
    nbytes = args.calibrate_copy << 20
    rows = nbytes // (128 * 128 * 2)
    src = torch.ones((1, 1, rows, 128, 128), dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    with UlyssesContext(1, device=0) as ctx:
        for _ in range(args.warmup + args.steps):
            ctx.scatter_qkv(q=src, out=(dst, None, None))
            ctx.wait()
        torch.cuda.synchronize()
    print(json.dumps({"calibration": "relayout_kernel plain copy", "bytes_read_per_launch": nbytes,
                      "bytes_written_per_launch": nbytes, "launches": args.warmup + args.steps}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold", action="store_true",
                    help="also time each step after a 1 GiB scrub of the caches (event-timed, reported apart)")
    ap.add_argument("--no-profile", action="store_true", help="do not bracket launches with timing events")
    ap.add_argument("--no-two-stream", action="store_true",
                    help="skip the two-stream comparison (profiling runs then hold only the headline step)")
    ap.add_argument("--calibrate-copy", type=int, metavar="MIB", default=0,
                    help="instead of the step, run a plain device copy of MIB MiB (the library's relayout with "
                         "one rank) to calibrate HBM byte counters against a known size")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build runs the emulated Ulysses group on one GPU; --gpus %d is not supported"
              % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    from sequence_attention_ulysses_amd import UlyssesContext, rope_table_1d, synth

    if args.calibrate_copy:
        calibrate_copy(args, torch, UlyssesContext)
        return

    w = synth.VIDEO_DIT
    P, B, S_l, H, D = w.P, w.B, w.S_l, w.Hq, w.D
    dev = torch.device("cuda", 0)
    elem = 2
    n_tensor = P * B * S_l * H * D * elem
    args.bytes_per_step = 3 * 2 * n_tensor + 2 * n_tensor          # QKV scatter (r+w) + output gather (r+w)
    print("bench: %s on %s, %d warmup + %d timed steps" % (w.name, torch.cuda.get_device_name(0),
                                                         args.warmup, args.steps), file=sys.stderr, flush=True)

    qkv = synth.normal((P, B, S_l, 3, H, D), "bf16", 0)
    w_q = synth.norm_weight(D, "bf16", 1)
    w_k = synth.norm_weight(D, "bf16", 2)
    o = synth.normal((P, B, P * S_l, H // P, D), "bf16", 3)
    cos, sin = rope_table_1d(P * S_l, D, theta=w.theta)
    g_qkv, g_wq, g_wk, g_o = qkv.to(dev), w_q.to(dev), w_k.to(dev), o.to(dev)
    g_cos, g_sin = cos.to(dev), sin.to(dev)
    q_in, k_in, v_in = g_qkv[:, :, :, 0], g_qkv[:, :, :, 1], g_qkv[:, :, :, 2]

    ctx = UlyssesContext(P, device=0)

    def step():
        ctx.fused_qk_norm_rope_scatter(q_in, k_in, g_wq, g_wk, g_cos, g_sin, eps=w.eps, v=v_in)
        ctx.wait()
        ctx.gather_out(g_o)

    def step_two_stream():
        ctx.scatter_qkv(v=v_in, tags=(None, None, "v2"))
        ctx.fused_qk_norm_rope_scatter(q_in, k_in, g_wq, g_wk, g_cos, g_sin, eps=w.eps)
        ctx.wait()
        ctx.gather_out(g_o)

    def timed(fn, steps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    for _ in range(args.warmup):
        step()
        if not args.no_two_stream:
            step_two_stream()
    torch.cuda.synchronize()
    if not args.no_profile:
        # time only the dominant kernel, one launch in PROFILE_EVERY: every event pair adds
        # latency between kernels
        ctx.profile(True, kinds=["norm_rope"], every=PROFILE_EVERY)
        ctx.profile_reset()
    wall = timed(step, args.steps)
    ms_per_step = wall * 1e3 / args.steps
    value = args.bytes_per_step / (wall / args.steps) / 1e9

    kernels = {}
    roofline = None
    if not args.no_profile:
        per_launch_bytes = {"norm_rope": 6 * n_tensor}
        for kind, nbytes in per_launch_bytes.items():
            ms, n = ctx.profile_read(kind)
            if n:
                avg_us = ms * 1e3 / n
                kernels[kind] = {"timed_launches": n, "launches": args.steps, "avg_us": round(avg_us, 2),
                                 "bytes_per_launch": nbytes,
                                 "GB_s": round(nbytes / (avg_us * 1e-6) / 1e9, 1)}
        ctx.profile(False)
        ctx.profile_reset()
        dom = kernels.get("norm_rope")
        if dom:
            achieved = dom["GB_s"]
            roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_from_profiles(w.name),
                        "kernel": "norm_rope_kernel<16,bf16> (Q/K RMSNorm+RoPE scatter with V in the same grid)",
                        "algorithmic_bytes_per_launch": dom["bytes_per_launch"], "avg_us": dom["avg_us"]}

    # the two-stream form of the same step, timed the same way (no events)
    two_stream = None
    if not args.no_two_stream:
        wall2 = timed(step_two_stream, args.steps)
        two_stream = {"ms_per_step": round(wall2 * 1e3 / args.steps, 5),
                      "GB_s": round(args.bytes_per_step / (wall2 / args.steps) / 1e9, 2)}

    cold = None
    if args.cold:
        scrub = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        times = []
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(20):
            scrub.fill_(1)
            e0.record()
            step()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        times.sort()
        med = times[len(times) // 2]
        cold = {"median_ms": round(med, 4), "GB_s": round(args.bytes_per_step / (med * 1e-3) / 1e9, 1),
                "p10_ms": round(times[2], 4), "p90_ms": round(times[17], 4)}

    ctx.close()

    cpu = None
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle on one step", file=sys.stderr, flush=True)
        cpu = cpu_baseline(args, (qkv, w_q, w_k, o))

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic N(0,1) activations, N(1,0.1) norm weights, 1-D RoPE theta 1e4 (seeded)",
        "config": {"workload": w.name, "P": P, "B": B, "S_local": S_l, "S": P * S_l, "H": H, "D": D,
                   "v_source": "strided from fused QKV [B,S_local,3,H,D]", "parallelism": "ulysses-p4-emulated",
                   "bytes_per_step": args.bytes_per_step},
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "roofline": roofline,
        "kernels": kernels,
        "two_stream": two_stream,
        "cpu_baseline": cpu,
    }
    if cold:
        rec["cold_cache"] = cold
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
