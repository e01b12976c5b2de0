#!/usr/bin/env python3
"""Benchmark of one Ulysses attention-front-end step on one MI355X.

A step is the whole hot path over one batch of synthetic inputs already
resident in HBM:
  1. V scattered from the fused QKV projection on the library's comm stream,
  2. Q/K RMSNorm + RoPE fused into their scatter on the caller's stream,
  3. the grouped wait (the caller stream joins the comm stream),
  4. the attention output gathered back from head-sharded to sequence-sharded.

Workload: the video-DiT block with P=4 emulated ranks, B=1, S_local=4096
(S=16384), H=24, D=128, bf16.  The metric is algorithmic bytes per step (each
input element read once and each output element written once: 805,306,368 B)
over wall time, in GB/s, and as a fraction of the 8 TB/s HBM peak.

Prints one JSON line (rank 0).  --gpus N with N > 1 exits: this build runs on
one GPU.
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


def cpu_baseline(args, inputs):
    """The CPU oracle, as it stands, on one full step of the same workload."""
    import numpy as np

    from oracle import oracle
    from sequence_attention_ulysses_amd import synth

    qkv, w_q, w_k, o = (synth.bits(t) for t in inputs)
    w = synth.VIDEO_DIT
    cos, sin = oracle.rope_table_1d(w.S, w.D, theta=w.theta)
    t0 = time.perf_counter()
    yv = oracle.scatter(np.ascontiguousarray(qkv[:, :, :, 2]))
    yq = oracle.fused_norm_rope_scatter(np.ascontiguousarray(qkv[:, :, :, 0]), "bf16", w_q, w.eps, cos, sin)
    yk = oracle.fused_norm_rope_scatter(np.ascontiguousarray(qkv[:, :, :, 1]), "bf16", w_k, w.eps, cos, sin)
    z = oracle.gather(o)
    dt = time.perf_counter() - t0
    del yv, yq, yk, z
    return {"value": round(args.bytes_per_step / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "one full step of the workload (V scatter, fused Q/K norm+RoPE scatter, output gather; "
                      "%d algorithmic bytes) in %.2f s, single-threaded C oracle in double" %
                      (args.bytes_per_step, dt)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold", action="store_true",
                    help="also time each step after a 1 GiB scrub of the caches (event-timed, reported apart)")
    ap.add_argument("--no-profile", action="store_true", help="do not bracket launches with timing events")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build runs the emulated Ulysses group on one GPU; --gpus %d is not supported"
              % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    from sequence_attention_ulysses_amd import UlyssesContext, rope_table_1d, synth

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
        ctx.scatter_qkv(v=v_in)
        ctx.fused_qk_norm_rope_scatter(q_in, k_in, g_wq, g_wk, g_cos, g_sin, eps=w.eps)
        ctx.wait()
        ctx.gather_out(g_o)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if not args.no_profile:
        ctx.profile(True)
        ctx.profile_reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    value = args.bytes_per_step / (wall / args.steps) / 1e9

    kernels = {}
    roofline = None
    if not args.no_profile:
        per_launch_bytes = {"norm_rope": 2 * 2 * n_tensor, "scatter": 2 * n_tensor, "gather": 2 * n_tensor}
        for kind, nbytes in per_launch_bytes.items():
            ms, n = ctx.profile_read(kind)
            if n:
                avg_us = ms * 1e3 / n
                kernels[kind] = {"launches": n, "avg_us": round(avg_us, 2), "bytes_per_launch": nbytes,
                                 "GB_s": round(nbytes / (avg_us * 1e-6) / 1e9, 1)}
        ctx.profile(False)
        dom = kernels.get("norm_rope")
        if dom:
            achieved = dom["GB_s"]
            roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_from_profiles(w.name),
                        "kernel": "norm_rope_kernel<16,bf16> (fused Q/K RMSNorm+RoPE scatter)",
                        "algorithmic_bytes_per_launch": dom["bytes_per_launch"], "avg_us": dom["avg_us"]}

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
        "cpu_baseline": cpu,
    }
    if cold:
        rec["cold_cache"] = cold
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
