#!/usr/bin/env python3
"""Benchmark of one Ulysses attention-front-end step on one MI355X.

A step is the whole hot path over one batch of synthetic inputs already
resident in HBM:
  1. Q/K RMSNorm + RoPE fused into their scatter, with V scattered in the
     same launch (one grid moves all of Q, K and V to head-sharded targets),
  2. the grouped wait,
  3. the attention output gathered back from head-sharded to
     sequence-sharded.

Workload: the video-DiT block with P=4 emulated ranks, B=1, S_local=4096
(S=16384), H=24, D=128, bf16, V strided from the fused QKV projection.  The
metric is algorithmic bytes per step (each input element read once and each
output element written once: 805,306,368 B) over the step's time, in GB/s,
and as a fraction of the 8 TB/s HBM peak.

Timing (flashinfer PR #6332 times with a cold L2, "Speedup", and gates its
records, "Export-protocol validation"):
  * the timed steps rotate over three independent sets of inputs and
    destinations (--sets), so nothing a step reads is still cached from the
    step before, and they run back to back with HIP events between them, so
    every byte a step writes is charged to the steps (a write-back still in
    flight when a step's last kernel ends delays the next step);
  * the headline is the median of exactly --steps such steps (p10 and p90
    beside it), after --warmup untimed steps and an untimed pre-heat (at
    least 0.2 s, until two passes of steps agree within 1 %) that lets the
    clocks settle under the load;
  * an A/A repeat of the same measurement that drifts by more than 2 %
    marks the record invalid, with the reason;
  * the dominant kernel is timed on at least 10 launches by the library's
    own events on the stream it runs on (the roofline figure);
  * reported beside it: the host's enqueue time per step, a warm wall-clock
    loop on one set, the step after a 1 GiB cache-evicting read with events
    around the step alone (that form lets dirty lines left in the caches be
    written back outside the events), the two-stream form of step 1 and
    copy controls.

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
AA_MAX_DRIFT = 0.02          # an A/A repeat further off than this voids the record
MIN_TIMED_LAUNCHES = 10      # launches of the dominant kernel timed whatever --steps is
PREHEAT_S = 0.2              # untimed steps run before the warmup: at least this long (s) ...
PREHEAT_MAX_S = 3.0          # ... and at most this long, until two passes agree within 1 %
# the kernels and the runtime that decides which kernel moves which operand
KERNEL_SOURCES = [os.path.join(ROOT, "sequence_attention_ulysses_amd", "csrc", f)
                  for f in ("uly_kernels.hip", "uly_internal.h", "fastdiv.h", "uly_runtime.cpp")]


def kernel_source_hash() -> str:
    """Hash of the kernel sources with comments and blank space removed, so that
    an edit of the comments alone keeps the committed counter runs valid."""
    import re
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
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


def host_cpu() -> str:
    """The host CPU's model name and the logical CPUs this process may use."""
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return "%s, %d logical CPUs available" % (model, n)


def cpu_baseline(args, inputs, min_seconds: float = 10.0):
    """The CPU oracle, as it stands, on whole steps of the same workload:
    first on every host core (one whole step per thread at a time; the oracle's
    C loops run outside the interpreter lock), then on one thread, each for
    about `min_seconds`."""
    import threading

    import numpy as np

    from oracle import oracle
    from sequence_attention_ulysses_amd import synth

    qkv, w_q, w_k, o = (synth.bits(t) for t in inputs)
    w = synth.VIDEO_DIT
    cos, sin = oracle.rope_table_1d(w.S, w.D, theta=w.theta)
    q_src, k_src, v_src = (np.ascontiguousarray(qkv[:, :, :, c]) for c in range(3))

    def one_step():
        yv = oracle.scatter(v_src)
        yq = oracle.fused_norm_rope_scatter(q_src, "bf16", w_q, w.eps, cos, sin)
        yk = oracle.fused_norm_rope_scatter(k_src, "bf16", w_k, w.eps, cos, sin)
        z = oracle.gather(o)
        del yv, yq, yk, z

    def run(threads):
        done = [0] * threads
        t0 = time.perf_counter()

        def worker(i):
            while time.perf_counter() - t0 < min_seconds:
                one_step()
                done[i] += 1

        pool = [threading.Thread(target=worker, args=(i,)) for i in range(threads)]
        for t in pool:
            t.start()
        for t in pool:
            t.join()
        return sum(done), time.perf_counter() - t0

    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    threads = max(1, min(cores, 16))
    steps_n, dt_n = run(threads)
    steps_1, dt_1 = run(1)
    return {"value": round(steps_n * args.bytes_per_step / dt_n / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": "%d full steps of the workload (V scatter, Q/K norm+RoPE scatter, output gather; "
                      "%d algorithmic bytes each) on %d threads in %.1f s, C oracle in double; host: %s"
                      % (steps_n, args.bytes_per_step, threads, dt_n, host_cpu()),
            "single_thread": {"value": round(steps_1 * args.bytes_per_step / dt_1 / 1e9, 4), "unit": "GB/s",
                              "sample": "%d full steps on 1 thread in %.1f s" % (steps_1, dt_1)}}


# ---------------------------------------------------------------------------
# Workloads.  Each setup builds `sets` independent sets of inputs and
# explicit destinations (different seeds, distinct buffers) and returns one
# step closure per set, so that consecutive timed steps touch disjoint memory
# and nothing a step reads is still in a cache from the step before (two
# other sets, >= 1.5 GiB, pass between two uses of a set: far more than the
# 256 MB Infinity Cache).  Also returned: the algorithmic bytes of a step
# (each input element read once, each output element written once, real
# tokens only), the dominant kernel (kind, bytes per launch, name) and the
# JSON config.
# ---------------------------------------------------------------------------
def _empty(torch, dev, shape, dtype):
    return torch.empty(tuple(shape), dtype=dtype, device=dev)


def setup_video_dit(torch, dev, synth, rope_table_1d, UlyssesContext, sets=3, dtype="bf16"):
    w = synth.VIDEO_DIT
    P, B, S_l, H, D = w.P, w.B, w.S_l, w.Hq, w.D
    n_tensor = P * B * S_l * H * D * 2
    tdt = synth.DTYPES[dtype]
    cos, sin = rope_table_1d(P * S_l, D, theta=w.theta)
    g_cos, g_sin = cos.to(dev), sin.to(dev)
    ctx = UlyssesContext(P, device=0)
    steps, two_stream, cpu_inputs = [], [], None
    for k in range(sets):
        if k == 0:       # set 0 is drawn on the host too: the CPU oracle times the same inputs
            qkv = synth.normal((P, B, S_l, 3, H, D), dtype, 0)
            w_q, w_k = synth.norm_weight(D, dtype, 1), synth.norm_weight(D, dtype, 2)
            o = synth.normal((P, B, P * S_l, H // P, D), dtype, 3)
            cpu_inputs = (qkv, w_q, w_k, o)
            g_qkv, g_wq, g_wk, g_o = qkv.to(dev), w_q.to(dev), w_k.to(dev), o.to(dev)
        else:
            g_qkv = synth.normal((P, B, S_l, 3, H, D), dtype, 10 * k, dev)
            g_wq, g_wk = synth.norm_weight(D, dtype, 10 * k + 1, dev), synth.norm_weight(D, dtype, 10 * k + 2, dev)
            g_o = synth.normal((P, B, P * S_l, H // P, D), dtype, 10 * k + 3, dev)
        yq, yk, yv = (_empty(torch, dev, (P, B, P * S_l, H // P, D), tdt) for _ in range(3))
        z = _empty(torch, dev, (P, B, S_l, H, D), tdt)

        def step(q=g_qkv[:, :, :, 0], k_=g_qkv[:, :, :, 1], v=g_qkv[:, :, :, 2], wq=g_wq, wk=g_wk, o=g_o,
                 outs=(yq, yk, yv), z=z):
            ctx.fused_qk_norm_rope_scatter(q, k_, wq, wk, g_cos, g_sin, eps=w.eps, v=v, out=outs)
            ctx.wait()
            ctx.gather_out(o, out=z)

        def step_two_stream(q=g_qkv[:, :, :, 0], k_=g_qkv[:, :, :, 1], v=g_qkv[:, :, :, 2], wq=g_wq, wk=g_wk,
                            o=g_o, outs=(yq, yk, yv), z=z):
            ctx.scatter_qkv(v=v, out=(None, None, outs[2]))
            ctx.fused_qk_norm_rope_scatter(q, k_, wq, wk, g_cos, g_sin, eps=w.eps, out=(outs[0], outs[1], None))
            ctx.wait()
            ctx.gather_out(o, out=z)

        steps.append(step)
        two_stream.append(step_two_stream)
    return {"workload": w, "ctx": ctx, "steps": steps, "two_stream": two_stream,
            "bytes_per_step": 3 * 2 * n_tensor + 2 * n_tensor,
            "dominant": ("norm_rope", 6 * n_tensor,
                         "norm_rope_kernel<16,bf16> (Q/K RMSNorm+RoPE scatter with V in the same grid)"),
            "cpu_inputs": cpu_inputs, "dtype": dtype,
            "data": "synthetic N(0,1) activations, N(1,0.1) norm weights, 1-D RoPE theta 1e4 (seeded)",
            "config": {"workload": w.name, "P": P, "B": B, "S_local": S_l, "S": P * S_l, "H": H, "D": D,
                       "v_source": "strided from fused QKV [B,S_local,3,H,D]", "parallelism": "ulysses-p4-emulated",
                       "bytes_per_step": 3 * 2 * n_tensor + 2 * n_tensor}}


def setup_wan_long(torch, dev, synth, rope_table_1d, UlyssesContext, sets=3):
    from sequence_attention_ulysses_amd import rope_table_3d
    w = synth.WAN_LONG
    P, B, S_l, H, D, S = w.P, w.B, w.S_l, w.Hq, w.D, w.S_real
    _, Hh, Ww = w.grid
    ctx = UlyssesContext(P, device=0)
    cos, sin = (t.to(dev) for t in rope_table_3d(P * S_l, D, Hh, Ww, real_rows=S, theta=w.theta))
    real = B * S * H * D * 2
    steps = []
    for k in range(sets):
        # global sequences, padded and sharded once (the pad/trim kernels are not in the step)
        shards = [ctx.seq_pad_shard(synth.normal((B, S, H, D), "bf16", 30 + 10 * k + i, dev), S_l) for i in range(3)]
        w_q, w_k = synth.norm_weight(D, "bf16", 34 + 10 * k, dev), synth.norm_weight(D, "bf16", 35 + 10 * k, dev)
        o = synth.normal((P, B, P * S_l, H // P, D), "bf16", 36 + 10 * k, dev)
        outs = tuple(_empty(torch, dev, (P, B, P * S_l, H // P, D), torch.bfloat16) for _ in range(3))
        z = _empty(torch, dev, (P, B, S_l, H, D), torch.bfloat16)

        def step(sh=shards, wq=w_q, wk=w_k, o=o, outs=outs, z=z):
            ctx.fused_qk_norm_rope_scatter(sh[0], sh[1], wq, wk, cos, sin, eps=w.eps, v=sh[2], out=outs)
            ctx.wait()
            ctx.gather_out(o, out=z)

        steps.append(step)
    return {"workload": w, "ctx": ctx, "steps": steps, "bytes_per_step": 3 * 2 * real + 2 * real,
            "dominant": ("norm_rope", 4 * real,
                         "norm_rope_band_kernel<bf16> (Q/K, 3-D RoPE, padded sequence; V by the relayout kernel)"),
            "dtype": "bf16", "data": "synthetic N(0,1) activations, N(1,0.1) norm weights, 3-D RoPE 44/42/42",
            "config": {"workload": w.name, "P": P, "B": B, "S": S, "S_padded": P * S_l, "H": H, "D": D,
                       "bytes_per_step": 3 * 2 * real + 2 * real, "bytes_count": "real tokens only"}}


def setup_gqa(torch, dev, synth, rope_table_1d, UlyssesContext, sets=3):
    w = synth.GQA
    P, B, S_l, Hq, Hkv, D = w.P, w.B, w.S_l, w.Hq, w.Hkv, w.D
    ctx = UlyssesContext(P, device=0)
    nq, nkv = P * B * S_l * Hq * D * 2, P * B * S_l * Hkv * D * 2
    steps = []
    for k in range(sets):
        q = synth.normal((P, B, S_l, Hq, D), "bf16", 40 + 10 * k, dev)
        k_ = synth.normal((P, B, S_l, Hkv, D), "bf16", 41 + 10 * k, dev)
        v = synth.normal((P, B, S_l, Hkv, D), "bf16", 42 + 10 * k, dev)
        o = synth.normal((P, B, P * S_l, Hq // P, D), "bf16", 43 + 10 * k, dev)
        outs = (_empty(torch, dev, (P, B, P * S_l, Hq // P, D), torch.bfloat16),
                _empty(torch, dev, (P, B, P * S_l, Hkv // P, D), torch.bfloat16),
                _empty(torch, dev, (P, B, P * S_l, Hkv // P, D), torch.bfloat16))
        z = _empty(torch, dev, (P, B, S_l, Hq, D), torch.bfloat16)

        def step(q=q, k_=k_, v=v, o=o, outs=outs, z=z):
            ctx.scatter_qkv(q, k_, v, out=outs)
            ctx.wait()
            ctx.gather_out(o, out=z)

        steps.append(step)
    return {"workload": w, "ctx": ctx, "steps": steps, "bytes_per_step": 2 * (nq + 2 * nkv) + 2 * nq,
            "dominant": ("scatter", 2 * (nq + 2 * nkv), "relayout_kernel (grouped Q/K/V scatter, one launch)"),
            "dtype": "bf16", "data": "synthetic N(0,1) activations",
            "config": {"workload": w.name, "P": P, "B": B, "S_local": S_l, "Hq": Hq, "Hkv": Hkv, "D": D,
                       "bytes_per_step": 2 * (nq + 2 * nkv) + 2 * nq}}


def setup_tiny(torch, dev, synth, rope_table_1d, UlyssesContext, sets=3):
    w = synth.TINY
    P, B, S_l, H, D = w.P, w.B, w.S_l, w.Hq, w.D
    ctx = UlyssesContext(P, device=0)
    n = P * B * S_l * H * D * 2
    steps = []
    for k in range(sets):
        q, k_, v = (synth.normal((P, B, S_l, H, D), "f16", 50 + 10 * k + i, dev) for i in range(3))
        o = synth.normal((P, B, P * S_l, H // P, D), "f16", 53 + 10 * k, dev)
        outs = tuple(_empty(torch, dev, (P, B, P * S_l, H // P, D), torch.float16) for _ in range(3))
        z = _empty(torch, dev, (P, B, S_l, H, D), torch.float16)

        def step(q=q, k_=k_, v=v, o=o, outs=outs, z=z):
            ctx.scatter_qkv(q, k_, v, out=outs)
            ctx.wait()
            ctx.gather_out(o, out=z)

        steps.append(step)
    return {"workload": w, "ctx": ctx, "steps": steps, "bytes_per_step": 3 * 2 * n + 2 * n,
            "dominant": ("scatter", 6 * n, "relayout_kernel (grouped Q/K/V scatter, one launch)"),
            "dtype": "f16", "data": "synthetic N(0,1) activations",
            "config": {"workload": w.name, "P": P, "B": B, "S_local": S_l, "H": H, "D": D,
                       "bytes_per_step": 3 * 2 * n + 2 * n, "note": "launch-bound"}}


def setup_spatial(torch, dev, synth, rope_table_1d, UlyssesContext, sets=3):
    from sequence_attention_ulysses_amd import height_split
    w = synth.SPATIAL
    ctx = UlyssesContext(w.P, device=0)
    lead, (Hh, W) = w.shape[:-2], w.shape[-2:]
    N = 1
    for x in lead:
        N *= x
    h, hmax = height_split(Hh, w.P)
    halo_rows = sum(min(w.halo, sum(h[:r])) + min(w.halo, Hh - sum(h[:r + 1])) for r in range(w.P))
    row = W * 2
    # split: read every source row once per use (core rows once, halo rows again), write the shards;
    # gather: read core rows, write the stacked buffer; trim/concat: read core rows, write the full tensor
    split = N * row * (Hh + halo_rows) + N * row * w.P * (hmax + 2 * w.halo)
    gather = N * row * Hh + N * row * w.P * hmax
    trim = N * row * Hh * 2
    steps = []
    for k in range(sets):
        full = synth.normal(w.shape, w.dtype, 60 + k, dev)
        bufs = [_empty(torch, dev, (w.P,) + lead + (hmax + 2 * w.halo, W), full.dtype),
                _empty(torch, dev, (w.P,) + lead + (hmax, W), full.dtype),
                _empty(torch, dev, w.shape, full.dtype)]

        def step(full=full, bufs=bufs):
            sh = ctx.spatial_split_halo(full, halo=w.halo, out=bufs[0])
            st = ctx.spatial_gather_stacked(sh, Hh, halo=w.halo, out=bufs[1])
            ctx.spatial_trim_concat(st, Hh, out=bufs[2])

        steps.append(step)
    return {"workload": w, "ctx": ctx, "steps": steps, "bytes_per_step": split + gather + trim,
            "dominant": ("spatial", (split + gather + trim) // 3, "rowmap_kernel (average of the three launches)"),
            "dtype": "bf16", "data": "synthetic N(0,1) latent",
            "config": {"workload": w.name, "P": w.P, "shape": list(w.shape), "heights": h, "halo": w.halo,
                       "bytes_per_step": split + gather + trim, "note": "cache-resident"}}


MFMA_BF16_PEAK_TFLOPS = 2500.0


def _setup_proj(torch, dev, synth, rope_table_1d, UlyssesContext, w, seed, name, sets=3):
    """The attention front end with the QKV projection fused in: one launch
    projects x, normalises and rotates q/k and stores every head band into
    its head-sharded target (flashinfer PR #6332's fused call), then the wait
    and the output gather.  Timed beside it: the per-operator path, a library
    GEMM (torch, hipBLASLt) writing qkv, then the fused norm/RoPE scatter."""
    import torch.nn.functional as F
    P, B, S_l, Hq, Hkv, D = w.P, w.B, w.S_l, w.Hq, w.Hkv, w.D
    hidden, N = Hq * D, (Hq + 2 * Hkv) * D
    M = P * B * S_l
    w_qkv = synth.normal((N, hidden), "bf16", seed + 1, dev, std=hidden ** -0.5)
    w_q, w_k = synth.norm_weight(D, "bf16", seed + 2, dev), synth.norm_weight(D, "bf16", seed + 3, dev)
    cos, sin = (t.to(dev) for t in rope_table_1d(P * S_l, D, theta=w.theta))
    ctx = UlyssesContext(P, device=0)
    flops = 2 * M * N * hidden
    bf = torch.bfloat16
    steps, per_op, x0 = [], [], None
    for k in range(sets):
        x = synth.normal((P, B, S_l, hidden), "bf16", seed + 10 * k, dev)
        x0 = x if k == 0 else x0
        o = synth.normal((P, B, P * S_l, Hq // P, D), "bf16", seed + 10 * k + 4, dev)
        outs = (_empty(torch, dev, (P, B, P * S_l, Hq // P, D), bf),
                _empty(torch, dev, (P, B, P * S_l, Hkv // P, D), bf),
                _empty(torch, dev, (P, B, P * S_l, Hkv // P, D), bf))
        z = _empty(torch, dev, (P, B, S_l, Hq, D), bf)
        y = _empty(torch, dev, (M, N), bf)
        y4 = y.view(P, B, S_l, N)
        yq = y4[..., :Hq * D].unflatten(-1, (Hq, D))
        yk = y4[..., Hq * D:(Hq + Hkv) * D].unflatten(-1, (Hkv, D))
        yv = y4[..., (Hq + Hkv) * D:].unflatten(-1, (Hkv, D))

        def step(x=x, o=o, outs=outs, z=z):
            ctx.fused_qkv_proj_norm_rope_scatter(x, w_qkv, Hq, Hkv, w_q, w_k, cos, sin, eps=w.eps, out=outs)
            ctx.wait()
            ctx.gather_out(o, out=z)

        def step_per_operator(x2=x.view(M, hidden), y=y, yq=yq, yk=yk, yv=yv, o=o, outs=outs, z=z):
            F.linear(x2, w_qkv, out=y)
            ctx.fused_qk_norm_rope_scatter(yq, yk, w_q, w_k, cos, sin, eps=w.eps, v=yv, out=outs)
            ctx.wait()
            ctx.gather_out(o, out=z)

        steps.append(step)
        per_op.append(step_per_operator)
    return {"workload": w, "name": name, "ctx": ctx, "steps": steps, "per_operator": per_op,
            "bytes_per_step": flops, "unit": "TFLOP/s", "unit_div": 1e12,
            "metric": "QKV projection + QK-norm + RoPE + Ulysses scatter + output gather, projection TFLOP/s "
                      "over the step, P=%d bf16, 1 MI355X" % P,
            "dominant": ("proj", flops, "proj_kernel<bf16> (MFMA QKV projection with norm/RoPE/band-store "
                         "epilogue)", "mfma", MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"),
            "cpu_proj": (x0, w_qkv, w_q, w_k, Hq, Hkv, w.eps, w.theta),
            "dtype": "bf16", "data": "synthetic N(0,1) activations, N(0,1/hidden) QKV weight, N(1,0.1) norm "
                                     "weights, 1-D RoPE theta 1e4 (seeded)",
            "config": {"workload": name, "P": P, "B": B, "S_local": S_l, "S": P * S_l, "Hq": Hq, "Hkv": Hkv,
                       "D": D, "hidden": hidden, "M": M, "N": N, "flops_per_step": flops,
                       "parallelism": "ulysses-p%d-emulated" % P}}


def setup_video_dit_proj(torch, dev, synth, rope_table_1d, UlyssesContext, sets=3):
    return _setup_proj(torch, dev, synth, rope_table_1d, UlyssesContext, synth.VIDEO_DIT, 70,
                       "video_dit_proj_p4_s16384_h24_hidden3072_bf16", sets)


def setup_gqa_proj(torch, dev, synth, rope_table_1d, UlyssesContext, sets=3):
    return _setup_proj(torch, dev, synth, rope_table_1d, UlyssesContext, synth.GQA, 80,
                       "gqa_proj_p8_b2_s65536_hq32_hkv8_hidden4096_bf16", sets)


def cpu_baseline_proj(args, proj_inputs, min_seconds: float = 10.0):
    """The CPU oracle on a bounded sample of the projection workload: the
    projection, QK-norm and RoPE of 16 token rows at a time, repeated for
    about `min_seconds`; the rate counts the projection's flops."""
    import numpy as np

    from oracle import oracle
    from sequence_attention_ulysses_amd import synth

    x, w_qkv, w_q, w_k, Hq, Hkv, eps, theta = proj_inputs
    P, B, S_l, hidden = x.shape
    D = w_q.numel()
    xb, wb = synth.bits(x.cpu()).reshape(-1, hidden), synth.bits(w_qkv.cpu())
    wqb, wkb = synth.bits(w_q.cpu()), synth.bits(w_k.cpu())
    cos, sin = oracle.rope_table_1d(P * S_l, D, theta=theta)
    rng = np.random.default_rng(0)
    n, reps, dt = 16, 0, 0.0
    while dt < min_seconds:
        rows = rng.integers(0, xb.shape[0], size=n)
        pos = (rows // (B * S_l)) * S_l + rows % S_l
        t0 = time.perf_counter()
        oracle.qkv_proj_norm_rope_rows(xb[rows], "bf16", wb, Hq, Hkv, D, wqb, wkb, eps, cos, sin, pos)
        dt += time.perf_counter() - t0
        reps += 1
    flops = 2.0 * reps * n * wb.shape[0] * hidden
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": "%d batches of %d random token rows through the projection, QK-norm and RoPE "
                      "(%d x %d weight) in %.1f s, single-threaded C oracle in double; host: %s"
                      % (reps, n, wb.shape[0], hidden, dt, host_cpu())}


WORKLOADS = {"video_dit": setup_video_dit, "wan_long": setup_wan_long, "gqa": setup_gqa, "tiny": setup_tiny,
             "spatial": setup_spatial, "video_dit_proj": setup_video_dit_proj, "gqa_proj": setup_gqa_proj}


def pick(sorted_vals, q):
    """The q-quantile of an ascending list (nearest rank)."""
    return sorted_vals[min(len(sorted_vals) - 1, int(q * len(sorted_vals)))]


class FenceFreeEvents:
    """HIP timing events created with hipEventDisableSystemFence, recorded on the
    current stream.  A default event's system-scope release writes the L2 back
    each time it is recorded; between back-to-back steps that would add work a
    real pipeline does not have.  HIP is reached through the runtime torch has
    already loaded (measurement plumbing only)."""
    FLAGS = 0x20000000       # hipEventDisableSystemFence

    def __init__(self, torch, n):
        import ctypes
        self.torch = torch
        self.hip = ctypes.CDLL("libamdhip64.so.7", mode=ctypes.RTLD_GLOBAL)
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.FLAGS) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.ev.append(e)
        self._c = ctypes

    def record(self, i):
        st = self.torch.cuda.current_stream().cuda_stream
        if self.hip.hipEventRecord(self.ev[i], self._c.c_void_p(st)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed(self, i, j):
        ms = self._c.c_float()
        if self.hip.hipEventElapsedTime(self._c.byref(ms), self.ev[i], self.ev[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []


def back_to_back(torch, fns, n):
    """Run n steps back to back, step i on input/output set i % len(fns), with
    a fence-free HIP event on the current stream before every step and after the last:
    step i's time is the interval between its event and the next one, so the
    work a step leaves behind (a write-back still under way, say) is charged
    to the steps, and the host enqueues ahead of the GPU without waiting.
    Returns the sorted per-step times (ms), the sorted host enqueue times per
    step (s) and the events' total over the n steps (ms)."""
    ev = FenceFreeEvents(torch, n + 1)
    host = []
    torch.cuda.synchronize()
    for i in range(n):
        ev.record(i)
        h0 = time.perf_counter()
        fns[i % len(fns)]()
        host.append(time.perf_counter() - h0)
    ev.record(n)
    torch.cuda.synchronize()
    times = sorted(ev.elapsed(i, i + 1) for i in range(n))
    total = ev.elapsed(0, n)
    ev.close()
    return times, sorted(host), total


def cold_steps(torch, fn, n, scrub):
    """Run `fn` n times, each after a read of the 1 GiB `scrub` buffer (which
    evicts the L2s and the Infinity Cache), with HIP events around the step
    alone.  Unlike `back_to_back`, whatever a step leaves in the caches to be
    written back is written back during the next scrub, outside the events."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for e0, e1 in ev:
        scrub.max()
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return sorted(e0.elapsed_time(e1) for e0, e1 in ev)


def spread(times_ms, work, unit_div, unit):
    """Median, p10 and p90 of per-step times, and the rate at the median."""
    med = pick(times_ms, 0.5)
    return {"samples": len(times_ms), "median_us": round(med * 1e3, 2),
            "p10_us": round(pick(times_ms, 0.1) * 1e3, 2), "p90_us": round(pick(times_ms, 0.9) * 1e3, 2),
            unit.replace("/", "_") + "_at_median": round(work / (med * 1e-3) / unit_div, 2)}


def measure_protocol(args, torch, dev, setup, headline_gbs):
    """Controls beside the headline, timed the same way (back to back over
    rotating buffer sets): a device copy of the step's bytes by torch, the same
    bytes through the library's own relayout kernel as an identity copy (this
    box's copy roof), and the same step in fp16 (a relayout moves bytes, so the
    rate must not depend on the 16-bit type)."""
    from sequence_attention_ulysses_amd import UlyssesContext, rope_table_1d, synth

    nbytes = setup["bytes_per_step"]
    n = max(MIN_TIMED_LAUNCHES, args.steps)
    R = len(setup["steps"])

    pairs = [(torch.empty(nbytes // 2, dtype=torch.uint8, device=dev).fill_(1),
              torch.empty(nbytes // 2, dtype=torch.uint8, device=dev)) for _ in range(R)]
    t, _, _ = back_to_back(torch, [lambda s=s, d=d: d.copy_(s) for s, d in pairs], n)
    copy = {"bytes_copied": nbytes // 2, "median_us": round(pick(t, 0.5) * 1e3, 2),
            "GB_s": round(nbytes / (pick(t, 0.5) * 1e-3) / 1e9, 1)}
    del pairs

    # the same bytes through the library's relayout kernel as a plain copy (one
    # rank: the identity map) on the caller's stream
    rows = (nbytes // 2) // (128 * 128 * 2)
    pairs = [(torch.ones((1, 1, rows, 128, 128), dtype=torch.bfloat16, device=dev),
              torch.empty((1, 1, rows, 128, 128), dtype=torch.bfloat16, device=dev)) for _ in range(R)]
    with UlyssesContext(1, device=0) as cctx:
        cctx.set_route("caller")
        fns = [lambda s=s, d=d: cctx.scatter_qkv(q=s, out=(d, None, None)) for s, d in pairs]
        for i in range(max(args.warmup, R)):
            fns[i % R]()
        t, _, _ = back_to_back(torch, fns, n)
    cbytes = 2 * pairs[0][0].numel() * 2
    copy_roof = {"kernel": "relayout_kernel, one rank (identity map)", "bytes_moved": cbytes,
                 "median_us": round(pick(t, 0.5) * 1e3, 2),
                 "GB_s": round(cbytes / (pick(t, 0.5) * 1e-3) / 1e9, 1)}
    copy_roof["step_over_copy_roof"] = round(headline_gbs / copy_roof["GB_s"], 4)
    del pairs

    f16 = setup_video_dit(torch, dev, synth, rope_table_1d, UlyssesContext, sets=R, dtype="f16")
    for i in range(max(args.warmup, R)):
        f16["steps"][i % R]()
    t, _, _ = back_to_back(torch, f16["steps"], n)
    f16["ctx"].close()
    del f16
    fp16 = spread(t, nbytes, 1e9, "GB/s")
    return {"device_copy_control": copy, "copy_roof": copy_roof, "fp16_same_shape": fp16}


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
    ap.add_argument("--workload", default="video_dit", choices=sorted(WORKLOADS),
                    help="video_dit (the headline, default) or another workload recorded for reference")
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sets", type=int, default=3,
                    help="independent input/output buffer sets the timed steps rotate over (1: every step reuses "
                         "the same buffers, so data stays in the caches between steps)")
    ap.add_argument("--no-profile", action="store_true", help="do not bracket launches with timing events")
    ap.add_argument("--headline-only", action="store_true",
                    help="run the warmup and the headline steps only (for counter collection); the record is "
                         "marked invalid")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step per buffer set into a HIP graph and time their replays (no per-launch "
                         "host work; implies --no-profile)")
    ap.add_argument("--two-stream", action="store_true",
                    help="also time the two-stream form of step 1 (V scattered on the library's comm stream beside "
                         "the fused Q/K launch); off by default so that every fused launch of the run is the same "
                         "launch and a kernel trace of the run averages that launch alone")
    ap.add_argument("--route", choices=("kernel", "copy_engine", "caller"), default=None,
                    help="how the plain Q/K/V scatter moves its operands (the library default: kernel on the "
                         "comm stream); the workloads that use it are gqa and tiny")
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

    dev = torch.device("cuda", 0)
    setup = WORKLOADS[args.workload](torch, dev, synth, rope_table_1d, UlyssesContext, sets=args.sets)
    w = setup["workload"]
    ctx = setup["ctx"]
    if args.route:
        ctx.set_route(args.route)
        setup["config"]["scatter_route"] = args.route
    steps, steps_two_stream = setup["steps"], setup.get("two_stream")
    steps_per_operator = setup.get("per_operator")
    R = len(steps)
    args.bytes_per_step = setup["bytes_per_step"]        # the step's work: bytes, or flops for TFLOP/s
    unit, unit_div = setup.get("unit", "GB/s"), setup.get("unit_div", 1e9)
    name = setup.get("name", w.name)
    args.no_two_stream = steps_two_stream is None or not args.two_stream
    print("bench: %s on %s, %d warmup + %d timed steps over %d buffer sets" % (
        name, torch.cuda.get_device_name(0), args.warmup, args.steps, R), file=sys.stderr, flush=True)

    def timed(fn, n):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    if args.graph:
        args.no_profile = args.no_two_stream = True
        steps_per_operator = None
    # Pre-heat: untimed passes of back-to-back steps before the warmup until the
    # clocks have settled under this load: at least PREHEAT_S of wall time and
    # two consecutive passes within 1 % of each other, at most PREHEAT_MAX_S
    # (the MFMA-bound projection runs its first ~15 ms of back-to-back steps
    # up to 9 % slower than the rest).
    t0, n_pre, prev, settled = time.perf_counter(), 0, None, False
    per_pass = max(R, 10)
    while time.perf_counter() - t0 < PREHEAT_MAX_S:
        _, _, tot = back_to_back(torch, steps, per_pass)
        n_pre += per_pass
        settled = prev is not None and abs(tot / prev - 1.0) < 0.01
        prev = tot
        if settled and time.perf_counter() - t0 >= PREHEAT_S:
            break
    preheat = {"steps": n_pre, "s": round(time.perf_counter() - t0, 3), "settled": settled}
    # (the forms timed beside the headline get their own warmup right before
    # their measurement: interleaving another path's kernels here, a library
    # GEMM say, leaves the next ~20 fused projection steps up to 20 % slower)
    for i in range(max(args.warmup, R)):
        steps[i % R]()
    torch.cuda.synchronize()
    if args.graph:
        # the library's calls are capturable: a step with explicit destinations
        # allocates nothing, and the warmup filled the context's event pools
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        graphs = []
        for fn in steps:
            with torch.cuda.stream(cap):
                fn()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                fn()
            torch.cuda.synchronize()
            graphs.append(g)
        steps = [g.replay for g in graphs]
        for i in range(max(args.warmup, R)):
            steps[i % R]()
        torch.cuda.synchronize()
        setup["config"]["launch"] = "hip_graph"
    dom_kind, dom_bytes, dom_name = setup["dominant"][:3]
    dom_bound, dom_peak, dom_unit = (setup["dominant"][3:] if len(setup["dominant"]) > 3
                                     else ("hbm", HBM_PEAK_GBS, "GB/s"))
    work = args.bytes_per_step
    ukey = unit.replace("/", "_")

    # the headline: exactly --steps steps back to back over the rotating sets
    t_a, host_a, total_a = back_to_back(torch, steps, args.steps)
    med = pick(t_a, 0.5)
    ms_per_step = med
    value = work / (med * 1e-3) / unit_div
    headline = spread(t_a, work, unit_div, unit)
    headline["mean_us"] = round(total_a * 1e3 / args.steps, 2)
    host_us = pick(host_a, 0.5) * 1e6
    host = {"median_us": round(host_us, 2), "p90_us": round(pick(host_a, 0.9) * 1e6, 2),
            "frac_of_step": round(host_us / (med * 1e3), 3)}

    invalid = []
    if args.headline_only:
        # counter runs: the warmup and the headline steps alone
        args.no_profile = args.no_two_stream = True
        steps_per_operator = None
        invalid.append("headline steps only (a counter-collection run)")
        aa = None
    else:
        # A/A control: the same measurement again; a drift over 2 % voids the record
        t_b, _, _ = back_to_back(torch, steps, args.steps)
        drift = pick(t_b, 0.5) / med - 1.0
        aa = dict(spread(t_b, work, unit_div, unit), drift=round(drift, 4))
        if abs(drift) > AA_MAX_DRIFT:
            invalid.append("A/A repeat drifted %+.1f %% (limit %.0f %%)" % (100 * drift, 100 * AA_MAX_DRIFT))

    # every kernel of at least 10 steps bracketed by the library's own events on
    # the stream it runs on: the dominant kernel's average is the roofline figure
    kernels = {}
    roofline = None
    if not args.no_profile:
        n_dom = max(MIN_TIMED_LAUNCHES, args.steps)
        ctx.profile(True, every=1)
        ctx.profile_reset()
        back_to_back(torch, steps, n_dom)
        from sequence_attention_ulysses_amd._lib import KERNEL_KINDS
        for kind in KERNEL_KINDS:
            ms, n = ctx.profile_read(kind)
            if n:
                kernels[kind] = {"timed_launches": n, "avg_us": round(ms * 1e3 / n, 2)}
        ctx.profile(False)
        ctx.profile_reset()
        dom = kernels.get(dom_kind)
        if dom is None or dom["timed_launches"] < MIN_TIMED_LAUNCHES:
            invalid.append("fewer than %d timed launches of the dominant kernel" % MIN_TIMED_LAUNCHES)
        if dom:
            div = 1e9 if dom_unit == "GB/s" else 1e12
            achieved = round(dom_bytes / (dom["avg_us"] * 1e-6) / div, 1)
            dom.update(work_per_launch=dom_bytes, **{dom_unit.replace("/", "_"): achieved})
            roofline = {"bound": dom_bound, "achieved": achieved, "peak": dom_peak, "unit": dom_unit,
                        "frac": round(achieved / dom_peak, 4),
                        "traffic": traffic_from_profiles(name) if dom_bound == "hbm" else None,
                        "kernel": dom_name, "avg_us": dom["avg_us"], "timed_launches": dom["timed_launches"],
                        ("algorithmic_bytes_per_launch" if dom_bound == "hbm" else "flops_per_launch"): dom_bytes}

    # cross-checks: a wall-clock loop on one set (its data stays warm in the
    # caches between steps), and each step after a 1 GiB cache-evicting read
    warm = scrub_cold = None
    if not args.headline_only:
        wall_w = timed(steps[0], args.steps)
        warm = {"ms_per_step": round(wall_w * 1e3 / args.steps, 5),
                ukey: round(work / (wall_w / args.steps) / unit_div, 2)}
        scrub = torch.ones(1 << 27, dtype=torch.int64, device=dev)
        scrub_cold = spread(cold_steps(torch, steps[0], max(MIN_TIMED_LAUNCHES, args.steps), scrub), work,
                            unit_div, unit)
        del scrub

    # the two-stream form of the same step, timed like the headline
    two_stream = None
    if not args.no_two_stream:
        for i in range(max(args.warmup, R)):
            steps_two_stream[i % R]()
        t2, _, _ = back_to_back(torch, steps_two_stream, args.steps)
        two_stream = spread(t2, work, unit_div, unit)

    per_operator = None
    if steps_per_operator is not None:
        back_to_back(torch, steps_per_operator, max(args.steps, 2 * R))      # its warmup (~20 steps settle)
        t3, _, _ = back_to_back(torch, steps_per_operator, args.steps)
        per_operator = dict(spread(t3, work, unit_div, unit),
                            path="torch linear (hipBLASLt) writing qkv, then fused_qk_norm_rope_scatter, wait, gather",
                            fused_speedup=round(pick(t3, 0.5) / med, 4))

    ctx.close()
    del steps, steps_two_stream, steps_per_operator
    setup.pop("steps", None), setup.pop("two_stream", None), setup.pop("per_operator", None)
    extra = (measure_protocol(args, torch, dev, dict(setup, steps=[None] * R), work / (med * 1e-3) / 1e9)
             if args.workload == "video_dit" and not (args.graph or args.headline_only) else None)

    cpu = None
    if not args.no_cpu_baseline and "cpu_inputs" in setup:
        print("bench: timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(args, setup["cpu_inputs"])
    elif not args.no_cpu_baseline and "cpu_proj" in setup:
        print("bench: timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline_proj(args, setup["cpu_proj"])

    rec = {
        "metric": (METRIC if args.workload == "video_dit"
                   else setup.get("metric", "Ulysses exchange GB/s, workload %s" % name)),
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": setup["dtype"],
        "data": setup["data"],
        "config": setup["config"],
        "roofline": roofline,
        "cpu_baseline": cpu,
        "valid": not invalid,
        "preheat": preheat,
        "timing": "median of %d steps run back to back over %d rotating input/output sets (no data a step "
                  "reads is cached from the step before), HIP events between the steps" % (args.steps, R),
        "step_spread": headline,
        "aa_repeat": aa,
        "host_enqueue": host,
        "kernels": kernels,
        "warm_loop": warm,
        "scrub_cold": scrub_cold,
        "two_stream": two_stream,
    }
    if invalid:
        rec["invalid_reason"] = "; ".join(invalid)
    if unit == "GB/s":
        rec["hbm_frac"] = round(value / HBM_PEAK_GBS, 4)
    if per_operator:
        rec["per_operator"] = per_operator
    if extra:
        rec.update(extra)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
