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
PROFILE_EVERY = 16
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
# Workloads.  Each setup returns the context, the step (and its two-stream
# form where there is one), the algorithmic bytes of a step (each input
# element read once, each output element written once, real tokens only),
# the dominant kernel (kind, bytes per launch, name) and the JSON config.
# ---------------------------------------------------------------------------
def setup_video_dit(torch, dev, synth, rope_table_1d, UlyssesContext, dtype="bf16"):
    w = synth.VIDEO_DIT
    P, B, S_l, H, D = w.P, w.B, w.S_l, w.Hq, w.D
    n_tensor = P * B * S_l * H * D * 2
    qkv = synth.normal((P, B, S_l, 3, H, D), dtype, 0)
    w_q, w_k = synth.norm_weight(D, dtype, 1), synth.norm_weight(D, dtype, 2)
    o = synth.normal((P, B, P * S_l, H // P, D), dtype, 3)
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

    return {"workload": w, "ctx": ctx, "step": step, "step_two_stream": step_two_stream,
            "bytes_per_step": 3 * 2 * n_tensor + 2 * n_tensor,
            "dominant": ("norm_rope", 6 * n_tensor,
                         "norm_rope_kernel<16,bf16> (Q/K RMSNorm+RoPE scatter with V in the same grid)"),
            "cpu_inputs": (qkv, w_q, w_k, o), "dtype": dtype,
            "data": "synthetic N(0,1) activations, N(1,0.1) norm weights, 1-D RoPE theta 1e4 (seeded)",
            "config": {"workload": w.name, "P": P, "B": B, "S_local": S_l, "S": P * S_l, "H": H, "D": D,
                       "v_source": "strided from fused QKV [B,S_local,3,H,D]", "parallelism": "ulysses-p4-emulated",
                       "bytes_per_step": 3 * 2 * n_tensor + 2 * n_tensor}}


def setup_wan_long(torch, dev, synth, rope_table_1d, UlyssesContext):
    from sequence_attention_ulysses_amd import rope_table_3d
    w = synth.WAN_LONG
    P, B, S_l, H, D, S = w.P, w.B, w.S_l, w.Hq, w.D, w.S_real
    _, Hh, Ww = w.grid
    ctx = UlyssesContext(P, device=0)
    # global sequences, padded and sharded once (the pad/trim kernels are not in the step)
    shards = [ctx.seq_pad_shard(synth.normal((B, S, H, D), "bf16", 30 + i, dev), S_l) for i in range(3)]
    w_q, w_k = synth.norm_weight(D, "bf16", 31, dev), synth.norm_weight(D, "bf16", 32, dev)
    cos, sin = (t.to(dev) for t in rope_table_3d(P * S_l, D, Hh, Ww, real_rows=S, theta=w.theta))
    o = synth.normal((P, B, P * S_l, H // P, D), "bf16", 33, dev)
    real = B * S * H * D * 2

    def step():
        ctx.fused_qk_norm_rope_scatter(shards[0], shards[1], w_q, w_k, cos, sin, eps=w.eps, v=shards[2])
        ctx.wait()
        ctx.gather_out(o)

    return {"workload": w, "ctx": ctx, "step": step, "bytes_per_step": 3 * 2 * real + 2 * real,
            "dominant": ("norm_rope", 6 * real, "norm_rope_kernel<16,bf16> (3-D RoPE, padded sequence)"),
            "dtype": "bf16", "data": "synthetic N(0,1) activations, N(1,0.1) norm weights, 3-D RoPE 44/42/42",
            "config": {"workload": w.name, "P": P, "B": B, "S": S, "S_padded": P * S_l, "H": H, "D": D,
                       "bytes_per_step": 3 * 2 * real + 2 * real, "bytes_count": "real tokens only"}}


def setup_gqa(torch, dev, synth, rope_table_1d, UlyssesContext):
    w = synth.GQA
    P, B, S_l, Hq, Hkv, D = w.P, w.B, w.S_l, w.Hq, w.Hkv, w.D
    q = synth.normal((P, B, S_l, Hq, D), "bf16", 40, dev)
    k = synth.normal((P, B, S_l, Hkv, D), "bf16", 41, dev)
    v = synth.normal((P, B, S_l, Hkv, D), "bf16", 42, dev)
    o = synth.normal((P, B, P * S_l, Hq // P, D), "bf16", 43, dev)
    ctx = UlyssesContext(P, device=0)
    nq, nkv = P * B * S_l * Hq * D * 2, P * B * S_l * Hkv * D * 2

    def step():
        ctx.scatter_qkv(q, k, v)
        ctx.wait()
        ctx.gather_out(o)

    return {"workload": w, "ctx": ctx, "step": step, "bytes_per_step": 2 * (nq + 2 * nkv) + 2 * nq,
            "dominant": ("scatter", 2 * (nq + 2 * nkv), "relayout_kernel (grouped Q/K/V scatter, one launch)"),
            "dtype": "bf16", "data": "synthetic N(0,1) activations",
            "config": {"workload": w.name, "P": P, "B": B, "S_local": S_l, "Hq": Hq, "Hkv": Hkv, "D": D,
                       "bytes_per_step": 2 * (nq + 2 * nkv) + 2 * nq}}


def setup_tiny(torch, dev, synth, rope_table_1d, UlyssesContext):
    w = synth.TINY
    P, B, S_l, H, D = w.P, w.B, w.S_l, w.Hq, w.D
    q, k, v = (synth.normal((P, B, S_l, H, D), "f16", 50 + i, dev) for i in range(3))
    o = synth.normal((P, B, P * S_l, H // P, D), "f16", 53, dev)
    ctx = UlyssesContext(P, device=0)
    n = P * B * S_l * H * D * 2

    def step():
        ctx.scatter_qkv(q, k, v)
        ctx.wait()
        ctx.gather_out(o)

    return {"workload": w, "ctx": ctx, "step": step, "bytes_per_step": 3 * 2 * n + 2 * n,
            "dominant": ("scatter", 6 * n, "relayout_kernel (grouped Q/K/V scatter, one launch)"),
            "dtype": "f16", "data": "synthetic N(0,1) activations",
            "config": {"workload": w.name, "P": P, "B": B, "S_local": S_l, "H": H, "D": D,
                       "bytes_per_step": 3 * 2 * n + 2 * n, "note": "launch-bound"}}


def setup_spatial(torch, dev, synth, rope_table_1d, UlyssesContext):
    from sequence_attention_ulysses_amd import height_split
    w = synth.SPATIAL
    full = synth.normal(w.shape, w.dtype, 60, dev)
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

    def step():
        sh = ctx.spatial_split_halo(full, halo=w.halo, out=bufs[0])
        st = ctx.spatial_gather_stacked(sh, Hh, halo=w.halo, out=bufs[1])
        ctx.spatial_trim_concat(st, Hh, out=bufs[2])

    bufs = [torch.empty((w.P,) + lead + (hmax + 2 * w.halo, W), dtype=full.dtype, device=dev),
            torch.empty((w.P,) + lead + (hmax, W), dtype=full.dtype, device=dev),
            torch.empty(w.shape, dtype=full.dtype, device=dev)]
    return {"workload": w, "ctx": ctx, "step": step, "bytes_per_step": split + gather + trim,
            "dominant": ("spatial", (split + gather + trim) // 3, "rowmap_kernel (average of the three launches)"),
            "dtype": "bf16", "data": "synthetic N(0,1) latent",
            "config": {"workload": w.name, "P": w.P, "shape": list(w.shape), "heights": h, "halo": w.halo,
                       "bytes_per_step": split + gather + trim, "note": "cache-resident"}}


MFMA_BF16_PEAK_TFLOPS = 2500.0


def _setup_proj(torch, dev, synth, rope_table_1d, UlyssesContext, w, seed, name):
    """The attention front end with the QKV projection fused in: one launch
    projects x, normalises and rotates q/k and stores every head band into
    its head-sharded target (flashinfer PR #6332's fused call), then the wait
    and the output gather.  Timed beside it: the per-operator path, a library
    GEMM (torch, hipBLASLt) writing qkv, then the fused norm/RoPE scatter."""
    import torch.nn.functional as F
    P, B, S_l, Hq, Hkv, D = w.P, w.B, w.S_l, w.Hq, w.Hkv, w.D
    hidden, N = Hq * D, (Hq + 2 * Hkv) * D
    M = P * B * S_l
    x = synth.normal((P, B, S_l, hidden), "bf16", seed, dev)
    w_qkv = synth.normal((N, hidden), "bf16", seed + 1, dev, std=hidden ** -0.5)
    w_q, w_k = synth.norm_weight(D, "bf16", seed + 2, dev), synth.norm_weight(D, "bf16", seed + 3, dev)
    cos, sin = (t.to(dev) for t in rope_table_1d(P * S_l, D, theta=w.theta))
    o = synth.normal((P, B, P * S_l, Hq // P, D), "bf16", seed + 4, dev)
    ctx = UlyssesContext(P, device=0)
    flops = 2 * M * N * hidden
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    y4 = y.view(P, B, S_l, N)
    yq = y4[..., :Hq * D].unflatten(-1, (Hq, D))
    yk = y4[..., Hq * D:(Hq + Hkv) * D].unflatten(-1, (Hkv, D))
    yv = y4[..., (Hq + Hkv) * D:].unflatten(-1, (Hkv, D))
    x2 = x.view(M, hidden)

    def step():
        ctx.fused_qkv_proj_norm_rope_scatter(x, w_qkv, Hq, Hkv, w_q, w_k, cos, sin, eps=w.eps)
        ctx.wait()
        ctx.gather_out(o)

    def step_per_operator():
        F.linear(x2, w_qkv, out=y)
        ctx.fused_qk_norm_rope_scatter(yq, yk, w_q, w_k, cos, sin, eps=w.eps, v=yv, tags=("pq", "pk", "pv"))
        ctx.wait()
        ctx.gather_out(o)

    return {"workload": w, "name": name, "ctx": ctx, "step": step,
            "step_per_operator": step_per_operator,
            "bytes_per_step": flops, "unit": "TFLOP/s", "unit_div": 1e12,
            "metric": "QKV projection + QK-norm + RoPE + Ulysses scatter + output gather, projection TFLOP/s "
                      "over the step, P=%d bf16, 1 MI355X" % P,
            "dominant": ("proj", flops, "proj_kernel<bf16> (MFMA QKV projection with norm/RoPE/band-store "
                         "epilogue)", "mfma", MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"),
            "cpu_proj": (x, w_qkv, w_q, w_k, Hq, Hkv, w.eps, w.theta),
            "dtype": "bf16", "data": "synthetic N(0,1) activations, N(0,1/hidden) QKV weight, N(1,0.1) norm "
                                     "weights, 1-D RoPE theta 1e4 (seeded)",
            "config": {"workload": name, "P": P, "B": B, "S_local": S_l, "S": P * S_l, "Hq": Hq, "Hkv": Hkv,
                       "D": D, "hidden": hidden, "M": M, "N": N, "flops_per_step": flops,
                       "parallelism": "ulysses-p%d-emulated" % P}}


def setup_video_dit_proj(torch, dev, synth, rope_table_1d, UlyssesContext):
    return _setup_proj(torch, dev, synth, rope_table_1d, UlyssesContext, synth.VIDEO_DIT, 70,
                       "video_dit_proj_p4_s16384_h24_hidden3072_bf16")


def setup_gqa_proj(torch, dev, synth, rope_table_1d, UlyssesContext):
    return _setup_proj(torch, dev, synth, rope_table_1d, UlyssesContext, synth.GQA, 80,
                       "gqa_proj_p8_b2_s65536_hq32_hkv8_hidden4096_bf16")


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


def measure_protocol(args, torch, dev, setup, step, timed, samples: int = 100):
    """The rest of the timing protocol, outside the timed region: the spread
    of single steps (events on the stream every kernel of the step runs on),
    an A/A repeat of the timed loop, a plain device copy of the step's bytes
    (torch's, and the library's own relayout kernel as an identity copy: the
    copy roof of this box), and the same step in fp16 (a relayout moves bytes,
    so the rate must not depend on the 16-bit type)."""
    from sequence_attention_ulysses_amd import UlyssesContext, rope_table_1d, synth

    nbytes = setup["bytes_per_step"]
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(samples)]
    for e0, e1 in ev:
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    t = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    pick = lambda q: t[min(len(t) - 1, int(q * len(t)))]
    spread = {"samples": samples, "median_us": round(pick(0.5) * 1e3, 2), "p10_us": round(pick(0.1) * 1e3, 2),
              "p90_us": round(pick(0.9) * 1e3, 2), "GB_s_at_median": round(nbytes / (pick(0.5) * 1e-3) / 1e9, 1)}

    wall = timed(step, args.steps)
    aa = {"ms_per_step": round(wall * 1e3 / args.steps, 5), "GB_s": round(nbytes / (wall / args.steps) / 1e9, 2)}

    # a device-to-device copy moving the same bytes (half read, half written)
    src = torch.empty(nbytes // 2, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    wall = timed(lambda: dst.copy_(src), args.steps)
    copy = {"bytes_copied": nbytes // 2, "ms": round(wall * 1e3 / args.steps, 5),
            "GB_s": round(nbytes / (wall / args.steps) / 1e9, 2)}
    del src, dst

    # the same bytes through the library's own relayout kernel as a plain copy
    # (one rank: the identity map), on the caller's stream: this box's copy roof
    rows = (nbytes // 2) // (128 * 128 * 2)
    csrc = torch.ones((1, 1, rows, 128, 128), dtype=torch.bfloat16, device=dev)
    cdst = torch.empty_like(csrc)
    with UlyssesContext(1, device=0) as cctx:
        cctx.set_route("caller")
        for _ in range(args.warmup):
            cctx.scatter_qkv(q=csrc, out=(cdst, None, None))
        wall = timed(lambda: cctx.scatter_qkv(q=csrc, out=(cdst, None, None)), args.steps)
    cbytes = 2 * csrc.numel() * 2
    copy_roof = {"kernel": "relayout_kernel, one rank (identity map)", "bytes_moved": cbytes,
                 "us": round(wall * 1e6 / args.steps, 2), "GB_s": round(cbytes / (wall / args.steps) / 1e9, 1)}
    del csrc, cdst

    f16 = setup_video_dit(torch, dev, synth, rope_table_1d, UlyssesContext, dtype="f16")
    for _ in range(args.warmup):
        f16["step"]()
    wall = timed(f16["step"], args.steps)
    f16["ctx"].close()
    fp16 = {"ms_per_step": round(wall * 1e3 / args.steps, 5), "GB_s": round(nbytes / (wall / args.steps) / 1e9, 2)}
    copy_roof["step_over_copy_roof"] = round(aa["GB_s"] / copy_roof["GB_s"], 4)
    return {"step_spread": spread, "aa_repeat": aa, "device_copy_control": copy, "copy_roof": copy_roof,
            "fp16_same_shape": fp16}


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
    ap.add_argument("--cold", action="store_true",
                    help="also time each step after a 1 GiB read that evicts the caches (event-timed, reported apart)")
    ap.add_argument("--no-profile", action="store_true", help="do not bracket launches with timing events")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step into a HIP graph and time its replays (no per-launch host work; "
                         "implies --no-profile and --no-two-stream)")
    ap.add_argument("--no-two-stream", action="store_true",
                    help="skip the two-stream comparison (profiling runs then hold only the headline step)")
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
    setup = WORKLOADS[args.workload](torch, dev, synth, rope_table_1d, UlyssesContext)
    w = setup["workload"]
    ctx = setup["ctx"]
    if args.route:
        ctx.set_route(args.route)
        setup["config"]["scatter_route"] = args.route
    step, step_two_stream = setup["step"], setup.get("step_two_stream")
    step_per_operator = setup.get("step_per_operator")
    args.bytes_per_step = setup["bytes_per_step"]        # the step's work: bytes, or flops for TFLOP/s
    unit, unit_div = setup.get("unit", "GB/s"), setup.get("unit_div", 1e9)
    name = setup.get("name", w.name)
    if step_two_stream is None:
        args.no_two_stream = True
    print("bench: %s on %s, %d warmup + %d timed steps" % (name, torch.cuda.get_device_name(0),
                                                         args.warmup, args.steps), file=sys.stderr, flush=True)

    def timed(fn, steps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    if args.graph:
        args.no_profile = args.no_two_stream = True
        step_per_operator = None
    for _ in range(args.warmup):
        step()
        if not args.no_two_stream:
            step_two_stream()
        if step_per_operator is not None:
            step_per_operator()
    torch.cuda.synchronize()
    if args.graph:
        # the library's calls are capturable: its targets are registered and its
        # event pools filled by the warmup steps, and a step allocates nothing
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=cap):
            step()
        torch.cuda.synchronize()
        step = graph.replay
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        setup["config"]["launch"] = "hip_graph"
    dom_kind, dom_bytes, dom_name = setup["dominant"][:3]
    dom_bound, dom_peak, dom_unit = (setup["dominant"][3:] if len(setup["dominant"]) > 3
                                     else ("hbm", HBM_PEAK_GBS, "GB/s"))
    if not args.no_profile:
        # time only the dominant kernel, one launch in PROFILE_EVERY: every event pair adds
        # latency between kernels
        ctx.profile(True, kinds=[dom_kind], every=PROFILE_EVERY)
        ctx.profile_reset()
    wall = timed(step, args.steps)
    ms_per_step = wall * 1e3 / args.steps
    value = args.bytes_per_step / (wall / args.steps) / unit_div

    kernels = {}
    roofline = None
    if not args.no_profile:
        ms, n = ctx.profile_read(dom_kind)
        if n:
            avg_us = ms * 1e3 / n
            div = 1e9 if dom_unit == "GB/s" else 1e12
            kernels[dom_kind] = {"timed_launches": n, "launches": args.steps, "avg_us": round(avg_us, 2),
                                 "work_per_launch": dom_bytes,
                                 dom_unit.replace("/", "_"): round(dom_bytes / (avg_us * 1e-6) / div, 1)}
        ctx.profile(False)
        ctx.profile_reset()
        dom = kernels.get(dom_kind)
        if dom:
            achieved = dom[dom_unit.replace("/", "_")]
            roofline = {"bound": dom_bound, "achieved": achieved, "peak": dom_peak, "unit": dom_unit,
                        "frac": round(achieved / dom_peak, 4),
                        "traffic": traffic_from_profiles(name) if dom_bound == "hbm" else None,
                        "kernel": dom_name, "avg_us": dom["avg_us"],
                        ("algorithmic_bytes_per_launch" if dom_bound == "hbm" else "flops_per_launch"): dom_bytes}

    # the two-stream form of the same step, timed the same way (no events)
    two_stream = None
    if not args.no_two_stream:
        wall2 = timed(step_two_stream, args.steps)
        two_stream = {"ms_per_step": round(wall2 * 1e3 / args.steps, 5),
                      "GB_s": round(args.bytes_per_step / (wall2 / args.steps) / 1e9, 2)}

    per_operator = None
    if step_per_operator is not None:
        wall3 = timed(step_per_operator, args.steps)
        per_operator = {"path": "torch linear (hipBLASLt) writing qkv, then fused_qk_norm_rope_scatter, wait, gather",
                        "ms_per_step": round(wall3 * 1e3 / args.steps, 5),
                        unit.replace("/", "_"): round(args.bytes_per_step / (wall3 / args.steps) / unit_div, 2),
                        "fused_speedup": round(wall3 / wall, 4)}

    cold = None
    if args.cold:
        # Reading 1 GiB evicts the L2s and the 256 MB Infinity Cache without
        # leaving dirty lines whose write-back would overlap the timed step.
        scrub = torch.ones(1 << 27, dtype=torch.int64, device=dev)
        torch.cuda.synchronize()
        times = []
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(20):
            # no wait between the scrub and the step: the host enqueues the
            # step while the scrub runs, so the events time the GPU, not the
            # host's launch latency
            scrub.max()
            e0.record()
            step()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        times.sort()
        med = times[len(times) // 2]
        cold = {"median_ms": round(med, 4),
                unit.replace("/", "_"): round(args.bytes_per_step / (med * 1e-3) / unit_div, 1),
                "p10_ms": round(times[2], 4), "p90_ms": round(times[17], 4)}
        # the same cold steps again, each kernel bracketed by the library's own events
        if not args.no_profile:
            ctx.profile(True, every=1)
            ctx.profile_reset()
            for _ in range(20):
                scrub.max()
                torch.cuda.synchronize()
                step()
                torch.cuda.synchronize()
            per_kernel = {}
            from sequence_attention_ulysses_amd._lib import KERNEL_KINDS
            for kind in KERNEL_KINDS:
                ms, n = ctx.profile_read(kind)
                if n:
                    per_kernel[kind] = round(ms * 1e3 / n, 2)
            ctx.profile(False)
            ctx.profile_reset()
            cold["kernel_avg_us"] = per_kernel
        del scrub

    extra = (measure_protocol(args, torch, dev, setup, step, timed)
             if args.workload == "video_dit" and not args.graph else None)

    ctx.close()

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
        "kernels": kernels,
        "two_stream": two_stream,
        "cpu_baseline": cpu,
    }
    if unit == "GB/s":
        rec["hbm_frac"] = round(value / HBM_PEAK_GBS, 4)
    if per_operator:
        rec["per_operator"] = per_operator
    if cold:
        rec["cold_cache"] = cold
    if extra:
        rec.update(extra)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
