"""GPU parity of the HIP path against the CPU oracle (needs an MI355X).

Relayouts are compared bit for bit.  The fused Q/K RMSNorm + RoPE scatter is
compared element by element against the oracle's double-precision result:
every element within half a 16-bit ulp of it plus a derived fp32 evaluation
bound (one rounding to nearest even), max-abs error <= 2e-2 (bf16) / 2e-3
(fp16) everywhere below |y| = 8, where half an ulp alone is smaller than the
tolerance (flashinfer PR #6332, "Tolerance", classifies such elements instead
of loosening the tolerance), and the rounding error unbiased with a single
rounding's spread.  Small cases span several blocks with ragged tails; the five
workloads run at their full sizes in the launch configuration the benchmark
times, compared in full where the oracle finishes in seconds and on sampled
token windows otherwise.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from sequence_attention_ulysses_amd import (UlyssesContext, rope_table_1d, rope_table_3d, synth)
from tests.tolerance import Check16, check16, proj_bounds

pytestmark = pytest.mark.gpu

# host threads for the oracle side of whole-output comparisons (the GPU machines give 16)
HOST_THREADS = max(1, min(16, os.cpu_count() or 1))

@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def to_bits(t: torch.Tensor) -> np.ndarray:
    return synth.bits(t.detach().cpu())


def assert_close16(got: torch.Tensor, ref: np.ndarray, dtype: str, what: str, E=None, stats: bool = True):
    """Every element within half a 16-bit ulp of the exact oracle value plus the derived
    fp32 evaluation bound E (a single round-to-nearest-even of an fp32 evaluation), the
    stated max-abs tolerance everywhere below |y| = 8, and an unbiased rounding error
    of a single rounding's spread (tests/tolerance.py gives the derivation)."""
    out = check16(got.detach().cpu().double().numpy(), ref, dtype, what, E=E, stats=stats)
    return out["max_abs"]


def contiguous_qkv(P, B, S_l, H, D, dtype, seed, device, Hkv=None):
    Hkv = H if Hkv is None else Hkv
    q = synth.normal((P, B, S_l, H, D), dtype, seed, device)
    k = synth.normal((P, B, S_l, Hkv, D), dtype, seed + 1, device)
    v = synth.normal((P, B, S_l, Hkv, D), dtype, seed + 2, device)
    return q, k, v


# ---------------------------------------------------------------------------
# plain scatter / gather
# ---------------------------------------------------------------------------
SMALL = [
    # P, B, S_l, Hq, Hkv, D, dtype
    (1, 1, 33, 4, 4, 128, "bf16"),
    (2, 1, 128, 8, 8, 64, "f16"),          # the tiny round-trip workload
    (2, 2, 200, 8, 4, 128, "bf16"),        # S_local = 200 tail
    (3, 1, 7, 6, 3, 64, "f16"),
    (4, 1, 1, 8, 4, 128, "bf16"),
    (4, 2, 777, 24, 8, 128, "bf16"),       # several blocks, ragged tail
    (8, 1, 65, 32, 8, 128, "bf16"),        # one K/V head per rank
    (8, 2, 3, 16, 8, 256, "f16"),
]


@pytest.mark.parametrize("P,B,S_l,Hq,Hkv,D,dtype", SMALL)
def test_scatter_gather_small(dev, orc, P, B, S_l, Hq, Hkv, D, dtype):
    q, k, v = contiguous_qkv(P, B, S_l, Hq, D, dtype, 10 + P, dev, Hkv)
    with UlyssesContext(P, device=0) as ctx:
        yq, yk, yv = ctx.scatter_qkv(q, k, v)
        ctx.wait()
        torch.cuda.synchronize()
        for x, y in ((q, yq), (k, yk), (v, yv)):
            np.testing.assert_array_equal(to_bits(y), orc.scatter(to_bits(x)))
        # inverse: gather(scatter(x)) = x, and the oracle's gather of an independent output
        z = ctx.gather_out(yq, tag="rt")
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_bits(z), to_bits(q))
        o = synth.normal((P, B, P * S_l, Hq // P, D), dtype, 99, dev)
        z2 = ctx.gather_out(o, tag="out")
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_bits(z2), orc.gather(to_bits(o)))


def test_tiny_round_trip(dev, orc):
    """B=1, P=2, S_l=128, H=8, D=64 fp16 contiguous Q/K/V: scatter then inverse gather."""
    w = synth.TINY
    q, k, v = contiguous_qkv(w.P, w.B, w.S_l, w.Hq, w.D, w.dtype, 0, dev)
    with UlyssesContext(w.P, device=0) as ctx:
        ys = ctx.scatter_qkv(q, k, v)
        ctx.wait()
        for x, y, tag in zip((q, k, v), ys, ("oq", "ok", "ov")):
            np.testing.assert_array_equal(to_bits(y), orc.scatter(to_bits(x)))
            z = ctx.gather_out(y, tag=tag)
            torch.cuda.synchronize()
            assert torch.equal(z.view(torch.int16), x.view(torch.int16))


def test_bit_patterns_pass_unchanged(dev, orc):
    """NaN payloads, infinities, -0 and subnormals are moved as opaque bytes."""
    special = torch.tensor([0x7FC1, -1, -32768, 0x0001, 0x7F80, -128, 0x0000, 0x3F80], dtype=torch.int16)
    g = torch.Generator().manual_seed(5)
    idx = torch.randint(0, len(special), (4, 1, 37, 8, 128), generator=g)
    x = special[idx].view(torch.bfloat16).to(dev)
    with UlyssesContext(4, device=0) as ctx:
        (y,) = [t for t in ctx.scatter_qkv(v=x) if t is not None]
        ctx.wait()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_bits(y), orc.scatter(to_bits(x)))


def test_empty_operands_are_noops(dev):
    with UlyssesContext(2, device=0) as ctx:
        x = torch.empty((2, 1, 0, 4, 64), dtype=torch.float16, device=dev)
        out = torch.full((2, 1, 0, 2, 64), 1.0, dtype=torch.float16, device=dev)
        ctx.scatter_qkv(q=x, out=(out, None, None))
        ctx.wait()
        torch.cuda.synchronize()
        assert ctx.stats()["launches"] == 0


def test_guard_bands_and_prefill(dev, orc):
    """Targets inside larger buffers: the bytes around them are never written, and
    every element of the target is (a NaN prefill would otherwise survive)."""
    P, B, S_l, H, D = 4, 2, 300, 8, 128
    q = synth.normal((P, B, S_l, H, D), "bf16", 3, dev)
    n = P * B * S_l * H * D
    guard = 4096
    buf = torch.full((n + 2 * guard,), float("nan"), dtype=torch.bfloat16, device=dev)
    canary = buf.clone()
    out = buf[guard:guard + n].view(P, B, P * S_l, H // P, D)
    with UlyssesContext(P, device=0) as ctx:
        ctx.scatter_qkv(q=q, out=(out, None, None))
        ctx.wait()
        torch.cuda.synchronize()
    b = to_bits(buf)
    np.testing.assert_array_equal(b[:guard], to_bits(canary)[:guard])
    np.testing.assert_array_equal(b[guard + n:], to_bits(canary)[guard + n:])
    np.testing.assert_array_equal(to_bits(out), orc.scatter(to_bits(q)))


# ---------------------------------------------------------------------------
# fused Q/K RMSNorm + RoPE scatter
# ---------------------------------------------------------------------------
FUSED_SMALL = [
    # P, B, S_l, Hq, Hkv, D, dtype, fused_qkv_source
    (2, 1, 128, 8, 8, 64, "f16", False),      # fp16 at the tiny workload's shape
    (4, 1, 200, 24, 24, 128, "bf16", True),   # video-DiT head layout, S_local = 200 tail
    (4, 2, 37, 8, 4, 128, "bf16", False),     # GQA Q/K
    (2, 1, 50, 4, 4, 256, "f16", False),
    (4, 1, 29, 8, 8, 32, "bf16", True),
    (1, 1, 64, 4, 4, 128, "bf16", False),
    (2, 1, 40, 6, 2, 128, "bf16", False),     # head counts not a multiple of the groups per wave
    (3, 1, 16, 6, 3, 128, "f16", False),
]


@pytest.mark.parametrize("P,B,S_l,Hq,Hkv,D,dtype,fused", FUSED_SMALL)
def test_fused_norm_rope_small(dev, orc, P, B, S_l, Hq, Hkv, D, dtype, fused):
    if fused:
        qkv = synth.normal((P, B, S_l, 3, Hq, D), dtype, 21, dev)
        q, k, v = qkv[:, :, :, 0], qkv[:, :, :, 1], qkv[:, :, :, 2]
    else:
        q, k, v = contiguous_qkv(P, B, S_l, Hq, D, dtype, 21, dev, Hkv)
    w_q = synth.norm_weight(D, dtype, 1, dev)
    w_k = synth.norm_weight(D, dtype, 2, dev)
    rows = P * S_l + 5
    cos, sin = rope_table_1d(rows, D)
    ocos, osin = orc.rope_table_1d(rows, D)
    with UlyssesContext(P, device=0) as ctx:
        yq, yk, yv = ctx.fused_qk_norm_rope_scatter(q, k, w_q, w_k, cos.to(dev), sin.to(dev), v=v)
        ctx.wait()
        torch.cuda.synchronize()
        for x, w, y, name in ((q, w_q, yq, "q"), (k, w_k, yk, "k")):
            ref = orc.fused_norm_rope_scatter(to_bits(x), dtype, to_bits(w), 1e-6, ocos, osin)
            assert_close16(y, ref, dtype, name)
        # V rides in the same launch and is moved bit for bit
        np.testing.assert_array_equal(to_bits(yv), orc.scatter(to_bits(v)))
        # Q/K without V give the same bits as with it
        yq2, yk2, _ = ctx.fused_qk_norm_rope_scatter(q, k, w_q, w_k, cos.to(dev), sin.to(dev),
                                                     tags=("q2", "k2", None))
        torch.cuda.synchronize()
        assert torch.equal(yq2.view(torch.int16), yq.view(torch.int16))
        assert torch.equal(yk2.view(torch.int16), yk.view(torch.int16))


@pytest.mark.parametrize("P,B,S_l,Hq,Hkv", [(4, 1, 64, 24, 24), (8, 2, 16, 32, 8), (2, 1, 10, 40, 40), (1, 1, 6, 4, 2)])
def test_dense_and_interleaved_operands_agree(dev, orc, P, B, S_l, Hq, Hkv):
    """Dense Q/K/V tensors take the operand-major band kernel for Q/K and the relayout
    kernel for V (two launches), the same values as views of one interleaved tensor the
    token-tile kernel with V in the same launch: the per-row arithmetic is the same, so
    the results must agree bit for bit (and with the oracle)."""
    D = 128
    q, k, v = contiguous_qkv(P, B, S_l, Hq, D, "bf16", 77, dev, Hkv)
    # the same values, interleaved: [P, B, S_l, Hq + 2 Hkv, D] with q, k, v head ranges
    inter = torch.cat([q, k, v], dim=3).contiguous()
    qi, ki, vi = inter[:, :, :, :Hq], inter[:, :, :, Hq:Hq + Hkv], inter[:, :, :, Hq + Hkv:]
    w_q, w_k = synth.norm_weight(D, "bf16", 78, dev), synth.norm_weight(D, "bf16", 79, dev)
    cos, sin = (t.to(dev) for t in rope_table_1d(P * S_l, D))
    with UlyssesContext(P, device=0) as ctx:
        n0 = ctx.stats()["launches"]
        yd = ctx.fused_qk_norm_rope_scatter(q, k, w_q, w_k, cos, sin, v=v, tags=("dq", "dk", "dv"))
        n1 = ctx.stats()["launches"]
        yi = ctx.fused_qk_norm_rope_scatter(qi, ki, w_q, w_k, cos, sin, v=vi, tags=("iq", "ik", "iv"))
        assert (n1 - n0, ctx.stats()["launches"] - n1) == (2, 1)
        ctx.wait()
        torch.cuda.synchronize()
        for a, b_, name in zip(yd, yi, "qkv"):
            assert torch.equal(a.view(torch.int16), b_.view(torch.int16)), name
        ocos, osin = orc.rope_table_1d(P * S_l, D)
        assert_close16(yd[0], orc.fused_norm_rope_scatter(to_bits(q), "bf16", to_bits(w_q), 1e-6, ocos, osin), "bf16", "q")
        np.testing.assert_array_equal(to_bits(yd[2]), orc.scatter(to_bits(v)))


def test_fused_single_operand_and_determinism(dev, orc):
    P, B, S_l, H, D = 4, 1, 96, 8, 128
    k = synth.normal((P, B, S_l, H, D), "bf16", 8, dev)
    w = synth.norm_weight(D, "bf16", 9, dev)
    cos, sin = rope_table_1d(P * S_l, D)
    cos, sin = cos.to(dev), sin.to(dev)
    with UlyssesContext(P, device=0) as ctx:
        _, y1, _ = ctx.fused_qk_norm_rope_scatter(None, k, None, w, cos, sin, tags=(None, "k1"))
        _, y2, _ = ctx.fused_qk_norm_rope_scatter(None, k, None, w, cos, sin, tags=(None, "k2"))
        ctx.wait()
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
        ocos, osin = orc.rope_table_1d(P * S_l, D)
        assert_close16(y1, orc.fused_norm_rope_scatter(to_bits(k), "bf16", to_bits(w), 1e-6, ocos, osin),
                       "bf16", "k")


@pytest.mark.parametrize("layout", ["dense", "strided"])
def test_fused_v_only_is_a_plain_scatter(dev, orc, layout):
    """A fused call with V alone (no row is normalised) gives the bit-exact scatter.  A
    dense V goes through the relayout kernel alone; a strided one (a view into a wider
    tensor) through the token-tile kernel, which still reads a table row and a weight row
    per slot without a branch."""
    P, B, S_l, H, D = 4, 2, 40, 8, 128
    wide = synth.normal((P, B, S_l, 2 * H, D), "bf16", 12, dev)
    v = wide[:, :, :, :H].contiguous() if layout == "dense" else wide[:, :, :, H:]
    cos, sin = rope_table_1d(P * S_l, D)
    with UlyssesContext(P, device=0) as ctx:
        before = ctx.stats()["launches"]
        _, _, yv = ctx.fused_qk_norm_rope_scatter(None, None, None, None, cos.to(dev), sin.to(dev), v=v,
                                                  tags=(None, None, "v_only"))
        assert ctx.stats()["launches"] == before + 1
        ctx.wait()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_bits(yv), orc.scatter(to_bits(v)))


def test_fused_edge_rows(dev, orc):
    """Zero rows (padding) give exactly +-0; constant rows hit the closed form."""
    P, B, S_l, H, D = 2, 1, 16, 4, 128
    x = torch.zeros((P, B, S_l, H, D), dtype=torch.bfloat16)
    x[:, :, ::2] = 0.5
    x[1, 0, 3, 2] = -3.0
    xd = x.to(dev)
    w = synth.norm_weight(D, "bf16", 4, dev)
    cos, sin = rope_table_1d(P * S_l, D)
    with UlyssesContext(P, device=0) as ctx:
        (y, _, _) = ctx.fused_qk_norm_rope_scatter(xd, None, w, None, cos.to(dev), sin.to(dev))
        ctx.wait()
        torch.cuda.synchronize()
    ocos, osin = orc.rope_table_1d(P * S_l, D)
    ref = orc.fused_norm_rope_scatter(synth.bits(x), "bf16", to_bits(w), 1e-6, ocos, osin)
    assert_close16(y, ref, "bf16", "edge", stats=False)     # constant rows: not a random sample
    assert (y.float().abs().cpu().numpy()[ref == 0] == 0).all()


# ---------------------------------------------------------------------------
# full-size workloads, in the launch configuration the benchmark times
# ---------------------------------------------------------------------------
def _check_fused_whole(orc, x_bits, y_bits, dtype, w_bits, cos, sin, what, eps=1e-6, chunk=2048):
    """Every element of the head-sharded result y_bits[P(q), B, P*S_l, Hl, D] against the
    oracle's rows of x_bits[P(r), B, S_l, H, D] at positions r*S_l + s, computed in
    (source rank, token chunk) pieces on host threads (the C oracle runs outside the
    interpreter lock).  The rounding statistics are taken over the whole result."""
    P, B, S_l, H, D = x_bits.shape
    Hl = H // P
    w64 = orc.widen(w_bits, dtype)

    def job(r, s0):
        s1 = min(S_l, s0 + chunk)
        n = s1 - s0
        xs = orc.widen(x_bits[r, :, s0:s1], dtype).reshape(-1, D)
        pos = np.broadcast_to(r * S_l + np.arange(s0, s1)[None, :, None], (B, n, H)).reshape(-1)
        yo = orc.norm_rope_rows(xs, w64, eps, cos, sin, pos).reshape(B, n, P, Hl, D).transpose(2, 0, 1, 3, 4)
        c = Check16(dtype, what)
        c.add(orc.widen(y_bits[:, :, r * S_l + s0:r * S_l + s1], dtype), yo, where="r=%d s=[%d,%d)" % (r, s0, s1))
        return c

    total = Check16(dtype, what)
    with ThreadPoolExecutor(HOST_THREADS) as ex:
        for c in ex.map(lambda a: job(*a), [(r, s0) for r in range(P) for s0 in range(0, S_l, chunk)]):
            total.merge(c)
    out = total.done()
    print("%s: %d elements, max-abs %.3g, bias %+.4f ulp, rms %.4f ulp, %d classified" % (
        what, out["elements"], out["max_abs"], out.get("bias_ulp", 0.0), out.get("rms_ulp", 0.0),
        out["classified"]), flush=True)
    return out


def test_offsets_beyond_4gib(dev, orc):
    """Rank slabs and targets larger than 4 GiB (P=2, S_l=2^19+32, H=32, D=128 bf16:
    4 GiB per slab, 8 GiB per tensor), so every byte offset past 2^32 must be formed in
    64 bits: the plain scatter, the fused Q/K/V launch and the gather, checked against
    the oracle on token windows at the start, middle and end of each slab, and the
    gather of the scattered V against V itself in full."""
    P, B, S_l, H, D = 2, 1, (1 << 19) + 32, 32, 128
    n = P * B * S_l * H * D * 2
    assert n // P > 1 << 32
    free, _ = torch.cuda.mem_get_info()
    if free < 10 * n:
        pytest.skip("needs %.0f GiB of free device memory" % (10 * n / 2 ** 30))
    print("beyond-4GiB case: P=%d S_l=%d H=%d D=%d bf16, %.1f GiB per tensor" % (P, S_l, H, D, n / 2 ** 30), flush=True)
    q, k, v = contiguous_qkv(P, B, S_l, H, D, "bf16", 4000, dev)
    w_q, w_k = synth.norm_weight(D, "bf16", 4003, dev), synth.norm_weight(D, "bf16", 4004, dev)
    cos, sin = rope_table_1d(P * S_l, D)
    ocos, osin = orc.rope_table_1d(P * S_l, D)
    win = [(0, 32), (S_l // 2 - 16, S_l // 2 + 16), (S_l - 32, S_l)]
    with UlyssesContext(P, device=0) as ctx:
        _, _, yv = ctx.scatter_qkv(v=v, tags=(None, None, "v_plain"))
        yq, yk, yv2 = ctx.fused_qk_norm_rope_scatter(q, k, w_q, w_k, cos.to(dev), sin.to(dev), v=v)
        ctx.wait()
        z = ctx.gather_out(yv, tag="out")
        torch.cuda.synchronize()
        assert torch.equal(z.view(torch.int16), v.view(torch.int16))
        assert torch.equal(yv2.view(torch.int16), yv.view(torch.int16))
        for s0, s1 in win:
            rows = torch.cat([torch.arange(r * S_l + s0, r * S_l + s1) for r in range(P)]).to(dev)
            np.testing.assert_array_equal(to_bits(yv.index_select(2, rows)), orc.scatter(to_bits(v[:, :, s0:s1])))
        for x, w, y, name in ((q, w_q, yq, "q"), (k, w_k, yk, "k")):
            for s0, s1 in win:
                xs = orc.widen(to_bits(x[:, :, s0:s1]), "bf16")
                pos = np.broadcast_to(np.arange(P)[:, None, None, None] * S_l + np.arange(s0, s1)[None, None, :, None],
                                      (P, B, s1 - s0, H)).reshape(-1)
                yo = orc.norm_rope_rows(xs.reshape(-1, D), orc.widen(to_bits(w), "bf16"), 1e-6, ocos, osin, pos)
                yo = yo.reshape(P, B, s1 - s0, H, D)
                for r in range(P):
                    sub = y.index_select(2, torch.arange(r * S_l + s0, r * S_l + s1, device=dev))
                    want = yo[r].reshape(B, s1 - s0, P, H // P, D).transpose(2, 0, 1, 3, 4)
                    assert_close16(sub, want, "bf16", "%s r=%d s=[%d,%d)" % (name, r, s0, s1))


@pytest.mark.parametrize("seed", range(5))
def test_video_dit_block_full(dev, orc, seed):
    """P=4, S_l=4096, H=24, D=128 bf16; V strided from fused QKV on the comm stream,
    fused Q/K norm + RoPE on the caller stream, grouped wait, output gather; every
    output element compared, seeds 0-4."""
    w = synth.VIDEO_DIT
    P, B, S_l, H, D = w.P, w.B, w.S_l, w.Hq, w.D
    base = 100 * seed
    print("video-DiT two-stream seed %d" % seed, flush=True)
    qkv = synth.normal((P, B, S_l, 3, H, D), "bf16", base, dev)
    w_q, w_k = synth.norm_weight(D, "bf16", base + 1, dev), synth.norm_weight(D, "bf16", base + 2, dev)
    cos, sin = rope_table_1d(P * S_l, D, theta=w.theta)
    o = synth.normal((P, B, P * S_l, H // P, D), "bf16", base + 3, dev)
    with UlyssesContext(P, device=0) as ctx:
        _, _, yv = ctx.scatter_qkv(v=qkv[:, :, :, 2])
        yq, yk, _ = ctx.fused_qk_norm_rope_scatter(qkv[:, :, :, 0], qkv[:, :, :, 1], w_q, w_k,
                                                cos.to(dev), sin.to(dev), eps=w.eps)
        ctx.wait()
        z = ctx.gather_out(o)
        torch.cuda.synchronize()
        xb = to_bits(qkv)
        np.testing.assert_array_equal(to_bits(yv), orc.scatter(xb[:, :, :, 2]))
        np.testing.assert_array_equal(to_bits(z), orc.gather(to_bits(o)))
        ocos, osin = orc.rope_table_1d(P * S_l, D, theta=w.theta)
        for c, wt, y, name in ((0, w_q, yq, "q"), (1, w_k, yk, "k")):
            _check_fused_whole(orc, xb[:, :, :, c], to_bits(y), "bf16", to_bits(wt), ocos, osin,
                               "video-DiT %s seed %d" % (name, seed), eps=w.eps)


@pytest.mark.parametrize("seed", range(5))
def test_video_dit_block_single_launch_full(dev, orc, seed):
    """The same block with V scattered inside the fused Q/K launch (the launch the
    benchmark times); every output element compared, seeds 0-4."""
    w = synth.VIDEO_DIT
    P, B, S_l, H, D = w.P, w.B, w.S_l, w.Hq, w.D
    base = 100 * seed + 5
    print("video-DiT single launch seed %d" % seed, flush=True)
    qkv = synth.normal((P, B, S_l, 3, H, D), "bf16", base, dev)
    w_q, w_k = synth.norm_weight(D, "bf16", base + 1, dev), synth.norm_weight(D, "bf16", base + 2, dev)
    cos, sin = rope_table_1d(P * S_l, D, theta=w.theta)
    with UlyssesContext(P, device=0) as ctx:
        yq, yk, yv = ctx.fused_qk_norm_rope_scatter(qkv[:, :, :, 0], qkv[:, :, :, 1], w_q, w_k, cos.to(dev),
                                                    sin.to(dev), eps=w.eps, v=qkv[:, :, :, 2])
        ctx.wait()
        torch.cuda.synchronize()
        xb = to_bits(qkv)
        np.testing.assert_array_equal(to_bits(yv), orc.scatter(xb[:, :, :, 2]))
        ocos, osin = orc.rope_table_1d(P * S_l, D, theta=w.theta)
        for c, wt, y, name in ((0, w_q, yq, "q"), (1, w_k, yk, "k")):
            _check_fused_whole(orc, xb[:, :, :, c], to_bits(y), "bf16", to_bits(wt), ocos, osin,
                               "video-DiT single launch %s seed %d" % (name, seed), eps=w.eps)


@pytest.mark.parametrize("seed", range(2))
def test_wan_long_sequence_full(dev, orc, seed):
    """S = 75600 tokens (21x60x60 grid) padded to 75776 over P=4, H=40, D=128 bf16, 3-D
    RoPE, in the benchmark's single-launch form: pad + shard, the fused Q/K/V launch,
    the gather and trim; every output element compared, two seeds."""
    w = synth.WAN_LONG
    P, B, S_l, H, D, S = w.P, w.B, w.S_l, w.Hq, w.D, w.S_real
    assert orc.padded_local_len(S, P, 128) == S_l
    T_, Hh, Ww = w.grid
    base = 30 + 10 * seed
    print("Wan seed %d" % seed, flush=True)
    fulls = [synth.normal((B, S, H, D), "bf16", base + i, dev) for i in range(3)]
    w_q, w_k = synth.norm_weight(D, "bf16", base + 4, dev), synth.norm_weight(D, "bf16", base + 5, dev)
    cos, sin = rope_table_3d(P * S_l, D, Hh, Ww, real_rows=S)
    ocos, osin = orc.rope_table_3d(P * S_l, D, Hh, Ww, real_rows=S)
    with UlyssesContext(P, device=0) as ctx:
        shards = [ctx.seq_pad_shard(f, S_l) for f in fulls]
        yq, yk, yv = ctx.fused_qk_norm_rope_scatter(shards[0], shards[1], w_q, w_k, cos.to(dev), sin.to(dev),
                                                    v=shards[2])
        ctx.wait()
        z = ctx.gather_out(yv, tag="out")
        back = ctx.seq_unshard_trim(z, S)
        torch.cuda.synchronize()
        xbs = [to_bits(t) for t in shards]
        for f, xb in zip(fulls, xbs):           # pad + shard, zero pad rows
            np.testing.assert_array_equal(xb, orc.pad_shard(to_bits(f), P, S_l))
        np.testing.assert_array_equal(to_bits(yv), orc.scatter(xbs[2]))
        for xb, wt, y, name in ((xbs[0], w_q, yq, "q"), (xbs[1], w_k, yk, "k")):
            _check_fused_whole(orc, xb, to_bits(y), "bf16", to_bits(wt), ocos, osin, "Wan %s seed %d" % (name, seed))
        # inverse path: the gather of the head-sharded V, then the trim, is the original sequence
        np.testing.assert_array_equal(to_bits(z), orc.gather(to_bits(yv)))
        assert torch.equal(back.view(torch.int16), fulls[2].view(torch.int16))
        pad = z[P - 1, :, S_l - (P * S_l - S):]
        assert (pad.view(torch.int16) == 0).all()


@pytest.mark.parametrize("seed", range(2))
def test_gqa_twenty_steps_reuse_targets(dev, orc, seed):
    """B=2, P=8, S_l=8192, Hq=32, Hkv=8 bf16: tagged grouped scatter into 4 cached
    targets reused across 20 steps with fresh inputs, plus the output gather; no
    allocation after the first step; every output element compared at steps 0, 7
    and 19, two seeds."""
    w = synth.GQA
    P, B, S_l, Hq, Hkv, D = w.P, w.B, w.S_l, w.Hq, w.Hkv, w.D
    base = 1000 + 10000 * seed
    print("GQA seed %d" % seed, flush=True)
    with UlyssesContext(P, device=0) as ctx:
        ptrs = None
        for step in range(20):
            q, k, v = contiguous_qkv(P, B, S_l, Hq, D, "bf16", base + 3 * step, dev, Hkv)
            o = synth.normal((P, B, P * S_l, Hq // P, D), "bf16", base + 4000 + step, dev)
            if step == 1:
                torch.cuda.synchronize()
                alloc0 = torch.cuda.memory_stats()["allocation.all.allocated"]
            ys = ctx.scatter_qkv(q, k, v)
            ctx.wait()
            z = ctx.gather_out(o)
            if step == 1:
                torch.cuda.synchronize()
                # the step itself allocated nothing beyond this step's fresh inputs
                assert torch.cuda.memory_stats()["allocation.all.allocated"] == alloc0
            cur = [t.data_ptr() for t in ys] + [z.data_ptr()]
            if ptrs is None:
                ptrs = cur
            assert cur == ptrs, "cached targets moved"
            if step in (0, 7, 19):
                torch.cuda.synchronize()
                for x, y, name in zip((q, k, v), ys, "qkv"):
                    np.testing.assert_array_equal(to_bits(y), orc.scatter(to_bits(x)), err_msg="%s step %d" % (
                        name, step))
                np.testing.assert_array_equal(to_bits(z), orc.gather(to_bits(o)), err_msg="out step %d" % step)
                print("GQA seed %d step %d: q, k, v and out bit-exact" % (seed, step), flush=True)
        assert ctx.target_count() == 4
        assert ctx.stats()["registrations"] == 4


@pytest.mark.parametrize("seed", range(5))
def test_spatial_shards_full(dev, orc, seed):
    """latent [1,16,21,90,160] bf16, P=4 height shards 23/23/22/22 with 1-row halos,
    rank-major stacked gather, trim + concat; seeds 0-4."""
    w = synth.SPATIAL
    full = synth.normal(w.shape, w.dtype, 40 + 7 * seed, dev)
    with UlyssesContext(w.P, device=0) as ctx:
        sh = ctx.spatial_split_halo(full, halo=w.halo)
        st = ctx.spatial_gather_stacked(sh, w.shape[-2], halo=w.halo)
        back = ctx.spatial_trim_concat(st, w.shape[-2])
        torch.cuda.synchronize()
    fb = to_bits(full)
    osh = orc.spatial_split_halo(fb, w.P, halo=w.halo)
    np.testing.assert_array_equal(to_bits(sh), osh)
    np.testing.assert_array_equal(to_bits(st), orc.spatial_gather_stacked(osh, w.shape[-2], halo=w.halo))
    np.testing.assert_array_equal(to_bits(back), fb)


@pytest.mark.parametrize("shape,P,halo", [((2, 3, 1, 9, 8), 3, 1), ((1, 1, 2, 7, 64), 4, 2), ((1, 2, 1, 5, 8), 8, 0)])
def test_spatial_small(dev, orc, shape, P, halo):
    full = synth.normal(shape, "bf16", 41, dev)
    if shape[-2] < P:
        with UlyssesContext(P, device=0) as ctx, pytest.raises(ValueError):
            ctx.spatial_split_halo(full, halo=halo)
        return
    with UlyssesContext(P, device=0) as ctx:
        sh = ctx.spatial_split_halo(full, halo=halo)
        st = ctx.spatial_gather_stacked(sh, shape[-2], halo=halo)
        back = ctx.spatial_trim_concat(st, shape[-2])
        torch.cuda.synchronize()
    osh = orc.spatial_split_halo(to_bits(full), P, halo=halo)
    np.testing.assert_array_equal(to_bits(sh), osh)
    np.testing.assert_array_equal(to_bits(back), to_bits(full))


@pytest.mark.parametrize("P,B,S,R,S_l", [(4, 1, 75, 64, 19), (2, 2, 13, 8, 8), (3, 1, 10, 16, 4)])
def test_pad_shard_small(dev, orc, P, B, S, R, S_l):
    full = synth.normal((B, S, R), "f16", 42, dev)
    with UlyssesContext(P, device=0) as ctx:
        x = ctx.seq_pad_shard(full, S_l)
        back = ctx.seq_unshard_trim(x, S)
        torch.cuda.synchronize()
    np.testing.assert_array_equal(to_bits(x), orc.pad_shard(to_bits(full), P, S_l))
    np.testing.assert_array_equal(to_bits(back), to_bits(full))


# ---------------------------------------------------------------------------
# streams, handshake, reuse hazard, measurement and fail-stop on the device
# ---------------------------------------------------------------------------
def test_consumer_on_other_stream_sees_results(dev, orc):
    P, B, S_l, H, D = 4, 1, 512, 8, 128
    q, k, v = contiguous_qkv(P, B, S_l, H, D, "bf16", 50, dev)
    w_q, w_k = synth.norm_weight(D, "bf16", 51, dev), synth.norm_weight(D, "bf16", 52, dev)
    cos, sin = rope_table_1d(P * S_l, D)
    consumer = torch.cuda.Stream()
    with UlyssesContext(P, device=0) as ctx:
        _, _, yv = ctx.scatter_qkv(v=v)
        yq, yk, _ = ctx.fused_qk_norm_rope_scatter(q, k, w_q, w_k, cos.to(dev), sin.to(dev))
        ctx.wait(consumer)
        with torch.cuda.stream(consumer):
            snap = [yq.clone(), yk.clone(), yv.clone()]
        consumer.synchronize()
    np.testing.assert_array_equal(to_bits(snap[2]), orc.scatter(to_bits(v)))
    ocos, osin = orc.rope_table_1d(P * S_l, D)
    assert_close16(snap[0], orc.fused_norm_rope_scatter(to_bits(q), "bf16", to_bits(w_q), 1e-6, ocos, osin),
                   "bf16", "q")


def test_rejected_call_registers_nothing(dev):
    """A call the library rejects leaves the target cache as it was: new keys are
    registered only after the library accepted the call."""
    P, B, S_l, H, D = 2, 1, 16, 4, 128
    q = synth.normal((P, B, S_l, H, D), "bf16", 70, dev)
    w = synth.norm_weight(D, "bf16", 71, dev)
    cos, sin = (t.to(dev) for t in rope_table_1d(P * S_l, D))
    o = synth.normal((P, B, P * S_l, H // P, D), "bf16", 72, dev)
    with UlyssesContext(P, device=0) as ctx:
        with pytest.raises(ValueError, match="eps"):
            ctx.fused_qk_norm_rope_scatter(q, None, w, None, cos, sin, eps=0.0, tags=("qa", None, None))
        with pytest.raises(ValueError, match="table"):
            ctx.fused_qk_norm_rope_scatter(q, None, w, None, cos[:3], sin[:3], tags=("qb", None, None))
        with pytest.raises(ValueError):
            ctx.gather_out(o[:, :, :P * S_l - 1], tag="oa")          # sequence not divisible by P
        assert ctx.target_count() == 0 and ctx.stats()["registrations"] == 0
        (y, _, _) = ctx.fused_qk_norm_rope_scatter(q, None, w, None, cos, sin, tags=("qc", None, None))
        z = ctx.gather_out(o, tag="oc")
        (y2, _, _) = ctx.fused_qk_norm_rope_scatter(q, None, w, None, cos, sin, tags=("qc", None, None))
        torch.cuda.synchronize()
        assert ctx.target_count() == 2 and ctx.stats()["registrations"] == 2
        assert y2.data_ptr() == y.data_ptr() and torch.equal(y2.view(torch.int16), y.view(torch.int16))
        assert ctx.gather_out(o, tag="oc").data_ptr() == z.data_ptr()


def test_target_reuse_waits_for_consumer(dev, orc):
    """Step n+1's scatter into a cached target is ordered after step n's consumer
    on the caller stream, even when that consumer is slow."""
    P, B, S_l, H, D = 4, 1, 1024, 8, 128
    with UlyssesContext(P, device=0) as ctx:
        v1 = synth.normal((P, B, S_l, H, D), "bf16", 60, dev)
        v2 = synth.normal((P, B, S_l, H, D), "bf16", 61, dev)
        _, _, y = ctx.scatter_qkv(v=v1)
        ctx.wait()
        torch.cuda._sleep(20_000_000)          # a slow consumer ...
        snap = y.clone()                       # ... that reads step n's target
        ctx.scatter_qkv(v=v2)                  # step n+1 overwrites the same target
        ctx.wait()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_bits(snap), orc.scatter(to_bits(v1)))
        np.testing.assert_array_equal(to_bits(y), orc.scatter(to_bits(v2)))


def test_profiling_and_stats(dev):
    P = 4
    with UlyssesContext(P, device=0) as ctx:
        ctx.profile(True)
        q, k, v = contiguous_qkv(P, 1, 256, 8, 128, "bf16", 70, dev)
        ys = ctx.scatter_qkv(q, k, v)
        ctx.wait()
        ctx.gather_out(ys[0])
        ms, n = ctx.profile_read("scatter")
        assert n == 1 and ms > 0
        ms, n = ctx.profile_read("gather")
        assert n == 1 and ms > 0
        ctx.profile_reset()
        assert ctx.profile_read("scatter") == (0.0, 0)
        assert ctx.stats()["launches"] == 2
        # sampled: the first launch of a kind and then one in every 3
        ctx.profile(True, kinds=["gather"], every=3)
        for _ in range(7):
            ctx.gather_out(ys[0])
        ctx.scatter_qkv(q, k, v)
        ms, n = ctx.profile_read("gather")
        assert n == 3 and ms > 0
        assert ctx.profile_read("scatter") == (0.0, 0)


def test_device_fail_stop(dev):
    """An injected launch failure poisons the context without enqueueing anything."""
    from sequence_attention_ulysses_amd import UlyBroken, UlyHipError
    ctx = UlyssesContext(2, device=0)
    q = synth.normal((2, 1, 8, 4, 64), "f16", 80, dev)
    ctx.debug_fail_launch(0)
    with pytest.raises(UlyHipError):
        ctx.scatter_qkv(q=q)
    with pytest.raises(UlyBroken):
        ctx.scatter_qkv(q=q)
    ctx.close()


def test_two_stream_and_single_launch_agree(dev):
    """V on the comm stream and V inside the fused launch give the same bits, and so
    do the Q/K targets of both forms."""
    P, B, S_l, H, D = 4, 1, 256, 8, 128
    qkv = synth.normal((P, B, S_l, 3, H, D), "bf16", 90, dev)
    w_q, w_k = synth.norm_weight(D, "bf16", 91, dev), synth.norm_weight(D, "bf16", 92, dev)
    cos, sin = (t.to(dev) for t in rope_table_1d(P * S_l, D))
    with UlyssesContext(P, device=0) as ctx:
        a = ctx.fused_qk_norm_rope_scatter(qkv[:, :, :, 0], qkv[:, :, :, 1], w_q, w_k, cos, sin, v=qkv[:, :, :, 2],
                                           tags=("qa", "ka", "va"))
        (_, _, vb) = ctx.scatter_qkv(v=qkv[:, :, :, 2], tags=(None, None, "vb"))
        qb, kb, _ = ctx.fused_qk_norm_rope_scatter(qkv[:, :, :, 0], qkv[:, :, :, 1], w_q, w_k, cos, sin,
                                                   tags=("qb", "kb", None))
        ctx.wait()
        torch.cuda.synchronize()
        for x, y in zip(a, (qb, kb, vb)):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_two_contexts_in_flight(dev, orc):
    """Two groups on two streams, submissions interleaved, each consumed on its own stream."""
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    x1 = synth.normal((2, 1, 300, 8, 64), "f16", 93, dev)
    x2 = synth.normal((4, 2, 100, 8, 128), "bf16", 94, dev)
    torch.cuda.synchronize()
    c1, c2 = UlyssesContext(2, device=0), UlyssesContext(4, device=0)
    try:
        for _ in range(3):
            y1 = c1.scatter_qkv(q=x1, k=x1, stream=s1)
            y2 = c2.scatter_qkv(v=x2, stream=s2)
            c1.wait(s1)
            c2.wait(s2)
            with torch.cuda.stream(s1):
                z1 = c1.gather_out(y1[0], stream=s1)
            with torch.cuda.stream(s2):
                z2 = c2.gather_out(y2[2], stream=s2)
        s1.synchronize()
        s2.synchronize()
        np.testing.assert_array_equal(to_bits(y1[1]), orc.scatter(to_bits(x1)))
        np.testing.assert_array_equal(to_bits(y2[2]), orc.scatter(to_bits(x2)))
        assert torch.equal(z1.view(torch.int16), x1.view(torch.int16))
        assert torch.equal(z2.view(torch.int16), x2.view(torch.int16))
    finally:
        c1.close()
        c2.close()


@pytest.mark.parametrize("form", ["single", "two_stream", "dense"])
def test_graph_capture_replays(dev, form):
    """The step captured into a HIP graph: every replay, with fresh inputs written
    eagerly between replays, matches an eager run of the same step.  single: views of
    one fused QKV tensor, V in the fused launch; two_stream: V scattered on the comm
    stream; dense: separate Q/K/V tensors, the band kernel and then V by the relayout
    kernel, both inside the capture."""
    two_stream = form == "two_stream"
    P, B, S_l, H, D = 4, 1, 128, 8, 128
    qkv = synth.normal((P, B, S_l, 3, H, D), "bf16", 95, dev)
    o = synth.normal((P, B, P * S_l, H // P, D), "bf16", 96, dev)
    w_q, w_k = synth.norm_weight(D, "bf16", 97, dev), synth.norm_weight(D, "bf16", 98, dev)
    cos, sin = (t.to(dev) for t in rope_table_1d(P * S_l, D))
    if form == "dense":
        dense = [torch.empty((P, B, S_l, H, D), dtype=torch.bfloat16, device=dev) for _ in range(3)]
        q_in, k_in, v_in = dense
    else:
        q_in, k_in, v_in = qkv[:, :, :, 0], qkv[:, :, :, 1], qkv[:, :, :, 2]

    def refresh(seed):
        qkv.copy_(synth.normal(qkv.shape, "bf16", seed, dev))
        if form == "dense":
            for c in range(3):
                dense[c].copy_(qkv[:, :, :, c])

    refresh(95)
    ctx = UlyssesContext(P, device=0)
    try:
        def step(stream=None):
            if two_stream:
                ctx.scatter_qkv(v=v_in, stream=stream)
                outs = ctx.fused_qk_norm_rope_scatter(q_in, k_in, w_q, w_k, cos, sin, stream=stream)
                outs = (outs[0], outs[1], ctx.target("v", 0, torch.bfloat16, (B, P * S_l, H // P, D)))
            else:
                outs = ctx.fused_qk_norm_rope_scatter(q_in, k_in, w_q, w_k, cos, sin, v=v_in, stream=stream)
            ctx.wait(stream)
            z = ctx.gather_out(o, stream=stream)
            return list(outs) + [z]

        cap = torch.cuda.Stream()
        with torch.cuda.stream(cap):
            targets = step(cap)              # registers the targets and fills the event pools
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            step(cap)
        torch.cuda.synchronize()
        for rep in range(3):
            refresh(200 + rep)
            o.copy_(synth.normal(o.shape, "bf16", 300 + rep, dev))
            torch.cuda.synchronize()
            ref = [t.clone() for t in step()]        # eager, on the current stream
            torch.cuda.synchronize()
            for t in targets:
                t.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for t, r in zip(targets, ref):
                assert torch.equal(t.view(torch.int16), r.view(torch.int16)), "replay %d differs" % rep
    finally:
        torch.cuda.synchronize()
        ctx.close()


def _random_case(rng):
    P = int(rng.choice([1, 2, 3, 4, 6, 8]))
    D = int(rng.choice([32, 64, 128, 256]))
    Hl_q = int(rng.integers(1, 5))
    Hl_k = int(rng.integers(1, Hl_q + 1))
    B = int(rng.integers(1, 3))
    S_l = int(rng.integers(1, 97))
    dtype = str(rng.choice(["bf16", "f16"]))
    pad = int(rng.choice([0, 8, 64]))          # extra elements per token row: a strided source
    return P, B, S_l, P * Hl_q, P * Hl_k, D, dtype, pad


@pytest.mark.parametrize("seed", range(192))
def test_random_shapes_all_paths(dev, orc, seed):
    """Random world sizes, head counts, head dims, tails, dtypes and source row
    padding through the plain scatter, the fused norm + RoPE scatter (with V) and
    the gather, each against the oracle.  The fused call runs twice: on views of the
    one interleaved tensor (the token-tile kernel) and on dense copies (for D = 128
    and even S_l the band kernel with V by the relayout kernel); both give the same
    bits."""
    rng = np.random.default_rng(1000 + seed)
    P, B, S_l, Hq, Hk, D, dtype, pad = _random_case(rng)
    print("case P=%d B=%d S_l=%d Hq=%d Hk=%d D=%d %s pad=%d" % (P, B, S_l, Hq, Hk, D, dtype, pad), flush=True)
    row = (Hq + 2 * Hk) * D + pad
    base = synth.normal((P, B, S_l, row), dtype, 2000 + seed, dev)
    q = base[..., :Hq * D].unflatten(-1, (Hq, D))
    k = base[..., Hq * D:(Hq + Hk) * D].unflatten(-1, (Hk, D))
    v = base[..., (Hq + Hk) * D:(Hq + 2 * Hk) * D].unflatten(-1, (Hk, D))
    w_q, w_k = synth.norm_weight(D, dtype, 3000 + seed, dev), synth.norm_weight(D, dtype, 4000 + seed, dev)
    rows = P * S_l + int(rng.integers(0, 4))
    cos, sin = rope_table_1d(rows, D)
    ocos, osin = orc.rope_table_1d(rows, D)
    with UlyssesContext(P, device=0) as ctx:
        ys = ctx.scatter_qkv(q, k, v, tags=("pq", "pk", "pv"))
        yq, yk, yv = ctx.fused_qk_norm_rope_scatter(q, k, w_q, w_k, cos.to(dev), sin.to(dev), v=v)
        ctx.wait()
        z = ctx.gather_out(ys[0], tag="z")
        torch.cuda.synchronize()
        for x, y in zip((q, k, v), ys):
            np.testing.assert_array_equal(to_bits(y), orc.scatter(to_bits(x.contiguous())))
        np.testing.assert_array_equal(to_bits(yv), orc.scatter(to_bits(v.contiguous())))
        assert torch.equal(z.view(torch.int16), q.contiguous().view(torch.int16))
        for x, w, y, name in ((q, w_q, yq, "q"), (k, w_k, yk, "k")):
            ref = orc.fused_norm_rope_scatter(to_bits(x.contiguous()), dtype, to_bits(w), 1e-6, ocos, osin)
            assert_close16(y, ref, dtype, name)
        qd, kd, vd = (t.contiguous() for t in (q, k, v))
        yd = ctx.fused_qk_norm_rope_scatter(qd, kd, w_q, w_k, cos.to(dev), sin.to(dev), v=vd,
                                            tags=("dq", "dk", "dv"))
        ctx.wait()
        torch.cuda.synchronize()
        for a, b_, name in zip((yq, yk, yv), yd, "qkv"):
            assert torch.equal(a.view(torch.int16), b_.view(torch.int16)), name


def test_c_program_uses_the_abi_alone(dev):
    """A C program linked against libuly.so (built by __graft_entry__.build()) runs the
    scatter and gather through include/uly.h and checks them against the oracle."""
    import os
    import subprocess
    exe = os.path.join(os.path.dirname(__file__), "c_abi", "uly_c_smoke")
    assert os.path.exists(exe), "tests/c_abi/uly_c_smoke is not built; run __graft_entry__.build()"
    torch.cuda.synchronize()
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout + out.stderr


@pytest.mark.parametrize("P,B,S_l,Hq,Hkv,D,fused", [(4, 1, 4096, 24, 24, 128, True), (8, 2, 33, 32, 8, 128, False),
                                                    (1, 1, 17, 4, 4, 64, False), (2, 1, 1, 8, 8, 64, False)])
def test_copy_engine_route(dev, orc, P, B, S_l, Hq, Hkv, D, fused):
    """The copy-engine route moves the same bits as the kernel route."""
    if fused:
        qkv = synth.normal((P, B, S_l, 3, Hq, D), "bf16", 110, dev)
        q, k, v = qkv[:, :, :, 0], qkv[:, :, :, 1], qkv[:, :, :, 2]
    else:
        q, k, v = contiguous_qkv(P, B, S_l, Hq, D, "bf16", 111, dev, Hkv)
    with UlyssesContext(P, device=0) as ctx:
        ctx.set_route("copy_engine")
        ys = ctx.scatter_qkv(q, k, v)
        ctx.wait()
        torch.cuda.synchronize()
        for x, y in zip((q, k, v), ys):
            np.testing.assert_array_equal(to_bits(y), orc.scatter(to_bits(x.contiguous())))
        ctx.set_route("kernel")
        ys2 = ctx.scatter_qkv(q, k, v, tags=("q2", "k2", "v2"))
        ctx.wait()
        torch.cuda.synchronize()
        for y, y2 in zip(ys, ys2):
            assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
        # the caller route: the same kernel on the caller's stream, no events; a
        # consumer later on that stream sees the result without any wait
        ctx.set_route("caller")
        before = ctx.stats()["launches"]
        ys3 = ctx.scatter_qkv(q, k, v, tags=("q3", "k3", "v3"))
        sums = [y.float().sum() for y in ys3]         # consumer kernels on the same stream
        ctx.wait()
        torch.cuda.synchronize()
        assert ctx.stats()["launches"] == before + 1
        for y, y3, sm in zip(ys, ys3, sums):
            assert torch.equal(y.view(torch.int16), y3.view(torch.int16))
            assert torch.equal(sm, y.float().sum())


# ---------------------------------------------------------------------------
# 1-byte payloads, the packed receive layout, the destination-major exchange
# ---------------------------------------------------------------------------
BYTE_DTYPES = [torch.uint8, torch.int8, torch.float8_e4m3fn, torch.float8_e5m2]


@pytest.mark.parametrize("P,B,S_l,Hq,Hkv,D", [(4, 1, 33, 8, 8, 128), (8, 2, 5, 16, 8, 16), (2, 1, 200, 4, 2, 64),
                                              (4, 1, 4096, 24, 24, 128)])
def test_byte_payloads_bit_exact(dev, orc, P, B, S_l, Hq, Hkv, D):
    """flashinfer UlyssesCommunicator PR, 'What': fp8 / int8 move as opaque bytes,
    byte-exact in both directions."""
    for i, dt in enumerate(BYTE_DTYPES):
        q = synth.random_bytes((P, B, S_l, Hq, D), 40 + i, dt, dev)
        k = synth.random_bytes((P, B, S_l, Hkv, D), 50 + i, dt, dev)
        v = synth.random_bytes((P, B, S_l, Hkv, D), 60 + i, dt, dev)
        with UlyssesContext(P, device=0) as ctx:
            ys = ctx.scatter_qkv(q, k, v)
            ctx.wait()
            torch.cuda.synchronize()
            for x, y in zip((q, k, v), ys):
                assert y.dtype == dt
                np.testing.assert_array_equal(to_bits(y), orc.scatter(to_bits(x)))
            o = synth.random_bytes((P, B, P * S_l, Hq // P, D), 70 + i, dt, dev)
            z = ctx.gather_out(o)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(to_bits(z), orc.gather(to_bits(o)))


@pytest.mark.parametrize("P,B,S_l,H,D,dtype,fused", [(4, 1, 200, 24, 128, "bf16", True), (2, 1, 128, 8, 64, "f16", False),
                                                     (2, 2, 37, 6, 128, "bf16", False), (4, 1, 29, 8, 32, "bf16", True),
                                                     (2, 1, 50, 4, 256, "f16", False),
                                                     (4, 1, 4096, 24, 128, "bf16", True)])   # the video-DiT block
def test_packed_receive_layout(dev, orc, P, B, S_l, H, D, dtype, fused):
    """flashinfer PR #6332, 'Description' (Layouts): the fused [B, S, Hl, 3D] payload
    holds q, k and v side by side in every head row."""
    if fused:
        qkv = synth.normal((P, B, S_l, 3, H, D), dtype, 31, dev)
        q, k, v = qkv[:, :, :, 0], qkv[:, :, :, 1], qkv[:, :, :, 2]
    else:
        q, k, v = contiguous_qkv(P, B, S_l, H, D, dtype, 31, dev)
    w_q = synth.norm_weight(D, dtype, 3, dev)
    w_k = synth.norm_weight(D, dtype, 4, dev)
    rows = P * S_l
    cos, sin = rope_table_1d(rows, D)
    ocos, osin = orc.rope_table_1d(rows, D)
    with UlyssesContext(P, device=0) as ctx:
        y = ctx.fused_qkv_norm_rope_scatter_packed(q, k, v, w_q, w_k, cos.to(dev), sin.to(dev))
        assert tuple(y.shape) == (P, B, P * S_l, H // P, 3 * D)
        yq, yk, yv = ctx.fused_qk_norm_rope_scatter(q, k, w_q, w_k, cos.to(dev), sin.to(dev), v=v)
        ctx.wait()
        torch.cuda.synchronize()
        # the same arithmetic as the three-target layout, bit for bit
        assert torch.equal(y.view(torch.int16), torch.cat([yq, yk, yv], dim=-1).view(torch.int16))
        ref_q = orc.fused_norm_rope_scatter(to_bits(q), dtype, to_bits(w_q), 1e-6, ocos, osin)
        ref_k = orc.fused_norm_rope_scatter(to_bits(k), dtype, to_bits(w_k), 1e-6, ocos, osin)
        assert_close16(y[..., :D], ref_q, dtype, "q")
        assert_close16(y[..., D:2 * D], ref_k, dtype, "k")
        np.testing.assert_array_equal(to_bits(y[..., 2 * D:]), orc.scatter(to_bits(v)))
        # a second call reuses the cached packed target
        y2 = ctx.fused_qkv_norm_rope_scatter_packed(q, k, v, w_q, w_k, cos.to(dev), sin.to(dev))
        torch.cuda.synchronize()
        assert y2.data_ptr() == y.data_ptr()


@pytest.mark.parametrize("P,chunk", [(1, 4096), (2, 16), (4, 1 << 20), (8, 48), (4, 0)])
def test_exchange_chunks_bit_exact(dev, orc, P, chunk):
    """flashinfer UlyssesCommunicator PR, 'What' (Transforms): y[q, r] = x[r, q]."""
    x = synth.random_bytes((P, P, chunk), 80 + P, torch.uint8, dev)
    with UlyssesContext(P, device=0) as ctx:
        y = ctx.exchange_chunks(x)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y.cpu().numpy(), orc.exchange_chunks(x.cpu().numpy()))
        # bf16 payload of a pack that laid rows out destination-major
        if chunk and chunk % 2 == 0:
            xb = synth.normal((P, P, chunk // 2), "bf16", 90, dev)
            yb = ctx.exchange_chunks(xb)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(to_bits(yb), orc.exchange_chunks(to_bits(xb)))


# ---------------------------------------------------------------------------
# QKV projection (MFMA) with the norm + RoPE + scatter epilogue
# ---------------------------------------------------------------------------
def _proj_inputs(P, B, S_l, hidden, Hq, Hkv, dtype, seed, dev, D=128):
    x = synth.normal((P, B, S_l, hidden), dtype, seed, dev)
    w = synth.normal(((Hq + 2 * Hkv) * D, hidden), dtype, seed + 1, dev, std=hidden ** -0.5)
    wq = synth.norm_weight(D, dtype, seed + 2, dev)
    wk = synth.norm_weight(D, dtype, seed + 3, dev)
    return x, w, wq, wk


PROJ_SMALL = [
    # P, B, S_l, hidden, Hq, Hkv, dtype
    (2, 1, 40, 256, 4, 2, "bf16"),       # one ragged token tile
    (4, 1, 200, 512, 8, 4, "bf16"),      # S_local = 200 tail, tiles cross rank boundaries
    (1, 2, 33, 128, 2, 1, "f16"),
    (4, 2, 64, 384, 4, 4, "bf16"),       # B = 2, six K stages
    (8, 1, 32, 1024, 8, 8, "bf16"),
    (2, 1, 300, 192, 2, 2, "f16"),       # three K stages
    (1, 1, 70, 64, 3, 1, "bf16"),        # one K stage, five heads (last head block half empty)
]


@pytest.mark.parametrize("ring", [0, 3])
@pytest.mark.parametrize("P,B,S_l,hidden,Hq,Hkv,dtype", PROJ_SMALL)
def test_projection_small(dev, orc, P, B, S_l, hidden, Hq, Hkv, dtype, ring):
    """flashinfer PR #6332, 'Description' / 'Assumptions': projection -> QK-norm -> RoPE ->
    exchange, against the double-precision oracle element by element.  ring=3 forces the
    kernel with the three-stage token-row ring (chosen by itself only for operands beyond
    the Infinity Cache)."""
    x, w, wq, wk = _proj_inputs(P, B, S_l, hidden, Hq, Hkv, dtype, 60, dev)
    rows = P * S_l + 3
    cos, sin = rope_table_1d(rows, 128)
    ocos, osin = orc.rope_table_1d(rows, 128)
    with UlyssesContext(P, device=0) as ctx:
        ctx.debug_proj_ring(ring)
        yq, yk, yv = ctx.fused_qkv_proj_norm_rope_scatter(x, w, Hq, Hkv, wq, wk, cos.to(dev), sin.to(dev))
        ctx.wait()
        torch.cuda.synchronize()
        rq, rk, rv = orc.qkv_proj_norm_rope_scatter(to_bits(x), dtype, to_bits(w), Hq, Hkv, to_bits(wq),
                                                    to_bits(wk), 1e-6, ocos, osin)
        # fp32 evaluation bounds per token row, moved to the head-sharded layout like the results
        pos = np.broadcast_to(np.arange(P)[:, None, None] * S_l + np.arange(S_l)[None, None, :],
                              (P, B, S_l)).reshape(-1)
        E = _proj_row_bounds(orc, to_bits(x).reshape(-1, hidden), dtype, w, wq, wk, Hq, Hkv, ocos, osin, pos)
        for y, r_, e, H, name in ((yq, rq, E[0], Hq, "q"), (yk, rk, E[1], Hkv, "k"), (yv, rv, E[2], Hkv, "v")):
            assert_close16(y, r_, dtype, name, E=orc.scatter(e.reshape(P, B, S_l, H, 128)))
        # deterministic: a second call gives the same bits
        yq2, _, yv2 = ctx.fused_qkv_proj_norm_rope_scatter(x, w, Hq, Hkv, wq, wk, cos.to(dev), sin.to(dev),
                                                           tags=("q2", "k2", "v2"))
        torch.cuda.synchronize()
        assert torch.equal(yq2.view(torch.int16), yq.view(torch.int16))
        assert torch.equal(yv2.view(torch.int16), yv.view(torch.int16))


def _proj_row_bounds(orc, x_rows_bits, dtype, w, wq, wk, Hq, Hkv, cos, sin, pos):
    """The derived fp32 evaluation bound E of every output element of token rows
    x_rows_bits[n, hidden] (token-major [n, H, D] per output)."""
    exact = orc.qkv_proj_norm_rope_rows(x_rows_bits, dtype, to_bits(w), Hq, Hkv, 128, to_bits(wq), to_bits(wk),
                                        1e-6, cos, sin, pos)
    return proj_bounds(orc.widen(x_rows_bits, dtype), orc.widen(to_bits(w), dtype), Hq, Hkv, 128,
                       orc.widen(to_bits(wq), dtype), orc.widen(to_bits(wk), dtype), 1e-6, cos[pos], sin[pos],
                       exact)


def _check_proj_sampled(orc, x, w, wq, wk, ys, Hq, Hkv, dtype, cos, sin, windows):
    """Oracle rows for sampled tokens of every rank, compared at their destinations."""
    P, B, S_l, hidden = x.shape
    toks = [(r, b, s) for r in range(P) for b in range(B) for (s0, n) in windows for s in range(s0, s0 + n)]
    idx = torch.tensor([(r * B + b) * S_l + s for r, b, s in toks])
    x_rows = to_bits(x.reshape(-1, hidden)[idx.to(x.device)])
    pos = np.array([r * S_l + s for r, b, s in toks])
    ref = orc.qkv_proj_norm_rope_rows(x_rows, dtype, to_bits(w), Hq, Hkv, 128, to_bits(wq), to_bits(wk), 1e-6,
                                      cos, sin, pos)
    E = _proj_row_bounds(orc, x_rows, dtype, w, wq, wk, Hq, Hkv, cos, sin, pos)
    for y, r_, e, H in zip(ys, ref, E, (Hq, Hkv, Hkv)):
        Hl = H // P
        h = torch.arange(H)
        got = torch.stack([y[h // Hl, b, r * S_l + s, h % Hl] for r, b, s in toks])   # [n, H, D]
        assert_close16(got, r_, dtype, "sampled", E=e)


def test_projection_video_dit_full(dev, orc):
    """Video-DiT block (P=4, S=16384, H=24, D=128, hidden 3072, bf16) at full size, the
    launch the benchmark times; oracle rows on sampled token windows of every rank."""
    P, B, S_l, H, hidden = 4, 1, 4096, 24, 3072
    x, w, wq, wk = _proj_inputs(P, B, S_l, hidden, H, H, "bf16", 70, dev)
    cos, sin = rope_table_1d(P * S_l, 128)
    ocos, osin = orc.rope_table_1d(P * S_l, 128)
    with UlyssesContext(P, device=0) as ctx:
        ys = ctx.fused_qkv_proj_norm_rope_scatter(x, w, H, H, wq, wk, cos.to(dev), sin.to(dev))
        ctx.wait()
        torch.cuda.synchronize()
        _check_proj_sampled(orc, x, w, wq, wk, ys, H, H, "bf16", ocos, osin, [(0, 3), (2047, 2), (4093, 3)])


def test_projection_gqa_full(dev, orc):
    """GQA (P=8, B=2, S_l=8192, Hq=32, Hkv=8, hidden 4096, bf16) at full size, sampled."""
    P, B, S_l, Hq, Hkv, hidden = 8, 2, 8192, 32, 8, 4096
    x, w, wq, wk = _proj_inputs(P, B, S_l, hidden, Hq, Hkv, "bf16", 80, dev)
    cos, sin = rope_table_1d(P * S_l, 128)
    ocos, osin = orc.rope_table_1d(P * S_l, 128)
    with UlyssesContext(P, device=0) as ctx:
        ys = ctx.fused_qkv_proj_norm_rope_scatter(x, w, Hq, Hkv, wq, wk, cos.to(dev), sin.to(dev))
        ctx.wait()
        torch.cuda.synchronize()
        _check_proj_sampled(orc, x, w, wq, wk, ys, Hq, Hkv, "bf16", ocos, osin, [(0, 1), (8191, 1)])


def test_projection_wan_full(dev, orc):
    """Wan-style long sequence (P=4, S=75600 padded to 75776, H=40, hidden 5120, bf16, 3-D
    RoPE with pad rows) at full size, sampled; its 776 MB activations take the three-stage
    token-row ring."""
    from sequence_attention_ulysses_amd import rope_table_3d
    P, B, S_l, H, hidden = 4, 1, 18944, 40, 5120
    S_real, Hh, Ww = 75600, 60, 60
    x, w, wq, wk = _proj_inputs(P, B, S_l, hidden, H, H, "bf16", 90, dev)
    cos, sin = rope_table_3d(P * S_l, 128, Hh, Ww, real_rows=S_real)
    ocos, osin = orc.rope_table_3d(P * S_l, 128, Hh, Ww, real_rows=S_real)
    with UlyssesContext(P, device=0) as ctx:
        ys = ctx.fused_qkv_proj_norm_rope_scatter(x, w, H, H, wq, wk, cos.to(dev), sin.to(dev))
        ctx.wait()
        torch.cuda.synchronize()
        # on rank 3 the window at 18766 holds positions 75598..75601: two real rows, two pad rows
        _check_proj_sampled(orc, x, w, wq, wk, ys, H, H, "bf16", ocos, osin, [(0, 1), (9000, 1), (18766, 4)])
