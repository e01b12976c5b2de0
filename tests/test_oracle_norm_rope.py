"""Pins for the oracle's RMSNorm + interleaved RoPE and its rotary tables (CPU only).

flashinfer PR #6332, "Assumptions", fixes the operator: per-head RMSNorm with
eps 1e-6 and one [head_dim] weight, then interleaved (pairwise) RoPE from a
per-token fp32 cos/sin table, QK-norm before RoPE.  The checks below pin it
with a hand-worked fixture, closed forms of RMSNorm, complex multiplication
(numpy) for the rotation, and rotary invariants.
"""
import json
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
EPS = 1e-6


def _identity_table(rows, half):
    return np.ones((rows, half), np.float32), np.zeros((rows, half), np.float32)


def test_worked_fixture(orc):
    g = json.load(open(os.path.join(GOLDEN, "norm_rope_worked.json")))
    for case in g["cases"]:
        c = np.array([case["cos"]], np.float32)
        s = np.array([case["sin"]], np.float32)
        y = orc.norm_rope_rows(np.array([case["x"]], float), np.array(case["w"], float), g["eps"],
                               c, s, np.array([0]))
        np.testing.assert_allclose(y[0], case["expected"], rtol=0, atol=1e-12)


def test_rmsnorm_constant_row_closed_form(orc):
    """x = c everywhere: n_i = c / sqrt(c^2 + eps) * w_i (eps matters at small c)."""
    D = 16
    w = np.linspace(0.5, 2.0, D)     # asymmetric, catches a reversed weight index
    cos, sin = _identity_table(1, D // 2)
    for c in (1e-3, -0.25, 3.0):
        y = orc.norm_rope_rows(np.full((1, D), c), w, EPS, cos, sin, np.array([0]))
        np.testing.assert_allclose(y[0], c / math.sqrt(c * c + EPS) * w, rtol=1e-13)
    # c = 1e-3: eps doubles the denominator -> 1/sqrt(2)
    y = orc.norm_rope_rows(np.full((1, 2), 1e-3), np.ones(2), EPS, *_identity_table(1, 1), np.array([0]))
    np.testing.assert_allclose(y[0], [2 ** -0.5] * 2, rtol=1e-12)


def test_rmsnorm_zero_row_and_spike(orc):
    D = 8
    cos, sin = _identity_table(1, D // 2)
    y = orc.norm_rope_rows(np.zeros((1, D)), np.ones(D), EPS, cos, sin, np.array([0]))
    assert (y == 0).all()
    # one nonzero entry a at index k: ms = a^2 / D, n_k = a / sqrt(a^2/D + eps) * w_k
    x = np.zeros((1, D)); x[0, 5] = 2.0
    w = np.arange(1, D + 1, dtype=float)
    y = orc.norm_rope_rows(x, w, EPS, cos, sin, np.array([0]))
    want = np.zeros(D); want[5] = 2.0 / math.sqrt(4.0 / D + EPS) * w[5]
    np.testing.assert_allclose(y[0], want, rtol=1e-13, atol=0)


def test_rmsnorm_unit_weight_mean_square(orc):
    """With w = 1, mean(n^2) = ms / (ms + eps) exactly; scaling x leaves n nearly unchanged."""
    rng = np.random.default_rng(0)
    D = 128
    x = rng.standard_normal((64, D))
    cos, sin = _identity_table(1, D // 2)
    pos = np.zeros(64, np.int64)
    n = orc.norm_rope_rows(x, np.ones(D), EPS, cos, sin, pos)
    ms = (x ** 2).mean(axis=1)
    np.testing.assert_allclose((n ** 2).mean(axis=1), ms / (ms + EPS), rtol=1e-12)
    n7 = orc.norm_rope_rows(7.0 * x, np.ones(D), EPS, cos, sin, pos)
    np.testing.assert_allclose(n7, n, rtol=1e-5, atol=1e-6)


def _complex_reference(n, cos, sin):
    """Rotation of pair (n_2j, n_2j+1) as the complex product (n_2j + i n_2j+1) e^{i a_j}."""
    z = n[..., 0::2] + 1j * n[..., 1::2]
    z = z * (cos.astype(np.float64) + 1j * sin.astype(np.float64))
    out = np.empty_like(n)
    out[..., 0::2] = z.real
    out[..., 1::2] = z.imag
    return out


def test_rotation_is_complex_multiplication(orc):
    rng = np.random.default_rng(1)
    D, rows = 128, 40
    x = rng.standard_normal((rows, D))
    w = 1.0 + 0.1 * rng.standard_normal(D)
    cos, sin = orc.rope_table_1d(1000, D)
    pos = rng.integers(0, 1000, rows)
    y = orc.norm_rope_rows(x, w, EPS, cos, sin, pos)
    n = orc.norm_rope_rows(x, w, EPS, *_identity_table(1, D // 2), np.zeros(rows, np.int64))
    np.testing.assert_allclose(y, _complex_reference(n, cos[pos], sin[pos]), rtol=0, atol=1e-12)


def test_rotation_preserves_pair_norms_and_inverts(orc):
    rng = np.random.default_rng(2)
    D, rows = 64, 32
    x = rng.standard_normal((rows, D))
    w = 1.0 + 0.1 * rng.standard_normal(D)
    cos, sin = orc.rope_table_1d(4096, D)
    pos = rng.integers(0, 4096, rows)
    ident = _identity_table(1, D // 2)
    n = orc.norm_rope_rows(x, w, EPS, *ident, np.zeros(rows, np.int64))
    y = orc.norm_rope_rows(x, w, EPS, cos, sin, pos)
    pair = lambda a: a[:, 0::2] ** 2 + a[:, 1::2] ** 2
    # fp32 table: cos^2 + sin^2 = 1 to ~1e-7, so norms agree to that order
    np.testing.assert_allclose(pair(y), pair(n), rtol=3e-7, atol=1e-12)
    # rotating back with -sin (the inverse rotation) recovers n, up to the fp32
    # table's unit-modulus error
    back = _complex_reference(y, cos[pos], -sin[pos])
    np.testing.assert_allclose(back, n, rtol=0, atol=1e-6)


def test_position_zero_is_identity(orc):
    rng = np.random.default_rng(3)
    D = 128
    x = rng.standard_normal((4, D))
    w = 1.0 + 0.1 * rng.standard_normal(D)
    cos, sin = orc.rope_table_1d(8, D)
    assert (cos[0] == 1).all() and (sin[0] == 0).all()
    y0 = orc.norm_rope_rows(x, w, EPS, cos, sin, np.zeros(4, np.int64))
    n = orc.norm_rope_rows(x, w, EPS, *_identity_table(1, D // 2), np.zeros(4, np.int64))
    np.testing.assert_array_equal(y0, n)


def test_relative_position_invariance(orc):
    """<R_m q, R_n k> depends only on n - m (1-D table)."""
    rng = np.random.default_rng(4)
    D = 64
    q = rng.standard_normal((1, D))
    k = rng.standard_normal((1, D))
    ones = np.ones(D)
    cos, sin = orc.rope_table_1d(300, D)
    dots = []
    for m, n in [(3, 10), (50, 57), (200, 207)]:
        rq = orc.norm_rope_rows(q, ones, EPS, cos, sin, np.array([m]))
        rk = orc.norm_rope_rows(k, ones, EPS, cos, sin, np.array([n]))
        dots.append(float((rq * rk).sum()))
    np.testing.assert_allclose(dots, dots[0], rtol=1e-5)


def test_table_1d_closed_forms(orc):
    D = 128
    cos, sin = orc.rope_table_1d(5, D)
    np.testing.assert_allclose(cos ** 2 + sin ** 2, 1.0, atol=2e-7)
    # pair 0 has unit frequency: angle = g
    for g in range(5):
        assert cos[g, 0] == np.float32(math.cos(g)) and sin[g, 0] == np.float32(math.sin(g))
    # last pair: frequency theta^(-(D-2)/D)
    f = 1e4 ** (-(D - 2) / D)
    assert sin[3, D // 2 - 1] == np.float32(math.sin(3 * f))
    # padding rows are the identity rotation
    c2, s2 = orc.rope_table_1d(6, D, real_rows=4)
    assert (c2[4:] == 1).all() and (s2[4:] == 0).all()
    np.testing.assert_array_equal(c2[:4], orc.rope_table_1d(4, D)[0])


def test_table_3d_reduces_to_1d_on_time_axis(orc):
    """Tokens with h = w = 0 rotate the t band like a 1-D table of width 44; the
    h and w bands are the identity there."""
    D, Hh, Ww = 128, 60, 60
    rows = 3 * Hh * Ww
    cos, sin = orc.rope_table_3d(rows, D, Hh, Ww)
    c1, s1 = orc.rope_table_1d(3, 44)
    for t in range(3):
        g = t * Hh * Ww
        np.testing.assert_array_equal(cos[g, :22], c1[t])
        np.testing.assert_array_equal(sin[g, :22], s1[t])
        assert (cos[g, 22:] == 1).all() and (sin[g, 22:] == 0).all()
    # token (t=0, h=5, w=0) rotates only the h band, like a 1-D table of width 42 at position 5
    c42, s42 = orc.rope_table_1d(6, 42)
    g = 5 * Ww
    np.testing.assert_array_equal(cos[g, 22:43], c42[5])
    np.testing.assert_array_equal(sin[g, 22:43], s42[5])
    assert (cos[g, :22] == 1).all() and (cos[g, 43:] == 1).all()
    # token (0, 0, w=7): only the w band
    g = 7
    np.testing.assert_array_equal(sin[g, 43:], orc.rope_table_1d(8, 42)[1][7])
    assert (sin[g, :43] == 0).all()
    np.testing.assert_allclose(cos ** 2 + sin ** 2, 1.0, atol=2e-7)


def test_sharded_positions_equal_unsharded_sequence(orc):
    """QK-norm -> RoPE -> exchange equals QK-norm -> RoPE on the whole sequence
    (positions 0..S-1) followed by taking each rank's head band: pins the global
    position r*S_l + s and the head band of the exchange."""
    rng = np.random.default_rng(5)
    P, B, S_l, H, D = 4, 2, 6, 8, 16
    x = rng.standard_normal((P, B, S_l, H, D)).astype(np.float32)
    bits = x.view(np.uint32) >> 16               # bf16 truncation: any 16-bit pattern will do
    bits = bits.astype(np.uint16)
    w_bits = (np.float32(1.1) * np.ones(D, np.float32)).view(np.uint32) >> 16
    w_bits = w_bits.astype(np.uint16)
    cos, sin = orc.rope_table_1d(P * S_l, D)
    y = orc.fused_norm_rope_scatter(bits, "bf16", w_bits, EPS, cos, sin)
    full = np.concatenate([bits[r] for r in range(P)], axis=1)          # [B, S, H, D]
    x64 = orc.widen(full, "bf16").reshape(-1, D)
    pos = np.broadcast_to(np.arange(P * S_l).reshape(1, -1, 1), (B, P * S_l, H)).reshape(-1)
    ref = orc.norm_rope_rows(x64, orc.widen(w_bits, "bf16"), EPS, cos, sin, pos).reshape(B, P * S_l, H, D)
    Hl = H // P
    for q in range(P):
        np.testing.assert_array_equal(y[q], ref[:, :, q * Hl:(q + 1) * Hl])


def test_widen_exact(orc):
    vals = np.array([1.0, -2.5, 3.140625, 65504.0, 2 ** -24], np.float16)
    np.testing.assert_array_equal(orc.widen(vals.view(np.uint16), "f16"), vals.astype(np.float64))
    b = np.array([0x3F80, 0xC020, 0x0001], np.uint16)        # 1.0, -2.5, smallest subnormal
    np.testing.assert_array_equal(orc.widen(b, "bf16"), [1.0, -2.5, 2.0 ** -133])
