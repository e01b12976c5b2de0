"""The element-wise checker the GPU parity tests use, checked on the CPU.

A checker that lets a wrong rounding through proves nothing.  These tests
build 16-bit results on the CPU from the oracle's exact values and check
that the checker
  * accepts a correct single rounding of an fp32 evaluation (numpy float32
    arithmetic standing in for the kernel: its error must sit inside the
    derived fp32 bound),
  * rejects truncation, the pages' bf16 reference arithmetic with its
    intermediate roundings (flashinfer PR #6332, "Tests": round before the
    scale and again at the output), a projection rounded before the norm,
    and single elements one ulp off,
  * classifies, rather than rejects, correctly rounded elements at |y| >= 8,
    where half an ulp alone exceeds the stated tolerance ("Tolerance").
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import oracle
from tests.tolerance import Check16, ToleranceError, check16, norm_rope_eval_bound, proj_bounds, round16, ulp16

D = 128


def _rows(n, dtype, seed, spike=False):
    rng = np.random.default_rng(seed)
    x = round16(rng.standard_normal((n, D)), dtype)
    if spike:                       # one dominant element per row: |n_0| ~ sqrt(D) |w_0|
        x[:, 1:] *= 1e-3
        x = round16(x, dtype)
    w = round16(1.0 + 0.1 * rng.standard_normal(D), dtype)
    pos = rng.integers(0, 4096, n)
    cos, sin = oracle.rope_table_1d(4096, D)
    return x, w, pos, cos, sin


def _fp32_norm_rope(x, w, eps, cos, sin, pos):
    """The producer's arithmetic in numpy float32 (sum of squares, rsqrt, two products,
    the rotation), each operation rounded to fp32."""
    f = np.float32
    x32, w32 = x.astype(f), w.astype(f)
    ss = (x32 * x32).sum(axis=-1, dtype=f, keepdims=True)
    inv = (f(1) / np.sqrt(ss * f(1.0 / x.shape[-1]) + f(eps))).astype(f)
    n = (x32 * inv) * w32
    c, s = cos[pos], sin[pos]
    y = np.empty_like(n)
    y[:, 0::2] = n[:, 0::2] * c - n[:, 1::2] * s
    y[:, 1::2] = n[:, 0::2] * s + n[:, 1::2] * c
    return y.astype(np.float64)


def _rotate(n, cos, sin, pos):
    c, s = cos[pos].astype(np.float64), sin[pos].astype(np.float64)
    y = np.empty_like(n)
    y[:, 0::2] = n[:, 0::2] * c - n[:, 1::2] * s
    y[:, 1::2] = n[:, 0::2] * s + n[:, 1::2] * c
    return y


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_correct_single_rounding_passes(dtype):
    x, w, pos, cos, sin = _rows(2048, dtype, 1)
    exact = oracle.norm_rope_rows(x, w, 1e-6, cos, sin, pos)
    # the fp32 evaluation stays inside the derived bound (2) ...
    y32 = _fp32_norm_rope(x, w, 1e-6, cos, sin, pos)
    assert (np.abs(y32 - exact) <= norm_rope_eval_bound(exact)).all()
    # ... and its single rounding passes the checker, statistics included
    out = check16(round16(y32, dtype), exact, dtype, "rne")
    assert out["classified"] == 0
    assert abs(out["bias_ulp"]) < 0.01 and 0.28 < out["rms_ulp"] < 0.30
    # so does the rounding of the exact value itself
    check16(round16(exact, dtype), exact, dtype, "rne exact")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_truncation_fails(dtype):
    x, w, pos, cos, sin = _rows(2048, dtype, 2)
    exact = oracle.norm_rope_rows(x, w, 1e-6, cos, sin, pos)
    with pytest.raises(ToleranceError):
        check16(round16(exact, dtype, "trunc"), exact, dtype, "trunc")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_pages_reference_double_rounding_fails(dtype):
    """Round the normalised row, then the weighted row, then the rotated output:
    three roundings where the operator here rounds once."""
    x, w, pos, cos, sin = _rows(2048, dtype, 3)
    exact = oracle.norm_rope_rows(x, w, 1e-6, cos, sin, pos)
    ones = np.ones(D)
    ident_c, ident_s = np.ones_like(cos), np.zeros_like(sin)
    normed = oracle.norm_rope_rows(x, ones, 1e-6, ident_c, ident_s, pos)     # x * rsqrt(ms + eps)
    n = round16(round16(normed, dtype) * w, dtype)
    y = round16(_rotate(n, cos, sin, pos), dtype)
    with pytest.raises(ToleranceError):
        check16(y, exact, dtype, "double")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_double_rounding_within_the_stated_tolerance_fails(dtype):
    """Rounding through a format two bits wider first errs by up to 5/8 ulp: inside the
    stated max-abs tolerance everywhere below |y| = 4, so only the rounding model sees it."""
    x, w, pos, cos, sin = _rows(2048, dtype, 8)
    exact = oracle.norm_rope_rows(x, w, 1e-6, cos, sin, pos)
    wide = np.round(exact / (ulp16(np.abs(exact), dtype) / 4)) * (ulp16(np.abs(exact), dtype) / 4)
    y = round16(wide, dtype)
    small = np.abs(exact) < 4
    assert (np.abs(y - exact)[small] <= {"bf16": 2e-2, "f16": 2e-3}[dtype]).all()
    assert (y != round16(exact, dtype)).any()
    with pytest.raises(ToleranceError):
        check16(y, exact, dtype, "double via a wider format", stats=False)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_single_element_one_ulp_off_fails(dtype):
    x, w, pos, cos, sin = _rows(64, dtype, 4)
    exact = oracle.norm_rope_rows(x, w, 1e-6, cos, sin, pos)
    y = round16(exact, dtype)
    i = np.unravel_index(np.argmax(np.abs(exact) < 1.0), exact.shape)
    y[i] += np.sign(exact[i] - y[i] or 1.0) * -ulp16(np.abs(y[i]), dtype)    # one ulp further away
    with pytest.raises(ToleranceError):
        check16(y, exact, dtype, "one ulp", stats=False)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_large_values_are_classified_not_rejected(dtype):
    x, w, pos, cos, sin = _rows(256, dtype, 5, spike=True)
    exact = oracle.norm_rope_rows(x, w, 1e-6, cos, sin, pos)
    assert np.abs(exact).max() >= 8
    y = round16(_fp32_norm_rope(x, w, 1e-6, cos, sin, pos), dtype)
    out = check16(y, exact, dtype, "spike", stats=False)
    big = np.abs(exact) >= 8
    if (np.abs(y - exact)[big] > {"bf16": 2e-2, "f16": 2e-3}[dtype]).any():
        assert out["classified"] > 0
    # a one-ulp miss there is still a miss
    i = np.unravel_index(np.argmax(np.abs(exact)), exact.shape)
    r = round16(exact[i], dtype)
    y[i] = r + (np.sign(r - exact[i]) or 1.0) * ulp16(np.abs(r), dtype)
    with pytest.raises(ToleranceError):
        check16(y, exact, dtype, "spike one ulp", stats=False)


def test_nan_fails():
    x, w, pos, cos, sin = _rows(16, "bf16", 6)
    exact = oracle.norm_rope_rows(x, w, 1e-6, cos, sin, pos)
    y = round16(exact, "bf16")
    y[3, 7] = np.nan
    with pytest.raises(ToleranceError):
        check16(y, exact, "bf16", "nan", stats=False)


def _proj_case(dtype, n=512, K=512, Hq=2, Hkv=1, seed=7):
    rng = np.random.default_rng(seed)
    x = round16(rng.standard_normal((n, K)), dtype)
    W = round16(rng.standard_normal(((Hq + 2 * Hkv) * D, K)) * K ** -0.5, dtype)
    wq = round16(1.0 + 0.1 * rng.standard_normal(D), dtype)
    wk = round16(1.0 + 0.1 * rng.standard_normal(D), dtype)
    pos = rng.integers(0, 4096, n)
    cos, sin = oracle.rope_table_1d(4096, D)
    return x, W, wq, wk, pos, cos, sin


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_projection_fp32_passes_and_early_rounding_fails(dtype):
    Hq, Hkv = 2, 1
    x, W, wq, wk, pos, cos, sin = _proj_case(dtype)
    xb = _bits(x, dtype)
    Wb = _bits(W, dtype)
    exact = oracle.qkv_proj_norm_rope_rows(xb, dtype, Wb, Hq, Hkv, D, _bits(wq, dtype), _bits(wk, dtype), 1e-6,
                                           cos, sin, pos)
    E = proj_bounds(x, W, Hq, Hkv, D, wq, wk, 1e-6, cos[pos], sin[pos], exact)
    # fp32 projection (numpy float32 sums of exact products), fp32 norm + rotation, one rounding
    pre32 = (x.astype(np.float32) @ W.astype(np.float32).T).astype(np.float32)
    q32 = pre32[:, :Hq * D].reshape(-1, D)
    k32 = pre32[:, Hq * D:(Hq + Hkv) * D].reshape(-1, D)
    v32 = pre32[:, (Hq + Hkv) * D:].astype(np.float64).reshape(len(x), Hkv, D)
    yq = _fp32_norm_rope(q32.astype(np.float64), wq, 1e-6, cos, sin, np.repeat(pos, Hq)).reshape(len(x), Hq, D)
    yk = _fp32_norm_rope(k32.astype(np.float64), wk, 1e-6, cos, sin, np.repeat(pos, Hkv)).reshape(len(x), Hkv, D)
    for got, ref, e, name in zip((yq, yk, v32), exact, E, "qkv"):
        check16(round16(got, dtype), ref, dtype, "proj " + name, E=e)
    # the projection rounded to 16 bits before the norm: a second rounding
    q16 = round16(q32.astype(np.float64), dtype)
    yq2 = _fp32_norm_rope(q16, wq, 1e-6, cos, sin, np.repeat(pos, Hq)).reshape(len(x), Hq, D)
    with pytest.raises(ToleranceError):
        check16(round16(yq2, dtype), exact[0], dtype, "proj q early", E=E[0])
    # truncated V
    with pytest.raises(ToleranceError):
        check16(round16(v32, dtype, "trunc"), exact[2], dtype, "proj v trunc", E=E[2])


def _bits(v: np.ndarray, dtype: str) -> np.ndarray:
    """16-bit storage words of values already on the format's grid."""
    if dtype == "f16":
        return v.astype(np.float16).view(np.uint16)
    return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_chunked_checker_matches_the_whole():
    x, w, pos, cos, sin = _rows(1024, "bf16", 9)
    exact = oracle.norm_rope_rows(x, w, 1e-6, cos, sin, pos)
    y = round16(_fp32_norm_rope(x, w, 1e-6, cos, sin, pos), "bf16")
    whole = check16(y, exact, "bf16", "whole")
    total = Check16("bf16", "chunks")
    for lo in range(0, 1024, 256):
        part = Check16("bf16", "chunk")
        part.add(y[lo:lo + 256], exact[lo:lo + 256])
        total.merge(part)
    out = total.done()
    assert out["elements"] == whole["elements"] and out["max_abs"] == whole["max_abs"]
    assert abs(out["bias_ulp"] - whole["bias_ulp"]) < 1e-12 and abs(out["rms_ulp"] - whole["rms_ulp"]) < 1e-12
    # a bias spread thinly over chunks is still caught once they are folded together
    t = round16(exact, "bf16", "trunc")
    total = Check16("bf16", "trunc chunks")
    with pytest.raises(ToleranceError):
        for lo in range(0, 1024, 256):
            total.add(t[lo:lo + 256], exact[lo:lo + 256])
        total.done()
