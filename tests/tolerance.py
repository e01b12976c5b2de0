"""Element-wise checker for 16-bit results that the kernels compute in fp32 and round once.

Test infrastructure only.  The fused Q/K RMSNorm + RoPE producer (flashinfer
PR #6332, "Assumptions") and the QKV projection in front of it evaluate in
fp32 and round each output once, to nearest even, to bf16 or fp16.  Against
the exact (double-precision) oracle value y, a correct result y_hat obeys

    |y_hat - y| <= E + ulp16(|y| + E) / 2                                (1)

where E bounds the fp32 evaluation error before the rounding and
ulp16(v) is the spacing of the 16-bit format at magnitude v.  The bound on E
is derived from the operations the producer performs (u = 2^-24, the unit
roundoff of fp32):

* norm + rotation of one row of D values:
    - sum of D squares, any order:            relative error <= (D-1) u / (1 - (D-1) u)
    - mean + eps by one fused multiply-add:   + u
    - reciprocal square root (v_rsq_f32, 1 ulp): relative 2u, and the square root
      halves the relative error of its argument
    - n_i = x_i * inv * w_i, two roundings:   + 2u
    so n carries a relative error delta_n <= (D/2 + 5) u; the rotated
    y_2j = n_2j c - n_2j+1 s (and its twin) adds two roundings of magnitude
    M = |n_2j c| + |n_2j+1 s| <= |(y_2j, y_2j+1)|, hence

        E_norm = (D/2 + 8) u * |(y_2j, y_2j+1)|                          (2)

  (the weights, the inputs and the fp32 cos/sin table are the same exact
  values on both sides, so they contribute nothing).

* projection q = x . W^T over K terms in fp32 (products of two 16-bit values
  are exact in fp32; any summation order, one rounding per addition):

        e_i = gamma_K * sum_k |x_k W_ik|,  gamma_K = K u / (1 - K u)       (3)

  propagated to first order through the norm,
        |dn_i| <= |w_i| inv (e_i + |q_i| inv^2 sum_j |q_j| e_j / D),
  and through the rotation, |dy_2j| <= |c| |dn_2j| + |s| |dn_2j+1| (and the
  twin), with a 5 % margin for the second-order terms; E = E_norm + that
  (E_norm from the exact result as in (2)).

The tolerance the pages' operator is held to (max-abs 2e-2 for bf16, 2e-3
for fp16) is never loosened.  Half an ulp alone exceeds it only from |y| = 8
up, in both formats (bf16: 2^-5 = 0.03125 > 2e-2; fp16: 2^-8 = 0.0039 >
2e-3), so only elements at |y| >= 8 may exceed it;
they are counted and reported (PR #6332, "Tolerance": classify such
elements explicitly instead of loosening the tolerance), and they still
obey (1).

Bound (1) admits one rounding; it does not by itself rule out a biased one.
For random data the signed rounding error in ulps, t = (y_hat - y) / ulp16(|y|),
is uniform on [-1/2, 1/2] for a correct single rounding (mean 0, rms
1/sqrt(12) = 0.289); truncation shifts its mean toward zero by 1/2, and an
extra intermediate rounding (for instance of the normalised value before the
rotation, as the pages' own bf16 reference does) raises its rms.  With
enough elements the checker therefore also bounds |mean(t * sign(y))| and
rms(t).  These statistics skip elements where the rotation cancels
(|y_2j| < |(y_2j, y_2j+1)| / 16): there the fp32 error of the two products,
though within (2), is no longer small against an ulp of the small result,
and it would widen the spread of a correct rounding (bf16 at D = 128: the
bound E is at most 0.018 ulp on the kept elements, fp16 0.14 ulp).
"""
from __future__ import annotations

import numpy as np

from oracle import oracle

U32 = 2.0 ** -24                     # unit roundoff of fp32
TOL = {"bf16": 2e-2, "f16": 2e-3}    # the operator's stated max-abs tolerance
MANT = {"bf16": 7, "f16": 10}        # explicit mantissa bits
EMIN = {"bf16": -126, "f16": -14}    # smallest normal exponent

# statistics are applied from this many nonzero elements on; the limits sit
# many standard errors away from a correct rounding's values at that size
STATS_MIN = 4096
BIAS_MAX = 0.03          # |mean(t * sign(y))|, correct: 0 +- 0.0045 at 4096
RMS_MAX = 0.31           # rms(t), correct: 0.2887 +- 0.002 at 4096


def ulp16(mag: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the 16-bit format at magnitude `mag` (subnormal spacing below the normals)."""
    mag = np.asarray(mag, np.float64)
    e = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
    e = np.maximum(np.where(mag > 0, e, EMIN[dtype]), EMIN[dtype])
    return np.exp2(e - MANT[dtype])


def round16(v: np.ndarray, dtype: str, mode: str = "rne") -> np.ndarray:
    """Round float64 values once to the 16-bit format's grid (no overflow handling).

    mode "rne" rounds to nearest even (numpy's round is half-to-even), "trunc" toward zero."""
    v = np.asarray(v, np.float64)
    q = ulp16(np.abs(v), dtype)
    f = np.round if mode == "rne" else np.trunc
    return f(v / q) * q


def pair_magnitude(y: np.ndarray) -> np.ndarray:
    """|(y_2j, y_2j+1)| repeated onto both elements of each interleaved pair."""
    p = np.sqrt(y[..., 0::2] ** 2 + y[..., 1::2] ** 2)
    return np.repeat(p, 2, axis=-1)


def norm_rope_eval_bound(y: np.ndarray) -> np.ndarray:
    """E of (2) for rows of the fused norm + rotation, from the exact result y[..., D]."""
    D = y.shape[-1]
    return (D / 2 + 8) * U32 * pair_magnitude(y)


def proj_eval_bound(q: np.ndarray, abs_sum: np.ndarray, K: int, w: np.ndarray | None = None,
                    eps: float = 1e-6, cos: np.ndarray | None = None, sin: np.ndarray | None = None) -> np.ndarray:
    """The accumulation part of E for projected rows q[n, H, D] (exact projection,
    double) whose fp32 sums over K terms err by at most (3), with
    abs_sum[n, H, D] = sum_k |x_k W_ik|.

    Without a weight (the V columns, rounded straight from the accumulators) it is
    (3) itself.  With the norm weight w[D], eps and the rotation cos/sin[n, D/2]
    it is (3) propagated through the norm and the rotation, with a 5 % margin;
    the caller adds E_norm of (2) for the norm's own fp32 evaluation."""
    gamma = K * U32 / (1.0 - K * U32)
    e = gamma * abs_sum
    if w is None:
        return e
    D = q.shape[-1]
    inv = 1.0 / np.sqrt((q * q).mean(axis=-1, keepdims=True) + eps)
    coupled = np.abs(q) * inv ** 2 * (np.abs(q) * e).sum(axis=-1, keepdims=True) / D
    dn = np.abs(w) * inv * (e + coupled)
    c = np.abs(cos)[:, None, :]
    s = np.abs(sin)[:, None, :]
    d0, d1 = dn[..., 0::2], dn[..., 1::2]
    dy = np.empty_like(dn)
    dy[..., 0::2] = c * d0 + s * d1
    dy[..., 1::2] = s * d0 + c * d1
    return 1.05 * dy


def proj_bounds(x64: np.ndarray, w64: np.ndarray, Hq: int, Hkv: int, D: int, wq64: np.ndarray,
                wk64: np.ndarray, eps: float, cos_rows: np.ndarray, sin_rows: np.ndarray, exact) -> tuple:
    """E for the projection's q, k and v outputs of token rows x64[n, K] with weight
    w64[(Hq + 2 Hkv) D, K]: E_norm of (2) plus the propagated accumulation bound (3)
    for q and k, (3) alone for v.  cos_rows/sin_rows[n, D/2] are the table rows of the
    tokens; `exact` is the oracle's (q, k, v), each [n, H, D].  The projection and
    the absolute sums are the oracle's own matrix product."""
    n, K = x64.shape
    pre = oracle.linear(x64, w64)
    absum = oracle.linear(np.abs(x64), np.abs(w64))
    cut = (Hq * D, (Hq + Hkv) * D)
    out = []
    for i, (p, a) in enumerate(zip(np.split(pre, cut, axis=1), np.split(absum, cut, axis=1))):
        H = p.shape[1] // D
        p, a = p.reshape(n, H, D), a.reshape(n, H, D)
        if i == 2:
            out.append(proj_eval_bound(p, a, K))
        else:
            w = wq64 if i == 0 else wk64
            out.append(proj_eval_bound(p, a, K, w, eps, cos_rows, sin_rows) + norm_rope_eval_bound(exact[i]))
    return tuple(out)


class ToleranceError(AssertionError):
    pass


class Check16:
    """Accumulating form of `check16` for results compared chunk by chunk: every chunk
    is held to (1) and to the stated tolerance at once; the rounding statistics are
    taken over all chunks together by `done()`."""

    def __init__(self, dtype: str, what: str, stats: bool = True, verbose: bool = True):
        self.dtype, self.what, self.stats, self.verbose = dtype, what, stats, verbose
        self.n = self.nz = self.classified = 0
        self.max_abs = 0.0
        self.min_classified = np.inf
        self.sum_t = self.sum_t2 = 0.0

    def add(self, got: np.ndarray, ref: np.ndarray, E: np.ndarray | None = None, where: str = "") -> None:
        dtype, what = self.dtype, self.what + (" " + where if where else "")
        g = np.asarray(got, np.float64)
        ref = np.asarray(ref, np.float64)
        if g.shape != ref.shape:
            raise ToleranceError("%s: shape %s against %s" % (what, g.shape, ref.shape))
        if E is None:
            E = norm_rope_eval_bound(ref)
        mag = np.abs(ref)
        err = np.abs(g - ref)
        half = 0.5 * ulp16(mag + E, dtype)
        bound = E + half
        bad = ~(err <= bound)                               # NaN in got fails too
        if bad.any():
            i = np.flatnonzero(bad.reshape(-1))[0]
            raise ToleranceError("%s: %d elements beyond half an ulp + fp32 bound; first at flat %d: got %r, "
                                 "exact %r, error %g > %g (half ulp %g, E %g)" % (
                                     what, int(bad.sum()), i, float(g.reshape(-1)[i]), float(ref.reshape(-1)[i]),
                                     float(err.reshape(-1)[i]), float(bound.reshape(-1)[i]),
                                     float(half.reshape(-1)[i]),
                                     float(np.broadcast_to(E, ref.shape).reshape(-1)[i])))
        tol = TOL[dtype]
        classified = 0.5 * ulp16(mag, dtype) > tol          # half an ulp alone exceeds it: |y| >= 8
        over = err > tol
        if (over & ~classified).any():
            raise ToleranceError("%s: max-abs %g > %g at |y| = %g" % (
                what, float(err[over & ~classified].max()), tol, float(mag[over & ~classified][0])))
        n_class = int((over & classified).sum())
        if n_class:
            self.classified += n_class
            self.min_classified = min(self.min_classified, float(mag[over].min()))
        self.n += int(err.size)
        if err.size:
            self.max_abs = max(self.max_abs, float(err.max()))
        # statistics over elements whose rotation does not cancel (|y| >= 1/16 of its pair's
        # magnitude): there the fp32 evaluation error is a negligible part of an ulp of y
        nz = (mag > 0) & (mag >= pair_magnitude(ref) / 16)
        if self.stats:
            t = (g[nz] - ref[nz]) / ulp16(mag[nz], dtype)
            self.nz += int(nz.sum())
            self.sum_t += float(np.sum(t * np.sign(ref[nz])))
            self.sum_t2 += float(np.sum(t * t))

    def merge(self, other: "Check16") -> None:
        """Fold in the counts of a checker that saw other chunks of the same result."""
        self.n += other.n
        self.nz += other.nz
        self.classified += other.classified
        self.max_abs = max(self.max_abs, other.max_abs)
        self.min_classified = min(self.min_classified, other.min_classified)
        self.sum_t += other.sum_t
        self.sum_t2 += other.sum_t2

    def done(self) -> dict:
        out = {"max_abs": self.max_abs, "classified": self.classified, "elements": self.n}
        if self.classified and self.verbose:
            print("%s: %d elements above the %g tolerance at |y| >= %g, each within (1) (classified)"
                  % (self.what, self.classified, TOL[self.dtype], self.min_classified), flush=True)
        if self.stats and self.nz >= STATS_MIN:
            bias = self.sum_t / self.nz
            rms = float(np.sqrt(self.sum_t2 / self.nz))
            out.update(bias_ulp=bias, rms_ulp=rms)
            if abs(bias) > BIAS_MAX:
                raise ToleranceError("%s: rounding biased toward %s by %.3f ulp (limit %g)" % (
                    self.what, "zero" if bias < 0 else "infinity", abs(bias), BIAS_MAX))
            if rms > RMS_MAX:
                raise ToleranceError("%s: rms rounding error %.3f ulp > %g (a single rounding gives 0.289)" % (
                    self.what, rms, RMS_MAX))
        return out


def check16(got: np.ndarray, ref: np.ndarray, dtype: str, what: str, E: np.ndarray | None = None,
            stats: bool = True, verbose: bool = True) -> dict:
    """Check 16-bit results `got` (widened to float64) against the exact `ref`.

    E: per-element fp32 evaluation bound (default: the fused norm + rotation's (2)).
    Raises ToleranceError on any element beyond (1), any element beyond the stated
    tolerance where half an ulp does not itself exceed it, or (with `stats` and
    enough elements) a biased or over-dispersed rounding error."""
    c = Check16(dtype, what, stats, verbose)
    c.add(got, ref, E)
    return c.done()
