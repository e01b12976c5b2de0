"""CPU oracle for the Ulysses exchange and the fused Q/K RMSNorm + RoPE producer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, the package smoke check and the
CPU-baseline leg of ``bench.py`` may import this module.  It shares no code
with the HIP library (``sequence_attention_ulysses_amd``): the arithmetic
lives in ``uly_oracle.c`` (plain loops, double precision) and this module
only marshals numpy arrays into it, widens 16-bit storage exactly, and
composes the steps in the pages' order.

Sources are cited by page title and section:

* [CA] TeleFuser documentation, "Communication Architecture" —
  "Sequence Parallel Communication / Ulysses", "Shared Collective
  Primitives / Equal-shape gather", "Spatial VAE Communication".
* [QN] flashinfer PR #6332 (QkvNormRopeExchangeOverlap) — "Description",
  "Assumptions", "Tolerance".
* [UC] flashinfer ``UlyssesCommunicator(backend="pcie")`` PR — "What"
  (world size 1 is the identity route; the transport moves opaque bytes).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "uly_oracle.c")
# ULY_ORACLE_LIB points the oracle at another build of uly_oracle.c (the
# mutation tests load deliberately broken copies to show the pins catch them).
_LIB = os.environ.get("ULY_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile ``uly_oracle.c`` with the host C compiler into ``liboracle.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wl,-soname,liboracle.so",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
        lib.oracle_scatter.argtypes = [vp, vp, sz, i64, i64, i64, i64, i64]
        lib.oracle_scatter.restype = ctypes.c_int
        lib.oracle_gather.argtypes = [vp, vp, sz, i64, i64, i64, i64, i64]
        lib.oracle_gather.restype = ctypes.c_int
        lib.oracle_linear.argtypes = [vp, vp, vp, i64, i64, i64]
        lib.oracle_linear.restype = None
        lib.oracle_exchange_chunks.argtypes = [vp, vp, i64, i64]
        lib.oracle_exchange_chunks.restype = None
        lib.oracle_norm_rope_rows.argtypes = [vp, vp, i64, i64, vp, ctypes.c_double, vp, vp, i64, vp]
        lib.oracle_norm_rope_rows.restype = ctypes.c_int
        lib.oracle_rope_table_1d.argtypes = [vp, vp, i64, i64, i64, ctypes.c_double]
        lib.oracle_rope_table_1d.restype = None
        lib.oracle_rope_table_3d.argtypes = [vp, vp, i64, i64, i64, i64, i64, i64, i64, i64, ctypes.c_double]
        lib.oracle_rope_table_3d.restype = None
        lib.oracle_pad_shard.argtypes = [vp, vp, sz, i64, i64, i64, i64, i64]
        lib.oracle_pad_shard.restype = None
        lib.oracle_unshard_trim.argtypes = [vp, vp, sz, i64, i64, i64, i64, i64]
        lib.oracle_unshard_trim.restype = None
        lib.oracle_spatial_split_halo.argtypes = [vp, vp, sz, i64, i64, i64, i64, vp, vp, i64, i64]
        lib.oracle_spatial_split_halo.restype = None
        lib.oracle_spatial_gather_stacked.argtypes = [vp, vp, sz, i64, i64, i64, vp, i64, i64]
        lib.oracle_spatial_gather_stacked.restype = None
        lib.oracle_spatial_trim_concat.argtypes = [vp, vp, sz, i64, i64, i64, i64, vp, vp, i64]
        lib.oracle_spatial_trim_concat.restype = None
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


# --------------------------------------------------------------------------
# 16-bit storage.  bf16 arrives as uint16 bit patterns (numpy has no bf16);
# fp16 as float16 or uint16.  Widening to double is exact in both cases.
# --------------------------------------------------------------------------
def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of 16-bit storage (``"bf16"`` or ``"f16"``) to float64."""
    b = np.ascontiguousarray(bits)
    if dtype == "bf16":
        u = b.view(np.uint16).astype(np.uint32) << 16
        return u.view(np.float32).astype(np.float64)
    if dtype == "f16":
        return b.view(np.float16).astype(np.float64)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# Relayout [CA "Ulysses"].
# --------------------------------------------------------------------------
def scatter(x: np.ndarray) -> np.ndarray:
    """Sequence-sharded x[P,B,S_l,H,D] -> head-sharded y[P,B,P*S_l,H/P,D].

    Rank q receives head band [q*H/P, (q+1)*H/P) of every token; token s of
    rank r lands at global row r*S_l + s.  Opaque byte copy of any dtype.
    """
    x = np.ascontiguousarray(x)
    P, B, S_l, H, D = x.shape
    if H % P:
        raise ValueError("heads %d not divisible by world size %d" % (H, P))
    y = np.empty((P, B, P * S_l, H // P, D), dtype=x.dtype)
    rc = _load().oracle_scatter(_p(x), _p(y), x.itemsize, P, B, S_l, H, D)
    assert rc == 0
    return y


def gather(o: np.ndarray) -> np.ndarray:
    """Head-sharded o[P,B,S,Hl,D] -> sequence-sharded z[P,B,S/P,P*Hl,D] (the inverse)."""
    o = np.ascontiguousarray(o)
    P, B, S, Hl, D = o.shape
    if S % P:
        raise ValueError("gathered sequence %d not divisible by world size %d" % (S, P))
    z = np.empty((P, B, S // P, P * Hl, D), dtype=o.dtype)
    rc = _load().oracle_gather(_p(o), _p(z), o.itemsize, P, B, S, Hl, D)
    assert rc == 0
    return z


def exchange_chunks(x: np.ndarray) -> np.ndarray:
    """x[P, P, ...] destination-major payloads -> y[P, P, ...], y[q, r] = x[r, q] (opaque bytes)."""
    x = np.ascontiguousarray(x)
    P = x.shape[0]
    assert x.shape[1] == P
    y = np.empty_like(x)
    chunk = x.nbytes // (P * P) if P else 0
    _load().oracle_exchange_chunks(_p(x), _p(y), P, chunk)
    return y


def pack_qkv(yq: np.ndarray, yk: np.ndarray, yv: np.ndarray) -> np.ndarray:
    """The packed receive layout: head rows hold q, k and v side by side ([..., 3*D])."""
    return np.concatenate([yq, yk, yv], axis=-1)


# --------------------------------------------------------------------------
# RMSNorm + interleaved RoPE [QN "Assumptions"].
# --------------------------------------------------------------------------
def norm_rope_rows(x64: np.ndarray, w64: np.ndarray, eps: float, cos_tab: np.ndarray,
                   sin_tab: np.ndarray, pos: np.ndarray) -> np.ndarray:
    """Rows x64[n, D] (float64) -> RMSNorm(w, eps) then rotation by table row pos[n]."""
    x64 = np.ascontiguousarray(x64, dtype=np.float64)
    n, D = x64.shape
    w64 = np.ascontiguousarray(w64, dtype=np.float64)
    cos_tab = np.ascontiguousarray(cos_tab, dtype=np.float32)
    sin_tab = np.ascontiguousarray(sin_tab, dtype=np.float32)
    assert cos_tab.shape == sin_tab.shape and cos_tab.shape[1] == D // 2 and w64.shape == (D,)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    assert pos.shape == (n,)
    y = np.empty_like(x64)
    rc = _load().oracle_norm_rope_rows(_p(x64), _p(y), n, D, _p(w64), float(eps),
                                      _p(cos_tab), _p(sin_tab), cos_tab.shape[0], _p(pos))
    if rc != 0:
        raise ValueError("oracle_norm_rope_rows rc=%d" % rc)
    return y


def norm_rope_sharded(x_bits: np.ndarray, dtype: str, w_bits: np.ndarray, eps: float,
                      cos_tab: np.ndarray, sin_tab: np.ndarray) -> np.ndarray:
    """QK-norm then RoPE on every rank's rows, positions r*S_l + s, in source layout.

    x_bits[P,B,S_l,H,D] 16-bit storage; returns float64 of the same shape.
    """
    P, B, S_l, H, D = x_bits.shape
    x64 = widen(x_bits, dtype).reshape(-1, D)
    w64 = widen(w_bits, dtype)
    r = np.arange(P).reshape(P, 1, 1, 1)
    s = np.arange(S_l).reshape(1, 1, S_l, 1)
    pos = np.broadcast_to(r * S_l + s, (P, B, S_l, H)).reshape(-1)
    y = norm_rope_rows(x64, w64, eps, cos_tab, sin_tab, pos)
    return y.reshape(P, B, S_l, H, D)


def fused_norm_rope_scatter(x_bits: np.ndarray, dtype: str, w_bits: np.ndarray, eps: float,
                            cos_tab: np.ndarray, sin_tab: np.ndarray) -> np.ndarray:
    """QK-norm -> RoPE -> head exchange, in that order; float64 head-sharded result."""
    return scatter(norm_rope_sharded(x_bits, dtype, w_bits, eps, cos_tab, sin_tab))


# --------------------------------------------------------------------------
# QKV projection ahead of the norm, rotation and exchange [QN "Description",
# "Assumptions": projection -> QK-norm -> RoPE; every rank holds a token
# shard and the full QKV weight].
# --------------------------------------------------------------------------
def linear(x64: np.ndarray, w64: np.ndarray) -> np.ndarray:
    """y[m, n] = sum_k x[m, k] * w[n, k] in double (weight stored [out, in])."""
    x64 = np.ascontiguousarray(x64, dtype=np.float64)
    w64 = np.ascontiguousarray(w64, dtype=np.float64)
    M, K = x64.shape
    N, K2 = w64.shape
    assert K == K2
    y = np.empty((M, N), np.float64)
    _load().oracle_linear(_p(x64), _p(w64), _p(y), M, N, K)
    return y


def qkv_proj_norm_rope_rows(x_rows: np.ndarray, dtype: str, w_qkv: np.ndarray, Hq: int, Hkv: int, D: int,
                            wq_bits: np.ndarray, wk_bits: np.ndarray, eps: float, cos_tab: np.ndarray,
                            sin_tab: np.ndarray, pos: np.ndarray):
    """Projection, then QK-norm and RoPE at global positions `pos`, for token rows
    x_rows[n, hidden] (16-bit storage).  The weight's output rows hold q's Hq*D
    columns, then k's Hkv*D, then v's Hkv*D.  Returns float64 q [n, Hq, D],
    k [n, Hkv, D] and v [n, Hkv, D] in source (token-major) layout."""
    n, hidden = x_rows.shape
    assert w_qkv.shape == ((Hq + 2 * Hkv) * D, hidden)
    y = linear(widen(x_rows, dtype), widen(w_qkv, dtype))
    q = y[:, :Hq * D].reshape(n, Hq, D)
    k = y[:, Hq * D:(Hq + Hkv) * D].reshape(n, Hkv, D)
    v = y[:, (Hq + Hkv) * D:].reshape(n, Hkv, D)
    pos = np.asarray(pos, np.int64)

    def nr(t, w_bits):
        H = t.shape[1]
        rows = norm_rope_rows(t.reshape(-1, D), widen(w_bits, dtype), eps, cos_tab, sin_tab,
                              np.repeat(pos, H))
        return rows.reshape(n, H, D)

    return nr(q, wq_bits), nr(k, wk_bits), np.ascontiguousarray(v)


def qkv_proj_norm_rope_scatter(x_bits: np.ndarray, dtype: str, w_qkv: np.ndarray, Hq: int, Hkv: int,
                               wq_bits: np.ndarray, wk_bits: np.ndarray, eps: float, cos_tab: np.ndarray,
                               sin_tab: np.ndarray):
    """The whole front end for x_bits[P, B, S_l, hidden]: projection -> QK-norm ->
    RoPE (positions r*S_l + s) -> head exchange.  float64 (q, k, v) head-sharded."""
    P, B, S_l, hidden = x_bits.shape
    D = w_qkv.shape[0] // (Hq + 2 * Hkv)
    r = np.arange(P).reshape(P, 1, 1)
    s = np.arange(S_l).reshape(1, 1, S_l)
    pos = np.broadcast_to(r * S_l + s, (P, B, S_l)).reshape(-1)
    q, k, v = qkv_proj_norm_rope_rows(x_bits.reshape(-1, hidden), dtype, w_qkv, Hq, Hkv, D, wq_bits, wk_bits,
                                      eps, cos_tab, sin_tab, pos)
    return tuple(scatter(t.reshape(P, B, S_l, t.shape[1], D)) for t in (q, k, v))


# --------------------------------------------------------------------------
# Rotary tables (the per-token fp32 cos/sin table the operator consumes).
# --------------------------------------------------------------------------
def rope_table_1d(rows: int, D: int, theta: float = 1e4, real_rows: int | None = None):
    real_rows = rows if real_rows is None else real_rows
    c = np.empty((rows, D // 2), np.float32)
    s = np.empty((rows, D // 2), np.float32)
    _load().oracle_rope_table_1d(_p(c), _p(s), rows, real_rows, D, float(theta))
    return c, s


def rope_table_3d(rows: int, D: int, grid_h: int, grid_w: int, pairs=(22, 21, 21),
                  theta: float = 1e4, real_rows: int | None = None):
    real_rows = rows if real_rows is None else real_rows
    c = np.empty((rows, D // 2), np.float32)
    s = np.empty((rows, D // 2), np.float32)
    _load().oracle_rope_table_3d(_p(c), _p(s), rows, real_rows, D, grid_h, grid_w,
                                 pairs[0], pairs[1], pairs[2], float(theta))
    return c, s


# --------------------------------------------------------------------------
# Sequence padding / restoration.
# --------------------------------------------------------------------------
def padded_local_len(S: int, P: int, tile: int = 128) -> int:
    """S_l after padding S up to a multiple of P*tile."""
    unit = P * tile
    return (S + unit - 1) // unit * unit // P


def pad_shard(full: np.ndarray, P: int, S_l: int) -> np.ndarray:
    """full[B,S,...] -> x[P,B,S_l,...] with zero rows past S."""
    full = np.ascontiguousarray(full)
    B, S = full.shape[:2]
    rest = full.shape[2:]
    R = int(np.prod(rest)) if rest else 1
    x = np.empty((P, B, S_l) + rest, dtype=full.dtype)
    _load().oracle_pad_shard(_p(full), _p(x), full.itemsize, P, B, S, S_l, R)
    return x


def unshard_trim(x: np.ndarray, S: int) -> np.ndarray:
    """x[P,B,S_l,...] -> full[B,S,...] (concatenate along the sequence, keep [0,S))."""
    x = np.ascontiguousarray(x)
    P, B, S_l = x.shape[:3]
    rest = x.shape[3:]
    R = int(np.prod(rest)) if rest else 1
    full = np.empty((B, S) + rest, dtype=x.dtype)
    _load().oracle_unshard_trim(_p(x), _p(full), x.itemsize, P, B, S, S_l, R)
    return full


# --------------------------------------------------------------------------
# Height-sharded spatial tensors [CA "Spatial VAE Communication"].
# --------------------------------------------------------------------------
def height_split(Hh: int, P: int):
    """Heights and offsets: the first Hh % P ranks take one extra row."""
    base, extra = divmod(Hh, P)
    h = np.array([base + (1 if r < extra else 0) for r in range(P)], np.int64)
    o = np.concatenate([[0], np.cumsum(h)[:-1]]).astype(np.int64)
    return h, o


def spatial_split_halo(full: np.ndarray, P: int, halo: int = 1) -> np.ndarray:
    """full[..., Hh, W] -> shards[P, ..., hmax+2*halo, W] with zero halos at image edges."""
    full = np.ascontiguousarray(full)
    lead = full.shape[:-2]
    Hh, W = full.shape[-2:]
    N = int(np.prod(lead)) if lead else 1
    h, o = height_split(Hh, P)
    hmax = int(h.max())
    sh = np.empty((P,) + lead + (hmax + 2 * halo, W), dtype=full.dtype)
    _load().oracle_spatial_split_halo(_p(full), _p(sh), full.itemsize, P, N, Hh, W,
                                      _p(h), _p(o), hmax, halo)
    return sh


def spatial_gather_stacked(sh: np.ndarray, Hh: int, halo: int = 1) -> np.ndarray:
    """shards[P, ..., hmax+2*halo, W] -> stacked[P, ..., hmax, W] of core rows, zero-padded."""
    sh = np.ascontiguousarray(sh)
    P = sh.shape[0]
    lead = sh.shape[1:-2]
    W = sh.shape[-1]
    N = int(np.prod(lead)) if lead else 1
    h, _ = height_split(Hh, P)
    hmax = int(h.max())
    st = np.empty((P,) + lead + (hmax, W), dtype=sh.dtype)
    _load().oracle_spatial_gather_stacked(_p(sh), _p(st), sh.itemsize, P, N, W, _p(h), hmax, halo)
    return st


def spatial_trim_concat(st: np.ndarray, Hh: int) -> np.ndarray:
    """stacked[P, ..., hmax, W] -> full[..., Hh, W] (trim to each rank's height, concat)."""
    st = np.ascontiguousarray(st)
    P = st.shape[0]
    lead = st.shape[1:-2]
    hmax, W = st.shape[-2:]
    N = int(np.prod(lead)) if lead else 1
    h, o = height_split(Hh, P)
    full = np.empty(lead + (Hh, W), dtype=st.dtype)
    _load().oracle_spatial_trim_concat(_p(st), _p(full), st.itemsize, P, N, Hh, W,
                                       _p(h), _p(o), hmax)
    return full
