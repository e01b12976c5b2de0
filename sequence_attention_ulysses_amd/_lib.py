"""ctypes declarations of ``include/uly.h`` and the loader of ``libuly.so``.

torch is imported before the library is opened so that ``libuly.so``
binds to the HIP runtime torch already loaded (both carry the soname
``libamdhip64.so.7``): streams and device pointers handed over from torch are
then valid inside the library.  There is no fallback: without the built
library every entry point raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime first, see above)

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libuly.so")

# status codes
OK = 0
E_INVAL = -1
E_DTYPE = -2
E_CACHE_FULL = -3
E_NOT_FOUND = -4
E_UNSUPPORTED = -5
E_HIP = -6
E_BROKEN = -7
E_OVERLAP = -8

F16 = 1
BF16 = 2
U8 = 3
MODE_SCATTER = 0
MODE_GATHER = 1
ROUTE_KERNEL = 0
ROUTE_COPY_ENGINE = 1
ROUTE_CALLER = 2

K_SCATTER, K_NORM_ROPE, K_GATHER, K_PAD, K_SPATIAL, K_PROJ = range(6)
KERNEL_KINDS = {"scatter": K_SCATTER, "norm_rope": K_NORM_ROPE, "gather": K_GATHER,
                "pad": K_PAD, "spatial": K_SPATIAL, "proj": K_PROJ}

# Every symbol include/uly.h declares.
EXPORTS = (
    "uly_create", "uly_destroy", "uly_target_register", "uly_target_lookup", "uly_target_count",
    "ulysses_scatter_qkv", "fused_qk_norm_rope_scatter", "fused_qkv_norm_rope_scatter_packed",
    "fused_qkv_proj_norm_rope_scatter", "uly_wait",
    "ulysses_gather_out", "uly_exchange_chunks",
    "uly_seq_pad_shard", "uly_seq_unshard_trim", "uly_spatial_split_halo",
    "uly_spatial_gather_stacked", "uly_spatial_trim_concat", "uly_rope_table_1d",
    "uly_rope_table_3d", "uly_profile_enable", "uly_profile_read", "uly_profile_reset",
    "uly_get_stats", "uly_comm_stream", "uly_set_route", "uly_debug_fail_launch", "uly_debug_proj_ring",
    "uly_last_error", "uly_status_string",
)


class UlyTensor(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("rank_stride", ctypes.c_int64),
        ("shape", ctypes.c_int64 * 4),
        ("stride", ctypes.c_int64 * 4),
    ]


class UlyStats(ctypes.Structure):
    _fields_ = [
        ("registrations", ctypes.c_int64),
        ("lookups", ctypes.c_int64),
        ("hits", ctypes.c_int64),
        ("launches", ctypes.c_int64),
    ]


class UlyError(RuntimeError):
    status = None


class UlyInvalidArgument(UlyError, ValueError):
    status = E_INVAL


class UlyDtypeError(UlyError, TypeError):
    status = E_DTYPE


class UlyCacheFull(UlyError):
    status = E_CACHE_FULL


class UlyNotFound(UlyError, LookupError):
    status = E_NOT_FOUND


class UlyUnsupported(UlyError, NotImplementedError):
    status = E_UNSUPPORTED


class UlyHipError(UlyError):
    status = E_HIP


class UlyBroken(UlyError):
    status = E_BROKEN


class UlyOverlap(UlyError, ValueError):
    status = E_OVERLAP


_ERRORS = {c.status: c for c in (UlyInvalidArgument, UlyDtypeError, UlyCacheFull, UlyNotFound,
                                 UlyUnsupported, UlyHipError, UlyBroken, UlyOverlap)}

_lib = None


def load() -> ctypes.CDLL:
    """Open ``libuly.so`` (built by ``__graft_entry__.build()``); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            "libuly.so is not built (%s); run __graft_entry__.build() or "
            "python -m sequence_attention_ulysses_amd._build" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, f64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_double
    cp = ctypes.c_char_p
    P_T = ctypes.POINTER(UlyTensor)
    P_I64 = ctypes.POINTER(ctypes.c_int64)
    TAGS = ctypes.POINTER(cp)
    OUTS = ctypes.POINTER(vp)
    sig = {
        "uly_create": [ctypes.POINTER(vp), i32, i32, i32],
        "uly_destroy": [vp],
        "uly_target_register": [vp, cp, i32, i32, P_I64, vp, ctypes.c_size_t],
        "uly_target_lookup": [vp, cp, i32, i32, P_I64, ctypes.POINTER(vp)],
        "uly_target_count": [vp, ctypes.POINTER(i32)],
        "ulysses_scatter_qkv": [vp, P_T, P_T, P_T, TAGS, OUTS, vp],
        "fused_qk_norm_rope_scatter": [vp, P_T, P_T, P_T, vp, vp, f32, vp, vp, i64, TAGS, OUTS, vp],
        "fused_qkv_norm_rope_scatter_packed": [vp, P_T, P_T, P_T, vp, vp, f32, vp, vp, i64, cp, vp, vp],
        "uly_exchange_chunks": [vp, vp, vp, i64, vp],
        "fused_qkv_proj_norm_rope_scatter": [vp, vp, i32, i64, i64, i64, vp, i64, i64, i64, vp, vp, f32, vp, vp,
                                             i64, TAGS, OUTS, vp],
        "uly_wait": [vp, vp],
        "ulysses_gather_out": [vp, P_T, cp, vp, vp],
        "uly_seq_pad_shard": [vp, vp, i32, i64, i64, i64, i64, vp, vp],
        "uly_seq_unshard_trim": [vp, vp, i32, i64, i64, i64, i64, vp, vp],
        "uly_spatial_split_halo": [vp, vp, i32, i64, i64, i64, i64, vp, vp],
        "uly_spatial_gather_stacked": [vp, vp, i32, i64, i64, i64, i64, vp, vp],
        "uly_spatial_trim_concat": [vp, vp, i32, i64, i64, i64, vp, vp],
        "uly_rope_table_1d": [vp, vp, i64, i64, i64, f64],
        "uly_rope_table_3d": [vp, vp, i64, i64, i64, i64, i64, i64, i64, i64, f64],
        "uly_profile_enable": [vp, i32, i32],
        "uly_profile_read": [vp, i32, ctypes.POINTER(f64), P_I64],
        "uly_profile_reset": [vp],
        "uly_get_stats": [vp, ctypes.POINTER(UlyStats)],
        "uly_comm_stream": [vp, ctypes.POINTER(vp)],
        "uly_set_route": [vp, i32],
        "uly_debug_fail_launch": [vp, i32],
        "uly_debug_proj_ring": [vp, i32],
    }
    for name, argtypes in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = ctypes.c_int
    lib.uly_last_error.argtypes = []
    lib.uly_last_error.restype = cp
    lib.uly_status_string.argtypes = [i32]
    lib.uly_status_string.restype = cp
    _lib = lib
    return lib


def check(status: int, what: str = "") -> None:
    """Raise the exception class of a failing status with the library's message."""
    if status == OK:
        return
    lib = load()
    msg = lib.uly_last_error().decode(errors="replace")
    name = lib.uly_status_string(status).decode()
    cls = _ERRORS.get(status, UlyError)
    raise cls("%s%s: %s" % (what + " " if what else "", name, msg))


def int64_array(values):
    return (ctypes.c_int64 * len(values))(*[int(v) for v in values])


_TAGS = {}


def tags_array(tags):
    """A C array of the tag strings (NULL for None).  The library only reads it, so one
    array per distinct tags tuple is built and reused."""
    tags = tuple(tags)
    arr = _TAGS.get(tags)
    if arr is None:
        if len(_TAGS) > 1024:
            _TAGS.clear()
        arr = _TAGS[tags] = (ctypes.c_char_p * len(tags))(*[t.encode() if t is not None else None for t in tags])
    return arr


_PTRS3 = ctypes.c_void_p * 3


def ptr_array(ptrs):
    if len(ptrs) == 3:
        return _PTRS3(ptrs[0] or None, ptrs[1] or None, ptrs[2] or None)
    return (ctypes.c_void_p * len(ptrs))(*[p if p else None for p in ptrs])
