"""Host-only checks of the C ABI (no GPU): exported symbols, argument
rejection before any launch, the tagged target cache, the fail-stop rule,
the division helper and the library's rotary tables against the oracle's.

A host-only context (device -1) runs every check a device context runs and
returns ULY_E_UNSUPPORTED where it would launch; the pointers below are
never dereferenced.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from sequence_attention_ulysses_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "uly.h")
BASE = 0x7F0000000000          # fake, 16-byte aligned device addresses
MiB = 1 << 20


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_symbols_exported(lib):
    names = header_functions()
    assert "ulysses_scatter_qkv" in names and "fused_qk_norm_rope_scatter" in names
    assert "ulysses_gather_out" in names
    out = subprocess.check_output(["nm", "-D", "--defined-only", _lib.LIB_PATH]).decode()
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert sorted(_lib.EXPORTS) == names


class Ctx:
    def __init__(self, lib, P, max_targets=12):
        self.lib = lib
        self.h = ctypes.c_void_p()
        assert lib.uly_create(ctypes.byref(self.h), -1, P, max_targets) == _lib.OK
        self.P = P

    def close(self):
        assert self.lib.uly_destroy(self.h) == _lib.OK


@pytest.fixture
def ctx4(lib):
    c = Ctx(lib, 4)
    yield c
    c.close()


def T(addr, shape, stride=None, rank_stride=None, dtype=_lib.BF16):
    """uly_tensor for a rank-major operand; contiguous strides by default."""
    B, S, H, D = shape
    if stride is None:
        stride = (S * H * D, H * D, D, 1)
    if rank_stride is None:
        rank_stride = B * S * H * D
    t = _lib.UlyTensor()
    t.data = addr
    t.dtype = dtype
    t.reserved = 0
    t.rank_stride = rank_stride
    for i in range(4):
        t.shape[i] = shape[i]
        t.stride[i] = stride[i]
    return t


def register(lib, c, tag, mode, shape, addr, dtype=_lib.BF16, nbytes=None):
    n = c.P * int(np.prod(shape)) * 2
    return lib.uly_target_register(c.h, tag.encode(), mode, dtype, _lib.int64_array(shape), addr,
                                   n if nbytes is None else nbytes)


def scatter(lib, c, q=None, k=None, v=None, tags=("q", "k", "v"), outs=(None, None, None)):
    args = [ctypes.byref(x) if x is not None else None for x in (q, k, v)]
    return lib.ulysses_scatter_qkv(c.h, *args, _lib.tags_array(tags), _lib.ptr_array(outs), None)


def test_create_arguments(lib):
    h = ctypes.c_void_p()
    assert lib.uly_create(ctypes.byref(h), -1, 0, 12) == _lib.E_INVAL
    assert lib.uly_create(ctypes.byref(h), -1, 4, 13) == _lib.E_INVAL      # at most 12 targets
    assert lib.uly_create(ctypes.byref(h), -1, 4, 0) == _lib.E_INVAL
    assert lib.uly_create(None, -1, 4, 12) == _lib.E_INVAL
    assert lib.uly_destroy(None) == _lib.OK


def test_scatter_valid_group_reaches_launch(lib, ctx4):
    shape = (1, 16, 8, 128)
    t_shape = (1, 64, 2, 128)
    for i, tag in enumerate("qkv"):
        assert register(lib, ctx4, tag, _lib.MODE_SCATTER, t_shape, BASE + (10 + i) * 64 * MiB) == _lib.OK
    q, k, v = (T(BASE + i * 64 * MiB, shape) for i in range(3))
    assert scatter(lib, ctx4, q, k, v) == _lib.E_UNSUPPORTED   # all checks passed, would launch


def test_divisibility_checked_before_launch(lib, ctx4):
    # heads 6 not divisible by P = 4
    st = scatter(lib, ctx4, q=T(BASE, (1, 16, 6, 128)), tags=("q", None, None), outs=(BASE + 64 * MiB, None, None))
    assert st == _lib.E_INVAL and b"divisible" in lib.uly_last_error()
    # gathered sequence 18 not divisible by P = 4
    o = T(BASE, (1, 18, 2, 128))
    st = lib.ulysses_gather_out(ctx4.h, ctypes.byref(o), None, BASE + 64 * MiB, None)
    assert st == _lib.E_INVAL and b"divisible" in lib.uly_last_error()


def test_group_rejected_as_a_whole(lib, ctx4):
    """A bad V leaves nothing launched for Q/K (no protocol mixing)."""
    shape = (1, 16, 8, 128)
    outs = (BASE + 10 * 64 * MiB, BASE + 11 * 64 * MiB, BASE + 12 * 64 * MiB)
    bad_v = T(BASE + 2 * 64 * MiB, (1, 16, 8, 128), dtype=_lib.F16)
    before = _stats(lib, ctx4)
    st = scatter(lib, ctx4, T(BASE, shape), T(BASE + 64 * MiB, shape), bad_v, outs=outs)
    assert st == _lib.E_DTYPE
    assert _stats(lib, ctx4)["launches"] == before["launches"]
    bad_v = T(BASE + 2 * 64 * MiB, (1, 17, 8, 128))                   # S_l differs
    assert scatter(lib, ctx4, T(BASE, shape), T(BASE + 64 * MiB, shape), bad_v, outs=outs) == _lib.E_INVAL


def _stats(lib, c):
    s = _lib.UlyStats()
    assert lib.uly_get_stats(c.h, ctypes.byref(s)) == _lib.OK
    return {f: getattr(s, f) for f, _ in s._fields_}


@pytest.mark.parametrize("mutate,code", [
    (lambda t: setattr(t, "data", BASE + 8), _lib.E_INVAL),                   # misaligned
    (lambda t: setattr(t, "data", 0), _lib.E_INVAL),                          # null
    (lambda t: t.stride.__setitem__(3, 2), _lib.E_INVAL),                     # head dim not contiguous
    (lambda t: t.shape.__setitem__(3, 36), _lib.E_INVAL),                     # D*2 % 16 != 0
    (lambda t: setattr(t, "dtype", 7), _lib.E_DTYPE),
    (lambda t: setattr(t, "reserved", 1), _lib.E_INVAL),
    (lambda t: t.stride.__setitem__(1, 8 * 128 + 4), _lib.E_INVAL),           # row pitch not 16-byte
    (lambda t: t.stride.__setitem__(2, 136), _lib.E_INVAL),                   # heads not packed
])
def test_operand_rejections(lib, ctx4, mutate, code):
    t = T(BASE, (1, 16, 8, 128))
    mutate(t)
    assert scatter(lib, ctx4, q=t, tags=("q", None, None), outs=(BASE + 64 * MiB, None, None)) == code


def test_overlap_rejected(lib, ctx4):
    t = T(BASE, (1, 16, 8, 128))
    assert scatter(lib, ctx4, q=t, tags=("q", None, None), outs=(BASE + 4096, None, None)) == _lib.E_OVERLAP
    # two members writing the same destination
    t2 = T(BASE + 64 * MiB, (1, 16, 8, 128))
    st = scatter(lib, ctx4, q=t, k=t2, tags=("q", "k", None), outs=(BASE + 128 * MiB, BASE + 128 * MiB, None))
    assert st == _lib.E_OVERLAP


def test_fused_qkv_strided_source_accepted(lib, ctx4):
    """V taken from a fused [B, S_l, 3, H, D] projection: stride[1] = 3*H*D, offset 2*H*D."""
    B, S, H, D = 1, 16, 8, 128
    rank = B * S * 3 * H * D
    v = T(BASE + 2 * H * D * 2, (B, S, H, D), stride=(S * 3 * H * D, 3 * H * D, D, 1), rank_stride=rank)
    assert scatter(lib, ctx4, v=v, tags=(None, None, "v"), outs=(None, None, BASE + 64 * MiB)) == _lib.E_UNSUPPORTED


def test_target_cache_policy(lib):
    c = Ctx(lib, 2, max_targets=12)
    try:
        for i in range(12):
            assert register(lib, c, "t%d" % i, _lib.MODE_SCATTER, (1, 8, 4, 64), BASE + i * MiB) == _lib.OK
        # a 13th key is refused (no eviction)
        assert register(lib, c, "t12", _lib.MODE_SCATTER, (1, 8, 4, 64), BASE + 12 * MiB) == _lib.E_CACHE_FULL
        n = ctypes.c_int()
        lib.uly_target_count(c.h, ctypes.byref(n))
        assert n.value == 12
        # lookups return the registered pointer, stable across calls
        for step in range(20):
            p = ctypes.c_void_p()
            assert lib.uly_target_lookup(c.h, b"t3", _lib.MODE_SCATTER, _lib.BF16, _lib.int64_array((1, 8, 4, 64)),
                                         ctypes.byref(p)) == _lib.OK
            assert p.value == BASE + 3 * MiB
        # every key component matters: mode, dtype and shape
        p = ctypes.c_void_p()
        for mode, dtype, shape in [(_lib.MODE_GATHER, _lib.BF16, (1, 8, 4, 64)),
                                   (_lib.MODE_SCATTER, _lib.F16, (1, 8, 4, 64)),
                                   (_lib.MODE_SCATTER, _lib.BF16, (1, 8, 4, 128))]:
            assert lib.uly_target_lookup(c.h, b"t3", mode, dtype, _lib.int64_array(shape),
                                         ctypes.byref(p)) == _lib.E_NOT_FOUND
        assert _stats(lib, c)["registrations"] == 12
    finally:
        c.close()


def test_target_register_rejections(lib, ctx4):
    shp = (1, 8, 4, 64)
    assert register(lib, ctx4, "a", _lib.MODE_SCATTER, shp, BASE + 8) == _lib.E_INVAL          # misaligned
    assert register(lib, ctx4, "a", _lib.MODE_SCATTER, shp, BASE, nbytes=100) == _lib.E_INVAL  # too small
    assert register(lib, ctx4, "x" * 64, _lib.MODE_SCATTER, shp, BASE) == _lib.E_INVAL        # tag too long
    assert register(lib, ctx4, "a", 5, shp, BASE) == _lib.E_INVAL
    assert register(lib, ctx4, "a", _lib.MODE_SCATTER, shp, BASE, dtype=9) == _lib.E_DTYPE
    assert register(lib, ctx4, "a", _lib.MODE_SCATTER, shp, BASE) == _lib.OK
    assert register(lib, ctx4, "a", _lib.MODE_SCATTER, shp, BASE + MiB) == _lib.E_INVAL       # duplicate key


def test_missing_and_mistyped_targets(lib, ctx4):
    q = T(BASE, (1, 16, 8, 128))
    assert scatter(lib, ctx4, q=q, tags=("q", None, None)) == _lib.E_NOT_FOUND
    # registered as fp16, called with bf16: a dtype error, not a miss
    assert register(lib, ctx4, "q", _lib.MODE_SCATTER, (1, 64, 2, 128), BASE + 64 * MiB, dtype=_lib.F16) == _lib.OK
    assert scatter(lib, ctx4, q=q, tags=("q", None, None)) == _lib.E_DTYPE


def _fused(lib, c, q, k, w=(BASE + 200 * MiB, BASE + 201 * MiB), eps=1e-6, rows=64,
           tabs=(BASE + 300 * MiB, BASE + 310 * MiB), outs=(BASE + 100 * MiB, BASE + 120 * MiB, BASE + 140 * MiB),
           v=None):
    args = [ctypes.byref(x) if x is not None else None for x in (q, k, v)]
    return lib.fused_qk_norm_rope_scatter(c.h, *args, w[0], w[1], eps, tabs[0], tabs[1], rows,
                                          _lib.tags_array(("q", "k", "v")), _lib.ptr_array(outs), None)


def test_fused_rejections(lib, ctx4):
    q, k = T(BASE, (1, 16, 8, 128)), T(BASE + 64 * MiB, (1, 16, 8, 128))
    assert _fused(lib, ctx4, q, k) == _lib.E_UNSUPPORTED                      # valid: would launch
    assert _fused(lib, ctx4, q, k, rows=63) == _lib.E_INVAL                   # positions reach 64
    assert _fused(lib, ctx4, q, k, eps=0.0) == _lib.E_INVAL
    assert _fused(lib, ctx4, q, k, eps=float("nan")) == _lib.E_INVAL
    assert _fused(lib, ctx4, q, k, w=(0, BASE)) == _lib.E_INVAL
    assert _fused(lib, ctx4, q, k, tabs=(BASE + 8, BASE)) == _lib.E_INVAL
    assert _fused(lib, ctx4, None, None) == _lib.E_INVAL
    k96 = T(BASE + 64 * MiB, (1, 16, 8, 96))
    assert _fused(lib, ctx4, q, k96) == _lib.E_INVAL                          # D differs
    q96 = T(BASE, (1, 16, 8, 96))
    assert _fused(lib, ctx4, q96, None) == _lib.E_UNSUPPORTED and b"head dim" in lib.uly_last_error()
    # GQA: Q and K may differ in heads
    k2 = T(BASE + 64 * MiB, (1, 16, 4, 128))
    assert _fused(lib, ctx4, q, k2) == _lib.E_UNSUPPORTED and b"host-only" in lib.uly_last_error()
    # V rides along unchanged; it needs no weight but must match B, S_l, D, dtype
    v = T(BASE + 80 * MiB, (1, 16, 4, 128))
    assert _fused(lib, ctx4, q, k2, v=v) == _lib.E_UNSUPPORTED
    assert _fused(lib, ctx4, None, None, v=v) == _lib.E_UNSUPPORTED
    v_bad = T(BASE + 80 * MiB, (1, 16, 4, 128), dtype=_lib.F16)
    assert _fused(lib, ctx4, q, k2, v=v_bad) == _lib.E_DTYPE
    v_over = T(BASE + 100 * MiB, (1, 16, 4, 128))         # reads what q's target is written to
    assert _fused(lib, ctx4, q, k2, v=v_over) == _lib.E_OVERLAP


def test_route_arguments(lib, ctx4):
    """Three routes for the plain scatter; anything else is refused and changes nothing."""
    q = T(BASE, (1, 16, 8, 128))
    for route in (_lib.ROUTE_KERNEL, _lib.ROUTE_COPY_ENGINE, _lib.ROUTE_CALLER):
        assert lib.uly_set_route(ctx4.h, route) == _lib.OK
        assert scatter(lib, ctx4, q=q, tags=(None, None, None), outs=(BASE + 64 * MiB, None, None)) == _lib.E_UNSUPPORTED
        assert b"host-only" in lib.uly_last_error()
    for bad in (-1, 3):
        assert lib.uly_set_route(ctx4.h, bad) == _lib.E_INVAL
    assert lib.uly_set_route(None, _lib.ROUTE_KERNEL) == _lib.E_INVAL


def test_launch_size_limits(lib, ctx4):
    """Flat 32-bit indices cover 2^31 16-byte vectors (32 GiB) per operand plan, and
    2^31 rows per fused launch: larger calls are refused before anything is enqueued."""
    GiB = 1 << 30
    # per rank [1, 2^21, 32, 128] bf16 = 16 GiB; 4 ranks = 64 GiB = 2^32 vectors: too large
    big = T(BASE, (1, 1 << 21, 32, 128))
    assert scatter(lib, ctx4, q=big, tags=(None, None, None), outs=(BASE + 256 * GiB, None, None)) == _lib.E_UNSUPPORTED
    assert b"too large" in lib.uly_last_error()
    # just under the limit: [1, 2^19, 32, 128] per rank, 2^30 vectors in all: accepted (would launch)
    ok = T(BASE, (1, 1 << 19, 32, 128))
    assert scatter(lib, ctx4, q=ok, tags=(None, None, None), outs=(BASE + 256 * GiB, None, None)) == _lib.E_UNSUPPORTED
    assert b"host-only" in lib.uly_last_error()
    # the inverse: head-sharded [1, 2^23, 8, 128] per rank is 2^32 vectors in all
    o = T(BASE, (1, 1 << 23, 8, 128))
    assert lib.ulysses_gather_out(ctx4.h, ctypes.byref(o), None, BASE + 256 * GiB, None) == _lib.E_UNSUPPORTED
    assert b"too large" in lib.uly_last_error()
    # fused: 4 * 2^24 tokens x 64 rows = 2^32 rows in one launch
    qf, kf = T(BASE, (1, 1 << 24, 32, 32)), T(BASE + 512 * GiB, (1, 1 << 24, 32, 32))
    assert _fused(lib, ctx4, qf, kf, rows=4 << 24, outs=(BASE + 1024 * GiB, BASE + 2048 * GiB)) == _lib.E_UNSUPPORTED
    assert b"too many rows" in lib.uly_last_error()


def test_wrapping_sizes_refused(lib, ctx4):
    """Extents whose products pass int64 are refused, never wrapped into a small launch."""
    huge = 1 << 62
    big_s = T(BASE, (1, huge, 8, 128), stride=(0, 1024, 128, 1), rank_stride=0)
    assert scatter(lib, ctx4, q=big_s, tags=(None, None, None), outs=(BASE + 64 * MiB, None, None)) == _lib.E_UNSUPPORTED
    assert b"too large" in lib.uly_last_error()
    # B * S * H * D * 2 wraps to exactly 2^64 * k: 2^16 * 2^16 * 2^16 * 2^16 * 2
    wrap = T(BASE, (1 << 16, 1 << 16, 1 << 16, 1 << 16))
    assert scatter(lib, ctx4, q=wrap, tags=(None, None, None), outs=(BASE + 64 * MiB, None, None)) == _lib.E_UNSUPPORTED
    # a stride whose span passes int64 once scaled by the element size
    far = T(BASE, (2, 16, 8, 128), stride=(huge, 1024, 128, 1))
    assert scatter(lib, ctx4, q=far, tags=(None, None, None), outs=(BASE + 64 * MiB, None, None)) == _lib.E_UNSUPPORTED
    o = T(BASE, (1 << 20, 1 << 22, 1 << 20, 128))
    assert lib.ulysses_gather_out(ctx4.h, ctypes.byref(o), None, BASE + 64 * MiB, None) == _lib.E_UNSUPPORTED
    qf = T(BASE, (1 << 30, 1 << 30, 32, 32))
    assert _fused(lib, ctx4, qf, qf, outs=(BASE + 64 * MiB, BASE + 128 * MiB)) == _lib.E_UNSUPPORTED
    assert b"too large" in lib.uly_last_error()
    qs, ks = T(BASE, (1, 16, 8, 128)), T(BASE + 8 * MiB, (1, 16, 8, 128))
    assert _fused(lib, ctx4, qs, ks, rows=huge) == _lib.E_UNSUPPORTED and b"table" in lib.uly_last_error()
    # projection: P * B * S_l and M * hidden would wrap
    assert _proj(lib, ctx4, B=1 << 40, S_l=1 << 40, rows=huge) == _lib.E_UNSUPPORTED
    assert _proj(lib, ctx4, B=1, S_l=1 << 20, hidden=1 << 50, rows=1 << 22) == _lib.E_UNSUPPORTED
    assert _proj(lib, ctx4, Hq=1 << 60, Hkv=4) == _lib.E_UNSUPPORTED
    # row maps, the chunk exchange and the host tables
    assert lib.uly_seq_pad_shard(ctx4.h, BASE, _lib.BF16, 1 << 40, 1 << 40, 64, 1 << 38, BASE + 64 * MiB,
                                 None) == _lib.E_INVAL
    assert lib.uly_seq_unshard_trim(ctx4.h, BASE, _lib.BF16, huge, 4, 64, 1, BASE + 64 * MiB, None) == _lib.E_INVAL
    assert lib.uly_spatial_split_halo(ctx4.h, BASE, _lib.BF16, 1 << 40, 1 << 40, 64, 0, BASE + 64 * MiB,
                                      None) == _lib.E_INVAL
    assert lib.uly_exchange_chunks(ctx4.h, BASE, BASE + 64 * MiB, 1 << 60, None) == _lib.E_UNSUPPORTED
    cos = np.zeros(4, np.float32)
    fp = cos.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    assert lib.uly_rope_table_1d(fp, fp, huge, 0, 128, 10000.0) == _lib.E_INVAL
    assert lib.uly_rope_table_3d(fp, fp, 1, 0, 128, huge, huge, 16, 24, 24, 10000.0) == _lib.E_INVAL
    # the world size is bounded
    h = ctypes.c_void_p()
    assert lib.uly_create(ctypes.byref(h), -1, 1 << 30, 12) == _lib.E_INVAL


def test_fail_stop_after_launch_failure(lib):
    c = Ctx(lib, 2)
    try:
        q = T(BASE, (1, 8, 4, 64))
        assert lib.uly_debug_fail_launch(c.h, 0) == _lib.OK
        st = scatter(lib, c, q=q, tags=("q", None, None), outs=(BASE + 64 * MiB, None, None))
        assert st == _lib.E_HIP
        # the context is poisoned: every later call refuses, even valid ones
        assert scatter(lib, c, q=q, tags=("q", None, None), outs=(BASE + 64 * MiB, None, None)) == _lib.E_BROKEN
        assert register(lib, c, "z", _lib.MODE_SCATTER, (1, 16, 2, 64), BASE) == _lib.E_BROKEN
        assert lib.uly_wait(c.h, None) == _lib.E_BROKEN
    finally:
        assert lib.uly_destroy(c.h) == _lib.OK      # destroy is still allowed


def test_argument_errors_leave_context_usable(lib, ctx4):
    q = T(BASE, (1, 16, 6, 128))
    assert scatter(lib, ctx4, q=q, tags=("q", None, None), outs=(BASE + 64 * MiB, None, None)) == _lib.E_INVAL
    q = T(BASE, (1, 16, 8, 128))
    assert scatter(lib, ctx4, q=q, tags=("q", None, None), outs=(BASE + 64 * MiB, None, None)) == _lib.E_UNSUPPORTED


def test_pad_and_spatial_rejections(lib, ctx4):
    # P*S_l must cover S
    assert lib.uly_seq_pad_shard(ctx4.h, BASE, _lib.BF16, 1, 100, 64, 24, BASE + 64 * MiB, None) == _lib.E_INVAL
    assert lib.uly_seq_pad_shard(ctx4.h, BASE, _lib.BF16, 1, 100, 64, 25, BASE + 64 * MiB, None) == _lib.E_UNSUPPORTED
    assert lib.uly_seq_pad_shard(ctx4.h, BASE, _lib.BF16, 1, 100, 12, 25, BASE + 64 * MiB, None) == _lib.E_INVAL
    assert lib.uly_seq_pad_shard(ctx4.h, BASE, _lib.BF16, 1, 100, 64, 25, BASE + 4096, None) == _lib.E_OVERLAP
    # spatial: W*2 multiple of 16, height >= P
    assert lib.uly_spatial_split_halo(ctx4.h, BASE, _lib.BF16, 336, 90, 160, 1, BASE + 64 * MiB, None) == _lib.E_UNSUPPORTED
    assert lib.uly_spatial_split_halo(ctx4.h, BASE, _lib.BF16, 336, 90, 150, 1, BASE + 64 * MiB, None) == _lib.E_INVAL
    assert lib.uly_spatial_split_halo(ctx4.h, BASE, _lib.BF16, 336, 3, 160, 1, BASE + 64 * MiB, None) == _lib.E_INVAL


def test_fastdiv_exhaustive_edges(tmp_path):
    """The kernels' division helper against integer division (host compiler)."""
    src = tmp_path / "t.cpp"
    src.write_text(r'''
#include "fastdiv.h"
#include <cstdio>
#include <random>
int main() {
    std::mt19937_64 rng(1);
    const uint32_t ds[] = {1, 2, 3, 5, 6, 7, 24, 40, 48, 96, 128, 160, 200, 4096, 18944, 75600, 75776,
                           65535, 65537, 0x7fffffffu, 0x80000000u, 0x80000001u, 0xfffffffeu, 0xffffffffu};
    long bad = 0;
    for (uint32_t d : ds) {
        uly::FastDiv f = uly::FastDiv::make(d);
        const uint32_t edge[] = {0u, 1u, d - 1, d, d + 1, 2 * d - 1, 0x7fffffffu, 0x80000000u, 0xfffffffeu, 0xffffffffu};
        for (uint32_t n : edge) { uint32_t q, r; f.divmod(n, q, r); bad += (q != n / d) || (r != n % d); }
        for (int i = 0; i < 200000; ++i) { uint32_t n = uint32_t(rng()); uint32_t q, r; f.divmod(n, q, r);
                                           bad += (q != n / d) || (r != n % d); }
    }
    for (int i = 0; i < 2000; ++i) {
        uint32_t d = uint32_t(rng()) >> (rng() % 32); if (!d) d = 1;
        uly::FastDiv f = uly::FastDiv::make(d);
        for (int j = 0; j < 2000; ++j) { uint32_t n = uint32_t(rng()); bad += f.div(n) != n / d; }
    }
    printf("%ld\n", bad);
    return bad != 0;
}
''')
    exe = tmp_path / "t"
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-I", os.path.join(ROOT, "sequence_attention_ulysses_amd", "csrc"),
                           str(src), "-o", str(exe)])
    assert subprocess.check_output([str(exe)]).decode().strip() == "0"


def test_library_rope_tables_match_oracle(orc):
    from sequence_attention_ulysses_amd import rope_table_1d, rope_table_3d
    c, s = rope_table_1d(4096 + 7, 128, real_rows=4096)
    oc, os_ = orc.rope_table_1d(4096 + 7, 128, real_rows=4096)
    # both evaluate in double and round once to fp32; allow one fp32 ulp for libm differences
    np.testing.assert_allclose(c.numpy(), oc, rtol=0, atol=6e-8)
    np.testing.assert_allclose(s.numpy(), os_, rtol=0, atol=6e-8)
    c3, s3 = rope_table_3d(2 * 3600 + 100, 128, 60, 60, real_rows=2 * 3600 + 50)
    oc3, os3 = orc.rope_table_3d(2 * 3600 + 100, 128, 60, 60, real_rows=2 * 3600 + 50)
    np.testing.assert_allclose(c3.numpy(), oc3, rtol=0, atol=6e-8)
    np.testing.assert_allclose(s3.numpy(), os3, rtol=0, atol=6e-8)


def test_python_binding_host_only():
    """The binding marshals arguments only; a host-only context exposes the cache."""
    import warnings

    from sequence_attention_ulysses_amd import UlyssesContext
    c = UlyssesContext(4, device=None)
    assert c.target_count() == 0
    c.close()
    c2 = UlyssesContext(2, device=None)
    with warnings.catch_warnings(record=True) as w:
        warnings.simplefilter("always")
        c2.__del__()
        assert any(issubclass(x.category, ResourceWarning) for x in w)
    c2.close()


def test_binding_table_checks():
    """The three norm + RoPE bindings pass cos's row count for both tables, so they
    refuse tables of different shapes (or the wrong width) before anything else."""
    import torch

    from sequence_attention_ulysses_amd import UlyssesContext
    c = UlyssesContext(2, device=None)
    try:
        q = torch.zeros((2, 1, 8, 2, 128), dtype=torch.bfloat16)
        w = torch.ones(128, dtype=torch.bfloat16)
        x = torch.zeros((2, 1, 8, 256), dtype=torch.bfloat16)
        wqkv = torch.zeros((6 * 128, 256), dtype=torch.bfloat16)
        good = torch.zeros((16, 64), dtype=torch.float32)
        for cos, sin, msg in ((good, torch.zeros((15, 64)), "differ"), (torch.zeros((16, 32)),) * 2 + ("D/2",),
                              (good, good.double(), "fp32")):
            with pytest.raises(ValueError, match=msg):
                c.fused_qkv_norm_rope_scatter_packed(q, q, q, w, w, cos, sin)
            with pytest.raises(ValueError, match=msg):
                c.fused_qkv_proj_norm_rope_scatter(x, wqkv, 2, 2, w, w, cos, sin)
            if msg != "D/2":       # this binding checks the width against each operand later
                with pytest.raises(ValueError, match=msg):
                    c.fused_qk_norm_rope_scatter(q, q, w, w, cos, sin)
    finally:
        c.close()


def test_binding_needs_tag_or_destination():
    """Without an explicit destination a member must name a cached target."""
    import torch

    from sequence_attention_ulysses_amd import UlyssesContext
    c = UlyssesContext(2, device=None)
    try:
        for tag in (None, ""):
            with pytest.raises(ValueError, match="needs a tag"):
                c.target(tag, _lib.MODE_SCATTER, torch.bfloat16, (1, 8, 2, 64))
    finally:
        c.close()


def test_profile_arguments(lib, ctx4):
    assert lib.uly_profile_enable(ctx4.h, 0x3, 0) == _lib.E_INVAL
    assert lib.uly_profile_enable(ctx4.h, 0x3, 4) == _lib.OK
    assert lib.uly_profile_enable(ctx4.h, 0, 1) == _lib.OK
    ms, n = ctypes.c_double(), ctypes.c_int64()
    assert lib.uly_profile_read(ctx4.h, 9, ctypes.byref(ms), ctypes.byref(n)) == _lib.E_INVAL
    assert lib.uly_profile_read(ctx4.h, 1, ctypes.byref(ms), ctypes.byref(n)) == _lib.OK and n.value == 0


# ---------------------------------------------------------------------------
# 1-byte payloads, the packed receive layout, the destination-major exchange
# ---------------------------------------------------------------------------
def test_byte_payloads_accepted_by_relayouts(lib, ctx4):
    """flashinfer UlyssesCommunicator PR, 'What': fp8 / int8 ride as opaque bytes."""
    shape, t_shape = (1, 16, 8, 128), (1, 64, 2, 128)
    assert register(lib, ctx4, "q", _lib.MODE_SCATTER, t_shape, BASE + 64 * MiB, dtype=_lib.U8,
                    nbytes=4 * 64 * 2 * 128) == _lib.OK
    q = T(BASE, shape, dtype=_lib.U8)
    assert scatter(lib, ctx4, q=q, tags=("q", None, None)) == _lib.E_UNSUPPORTED        # would launch
    # a 16-element head row is 16 bytes: the smallest one-byte row
    q16 = T(BASE, (1, 16, 8, 16), dtype=_lib.U8)
    st = scatter(lib, ctx4, q=q16, tags=("q", None, None), outs=(BASE + 64 * MiB, None, None))
    assert st == _lib.E_UNSUPPORTED
    q8 = T(BASE, (1, 16, 8, 8), dtype=_lib.U8)
    st = scatter(lib, ctx4, q=q8, tags=("q", None, None), outs=(BASE + 64 * MiB, None, None))
    assert st == _lib.E_INVAL and b"multiple of 16" in lib.uly_last_error()
    # storage is sized in bytes: the two-byte requirement would be twice as large
    assert register(lib, ctx4, "k", _lib.MODE_SCATTER, t_shape, BASE + 80 * MiB, dtype=_lib.U8,
                    nbytes=4 * 64 * 2 * 128 - 16) == _lib.E_INVAL
    # the overlap check counts bytes too: a destination one byte-slab past the source is fine
    src = T(BASE, shape, dtype=_lib.U8)
    st = scatter(lib, ctx4, q=src, tags=("q", None, None), outs=(BASE + 16 * 8 * 128, None, None))
    assert st == _lib.E_OVERLAP                  # source covers 4 ranks x 16 x 8 x 128 bytes
    st = scatter(lib, ctx4, q=src, tags=("q", None, None), outs=(BASE + 4 * 16 * 8 * 128, None, None))
    assert st == _lib.E_UNSUPPORTED
    o = T(BASE, (1, 64, 2, 128), dtype=_lib.U8)
    assert lib.ulysses_gather_out(ctx4.h, ctypes.byref(o), None, BASE + 64 * MiB, None) == _lib.E_UNSUPPORTED
    assert lib.uly_seq_pad_shard(ctx4.h, BASE, _lib.U8, 1, 100, 16, 25, BASE + 64 * MiB, None) == _lib.E_UNSUPPORTED
    assert lib.uly_seq_pad_shard(ctx4.h, BASE, _lib.U8, 1, 100, 8, 25, BASE + 64 * MiB, None) == _lib.E_INVAL


def test_fused_refuses_byte_payloads(lib, ctx4):
    q, k = T(BASE, (1, 16, 8, 128), dtype=_lib.U8), T(BASE + 64 * MiB, (1, 16, 8, 128), dtype=_lib.U8)
    assert _fused(lib, ctx4, q, k) == _lib.E_UNSUPPORTED and b"16-bit" in lib.uly_last_error()


def _packed(lib, c, q, k, v, out=BASE + 100 * MiB, tag=None, rows=64, eps=1e-6):
    args = [ctypes.byref(x) if x is not None else None for x in (q, k, v)]
    return lib.fused_qkv_norm_rope_scatter_packed(c.h, *args, BASE + 200 * MiB, BASE + 201 * MiB, eps,
                                                  BASE + 300 * MiB, BASE + 310 * MiB, rows,
                                                  tag.encode() if tag else None, out, None)


def test_packed_layout_checks(lib, ctx4):
    shape = (1, 16, 8, 128)
    q, k, v = T(BASE, shape), T(BASE + 64 * MiB, shape), T(BASE + 80 * MiB, shape)
    assert _packed(lib, ctx4, q, k, v) == _lib.E_UNSUPPORTED and b"host-only" in lib.uly_last_error()
    assert _packed(lib, ctx4, q, k, None) == _lib.E_INVAL                      # all three required
    assert _packed(lib, ctx4, None, k, v) == _lib.E_INVAL
    k4 = T(BASE + 64 * MiB, (1, 16, 4, 128))
    assert _packed(lib, ctx4, q, k4, v) == _lib.E_INVAL and b"same head count" in lib.uly_last_error()
    # the one packed target spans P * B * S * Hl * 3D elements: 4*64*2*384*2 bytes
    span = 4 * 64 * 2 * 384 * 2
    v_in_target = T(BASE + 100 * MiB + span - 4096, shape)
    assert _packed(lib, ctx4, q, k, v_in_target) == _lib.E_OVERLAP
    v_after = T(BASE + 100 * MiB + span, shape)
    assert _packed(lib, ctx4, q, k, v_after) == _lib.E_UNSUPPORTED
    # a tagged packed target is keyed by its [B, S, Hl, 3D] shape
    assert _packed(lib, ctx4, q, k, v, out=None, tag="qkv") == _lib.E_NOT_FOUND
    assert register(lib, ctx4, "qkv", _lib.MODE_SCATTER, (1, 64, 2, 128), BASE + 100 * MiB) == _lib.OK
    assert _packed(lib, ctx4, q, k, v, out=None, tag="qkv") == _lib.E_NOT_FOUND
    assert register(lib, ctx4, "qkv", _lib.MODE_SCATTER, (1, 64, 2, 384), BASE + 120 * MiB,
                    nbytes=span) == _lib.OK
    assert _packed(lib, ctx4, q, k, v, out=None, tag="qkv") == _lib.E_UNSUPPORTED


def test_exchange_chunks_checks(lib, ctx4):
    """flashinfer UlyssesCommunicator PR, 'What' (Transforms): a destination-major exchange."""
    ex = lib.uly_exchange_chunks
    assert ex(ctx4.h, BASE, BASE + 64 * MiB, 4096, None) == _lib.E_UNSUPPORTED       # would launch
    assert ex(ctx4.h, BASE, BASE + 64 * MiB, 24, None) == _lib.E_INVAL               # not 16-byte chunks
    assert ex(ctx4.h, BASE, BASE + 64 * MiB, -16, None) == _lib.E_INVAL
    assert ex(ctx4.h, BASE + 8, BASE + 64 * MiB, 16, None) == _lib.E_INVAL          # misaligned
    assert ex(ctx4.h, None, BASE, 16, None) == _lib.E_INVAL
    assert ex(ctx4.h, BASE, BASE + 16 * 4096 - 16, 4096, None) == _lib.E_OVERLAP   # 16 chunks of 4 KiB
    assert ex(ctx4.h, BASE, BASE + 16 * 4096, 4096, None) == _lib.E_UNSUPPORTED


# ---------------------------------------------------------------------------
# QKV projection with the norm + RoPE + scatter epilogue
# ---------------------------------------------------------------------------
def _proj(lib, c, B=1, S_l=16, hidden=256, Hq=8, Hkv=4, D=128, dtype=_lib.BF16, x=BASE,
          w=BASE + 32 * MiB, wn=(BASE + 200 * MiB, BASE + 201 * MiB), eps=1e-6, rows=64,
          tabs=(BASE + 300 * MiB, BASE + 310 * MiB),
          outs=(BASE + 100 * MiB, BASE + 120 * MiB, BASE + 140 * MiB), tags=("q", "k", "v")):
    return lib.fused_qkv_proj_norm_rope_scatter(c.h, x, dtype, B, S_l, hidden, w, Hq, Hkv, D, wn[0], wn[1], eps,
                                                tabs[0], tabs[1], rows, _lib.tags_array(tags),
                                                _lib.ptr_array(outs), None)


def test_projection_ring_hook(lib, ctx4):
    """The test hook that forces the projection's token-row ring depth takes 0, 2 or 3."""
    for depth in (0, 2, 3, 0):
        assert lib.uly_debug_proj_ring(ctx4.h, depth) == _lib.OK
    for depth in (1, 4, -1):
        assert lib.uly_debug_proj_ring(ctx4.h, depth) == _lib.E_INVAL
        assert b"ring depth" in lib.uly_last_error()
    assert lib.uly_debug_proj_ring(None, 0) == _lib.E_INVAL


def test_projection_checks(lib, ctx4):
    """flashinfer PR #6332, 'Description' / 'Assumptions': BF16 operands, head_dim 128,
    heads divisible by the world size, rejected before any launch."""
    assert _proj(lib, ctx4) == _lib.E_UNSUPPORTED and b"host-only" in lib.uly_last_error()
    assert _proj(lib, ctx4, dtype=_lib.F16) == _lib.E_UNSUPPORTED
    assert _proj(lib, ctx4, dtype=_lib.U8) == _lib.E_DTYPE
    assert _proj(lib, ctx4, Hq=6) == _lib.E_INVAL and b"divisible" in lib.uly_last_error()
    assert _proj(lib, ctx4, Hkv=2) == _lib.E_INVAL
    assert _proj(lib, ctx4, Hkv=0) == _lib.E_INVAL
    assert _proj(lib, ctx4, D=64) == _lib.E_UNSUPPORTED and b"head dim" in lib.uly_last_error()
    assert _proj(lib, ctx4, hidden=96) == _lib.E_INVAL                     # not a multiple of 64
    assert _proj(lib, ctx4, hidden=0) == _lib.E_INVAL
    assert _proj(lib, ctx4, eps=0.0) == _lib.E_INVAL
    assert _proj(lib, ctx4, x=BASE + 8) == _lib.E_INVAL                    # misaligned
    assert _proj(lib, ctx4, w=0) == _lib.E_INVAL
    assert _proj(lib, ctx4, wn=(BASE + 200 * MiB, 0)) == _lib.E_INVAL
    assert _proj(lib, ctx4, rows=63) == _lib.E_INVAL                       # positions reach 64
    assert _proj(lib, ctx4, B=-1) == _lib.E_INVAL
    # x spans 4 * 16 * 256 * 2 bytes; a q target inside it is an overlap
    assert _proj(lib, ctx4, outs=(BASE + 4096, BASE + 120 * MiB, BASE + 140 * MiB)) == _lib.E_OVERLAP
    # targets must not overlap each other (q spans 4 * 64 * 2 * 128 * 2 bytes)
    assert _proj(lib, ctx4, outs=(BASE + 100 * MiB, BASE + 100 * MiB + 4096, BASE + 140 * MiB)) == _lib.E_OVERLAP
    # tagged targets: q [1, 64, 2, 128], k and v [1, 64, 1, 128]
    tags = ("pq", "pk", "pv")
    assert _proj(lib, ctx4, outs=(None, None, None), tags=tags) == _lib.E_NOT_FOUND
    for i, (tag, hl) in enumerate(zip(tags, (2, 1, 1))):
        assert register(lib, ctx4, tag, _lib.MODE_SCATTER, (1, 64, hl, 128), BASE + (100 + 20 * i) * MiB) == _lib.OK
    assert _proj(lib, ctx4, outs=(None, None, None), tags=tags) == _lib.E_UNSUPPORTED
    # an empty batch checks everything and launches nothing
    assert _proj(lib, ctx4, B=0) == _lib.E_UNSUPPORTED
