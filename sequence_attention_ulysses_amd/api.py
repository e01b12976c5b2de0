"""Python binding of the Ulysses C ABI (``include/uly.h``).

Argument marshalling only: torch tensors are turned into pointers, strides
and stream handles, and every step of the exchange runs in ``libuly.so``'s
gfx950 kernels.  torch supplies device memory (target storage) and streams.

Operands are rank-major 5-D tensors ``[P, B, S, H, D]`` whose first axis is
the emulated rank; any strides are accepted as long as the head dimension is
contiguous (so a fused QKV projection ``[P, B, S_l, 3, H, D]`` is passed as
its views ``qkv[:, :, :, c]``).
"""
from __future__ import annotations

import ctypes
import math
import warnings

import torch

from . import _lib
from ._lib import check

_DTYPES = {torch.float16: _lib.F16, torch.bfloat16: _lib.BF16}
# 1-byte payloads (fp8, int8) move as opaque bytes
for _name in ("uint8", "int8", "float8_e4m3fn", "float8_e5m2", "float8_e4m3fnuz", "float8_e5m2fnuz"):
    if hasattr(torch, _name):
        _DTYPES[getattr(torch, _name)] = _lib.U8


def _dtype_code(t) -> int:
    dtype = t.dtype if isinstance(t, torch.Tensor) else t
    try:
        return _DTYPES[dtype]
    except KeyError:
        raise TypeError("supported: float16, bfloat16 and 1-byte types; got %s" % dtype) from None


# The current stream's raw handle without building a torch Stream object
# (torch.cuda.current_stream() costs ~3 us a call); torch's own compiled
# kernels read it the same way.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(stream, device=None) -> int:
    """The HIP stream handle of `stream`, or of the current stream of `device`."""
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None and device is not None:
        return _raw_stream(device)
    return torch.cuda.current_stream().cuda_stream


_I64x4 = ctypes.c_int64 * 4


def describe(t: torch.Tensor) -> _lib.UlyTensor:
    """uly_tensor of a rank-major [P, B, S, H, D] tensor (no copy)."""
    if t.dim() != 5:
        raise ValueError("operand must be 5-D [P, B, S, H, D], got shape %s" % (tuple(t.shape),))
    sh, st = t.shape, t.stride()
    return _lib.UlyTensor(t.data_ptr() if t.numel() else 0, _dtype_code(t), 0, st[0],
                          _I64x4(sh[1], sh[2], sh[3], sh[4]), _I64x4(st[1], st[2], st[3], st[4]))


def rope_table_1d(rows: int, D: int, theta: float = 1e4, real_rows: int | None = None):
    """Host fp32 cos/sin tables [rows, D/2] of the 1-D rotary (built by the library)."""
    real_rows = rows if real_rows is None else real_rows
    cos = torch.empty((rows, D // 2), dtype=torch.float32)
    sin = torch.empty((rows, D // 2), dtype=torch.float32)
    check(_lib.load().uly_rope_table_1d(cos.data_ptr(), sin.data_ptr(), rows, real_rows, D, float(theta)),
          "uly_rope_table_1d")
    return cos, sin


def rope_table_3d(rows: int, D: int, grid_h: int, grid_w: int, pairs=(22, 21, 21), theta: float = 1e4,
                  real_rows: int | None = None):
    """Host fp32 cos/sin tables [rows, D/2] of the 3-D (t, h, w) rotary of a row-major latent grid."""
    real_rows = rows if real_rows is None else real_rows
    cos = torch.empty((rows, D // 2), dtype=torch.float32)
    sin = torch.empty((rows, D // 2), dtype=torch.float32)
    check(_lib.load().uly_rope_table_3d(cos.data_ptr(), sin.data_ptr(), rows, real_rows, D, grid_h, grid_w,
                                         pairs[0], pairs[1], pairs[2], float(theta)), "uly_rope_table_3d")
    return cos, sin


def _check_tables(cos, sin, D: int | None) -> None:
    """cos and sin: contiguous fp32 [rows, D/2] of one shape (the library reads `rows` rows of each)."""
    for t in (cos, sin):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or not t.is_contiguous() or t.dim() != 2:
            raise ValueError("cos/sin tables must be contiguous fp32 [rows, D/2]")
    if cos.shape != sin.shape:
        raise ValueError("cos and sin tables differ in shape")
    if D is not None and cos.shape[1] * 2 != D:
        raise ValueError("cos/sin tables must have D/2 columns")


def height_split(Hh: int, P: int):
    """Heights of the P height shards (the first Hh % P ranks take one more row) and hmax."""
    base, extra = divmod(Hh, P)
    return [base + (1 if r < extra else 0) for r in range(P)], -(-Hh // P)


class UlyssesContext:
    """One Ulysses group of ``world_size`` emulated ranks on one GPU.

    Owns the library context (comm stream, events, tagged target cache).
    Targets are allocated by torch on first use of a key and registered with
    the library, so steady-state steps allocate nothing.
    """

    def __init__(self, world_size: int, device: int | None = 0, max_targets: int = 12):
        self._lib = _lib.load()
        self.world_size = int(world_size)
        self.device = device
        self._handle = ctypes.c_void_p()
        dev = -1 if device is None else int(device)
        check(self._lib.uly_create(ctypes.byref(self._handle), dev, self.world_size, int(max_targets)),
              "uly_create")
        self._targets: dict[tuple, torch.Tensor] = {}
        self._closed = False

    # -- lifetime -----------------------------------------------------------
    def close(self) -> None:
        if not self._closed:
            self._closed = True
            st = self._lib.uly_destroy(self._handle)
            self._handle = ctypes.c_void_p()
            self._targets.clear()
            check(st, "uly_destroy")

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        # Warn only; teardown from a finalizer could race the caller's streams.
        if not getattr(self, "_closed", True):
            warnings.warn("UlyssesContext was not closed; call close()", ResourceWarning, stacklevel=2)

    def _h(self):
        if self._closed:
            raise RuntimeError("UlyssesContext is closed")
        return self._handle

    def _on_device(self, *tensors) -> None:
        """Every tensor handed to the library must live on this context's GPU."""
        for t in tensors:
            if t is None:
                continue
            if not isinstance(t, torch.Tensor) or not t.is_cuda or t.get_device() != self.device:
                raise ValueError("tensor must be on cuda:%s, got %s" % (self.device, getattr(t, "device", type(t))))

    def _stream(self, stream) -> int:
        return _stream_handle(stream, self.device)

    @staticmethod
    def _check_out(out: torch.Tensor, like_dtype, numel: int, what: str) -> None:
        """An explicit destination must be contiguous, of the operand dtype and large enough."""
        if out.dtype != like_dtype or not out.is_contiguous() or out.numel() < numel:
            raise ValueError("%s: destination must be a contiguous %s tensor of >= %d elements, got %s %s"
                             % (what, like_dtype, numel, out.dtype, tuple(out.shape)))

    # -- targets ------------------------------------------------------------
    def target(self, tag: str, mode: int, dtype: torch.dtype, shape) -> torch.Tensor:
        """The cached target of (tag, mode, dtype, per-rank shape); allocated once.

        Returns a [P, *shape] view of the registered storage.  When the cache
        is full the returned tensor is a one-shot buffer (not cached).
        """
        if not tag:
            raise ValueError("a cached target needs a tag (or pass an explicit destination)")
        shape = tuple(int(s) for s in shape)
        code = _dtype_code(dtype)
        key = (tag, mode, code, shape)           # the library's key: 1-byte types share one code
        t = self._targets.get(key)
        if t is not None:
            return t if t.dtype == dtype else t.view(dtype)
        numel = self.world_size * math.prod(shape)
        buf = torch.empty(numel, dtype=dtype, device=torch.device("cuda", self.device))
        st = self._lib.uly_target_register(self._h(), tag.encode(), mode, code,
                                           _lib.int64_array(shape), buf.data_ptr(), buf.numel() * buf.element_size())
        view = buf.view((self.world_size,) + shape)
        if st == _lib.E_CACHE_FULL:
            warnings.warn("Ulysses target cache is full; '%s' uses a one-shot buffer" % tag, RuntimeWarning,
                          stacklevel=3)
            return view
        check(st, "uly_target_register")
        self._targets[key] = view
        return view

    def _resolve(self, tag, mode, like: torch.Tensor, shape, out, pending: dict):
        """A member's destination and the pointer the call passes for it.

        An explicit `out` is passed as a pointer.  A key already registered is
        passed as its tag alone (None), so the library resolves it from its cache.
        A new key gets fresh storage, passed as a pointer, and is recorded in
        `pending`: it is registered only once the library has accepted the call
        (`_register`), so a rejected call leaves the cache as it was."""
        if out is not None:
            self._on_device(out)
            self._check_out(out, like.dtype, self.world_size * math.prod(shape), tag or "out")
            return out, out.data_ptr()
        if not tag:
            raise ValueError("a cached target needs a tag (or pass an explicit destination)")
        key = (tag, mode, _dtype_code(like.dtype), shape)
        t = self._targets.get(key)
        if t is not None:
            return (t if t.dtype == like.dtype else t.view(like.dtype)), None
        t = pending.get(key)
        if t is None:
            t = torch.empty((self.world_size,) + shape, dtype=like.dtype,
                            device=torch.device("cuda", self.device))
            pending[key] = t
        return t, t.data_ptr()

    def _register(self, pending: dict) -> None:
        """Register the new targets of a call the library accepted."""
        for key, t in pending.items():
            tag, mode, code, shape = key
            st = self._lib.uly_target_register(self._h(), tag.encode(), mode, code, _lib.int64_array(shape),
                                               t.data_ptr(), t.numel() * t.element_size())
            if st == _lib.E_CACHE_FULL:
                warnings.warn("Ulysses target cache is full; '%s' used a one-shot buffer" % tag, RuntimeWarning,
                              stacklevel=3)
                continue
            check(st, "uly_target_register")
            self._targets[key] = t

    # -- the exchange -----------------------------------------------------------
    def scatter_qkv(self, q=None, k=None, v=None, tags=("q", "k", "v"), out=None, stream=None):
        """Sequence-sharded -> head-sharded for up to three operands, one launch (on the comm
        stream, or on the caller's stream with the "caller" route, see :meth:`set_route`).

        Returns the destination tensors [P, B, P*S_l, H/P, D] (None for absent members).
        Pair with :meth:`wait` before consuming them.
        """
        P = self.world_size
        mem = (q, k, v)
        self._on_device(*mem)
        descs, dests, ptrs, pending = [], [], [], {}
        for i, x in enumerate(mem):
            if x is None:
                descs.append(None); dests.append(None); ptrs.append(None)
                continue
            if x.dim() != 5 or x.shape[3] % P:
                # the library raises the precise error; shape here only sizes the target
                descs.append(describe(x)); dests.append(None); ptrs.append(None)
                continue
            sh = x.shape
            d, ptr = self._resolve(tags[i], _lib.MODE_SCATTER, x, (sh[1], sh[2] * P, sh[3] // P, sh[4]),
                                   None if out is None else out[i], pending)
            descs.append(describe(x)); dests.append(d); ptrs.append(ptr)
        args = [ctypes.byref(dd) if dd is not None else None for dd in descs]
        check(self._lib.ulysses_scatter_qkv(self._h(), *args, _lib.tags_array(tags), _lib.ptr_array(ptrs),
                                            self._stream(stream)), "ulysses_scatter_qkv")
        self._register(pending)
        return dests

    def fused_qk_norm_rope_scatter(self, q, k, w_q, w_k, cos, sin, eps: float = 1e-6, v=None,
                                   tags=("q", "k", "v"), out=None, stream=None):
        """Q/K RMSNorm + interleaved RoPE + scatter, fused in one kernel, on the caller's stream.

        v (optional) is scattered unchanged by the same call: in the same launch for
        interleaved operands, by the relayout kernel right after for dense ones.
        cos/sin: device fp32 [rows >= P*S_l, D/2] tables indexed by global position.
        Returns the destination tensors [P, B, P*S_l, H/P, D] of (q, k, v) (None for absent members).
        """
        P = self.world_size
        mem = (q, k, v)
        _check_tables(cos, sin, None)
        self._on_device(q, k, v, w_q, w_k, cos, sin)
        # every Python-side check before any destination is resolved
        for w, x in ((w_q, q), (w_k, k)):
            if x is not None and w is not None and (w.dtype != x.dtype or not w.is_contiguous()
                                                    or w.numel() != x.shape[-1]):
                raise ValueError("norm weights must be contiguous [D] tensors in the operand dtype")
        for x in (q, k, v):
            if x is not None and x.dim() == 5 and cos.shape[1] * 2 != x.shape[-1]:
                raise ValueError("cos/sin tables must have D/2 columns")
        tags = tuple(tags) + (None,) * (3 - len(tags))
        descs, dests, ptrs, pending = [], [], [], {}
        for i, x in enumerate(mem):
            if x is None:
                descs.append(None); dests.append(None); ptrs.append(None)
                continue
            if x.dim() != 5 or x.shape[3] % P:
                descs.append(describe(x)); dests.append(None); ptrs.append(None)
                continue
            sh = x.shape
            o_i = None if out is None or i >= len(out) else out[i]
            d, ptr = self._resolve(tags[i], _lib.MODE_SCATTER, x, (sh[1], sh[2] * P, sh[3] // P, sh[4]), o_i,
                                   pending)
            descs.append(describe(x)); dests.append(d); ptrs.append(ptr)
        args = [ctypes.byref(dd) if dd is not None else None for dd in descs]
        wq = w_q.data_ptr() if (w_q is not None and q is not None) else None
        wk = w_k.data_ptr() if (w_k is not None and k is not None) else None
        check(self._lib.fused_qk_norm_rope_scatter(self._h(), *args, wq, wk, float(eps), cos.data_ptr(),
                                                   sin.data_ptr(), cos.shape[0], _lib.tags_array(tags),
                                                   _lib.ptr_array(ptrs), self._stream(stream)),
              "fused_qk_norm_rope_scatter")
        self._register(pending)
        return dests

    def fused_qkv_proj_norm_rope_scatter(self, x, w_qkv, Hq: int, Hkv: int, w_q, w_k, cos, sin, eps: float = 1e-6,
                                         tags=("q", "k", "v"), out=None, stream=None):
        """QKV projection + Q/K RMSNorm + RoPE + scatter, one launch on the caller's stream.

        x: [P, B, S_l, hidden] token rows; w_qkv: [(Hq + 2*Hkv) * D, hidden] (q rows, then k,
        then v; no bias); w_q, w_k: [D] norm weights; cos/sin: fp32 [rows >= P*S_l, D/2].
        Returns the destination tensors (q, k, v), [P, B, P*S_l, H/P, D] each.
        """
        P = self.world_size
        _check_tables(cos, sin, w_q.numel())
        self._on_device(x, w_qkv, w_q, w_k, cos, sin)
        if x.dim() != 4 or not x.is_contiguous() or not w_qkv.is_contiguous() or w_qkv.dim() != 2:
            raise ValueError("x must be a contiguous [P, B, S_l, hidden] tensor and w_qkv a contiguous matrix")
        if x.shape[0] != P:
            raise ValueError("x must hold one slab per rank")
        D = w_q.numel()
        if w_qkv.shape != ((Hq + 2 * Hkv) * D, x.shape[3]) or w_qkv.dtype != x.dtype:
            raise ValueError("w_qkv must be [(Hq + 2*Hkv) * D, hidden] in the activation dtype")
        for w in (w_q, w_k):
            if w.dtype != x.dtype or not w.is_contiguous() or w.numel() != D:
                raise ValueError("norm weights must be contiguous [D] tensors in the activation dtype")
        B, S_l = x.shape[1], x.shape[2]
        dests, ptrs, pending = [], [], {}
        for i, H in enumerate((Hq, Hkv, Hkv)):
            if H % P:
                dests.append(None); ptrs.append(None)     # the library raises the precise error
                continue
            o_i = None if out is None else out[i]
            d, ptr = self._resolve(tags[i], _lib.MODE_SCATTER, x, (B, S_l * P, H // P, D), o_i, pending)
            dests.append(d); ptrs.append(ptr)
        check(self._lib.fused_qkv_proj_norm_rope_scatter(
            self._h(), x.data_ptr(), _dtype_code(x), B, S_l, x.shape[3], w_qkv.data_ptr(), Hq, Hkv, D,
            w_q.data_ptr(), w_k.data_ptr(), float(eps), cos.data_ptr(), sin.data_ptr(), cos.shape[0],
            _lib.tags_array(tags), _lib.ptr_array(ptrs), self._stream(stream)), "fused_qkv_proj_norm_rope_scatter")
        self._register(pending)
        return dests

    def fused_qkv_norm_rope_scatter_packed(self, q, k, v, w_q, w_k, cos, sin, eps: float = 1e-6, tag="qkv",
                                           out=None, stream=None):
        """Q/K norm + RoPE scatter with V into one packed target [P, B, P*S_l, H/P, 3*D]:
        each head row holds q, k and v side by side."""
        P = self.world_size
        _check_tables(cos, sin, q.shape[-1])
        self._on_device(q, k, v, w_q, w_k, cos, sin, out)
        for x in (q, k, v):
            if x.dim() != 5:
                raise ValueError("operands must be 5-D [P, B, S_l, H, D]")
        for w in (w_q, w_k):
            if w.dtype != q.dtype or not w.is_contiguous() or w.numel() != q.shape[-1]:
                raise ValueError("norm weights must be contiguous [D] tensors in the operand dtype")
        shape = (q.shape[1], q.shape[2] * P, q.shape[3] // P, 3 * q.shape[4])
        pending = {}
        if out is None and q.shape[3] % P:
            dest, ptr = None, None                        # the library raises the precise error
        else:
            dest, ptr = self._resolve(tag, _lib.MODE_SCATTER, q, shape, out, pending)
        check(self._lib.fused_qkv_norm_rope_scatter_packed(
            self._h(), ctypes.byref(describe(q)), ctypes.byref(describe(k)), ctypes.byref(describe(v)),
            w_q.data_ptr(), w_k.data_ptr(), float(eps), cos.data_ptr(), sin.data_ptr(), cos.shape[0],
            tag.encode() if tag else None, ptr, self._stream(stream)), "fused_qkv_norm_rope_scatter_packed")
        self._register(pending)
        return dest

    def exchange_chunks(self, x, out=None, stream=None):
        """Destination-major chunk exchange: x [P, P, ...] (rank r's chunk for q at x[r, q])
        -> y [P, P, ...] with y[q, r] = x[r, q]; opaque bytes."""
        P = self.world_size
        self._on_device(x, out)
        if x.dim() < 2 or x.shape[0] != P or x.shape[1] != P or not x.is_contiguous():
            raise ValueError("x must be a contiguous [P, P, ...] tensor")
        if out is None:
            out = torch.empty_like(x)
        elif out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous():
            raise ValueError("out must match x")
        chunk = x.numel() * x.element_size() // (P * P)
        check(self._lib.uly_exchange_chunks(self._h(), x.data_ptr() if x.numel() else None,
                                            out.data_ptr() if out.numel() else None, chunk,
                                            self._stream(stream)), "uly_exchange_chunks")
        return out

    def wait(self, stream=None) -> None:
        """Grouped handshake: ``stream`` (default: current) waits for all scatters since the last wait."""
        check(self._lib.uly_wait(self._h(), self._stream(stream)), "uly_wait")

    def gather_out(self, o, tag: str = "out", out=None, stream=None) -> torch.Tensor:
        """Head-sharded [P, B, S, Hl, D] -> sequence-sharded [P, B, S/P, P*Hl, D] on the caller's stream."""
        P = self.world_size
        self._on_device(o, out)
        if o.dim() != 5:
            raise ValueError("operand must be 5-D [P, B, S, Hl, D]")
        sh = o.shape
        shape = (sh[1], sh[2] // P, sh[3] * P, sh[4])
        pending = {}
        if out is None and sh[2] % P:
            dest, ptr = None, None                        # the library raises the precise error
        else:
            dest, ptr = self._resolve(tag, _lib.MODE_GATHER, o, shape, out, pending)
        check(self._lib.ulysses_gather_out(self._h(), ctypes.byref(describe(o)), tag.encode() if tag else None,
                                           ptr, self._stream(stream)), "ulysses_gather_out")
        self._register(pending)
        return dest

    # -- sequence padding ---------------------------------------------------------
    def seq_pad_shard(self, full: torch.Tensor, S_l: int, out=None, stream=None) -> torch.Tensor:
        """full [B, S, *row] -> rank-major [P, B, S_l, *row], zero rows past S."""
        self._on_device(full, out)
        B, S = full.shape[:2]
        row = tuple(full.shape[2:])
        if not full.is_contiguous():
            raise ValueError("full must be contiguous")
        if out is None:
            out = torch.empty((self.world_size, B, S_l) + row, dtype=full.dtype, device=full.device)
        self._check_out(out, full.dtype, self.world_size * B * S_l * math.prod(row), "seq_pad_shard")
        check(self._lib.uly_seq_pad_shard(self._h(), full.data_ptr(), _dtype_code(full), B, S,
                                          math.prod(row), S_l, out.data_ptr(), self._stream(stream)),
              "uly_seq_pad_shard")
        return out

    def seq_unshard_trim(self, x: torch.Tensor, S: int, out=None, stream=None) -> torch.Tensor:
        """rank-major [P, B, S_l, *row] -> [B, S, *row] (concat along the sequence, keep [0, S))."""
        self._on_device(x, out)
        P, B, S_l = x.shape[:3]
        row = tuple(x.shape[3:])
        if not x.is_contiguous() or P != self.world_size:
            raise ValueError("x must be contiguous with P = %d rank slabs" % self.world_size)
        if out is None:
            out = torch.empty((B, S) + row, dtype=x.dtype, device=x.device)
        self._check_out(out, x.dtype, B * S * math.prod(row), "seq_unshard_trim")
        check(self._lib.uly_seq_unshard_trim(self._h(), x.data_ptr(), _dtype_code(x), B, S, math.prod(row),
                                             S_l, out.data_ptr(), self._stream(stream)), "uly_seq_unshard_trim")
        return out

    # -- spatial height shards ----------------------------------------------------
    def spatial_split_halo(self, full: torch.Tensor, halo: int = 1, out=None, stream=None) -> torch.Tensor:
        """full [..., Hh, W] -> shards [P, ..., hmax + 2*halo, W]."""
        self._on_device(full, out)
        if not full.is_contiguous():
            raise ValueError("full must be contiguous")
        lead, (Hh, W) = tuple(full.shape[:-2]), tuple(full.shape[-2:])
        _, hmax = height_split(Hh, self.world_size)
        if out is None:
            out = torch.empty((self.world_size,) + lead + (hmax + 2 * halo, W), dtype=full.dtype,
                              device=full.device)
        self._check_out(out, full.dtype, self.world_size * math.prod(lead) * (hmax + 2 * halo) * W,
                        "spatial_split_halo")
        check(self._lib.uly_spatial_split_halo(self._h(), full.data_ptr(), _dtype_code(full), math.prod(lead),
                                               Hh, W, halo, out.data_ptr(), self._stream(stream)),
              "uly_spatial_split_halo")
        return out

    def spatial_gather_stacked(self, shards: torch.Tensor, Hh: int, halo: int = 1, out=None,
                               stream=None) -> torch.Tensor:
        """shards [P, ..., hmax + 2*halo, W] -> stacked core rows [P, ..., hmax, W] (zero-padded)."""
        self._on_device(shards, out)
        lead, W = tuple(shards.shape[1:-2]), shards.shape[-1]
        _, hmax = height_split(Hh, self.world_size)
        if (not shards.is_contiguous() or shards.shape[0] != self.world_size
                or shards.shape[-2] != hmax + 2 * halo):
            raise ValueError("shards must be contiguous [P, ..., hmax + 2*halo, W]")
        if out is None:
            out = torch.empty((self.world_size,) + lead + (hmax, W), dtype=shards.dtype, device=shards.device)
        self._check_out(out, shards.dtype, self.world_size * math.prod(lead) * hmax * W,
                        "spatial_gather_stacked")
        check(self._lib.uly_spatial_gather_stacked(self._h(), shards.data_ptr(), _dtype_code(shards),
                                                   math.prod(lead), Hh, W, halo, out.data_ptr(),
                                                   self._stream(stream)), "uly_spatial_gather_stacked")
        return out

    def spatial_trim_concat(self, stacked: torch.Tensor, Hh: int, out=None, stream=None) -> torch.Tensor:
        """stacked [P, ..., hmax, W] -> full [..., Hh, W]."""
        self._on_device(stacked, out)
        lead, W = tuple(stacked.shape[1:-2]), stacked.shape[-1]
        _, hmax = height_split(Hh, self.world_size)
        if (not stacked.is_contiguous() or stacked.shape[0] != self.world_size
                or stacked.shape[-2] != hmax):
            raise ValueError("stacked must be contiguous [P, ..., hmax, W]")
        if out is None:
            out = torch.empty(lead + (Hh, W), dtype=stacked.dtype, device=stacked.device)
        self._check_out(out, stacked.dtype, math.prod(lead) * Hh * W, "spatial_trim_concat")
        check(self._lib.uly_spatial_trim_concat(self._h(), stacked.data_ptr(), _dtype_code(stacked),
                                                math.prod(lead), Hh, W, out.data_ptr(), self._stream(stream)),
              "uly_spatial_trim_concat")
        return out

    # -- measurement --------------------------------------------------------------
    def profile(self, on: bool = True, kinds=None, every: int = 1) -> None:
        """Bracket launches with timing events: all kinds, or only `kinds` (names of KERNEL_KINDS);
        one launch in `every` of each kind is timed."""
        if not on:
            mask = 0
        elif kinds is None:
            mask = (1 << len(_lib.KERNEL_KINDS)) - 1
        else:
            mask = 0
            for k in kinds:
                mask |= 1 << _lib.KERNEL_KINDS[k]
        check(self._lib.uly_profile_enable(self._h(), mask, int(every)), "uly_profile_enable")

    def profile_read(self, kind: str):
        """(summed kernel ms, launches) of one kernel kind since the last reset."""
        ms = ctypes.c_double()
        n = ctypes.c_int64()
        check(self._lib.uly_profile_read(self._h(), _lib.KERNEL_KINDS[kind], ctypes.byref(ms), ctypes.byref(n)),
              "uly_profile_read")
        return ms.value, n.value

    def profile_reset(self) -> None:
        check(self._lib.uly_profile_reset(self._h()), "uly_profile_reset")

    def stats(self) -> dict:
        s = _lib.UlyStats()
        check(self._lib.uly_get_stats(self._h(), ctypes.byref(s)), "uly_get_stats")
        return {f: getattr(s, f) for f, _ in s._fields_}

    def target_count(self) -> int:
        n = ctypes.c_int()
        check(self._lib.uly_target_count(self._h(), ctypes.byref(n)), "uly_target_count")
        return n.value

    def comm_stream_handle(self) -> int:
        h = ctypes.c_void_p()
        check(self._lib.uly_comm_stream(self._h(), ctypes.byref(h)), "uly_comm_stream")
        return h.value or 0

    def set_route(self, route: str) -> None:
        """How scatter_qkv moves its operands: "kernel" (compute units, comm stream),
        "copy_engine" (copy engines, comm stream) or "caller" (compute units, caller stream)."""
        code = {"kernel": _lib.ROUTE_KERNEL, "copy_engine": _lib.ROUTE_COPY_ENGINE,
                "caller": _lib.ROUTE_CALLER}[route]
        check(self._lib.uly_set_route(self._h(), code), "uly_set_route")

    def debug_fail_launch(self, after: int = 0) -> None:
        check(self._lib.uly_debug_fail_launch(self._h(), int(after)), "uly_debug_fail_launch")

    def debug_proj_ring(self, depth: int = 0) -> None:
        """Test hook: force the projection's token-row ring depth (2 or 3), or 0 for automatic."""
        check(self._lib.uly_debug_proj_ring(self._h(), int(depth)), "uly_debug_proj_ring")
