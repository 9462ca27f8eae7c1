"""Split-KV grouped-query decode attention for MI355X (gfx950).

Thin ctypes binding of ``libsplitkv.so`` (C ABI in ``include/splitkv.h`` and
``include/splitkv_probe.h``). It only marshals arguments: it checks that the
torch tensors have the dtype, device, contiguity and sizes the C ABI expects,
passes their device pointers and the current HIP stream, and turns a negative
status into ``SplitKVError``. Every step of the computation runs in the HIP
kernels. There is no fallback: if the library is missing, every call raises.

Names follow the C ABI (``splitkv_`` dropped): ``decode_attn``,
``decode_attn_noalloc``, ``decode_step``, ``decode_attn_rows``,
``partial``, ``partial_rows``,
``partial_per_head``, ``combine``, ``append_kv``, ``partials_bytes``,
``pick_splits``, ``pick_splits_rows``, ``workgroups_per_cu``, ``strerror``,
``probe_read``, ``probe_copy``.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

__all__ = ["SplitKVError", "load", "abi_version", "strerror", "partials_bytes",
           "pick_splits", "pick_splits_rows", "partial", "partial_per_head",
           "partial_rows", "combine", "decode_attn", "decode_attn_noalloc",
           "decode_attn_rows", "NOALLOC_SCRATCH_BYTES",
           "decode_step", "append_kv", "workgroups_per_cu", "probe_read",
           "probe_copy", "LIB_PATH", "SUPPORTED_HEAD_DIMS", "MAX_GROUP"]

# SPLITKV_LIB names another build of the same library (the sanitizer build of
# `python -m decode_attention_gqa_amd.build --sanitize`); unset, the in-tree
# build is used.
LIB_PATH = os.environ.get("SPLITKV_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libsplitkv.so")
SUPPORTED_HEAD_DIMS = (8, 16, 32, 64, 128, 256)
MAX_GROUP = 8
ABI_VERSION = 3
NOALLOC_SCRATCH_BYTES = 16 << 20   # SPLITKV_NOALLOC_SCRATCH_BYTES

_lock = threading.Lock()
_lib = None

_vp = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t
_f = ctypes.c_float

# (name, restype, argtypes) of every symbol the headers declare.
SIGNATURES = {
    "splitkv_abi_version": (_i, []),
    "splitkv_strerror": (ctypes.c_char_p, [_i]),
    "splitkv_partials_bytes": (_sz, [_i, _i, _i, _i]),
    "splitkv_workgroups_per_cu": (_i, [_i, _i]),
    "splitkv_pick_splits": (_i, [_i, _i, _i, _i, _i, _i,
                                 ctypes.POINTER(_i), ctypes.POINTER(_i)]),
    "splitkv_pick_splits_rows": (_i, [_i, _i, _i, _i, _i, _i, _i,
                                      ctypes.POINTER(_i), ctypes.POINTER(_i)]),
    "splitkv_partial": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i,
                             _i, _f, _vp]),
    "splitkv_partial_rows": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i,
                                  _i, _i, _i, _f, _vp]),
    "splitkv_decode_attn_rows": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i,
                                      _i, _i, _i, _i, _i, _f, _vp]),
    "splitkv_partial_per_head": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i,
                                      _i, _i, _i, _f, _vp]),
    "splitkv_combine": (_i, [_vp, _vp, _i, _i, _i, _i, _vp]),
    "splitkv_decode_attn": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i,
                                 _i, _i, _i, _f, _vp]),
    "splitkv_decode_attn_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i,
                                         _i, _i, _i, _i, _f, _vp]),
    "splitkv_append_kv": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i,
                               _vp]),
    "splitkv_decode_step": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i,
                                 _i, _i, _i, _i, _i, _i, _f, _vp]),
    "splitkv_probe_read": (_i, [_vp, _sz, _vp, _i, _vp]),
    "splitkv_probe_copy": (_i, [_vp, _vp, _sz, _i, _vp]),
}


class SplitKVError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {strerror(status)} (status {status})")


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libsplitkv.so; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None and path == LIB_PATH:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with "
                "`python -m decode_attention_gqa_amd.build` (no fallback "
                "implementation exists)")
        # torch ships its own HIP runtime under the system runtime's soname.
        # Loaded first, the library would pull in the system runtime and
        # torch would then load a second one: kernels registered in one,
        # streams and memory from the other, and every launch fails. With
        # torch loaded first the library binds to torch's runtime.
        _torch()
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if lib.splitkv_abi_version() != ABI_VERSION:
            raise RuntimeError("libsplitkv.so ABI version mismatch")
        if path == LIB_PATH:
            _lib = lib
        return lib


def abi_version() -> int:
    return int(load().splitkv_abi_version())


def strerror(status: int) -> str:
    try:
        return load().splitkv_strerror(int(status)).decode()
    except RuntimeError:
        return f"status {status}"


def _check(status: int, what: str) -> None:
    if status != 0:
        raise SplitKVError(status, what)


def partials_bytes(batch: int, n_head: int, head_dim: int, n_splits: int) -> int:
    return int(load().splitkv_partials_bytes(batch, n_head, head_dim, n_splits))


def workgroups_per_cu(head_dim: int, group: int) -> int:
    """Resident partial-kernel workgroups per compute unit (0: unsupported)."""
    return load().splitkv_workgroups_per_cu(head_dim, group)


def pick_splits(batch: int, n_head: int, n_kv_head: int, head_dim: int,
                max_ctx: int, cu_count: int) -> tuple[int, int]:
    """(n_splits, block_len) chosen by the library's split heuristic."""
    s = _i(0)
    blk = _i(0)
    _check(load().splitkv_pick_splits(batch, n_head, n_kv_head, head_dim,
                                      max_ctx, cu_count, ctypes.byref(s),
                                      ctypes.byref(blk)), "pick_splits")
    return s.value, blk.value


def pick_splits_rows(batch: int, n_q: int, n_head: int, n_kv_head: int,
                     head_dim: int, max_ctx: int,
                     cu_count: int) -> tuple[int, int]:
    """(n_splits, block_len) for n_q query rows per sequence."""
    s = _i(0)
    blk = _i(0)
    _check(load().splitkv_pick_splits_rows(batch, n_q, n_head, n_kv_head,
                                           head_dim, max_ctx, cu_count,
                                           ctypes.byref(s), ctypes.byref(blk)),
           "pick_splits_rows")
    return s.value, blk.value


# -- torch marshalling ----------------------------------------------------
def _torch():
    import torch
    return torch


def _stream_ptr(stream) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _need(t, dtypes, what):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{what} must be on a GPU device")
    if t.dtype not in dtypes:
        raise TypeError(f"{what} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t.data_ptr()


def _shapes(q, k_cache, v_cache, positions):
    torch = _torch()
    _need(q, (torch.float32,), "q")
    _need(k_cache, (torch.float16, torch.int16, torch.uint16), "k_cache")
    _need(v_cache, (torch.float16, torch.int16, torch.uint16), "v_cache")
    _need(positions, (torch.int32,), "positions")
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [B][n_head][hd], k_cache [B][max_ctx][n_kv_head][hd]")
    B, nh, hd = q.shape
    kb, max_ctx, nkvh, khd = k_cache.shape
    if kb != B or khd != hd or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("q, k_cache and v_cache shapes disagree")
    if positions.numel() != B:
        raise ValueError("positions must hold one entry per sequence")
    return B, nh, nkvh, hd, max_ctx


def _partials_ok(partials, B, nh, hd, n_splits):
    torch = _torch()
    _need(partials, (torch.float32,), "partials")
    need = partials_bytes(B, nh, hd, n_splits)
    if partials.numel() * 4 < need:
        raise ValueError(f"partials holds {partials.numel() * 4} bytes, "
                         f"needs {need}")


def partial(q, k_cache, v_cache, positions, partials, n_splits: int,
            block_len: int = 0, scale: float | None = None, stream=None):
    """Partial kernel only (records into ``partials``)."""
    B, nh, nkvh, hd, max_ctx = _shapes(q, k_cache, v_cache, positions)
    _partials_ok(partials, B, nh, hd, n_splits)
    scale = 1.0 / math.sqrt(hd) if scale is None else float(scale)
    _check(load().splitkv_partial(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        positions.data_ptr(), partials.data_ptr(), B, nh, nkvh, hd, max_ctx,
        n_splits, block_len, scale, _stream_ptr(stream)), "splitkv_partial")


def _rows_shapes(q, k_cache, v_cache, positions):
    torch = _torch()
    _need(q, (torch.float32,), "q")
    if q.dim() != 4:
        raise ValueError("q must be [B][n_q][n_head][hd]")
    B, n_q, nh, hd = q.shape
    _need(k_cache, (torch.float16, torch.int16, torch.uint16), "k_cache")
    _need(v_cache, (torch.float16, torch.int16, torch.uint16), "v_cache")
    _need(positions, (torch.int32,), "positions")
    if k_cache.dim() != 4:
        raise ValueError("k_cache must be [B][max_ctx][n_kv_head][hd]")
    kb, max_ctx, nkvh, khd = k_cache.shape
    if kb != B or khd != hd or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("q, k_cache and v_cache shapes disagree")
    if positions.numel() != B:
        raise ValueError("positions must hold one entry per sequence")
    return B, n_q, nh, nkvh, hd, max_ctx


def partial_rows(q, k_cache, v_cache, positions, partials, n_splits: int,
                 block_len: int = 0, scale: float | None = None, stream=None):
    """Partial kernel for several query rows per sequence (q [B][n_q][nh][hd],
    causal within the rows; the records of ``partial`` with n_q*nh heads)."""
    B, n_q, nh, nkvh, hd, max_ctx = _rows_shapes(q, k_cache, v_cache, positions)
    _partials_ok(partials, B, n_q * nh, hd, n_splits)
    scale = 1.0 / math.sqrt(hd) if scale is None else float(scale)
    _check(load().splitkv_partial_rows(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        positions.data_ptr(), partials.data_ptr(), B, n_q, nh, nkvh, hd,
        max_ctx, n_splits, block_len, scale, _stream_ptr(stream)),
        "splitkv_partial_rows")


def decode_attn_rows(q, k_cache, v_cache, positions, partials, out,
                     n_splits: int, block_len: int = 0,
                     scale: float | None = None, stream=None):
    """Several query rows per sequence: partial then combine; out
    [B][n_q][n_head][hd]."""
    torch = _torch()
    B, n_q, nh, nkvh, hd, max_ctx = _rows_shapes(q, k_cache, v_cache, positions)
    _partials_ok(partials, B, n_q * nh, hd, n_splits)
    _need(out, (torch.float32,), "out")
    if tuple(out.shape) != (B, n_q, nh, hd):
        raise ValueError("out must be [B][n_q][n_head][hd]")
    scale = 1.0 / math.sqrt(hd) if scale is None else float(scale)
    _check(load().splitkv_decode_attn_rows(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        positions.data_ptr(), partials.data_ptr(), out.data_ptr(), B, n_q, nh,
        nkvh, hd, max_ctx, n_splits, block_len, scale, _stream_ptr(stream)),
        "splitkv_decode_attn_rows")


def partial_per_head(q, k_cache, v_cache, positions, partials, n_splits: int,
                     block_len: int = 0, scale: float | None = None,
                     stream=None):
    """Partial kernel, per-query-head grid (A/B baseline; same records)."""
    B, nh, nkvh, hd, max_ctx = _shapes(q, k_cache, v_cache, positions)
    _partials_ok(partials, B, nh, hd, n_splits)
    scale = 1.0 / math.sqrt(hd) if scale is None else float(scale)
    _check(load().splitkv_partial_per_head(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        positions.data_ptr(), partials.data_ptr(), B, nh, nkvh, hd, max_ctx,
        n_splits, block_len, scale, _stream_ptr(stream)),
        "splitkv_partial_per_head")


def combine(partials, out, n_splits: int, stream=None):
    """Combine kernel only: merges ``partials`` into ``out`` [B][n_head][hd]."""
    torch = _torch()
    _need(out, (torch.float32,), "out")
    if out.dim() != 3:
        raise ValueError("out must be [B][n_head][hd]")
    B, nh, hd = out.shape
    _partials_ok(partials, B, nh, hd, n_splits)
    _check(load().splitkv_combine(partials.data_ptr(), out.data_ptr(), B, nh,
                                  hd, n_splits, _stream_ptr(stream)),
           "splitkv_combine")


def decode_attn(q, k_cache, v_cache, positions, partials, out, n_splits: int,
                block_len: int = 0, scale: float | None = None, stream=None):
    """Whole operation: partial kernel then combine kernel on one stream."""
    torch = _torch()
    B, nh, nkvh, hd, max_ctx = _shapes(q, k_cache, v_cache, positions)
    _partials_ok(partials, B, nh, hd, n_splits)
    _need(out, (torch.float32,), "out")
    if tuple(out.shape) != (B, nh, hd):
        raise ValueError("out must be [B][n_head][hd]")
    scale = 1.0 / math.sqrt(hd) if scale is None else float(scale)
    _check(load().splitkv_decode_attn(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        positions.data_ptr(), partials.data_ptr(), out.data_ptr(), B, nh, nkvh,
        hd, max_ctx, n_splits, block_len, scale, _stream_ptr(stream)),
        "splitkv_decode_attn")


def decode_attn_noalloc(q, k_cache, v_cache, positions, out, n_splits: int,
                        block_len: int = 0, scale: float | None = None,
                        stream=None):
    """decode_attn without a caller records buffer: the library keeps the
    split records in its own device scratch (NOALLOC_SCRATCH_BYTES per GPU,
    shared by every call on that GPU: calls that overlap on one GPU race)."""
    torch = _torch()
    B, nh, nkvh, hd, max_ctx = _shapes(q, k_cache, v_cache, positions)
    _need(out, (torch.float32,), "out")
    if tuple(out.shape) != (B, nh, hd):
        raise ValueError("out must be [B][n_head][hd]")
    scale = 1.0 / math.sqrt(hd) if scale is None else float(scale)
    _check(load().splitkv_decode_attn_noalloc(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        positions.data_ptr(), out.data_ptr(), B, nh, nkvh, hd, max_ctx,
        n_splits, block_len, scale, _stream_ptr(stream)),
        "splitkv_decode_attn_noalloc")


def append_kv(k_new, v_new, k_cache, v_cache, positions, stream=None):
    """KV-cache append: new fp32 rows [B][n_rows][n_kv_head][hd] into the
    fp16 caches [B][max_ctx][n_kv_head][hd]; the last new row of sequence b
    lands at positions[b] (read on the device)."""
    torch = _torch()
    _need(k_new, (torch.float32,), "k_new")
    _need(v_new, (torch.float32,), "v_new")
    _need(k_cache, (torch.float16, torch.int16, torch.uint16), "k_cache")
    _need(v_cache, (torch.float16, torch.int16, torch.uint16), "v_cache")
    _need(positions, (torch.int32,), "positions")
    if k_new.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("k_new must be [B][n_rows][n_kv_head][hd], "
                         "k_cache [B][max_ctx][n_kv_head][hd]")
    B, n_rows, nkvh, hd = k_new.shape
    kb, max_ctx, knh, khd = k_cache.shape
    if (tuple(v_new.shape) != tuple(k_new.shape) or
            tuple(v_cache.shape) != tuple(k_cache.shape) or
            (kb, knh, khd) != (B, nkvh, hd)):
        raise ValueError("k_new, v_new, k_cache and v_cache shapes disagree")
    if positions.numel() != B:
        raise ValueError("positions must hold one entry per sequence")
    _check(load().splitkv_append_kv(
        k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(),
        v_cache.data_ptr(), positions.data_ptr(), B, n_rows, nkvh, hd, max_ctx,
        _stream_ptr(stream)), "splitkv_append_kv")


def decode_step(q, k_new, v_new, k_cache, v_cache, positions, partials, out,
                n_splits: int, block_len: int = 0, scale: float | None = None,
                stream=None):
    """One decode step: the new fp32 rows [B][1][n_kv_head][hd] go into the
    fp16 caches at positions[b], then attention over rows [0, positions[b]]
    (the append folded into the partial kernel for hd 64/128/256)."""
    torch = _torch()
    B, nh, nkvh, hd, max_ctx = _shapes(q, k_cache, v_cache, positions)
    _partials_ok(partials, B, nh, hd, n_splits)
    _need(out, (torch.float32,), "out")
    if tuple(out.shape) != (B, nh, hd):
        raise ValueError("out must be [B][n_head][hd]")
    _need(k_new, (torch.float32,), "k_new")
    _need(v_new, (torch.float32,), "v_new")
    if (tuple(k_new.shape) != (B, 1, nkvh, hd) or
            tuple(v_new.shape) != (B, 1, nkvh, hd)):
        raise ValueError("k_new and v_new must be [B][1][n_kv_head][hd]")
    scale = 1.0 / math.sqrt(hd) if scale is None else float(scale)
    _check(load().splitkv_decode_step(
        q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(),
        v_cache.data_ptr(), positions.data_ptr(), partials.data_ptr(),
        out.data_ptr(), B, nh, nkvh, hd, max_ctx, n_splits, block_len, scale,
        _stream_ptr(stream)), "splitkv_decode_step")


def probe_read(buf, sink, grid: int, stream=None):
    """HBM read-stream probe over ``buf`` (also the Infinity Cache flush)."""
    torch = _torch()
    _need(sink, (torch.int32, torch.uint32), "sink")
    if sink.numel() < grid:
        raise ValueError("sink must hold `grid` words")
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous tensor on a GPU device")
    nbytes = buf.numel() * buf.element_size()
    _check(load().splitkv_probe_read(buf.data_ptr(), nbytes, sink.data_ptr(),
                                     grid, _stream_ptr(stream)), "probe_read")


def probe_copy(src, dst, grid: int, stream=None):
    """Plain 16-byte copy of ``src`` into ``dst`` (same byte size)."""
    if not (src.is_cuda and dst.is_cuda and src.is_contiguous() and
            dst.is_contiguous()):
        raise ValueError("src and dst must be contiguous tensors on a GPU "
                         "device")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst is smaller than src")
    _check(load().splitkv_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes,
                                     grid, _stream_ptr(stream)), "probe_copy")
