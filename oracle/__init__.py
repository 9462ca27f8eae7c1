"""fp64 CPU oracle for split-KV grouped-query decode attention (ctypes binding).

TEST INFRASTRUCTURE ONLY: the test-suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers. The product path never
imports this package, and this package never imports the product package.

The arithmetic lives in ``oracle.c`` (plain C, double precision, one thread);
this module only builds it with gcc and marshals numpy arrays. Each function
cites the page passage it follows:

* "10 · R4 — decode split-attention dim-parallel rewrite", sections 2.1
  (definition, online-softmax triple, combine), 2.2 (live length from
  ``positions[0] + 1``, split rule, idle splits) and 3.2 (record layout).
* "Red Lite dev35 — long-context decode: grouped split-K attention", section
  Change (one workgroup per block and KV head, fixed block length).
* dotLLM issue #199 (tensor-core decode attention), comment 1: section 1 (the
  half-precision cache update ahead of attention in a decode step) and
  section 2 (several query rows with a causal mask from positionOffset).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# SPLITKV_ORACLE_LIB names a prebuilt copy (the sanitizer build); it is used
# as is, never rebuilt.
_ENV_LIB = os.environ.get("SPLITKV_ORACLE_LIB")
_lock = threading.Lock()
_lib = None

_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")


def build(out_path: str = _LIB, extra_flags: tuple = (),
          cc: str = "gcc") -> str:
    """Compile oracle.c (no fast-math: IEEE double throughout)."""
    cmd = [cc, "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
           *extra_flags, "-o", out_path, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return out_path


def load(path: str | None = None):
    """Load liboracle.so, building it first if it is missing."""
    global _lib
    with _lock:
        if path is None and _lib is not None:
            return _lib
        p = path or _ENV_LIB or _LIB
        if p == _ENV_LIB and path is None:
            if not os.path.exists(p):
                raise RuntimeError(f"SPLITKV_ORACLE_LIB={p} does not exist")
        elif not os.path.exists(p) or (
                path is None and os.path.getmtime(p) < os.path.getmtime(_SRC)):
            build(p)
        lib = ctypes.CDLL(p)
        lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_f64.restype = ctypes.c_double
        lib.oracle_live_length.argtypes = [ctypes.c_int32, ctypes.c_int32]
        lib.oracle_live_length.restype = ctypes.c_int
        lib.oracle_split_bounds.argtypes = [ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, _i32p, _i32p]
        lib.oracle_split_bounds.restype = None
        lib.oracle_decode_attn.argtypes = [
            _f32p, _u16p, _u16p, _i32p, _f64p, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float, _f64p]
        lib.oracle_decode_attn.restype = None
        lib.oracle_split_partials.argtypes = [
            _f32p, _u16p, _u16p, _i32p, _f64p, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_float, _f64p, _i32p]
        lib.oracle_split_partials.restype = None
        lib.oracle_combine.argtypes = [_f64p, _f64p, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int]
        lib.oracle_combine.restype = None
        lib.oracle_f32_to_f16.argtypes = [ctypes.c_float]
        lib.oracle_f32_to_f16.restype = ctypes.c_uint16
        lib.oracle_f32_to_f16_array.argtypes = [_f32p, _u16p, ctypes.c_size_t]
        lib.oracle_f32_to_f16_array.restype = None
        lib.oracle_append_kv.argtypes = [_f32p, _f32p, _u16p, _u16p, _i32p,
                                         ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int]
        lib.oracle_append_kv.restype = None
        lib.oracle_decode_attn_rows.argtypes = [
            _f32p, _u16p, _u16p, _i32p, _f64p, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_float, _f64p]
        lib.oracle_decode_attn_rows.restype = None
        if path is None:
            _lib = lib
        return lib


def _u16(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    return np.ascontiguousarray(a, dtype=np.uint16)


def f16_to_f64(bits, lib=None) -> np.ndarray:
    """Decode binary16 bit patterns with the oracle's own decoder."""
    lib = lib or load()
    flat = _u16(bits).ravel()
    out = np.array([lib.oracle_f16_to_f64(int(x)) for x in flat], np.float64)
    return out.reshape(np.shape(bits))


def live_length(position: int, max_ctx: int, lib=None) -> int:
    lib = lib or load()
    return int(lib.oracle_live_length(int(position), int(max_ctx)))


def split_bounds(nkv: int, n_splits: int, block_len: int = 0, lib=None):
    """(lo, hi) int32 arrays of length n_splits (R4 2.2; Red Lite Change)."""
    lib = lib or load()
    lo = np.zeros(n_splits, np.int32)
    hi = np.zeros(n_splits, np.int32)
    lib.oracle_split_bounds(int(nkv), int(n_splits), int(block_len), lo, hi)
    return lo, hi


def _shapes(q, k_cache, positions, n_kv_head):
    q = np.ascontiguousarray(q, dtype=np.float32)
    batch, n_head, head_dim = q.shape
    kb, max_ctx, nkvh, hd = k_cache.shape
    assert kb == batch and nkvh == n_kv_head and hd == head_dim
    assert n_head % n_kv_head == 0
    pos = np.ascontiguousarray(positions, dtype=np.int32).reshape(batch)
    return q, pos, batch, n_head, head_dim, max_ctx


def decode_attn(q, k_cache, v_cache, positions, n_kv_head: int, scale: float,
                lib=None) -> np.ndarray:
    """Unsplit softmax attention in double: out[b][h][d] (R4 2.1).

    q: fp32 [B][n_head][hd]; k_cache, v_cache: fp16 (or uint16 bits)
    [B][max_ctx][n_kv_head][hd]; positions: int32 [B].
    """
    lib = lib or load()
    q, pos, B, nh, hd, max_ctx = _shapes(q, k_cache, positions, n_kv_head)
    k = _u16(k_cache)
    v = _u16(v_cache)
    out = np.zeros((B, nh, hd), np.float64)
    work = np.zeros(max(max_ctx, 1), np.float64)
    lib.oracle_decode_attn(q, k, v, pos, out, B, nh, n_kv_head, hd, max_ctx,
                           float(np.float32(scale)), work)
    return out


def split_partials(q, k_cache, v_cache, positions, n_kv_head: int,
                   scale: float, n_splits: int, block_len: int = 0,
                   lib=None) -> np.ndarray:
    """Split records [B][S][n_head][4+hd] in double (R4 2.1, 2.2, 3.2)."""
    lib = lib or load()
    q, pos, B, nh, hd, max_ctx = _shapes(q, k_cache, positions, n_kv_head)
    k = _u16(k_cache)
    v = _u16(v_cache)
    rec = np.zeros((B, n_splits, nh, 4 + hd), np.float64)
    work = np.zeros(max(max_ctx, 1), np.float64)
    lohi = np.zeros(2 * n_splits, np.int32)
    lib.oracle_split_partials(q, k, v, pos, rec, B, nh, n_kv_head, hd, max_ctx,
                              int(n_splits), int(block_len),
                              float(np.float32(scale)), work, lohi)
    return rec


def combine(records, lib=None) -> np.ndarray:
    """Merge split records [B][S][n_head][4+hd] into out[B][n_head][hd]."""
    lib = lib or load()
    rec = np.ascontiguousarray(records, dtype=np.float64)
    B, S, nh, pstr = rec.shape
    hd = pstr - 4
    out = np.zeros((B, nh, hd), np.float64)
    lib.oracle_combine(rec, out, B, S, nh, hd)
    return out


def f32_to_f16(x, lib=None) -> np.ndarray:
    """binary32 -> binary16 bits, round to nearest even (the oracle's own
    conversion; #199 section 1 stores the cache in FP16)."""
    lib = lib or load()
    a = np.ascontiguousarray(x, dtype=np.float32)
    out = np.zeros(a.shape, np.uint16)
    lib.oracle_f32_to_f16_array(a.ravel(), out.ravel(), a.size)
    return out


def append_kv(k_new, v_new, k_cache, v_cache, positions, lib=None):
    """Caches after appending the new rows (#199 section 1): returns new
    (k_cache, v_cache) uint16 arrays; the inputs are not modified.

    k_new, v_new: fp32 [B][n_rows][n_kv_head][hd]; caches [B][max_ctx][nkvh][hd];
    the last new row of sequence b lands at positions[b]."""
    lib = lib or load()
    kn = np.ascontiguousarray(k_new, dtype=np.float32)
    vn = np.ascontiguousarray(v_new, dtype=np.float32)
    B, n_rows, nkvh, hd = kn.shape
    assert vn.shape == kn.shape
    k = _u16(k_cache).copy()
    v = _u16(v_cache).copy()
    kb, max_ctx, knh, khd = k.shape
    assert (kb, knh, khd) == (B, nkvh, hd) and v.shape == k.shape
    pos = np.ascontiguousarray(positions, dtype=np.int32).reshape(B)
    lib.oracle_append_kv(kn, vn, k, v, pos, B, n_rows, nkvh, hd, max_ctx)
    return k, v


def decode_attn_rows(q, k_cache, v_cache, positions, n_kv_head: int,
                     scale: float, lib=None) -> np.ndarray:
    """Several query rows per sequence with the causal mask of #199 section 2:
    q fp32 [B][n_q][n_head][hd] -> out[B][n_q][n_head][hd] in double; row t
    of sequence b sits at positions[b] - (n_q - 1 - t)."""
    lib = lib or load()
    q = np.ascontiguousarray(q, dtype=np.float32)
    B, n_q, nh, hd = q.shape
    kb, max_ctx, nkvh, khd = k_cache.shape
    assert kb == B and nkvh == n_kv_head and khd == hd and nh % nkvh == 0
    pos = np.ascontiguousarray(positions, dtype=np.int32).reshape(B)
    out = np.zeros((B, n_q, nh, hd), np.float64)
    work = np.zeros(max(max_ctx, 1), np.float64)
    lib.oracle_decode_attn_rows(q, _u16(k_cache), _u16(v_cache), pos, out, B,
                                n_q, nh, n_kv_head, hd, max_ctx,
                                float(np.float32(scale)), work)
    return out
