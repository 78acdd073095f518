"""fp64 CPU oracle for SAGA + Atop-N decode attention (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product
path (the HIP library and its binding) never imports it, and it imports
nothing from the product.

The arithmetic lives in ``oracle.c`` (plain C, double precision); this module
only builds that file with gcc and marshals numpy arrays.  Every function
takes bf16 data as ``uint16`` bit patterns, exactly the values the device
sees; the ``*_e4m3k`` variants take an fp8 E4M3 key cache as ``uint8`` codes
with one fp32 scale per (batch row, key head), and the ``*_e4m3kv`` variants
also an E4M3 value cache with one scale per (batch row, value head).  Citations of the pages are in
``oracle.c`` next to each function.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# The mutation tests point a child process at a deliberately broken build.
_LIB = os.environ.get("SAGA_ORACLE_LIBRARY", _LIB)


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc (OpenMP, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
             "-o", tmp, _SRC, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        i32, i64, dbl, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        lib.oracle_logits.argtypes = [i32, i32, i32, i32, i32, i64, i64, dbl, vp, vp, vp, i32]
        lib.oracle_nth_largest.argtypes = [vp, i64, i64]
        lib.oracle_nth_largest.restype = dbl
        lib.oracle_atopn_run.argtypes = [i32, i32, i32, i32, i32, i32, i64, i32, vp, dbl, i64,
                                         i64, vp, vp, vp, vp, vp, vp, vp, vp, i32]
        lib.oracle_masked.argtypes = [i32, i32, i32, i32, i32, i32, i64, i64, dbl, vp, vp, vp,
                                      vp, vp, vp, i32]
        lib.oracle_exact_topn.argtypes = [i32, i32, i32, i32, i32, i32, i64, i64, dbl, i64, vp,
                                          vp, vp, vp, i32]
        lib.oracle_full.argtypes = [i32, i32, i32, i32, i32, i32, i64, i64, dbl, vp, vp, vp, vp,
                                    i32]
        lib.oracle_logits_e4m3k.argtypes = [i32, i32, i32, i32, i32, i64, i64, dbl, vp, vp, vp,
                                            vp, i32]
        lib.oracle_atopn_run_e4m3k.argtypes = [i32, i32, i32, i32, i32, i32, i64, i32, vp, dbl,
                                               i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32]
        lib.oracle_masked_e4m3k.argtypes = [i32, i32, i32, i32, i32, i32, i64, i64, dbl, vp, vp,
                                            vp, vp, vp, vp, vp, i32]
        lib.oracle_atopn_run_e4m3kv.argtypes = [i32, i32, i32, i32, i32, i32, i64, i32, vp, dbl,
                                                i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                vp, i32]
        lib.oracle_masked_e4m3kv.argtypes = [i32, i32, i32, i32, i32, i32, i64, i64, dbl, vp,
                                             vp, vp, vp, vp, vp, vp, vp, i32]
        lib.oracle_e4m3_decode.argtypes = [vp, i64, vp]
        lib.oracle_e4m3_decode.restype = None
        lib.oracle_max_threads.restype = i32
        for name in ("oracle_logits", "oracle_atopn_run", "oracle_masked",
                     "oracle_exact_topn", "oracle_full", "oracle_logits_e4m3k",
                     "oracle_atopn_run_e4m3k", "oracle_masked_e4m3k", "oracle_atopn_run_e4m3kv",
                     "oracle_masked_e4m3kv"):
            getattr(lib, name).restype = i32
        _lib = lib
    return _lib


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"expected bf16 bit patterns as uint16, got {a.dtype}")
    return a


def _u8(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint8:
        raise TypeError(f"expected E4M3 codes as uint8, got {a.dtype}")
    return a


def _kscale(k_scale, B, hk) -> np.ndarray:
    k_scale = np.ascontiguousarray(k_scale, dtype=np.float32)
    if k_scale.shape != (B, hk):
        raise ValueError("k_scale must be [B][hk]")
    return k_scale


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _vscale(v_scale, B, hv) -> np.ndarray:
    v_scale = np.ascontiguousarray(v_scale, dtype=np.float32)
    if v_scale.shape != (B, hv):
        raise ValueError("v_scale must be [B][hv]")
    return v_scale


def _cache_shape(K, V):
    """(B, hk, hv, cache_len, d, dv): K and V share batch and rows; the key and
    value head dimensions d and dv are independent."""
    B, hk, cache_len, d = K.shape
    B2, hv, cache_len2, dv = V.shape
    if (B, cache_len) != (B2, cache_len2):
        raise ValueError("K and V caches disagree on batch or rows")
    return B, hk, hv, cache_len, d, dv


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def logits(q, K, ctx: int, scale: float = 1.0, nthreads: int = 0) -> np.ndarray:
    """fp64 logits ``[B][hq][ctx]`` of one step; q ``[B][hq][d]``, K ``[B][hk][rows][d]``."""
    q, K = _u16(q), _u16(K)
    B, hk, cache_len, d = K.shape
    hq = q.shape[1]
    out = np.empty((B, hq, ctx), dtype=np.float64)
    rc = _load().oracle_logits(B, hq, hk, hk, d, cache_len, ctx, scale, _ptr(q), _ptr(K),
                               _ptr(out), nthreads)
    if rc:
        raise ValueError("oracle_logits rejected its arguments")
    return out


def e4m3_decode(codes) -> np.ndarray:
    """Values (float64) of E4M3 codes, same shape; NaN for 0x7F and 0xFF."""
    codes = _u8(codes)
    out = np.empty(codes.shape, dtype=np.float64)
    _load().oracle_e4m3_decode(_ptr(codes), codes.size, _ptr(out))
    return out


def logits_e4m3k(q, K8, k_scale, ctx: int, scale: float = 1.0, nthreads: int = 0) -> np.ndarray:
    """fp64 logits ``[B][hq][ctx]`` with an E4M3 key cache ``K8 [B][hk][rows][d]``."""
    q, K8 = _u16(q), _u8(K8)
    B, hk, cache_len, d = K8.shape
    hq = q.shape[1]
    ks = _kscale(k_scale, B, hk)
    out = np.empty((B, hq, ctx), dtype=np.float64)
    rc = _load().oracle_logits_e4m3k(B, hq, hk, hk, d, cache_len, ctx, scale, _ptr(q), _ptr(K8),
                                     _ptr(ks), _ptr(out), nthreads)
    if rc:
        raise ValueError("oracle_logits_e4m3k rejected its arguments")
    return out


def nth_largest(s, N: int) -> float:
    """Exact N-th largest of a 1-D array (sorted), ``-inf`` when ``N >= len(s)``."""
    s = np.ascontiguousarray(s, dtype=np.float64)
    return float(_load().oracle_nth_largest(_ptr(s), s.size, N))


def atopn_run(q_steps, K, V, ctx_steps, top_n: int, refresh_n: int, scale: float = 1.0,
              want_sel: bool = False, want_logits: bool = False, nthreads: int = 0):
    """Atop-N over T steps of one layer.

    ``q_steps`` is ``[T][B][hq][d]``; ``ctx_steps`` the rows attended per step.
    Returns a dict with ``out [T][B][hq][dv]``, ``tau [T][B][hq]``,
    ``count [T][B][hq]`` and optionally ``sel``/``logits`` ``[T][B][hq][rows]``.
    """
    return _atopn(q_steps, _u16(K), None, V, ctx_steps, top_n, refresh_n, scale, want_sel,
                  want_logits, nthreads)


def atopn_run_e4m3k(q_steps, K8, k_scale, V, ctx_steps, top_n: int, refresh_n: int,
                    scale: float = 1.0, want_sel: bool = False, want_logits: bool = False,
                    nthreads: int = 0):
    """``atopn_run`` with an E4M3 key cache ``K8`` and scales ``k_scale [B][hk]``."""
    return _atopn(q_steps, _u8(K8), k_scale, V, ctx_steps, top_n, refresh_n, scale, want_sel,
                  want_logits, nthreads)


def atopn_run_e4m3kv(q_steps, K8, k_scale, V8, v_scale, ctx_steps, top_n: int, refresh_n: int,
                     scale: float = 1.0, want_sel: bool = False, want_logits: bool = False,
                     nthreads: int = 0):
    """``atopn_run`` with E4M3 key and value caches: ``K8`` with ``k_scale [B][hk]``,
    ``V8`` with ``v_scale [B][hv]`` (a value element is v_scale * e4m3(code))."""
    return _atopn(q_steps, _u8(K8), k_scale, V8, ctx_steps, top_n, refresh_n, scale, want_sel,
                  want_logits, nthreads, v_scale=v_scale)


def _atopn(q_steps, K, k_scale, V, ctx_steps, top_n, refresh_n, scale, want_sel, want_logits,
           nthreads, v_scale=None):
    q_steps = _u16(q_steps)
    V = _u16(V) if v_scale is None else _u8(V)
    B, hk, hv, cache_len, d, dv = _cache_shape(K, V)
    T, _, hq, _ = q_steps.shape
    ctx = np.ascontiguousarray(ctx_steps, dtype=np.int64)
    if ctx.shape != (T,):
        raise ValueError("ctx_steps must hold one length per step")
    out = np.empty((T, B, hq, dv), dtype=np.float64)
    tau = np.empty((T, B, hq), dtype=np.float64)
    count = np.empty((T, B, hq), dtype=np.int64)
    sel = np.empty((T, B, hq, cache_len), dtype=np.uint8) if want_sel else None
    lg = np.empty((T, B, hq, cache_len), dtype=np.float64) if want_logits else None
    tail = (_ptr(V), _ptr(out), _ptr(tau), _ptr(count),
            _ptr(sel) if sel is not None else None, _ptr(lg) if lg is not None else None,
            nthreads)
    if v_scale is not None:
        ks, vs = _kscale(k_scale, B, hk), _vscale(v_scale, B, hv)
        rc = _load().oracle_atopn_run_e4m3kv(B, hq, hk, hv, d, dv, cache_len, T, _ptr(ctx),
                                             scale, top_n, refresh_n, _ptr(q_steps), _ptr(K),
                                             _ptr(ks), _ptr(V), _ptr(vs), *tail[1:])
    elif k_scale is None:
        rc = _load().oracle_atopn_run(B, hq, hk, hv, d, dv, cache_len, T, _ptr(ctx), scale,
                                      top_n, refresh_n, _ptr(q_steps), _ptr(K), *tail)
    else:
        ks = _kscale(k_scale, B, hk)
        rc = _load().oracle_atopn_run_e4m3k(B, hq, hk, hv, d, dv, cache_len, T, _ptr(ctx),
                                            scale, top_n, refresh_n, _ptr(q_steps), _ptr(K),
                                            _ptr(ks), *tail)
    if rc:
        raise ValueError("oracle_atopn_run rejected its arguments")
    res = {"out": out, "tau": tau, "count": count}
    if sel is not None:
        res["sel"] = sel
    if lg is not None:
        res["logits"] = lg
    return res


def masked(q, K, V, ctx: int, bitmap, scale: float = 1.0, nthreads: int = 0):
    """One step over a caller-given selection bitmap ``[B][hq][ceil(rows/32)]`` (uint32)."""
    q, K, V = _u16(q), _u16(K), _u16(V)
    B, hk, hv, cache_len, d, dv = _cache_shape(K, V)
    hq = q.shape[1]
    bitmap = np.ascontiguousarray(bitmap, dtype=np.uint32)
    if bitmap.shape != (B, hq, (cache_len + 31) // 32):
        raise ValueError("bitmap must be [B][hq][ceil(rows/32)]")
    out = np.empty((B, hq, dv), dtype=np.float64)
    count = np.empty((B, hq), dtype=np.int64)
    rc = _load().oracle_masked(B, hq, hk, hv, d, dv, cache_len, ctx, scale, _ptr(q), _ptr(K),
                               _ptr(V), _ptr(bitmap), _ptr(out), _ptr(count), nthreads)
    if rc:
        raise ValueError("oracle_masked rejected its arguments")
    return out, count


def masked_e4m3k(q, K8, k_scale, V, ctx: int, bitmap, scale: float = 1.0, nthreads: int = 0):
    """``masked`` with an E4M3 key cache ``K8`` and scales ``k_scale [B][hk]``."""
    q, K8, V = _u16(q), _u8(K8), _u16(V)
    B, hk, hv, cache_len, d, dv = _cache_shape(K8, V)
    hq = q.shape[1]
    ks = _kscale(k_scale, B, hk)
    bitmap = np.ascontiguousarray(bitmap, dtype=np.uint32)
    if bitmap.shape != (B, hq, (cache_len + 31) // 32):
        raise ValueError("bitmap must be [B][hq][ceil(rows/32)]")
    out = np.empty((B, hq, dv), dtype=np.float64)
    count = np.empty((B, hq), dtype=np.int64)
    rc = _load().oracle_masked_e4m3k(B, hq, hk, hv, d, dv, cache_len, ctx, scale, _ptr(q), _ptr(K8),
                                     _ptr(ks), _ptr(V), _ptr(bitmap), _ptr(out), _ptr(count),
                                     nthreads)
    if rc:
        raise ValueError("oracle_masked_e4m3k rejected its arguments")
    return out, count


def masked_e4m3kv(q, K8, k_scale, V8, v_scale, ctx: int, bitmap, scale: float = 1.0,
                  nthreads: int = 0):
    """``masked`` with E4M3 key and value caches (scales ``[B][hk]`` and ``[B][hv]``)."""
    q, K8, V8 = _u16(q), _u8(K8), _u8(V8)
    B, hk, hv, cache_len, d, dv = _cache_shape(K8, V8)
    hq = q.shape[1]
    ks, vs = _kscale(k_scale, B, hk), _vscale(v_scale, B, hv)
    bitmap = np.ascontiguousarray(bitmap, dtype=np.uint32)
    if bitmap.shape != (B, hq, (cache_len + 31) // 32):
        raise ValueError("bitmap must be [B][hq][ceil(rows/32)]")
    out = np.empty((B, hq, dv), dtype=np.float64)
    count = np.empty((B, hq), dtype=np.int64)
    rc = _load().oracle_masked_e4m3kv(B, hq, hk, hv, d, dv, cache_len, ctx, scale, _ptr(q),
                                      _ptr(K8), _ptr(ks), _ptr(V8), _ptr(vs), _ptr(bitmap),
                                      _ptr(out), _ptr(count), nthreads)
    if rc:
        raise ValueError("oracle_masked_e4m3kv rejected its arguments")
    return out, count


def exact_topn(q, K, V, ctx: int, top_n: int, scale: float = 1.0, nthreads: int = 0):
    """Exact top-N attention of one step (index sort, first N, softmax)."""
    q, K, V = _u16(q), _u16(K), _u16(V)
    B, hk, hv, cache_len, d, dv = _cache_shape(K, V)
    hq = q.shape[1]
    out = np.empty((B, hq, dv), dtype=np.float64)
    rc = _load().oracle_exact_topn(B, hq, hk, hv, d, dv, cache_len, ctx, scale, top_n, _ptr(q),
                                   _ptr(K), _ptr(V), _ptr(out), nthreads)
    if rc:
        raise ValueError("oracle_exact_topn rejected its arguments")
    return out


def full(q, K, V, ctx: int, scale: float = 1.0, nthreads: int = 0):
    """Dense softmax attention of one step over all ``ctx`` rows."""
    q, K, V = _u16(q), _u16(K), _u16(V)
    B, hk, hv, cache_len, d, dv = _cache_shape(K, V)
    hq = q.shape[1]
    out = np.empty((B, hq, dv), dtype=np.float64)
    rc = _load().oracle_full(B, hq, hk, hv, d, dv, cache_len, ctx, scale, _ptr(q), _ptr(K),
                             _ptr(V), _ptr(out), nthreads)
    if rc:
        raise ValueError("oracle_full rejected its arguments")
    return out
