"""Python binding of libsaga.so: SAGA + Atop-N decode attention on MI355X.

Thin ctypes marshalling over the C ABI in ``include/saga.h``; every step of
the computation runs in the library's HIP kernels.  The function names are
the C names.  Tensors are torch CUDA (ROCm) tensors used only as device
memory; the stream is torch's current stream unless one is given.

There is no fallback: if ``libsaga.so`` has not been built, or a call
returns a non-zero status, an exception is raised.

    python -m sparse_decode_attention_atop_amd.build     # builds libsaga.so
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "SagaDims", "SagaError", "dims", "library", "saga_workspace_bytes", "alloc_workspace",
    "atopn_refresh_thresholds", "saga_decode_step", "atopn_refresh_decode_step",
    "SagaPaged", "paged", "atopn_refresh_thresholds_paged", "saga_decode_step_paged",
    "atopn_refresh_decode_step_paged", "atopn_refresh_thresholds_lq", "saga_decode_step_lq",
    "atopn_refresh_decode_step_lq", "alloc_workspace_lq", "atopn_refresh_thresholds_fp8k",
    "saga_decode_step_fp8k", "atopn_refresh_decode_step_fp8k", "saga_decode_step_fp8kv",
    "atopn_refresh_decode_step_fp8kv", "saga_full_attention",
    "saga_status_string", "saga_version", "LIB_PATH", "EXPORTED_SYMBOLS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsaga.so")
# Another build of the same library (e.g. with other tuning constants, from
# build.build(extra_flags=..., out=...)) for measurements; the in-tree build otherwise.
LIB_PATH = os.environ.get("SAGA_LIBRARY", LIB_PATH)
EXPORTED_SYMBOLS = ("saga_workspace_bytes", "atopn_refresh_thresholds", "saga_decode_step",
                    "atopn_refresh_decode_step", "atopn_refresh_thresholds_paged",
                    "saga_decode_step_paged", "atopn_refresh_decode_step_paged",
                    "atopn_refresh_thresholds_lq", "saga_decode_step_lq",
                    "atopn_refresh_decode_step_lq", "atopn_refresh_thresholds_fp8k",
                    "saga_decode_step_fp8k", "atopn_refresh_decode_step_fp8k",
                    "saga_decode_step_fp8kv", "atopn_refresh_decode_step_fp8kv",
                    "saga_full_attention", "saga_decode_step_noalloc", "saga_status_string",
                    "saga_version")

NOALLOC_SCRATCH_BYTES = 128 << 20    # SAGA_NOALLOC_SCRATCH_BYTES in include/saga.h

SAGA_OK = 0
SAGA_ERR_INVALID_ARGUMENT = 1
SAGA_ERR_UNSUPPORTED = 2
SAGA_ERR_WORKSPACE_TOO_SMALL = 3
SAGA_ERR_HIP = 4


class SagaDims(ctypes.Structure):
    """Mirror of ``saga_dims`` in include/saga.h."""
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("h_q", ctypes.c_int32),
        ("h_k", ctypes.c_int32),
        ("h_v", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("head_dim_v", ctypes.c_int32),
        ("ctx_len", ctypes.c_int64),
        ("cache_len", ctypes.c_int64),
        ("scale", ctypes.c_float),
        ("reserved2", ctypes.c_float),
    ]

    def __repr__(self):
        return (f"SagaDims(batch={self.batch}, h_q={self.h_q}, h_k={self.h_k}, h_v={self.h_v}, "
                f"head_dim={self.head_dim}, head_dim_v={self.head_dim_v}, ctx_len={self.ctx_len}, "
                f"cache_len={self.cache_len}, scale={self.scale})")


class SagaPaged(ctypes.Structure):
    """Mirror of ``saga_paged`` in include/saga.h (paged caches)."""
    _fields_ = [
        ("block_table_dev", ctypes.c_void_p),
        ("ctx_lens_dev", ctypes.c_void_p),
        ("page_rows", ctypes.c_int32),
        ("max_pages", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
        ("reserved", ctypes.c_int64),
    ]


class SagaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {saga_status_string(status)} (status {status})")


_lib = None


def library():
    """Load libsaga.so once (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m sparse_decode_attention_atop_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        pd = ctypes.POINTER(SagaDims)
        lib.saga_workspace_bytes.argtypes = [pd, i32]
        lib.saga_workspace_bytes.restype = sz
        lib.atopn_refresh_thresholds.argtypes = [pd, i32, vp, vp, vp, vp, vp, sz, vp]
        lib.atopn_refresh_thresholds.restype = ctypes.c_int
        lib.saga_decode_step.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.saga_decode_step.restype = ctypes.c_int
        lib.atopn_refresh_decode_step.argtypes = [pd, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.atopn_refresh_decode_step.restype = ctypes.c_int
        pp = ctypes.POINTER(SagaPaged)
        lib.atopn_refresh_thresholds_paged.argtypes = [pd, pp, i32, vp, vp, vp, vp, sz, vp]
        lib.atopn_refresh_thresholds_paged.restype = ctypes.c_int
        lib.saga_decode_step_paged.argtypes = [pd, pp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.saga_decode_step_paged.restype = ctypes.c_int
        lib.atopn_refresh_decode_step_paged.argtypes = [pd, pp, i32, vp, vp, vp, vp, vp, vp, vp,
                                                        sz, vp]
        lib.atopn_refresh_decode_step_paged.restype = ctypes.c_int
        lib.atopn_refresh_thresholds_lq.argtypes = [pd, i32, i32, vp, vp, vp, vp, sz, vp]
        lib.atopn_refresh_thresholds_lq.restype = ctypes.c_int
        lib.saga_decode_step_lq.argtypes = [pd, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.saga_decode_step_lq.restype = ctypes.c_int
        lib.atopn_refresh_decode_step_lq.argtypes = [pd, i32, i32, vp, vp, vp, vp, vp, vp, vp,
                                                     sz, vp]
        lib.atopn_refresh_decode_step_lq.restype = ctypes.c_int
        lib.atopn_refresh_thresholds_fp8k.argtypes = [pd, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.atopn_refresh_thresholds_fp8k.restype = ctypes.c_int
        lib.saga_decode_step_fp8k.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.saga_decode_step_fp8k.restype = ctypes.c_int
        lib.atopn_refresh_decode_step_fp8k.argtypes = [pd, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                                       sz, vp]
        lib.atopn_refresh_decode_step_fp8k.restype = ctypes.c_int
        lib.saga_decode_step_fp8kv.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                               vp]
        lib.saga_decode_step_fp8kv.restype = ctypes.c_int
        lib.atopn_refresh_decode_step_fp8kv.argtypes = [pd, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                                        vp, sz, vp]
        lib.atopn_refresh_decode_step_fp8kv.restype = ctypes.c_int
        lib.saga_full_attention.argtypes = [pd, vp, vp, vp, vp, vp, sz, vp]
        lib.saga_full_attention.restype = ctypes.c_int
        lib.saga_decode_step_noalloc.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp]
        lib.saga_decode_step_noalloc.restype = ctypes.c_int
        lib.saga_status_string.argtypes = [ctypes.c_int]
        lib.saga_status_string.restype = ctypes.c_char_p
        lib.saga_version.argtypes = []
        lib.saga_version.restype = ctypes.c_int
        _lib = lib
    return _lib


def dims(batch: int, h_q: int, h_k: int, h_v: int, head_dim: int, ctx_len: int,
         cache_len: int, scale: float = 1.0, head_dim_v: int = 0) -> SagaDims:
    """Shape of one layer call; head_dim is d_k, head_dim_v is d_v (0: same as d_k)."""
    return SagaDims(batch, h_q, h_k, h_v, head_dim, head_dim_v, ctx_len, cache_len, scale, 0.0)


def _dv(d: SagaDims) -> int:
    return d.head_dim_v or d.head_dim


def saga_status_string(status: int) -> str:
    return library().saga_status_string(int(status)).decode()


def saga_version() -> int:
    return int(library().saga_version())


def saga_workspace_bytes(d: SagaDims, top_n: int) -> int:
    return int(library().saga_workspace_bytes(ctypes.byref(d), int(top_n)))


def alloc_workspace(d: SagaDims, top_n: int, device="cuda") -> torch.Tensor:
    n = saga_workspace_bytes(d, top_n)
    if n == 0:
        raise SagaError(SAGA_ERR_INVALID_ARGUMENT, "saga_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _ptr(t: Optional[torch.Tensor], dtype, name: str):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (cuda/hip) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, numel: int, name: str):
    if t is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ws(workspace: torch.Tensor):
    return _ptr(workspace, torch.uint8, "workspace"), workspace.numel()


def _check(status: int, where: str):
    if status != SAGA_OK:
        raise SagaError(status, where)


def atopn_refresh_thresholds(d: SagaDims, top_n: int, q: torch.Tensor, k_cache: torch.Tensor,
                             thresholds: torch.Tensor, workspace: torch.Tensor,
                             logits_debug: Optional[torch.Tensor] = None, stream=None) -> None:
    """Exact top-N thresholds ``[B][h_q]`` (fp32) of this step's logits."""
    bh = d.batch * d.h_q
    _need(q, bh * d.head_dim, "q")
    _need(k_cache, d.batch * d.h_k * d.cache_len * d.head_dim, "k_cache")
    _need(thresholds, bh, "thresholds")
    _need(logits_debug, bh * d.ctx_len, "logits_debug")
    ws, nbytes = _ws(workspace)
    _check(library().atopn_refresh_thresholds(
        ctypes.byref(d), int(top_n), _ptr(q, torch.bfloat16, "q"),
        _ptr(k_cache, torch.bfloat16, "k_cache"), _ptr(thresholds, torch.float32, "thresholds"),
        _ptr(logits_debug, torch.float32, "logits_debug"), ws, nbytes, _stream(stream)),
        "atopn_refresh_thresholds")


def saga_decode_step(d: SagaDims, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                     thresholds: torch.Tensor, out: torch.Tensor, workspace: torch.Tensor,
                     sel_counts: Optional[torch.Tensor] = None,
                     sel_bitmap_debug: Optional[torch.Tensor] = None, stream=None) -> None:
    """One Atop-N decode step: out ``[B][h_q][d]`` (bf16) from the kept thresholds."""
    bh = d.batch * d.h_q
    _need(q, bh * d.head_dim, "q")
    _need(k_cache, d.batch * d.h_k * d.cache_len * d.head_dim, "k_cache")
    _need(v_cache, d.batch * d.h_v * d.cache_len * _dv(d), "v_cache")
    _need(thresholds, bh, "thresholds")
    _need(out, bh * _dv(d), "out")
    _need(sel_counts, bh, "sel_counts")
    _need(sel_bitmap_debug, bh * ((d.cache_len + 31) // 32), "sel_bitmap_debug")
    ws, nbytes = _ws(workspace)
    _check(library().saga_decode_step(
        ctypes.byref(d), _ptr(q, torch.bfloat16, "q"), _ptr(k_cache, torch.bfloat16, "k_cache"),
        _ptr(v_cache, torch.bfloat16, "v_cache"), _ptr(thresholds, torch.float32, "thresholds"),
        _ptr(out, torch.bfloat16, "out"), _ptr(sel_counts, torch.int32, "sel_counts"),
        _ptr(sel_bitmap_debug, torch.int32, "sel_bitmap_debug"), ws, nbytes, _stream(stream)),
        "saga_decode_step")


def atopn_refresh_decode_step(d: SagaDims, top_n: int, q: torch.Tensor, k_cache: torch.Tensor,
                              v_cache: torch.Tensor, thresholds: torch.Tensor, out: torch.Tensor,
                              workspace: torch.Tensor, sel_counts: Optional[torch.Tensor] = None,
                              stream=None) -> None:
    """A refresh step: fresh thresholds (kept for later steps) and this step's output."""
    bh = d.batch * d.h_q
    _need(q, bh * d.head_dim, "q")
    _need(k_cache, d.batch * d.h_k * d.cache_len * d.head_dim, "k_cache")
    _need(v_cache, d.batch * d.h_v * d.cache_len * _dv(d), "v_cache")
    _need(thresholds, bh, "thresholds")
    _need(out, bh * _dv(d), "out")
    _need(sel_counts, bh, "sel_counts")
    ws, nbytes = _ws(workspace)
    _check(library().atopn_refresh_decode_step(
        ctypes.byref(d), int(top_n), _ptr(q, torch.bfloat16, "q"),
        _ptr(k_cache, torch.bfloat16, "k_cache"), _ptr(v_cache, torch.bfloat16, "v_cache"),
        _ptr(thresholds, torch.float32, "thresholds"), _ptr(out, torch.bfloat16, "out"),
        _ptr(sel_counts, torch.int32, "sel_counts"), ws, nbytes, _stream(stream)),
        "atopn_refresh_decode_step")


def paged(block_table: torch.Tensor, ctx_lens: torch.Tensor, page_rows: int,
          num_pages: int) -> SagaPaged:
    """Describe paged caches: block_table int32 [B][max_pages], ctx_lens int32 [B]
    (device tensors, kept alive by the caller while calls use them)."""
    if block_table.dim() != 2 or ctx_lens.dim() != 1 or block_table.shape[0] != ctx_lens.shape[0]:
        raise ValueError("block_table must be [B][max_pages] and ctx_lens [B]")
    return SagaPaged(_ptr(block_table, torch.int32, "block_table").value,
                     _ptr(ctx_lens, torch.int32, "ctx_lens").value, int(page_rows),
                     int(block_table.shape[1]), int(num_pages), 0)


def _need_pool(t: torch.Tensor, d: SagaDims, p: SagaPaged, heads: int, dim: int, name: str):
    _need(t, p.num_pages * heads * p.page_rows * dim, name)


def atopn_refresh_thresholds_paged(d: SagaDims, p: SagaPaged, top_n: int, q: torch.Tensor,
                                   k_pages: torch.Tensor, thresholds: torch.Tensor,
                                   workspace: torch.Tensor, stream=None) -> None:
    """Exact top-N thresholds on paged caches (per-sequence lengths)."""
    _need(q, d.batch * d.h_q * d.head_dim, "q")
    _need_pool(k_pages, d, p, d.h_k, d.head_dim, "k_pages")
    _need(thresholds, d.batch * d.h_q, "thresholds")
    ws, nbytes = _ws(workspace)
    _check(library().atopn_refresh_thresholds_paged(
        ctypes.byref(d), ctypes.byref(p), int(top_n), _ptr(q, torch.bfloat16, "q"),
        _ptr(k_pages, torch.bfloat16, "k_pages"), _ptr(thresholds, torch.float32, "thresholds"),
        ws, nbytes, _stream(stream)), "atopn_refresh_thresholds_paged")


def saga_decode_step_paged(d: SagaDims, p: SagaPaged, q: torch.Tensor, k_pages: torch.Tensor,
                           v_pages: torch.Tensor, thresholds: torch.Tensor, out: torch.Tensor,
                           workspace: torch.Tensor, sel_counts: Optional[torch.Tensor] = None,
                           stream=None) -> None:
    """One Atop-N decode step on paged caches."""
    bh = d.batch * d.h_q
    _need(q, bh * d.head_dim, "q")
    _need_pool(k_pages, d, p, d.h_k, d.head_dim, "k_pages")
    _need_pool(v_pages, d, p, d.h_v, _dv(d), "v_pages")
    _need(thresholds, bh, "thresholds")
    _need(out, bh * _dv(d), "out")
    _need(sel_counts, bh, "sel_counts")
    ws, nbytes = _ws(workspace)
    _check(library().saga_decode_step_paged(
        ctypes.byref(d), ctypes.byref(p), _ptr(q, torch.bfloat16, "q"),
        _ptr(k_pages, torch.bfloat16, "k_pages"), _ptr(v_pages, torch.bfloat16, "v_pages"),
        _ptr(thresholds, torch.float32, "thresholds"), _ptr(out, torch.bfloat16, "out"),
        _ptr(sel_counts, torch.int32, "sel_counts"), ws, nbytes, _stream(stream)),
        "saga_decode_step_paged")


def atopn_refresh_decode_step_paged(d: SagaDims, p: SagaPaged, top_n: int, q: torch.Tensor,
                                    k_pages: torch.Tensor, v_pages: torch.Tensor,
                                    thresholds: torch.Tensor, out: torch.Tensor,
                                    workspace: torch.Tensor,
                                    sel_counts: Optional[torch.Tensor] = None,
                                    stream=None) -> None:
    """A refresh step on paged caches: fresh thresholds and this step's output."""
    bh = d.batch * d.h_q
    _need(q, bh * d.head_dim, "q")
    _need_pool(k_pages, d, p, d.h_k, d.head_dim, "k_pages")
    _need_pool(v_pages, d, p, d.h_v, _dv(d), "v_pages")
    _need(thresholds, bh, "thresholds")
    _need(out, bh * _dv(d), "out")
    _need(sel_counts, bh, "sel_counts")
    ws, nbytes = _ws(workspace)
    _check(library().atopn_refresh_decode_step_paged(
        ctypes.byref(d), ctypes.byref(p), int(top_n), _ptr(q, torch.bfloat16, "q"),
        _ptr(k_pages, torch.bfloat16, "k_pages"), _ptr(v_pages, torch.bfloat16, "v_pages"),
        _ptr(thresholds, torch.float32, "thresholds"), _ptr(out, torch.bfloat16, "out"),
        _ptr(sel_counts, torch.int32, "sel_counts"), ws, nbytes, _stream(stream)),
        "atopn_refresh_decode_step_paged")


def _lq_dims(d: SagaDims, l_q: int) -> SagaDims:
    return SagaDims(d.batch, d.h_q * l_q, d.h_k, d.h_v, d.head_dim, d.head_dim_v, d.ctx_len,
                    d.cache_len, d.scale, 0.0)


def alloc_workspace_lq(d: SagaDims, l_q: int, top_n: int, device="cuda") -> torch.Tensor:
    """Workspace for the *_lq calls (h_q * l_q virtual query heads)."""
    return alloc_workspace(_lq_dims(d, l_q), top_n, device)


def atopn_refresh_thresholds_lq(d: SagaDims, l_q: int, top_n: int, q: torch.Tensor,
                                k_cache: torch.Tensor, thresholds: torch.Tensor,
                                workspace: torch.Tensor, stream=None) -> None:
    """Thresholds [B][h_q][l_q] of a step with l_q query tokens per head."""
    n = d.batch * d.h_q * l_q
    _need(q, n * d.head_dim, "q")
    _need(k_cache, d.batch * d.h_k * d.cache_len * d.head_dim, "k_cache")
    _need(thresholds, n, "thresholds")
    ws, nbytes = _ws(workspace)
    _check(library().atopn_refresh_thresholds_lq(
        ctypes.byref(d), int(l_q), int(top_n), _ptr(q, torch.bfloat16, "q"),
        _ptr(k_cache, torch.bfloat16, "k_cache"), _ptr(thresholds, torch.float32, "thresholds"),
        ws, nbytes, _stream(stream)), "atopn_refresh_thresholds_lq")


def saga_decode_step_lq(d: SagaDims, l_q: int, q: torch.Tensor, k_cache: torch.Tensor,
                        v_cache: torch.Tensor, thresholds: torch.Tensor, out: torch.Tensor,
                        workspace: torch.Tensor, sel_counts: Optional[torch.Tensor] = None,
                        stream=None) -> None:
    """A decode step with l_q query tokens per head (causal among them)."""
    n = d.batch * d.h_q * l_q
    _need(q, n * d.head_dim, "q")
    _need(k_cache, d.batch * d.h_k * d.cache_len * d.head_dim, "k_cache")
    _need(v_cache, d.batch * d.h_v * d.cache_len * _dv(d), "v_cache")
    _need(thresholds, n, "thresholds")
    _need(out, n * _dv(d), "out")
    _need(sel_counts, n, "sel_counts")
    ws, nbytes = _ws(workspace)
    _check(library().saga_decode_step_lq(
        ctypes.byref(d), int(l_q), _ptr(q, torch.bfloat16, "q"),
        _ptr(k_cache, torch.bfloat16, "k_cache"), _ptr(v_cache, torch.bfloat16, "v_cache"),
        _ptr(thresholds, torch.float32, "thresholds"), _ptr(out, torch.bfloat16, "out"),
        _ptr(sel_counts, torch.int32, "sel_counts"), ws, nbytes, _stream(stream)),
        "saga_decode_step_lq")


def atopn_refresh_decode_step_lq(d: SagaDims, l_q: int, top_n: int, q: torch.Tensor,
                                 k_cache: torch.Tensor, v_cache: torch.Tensor,
                                 thresholds: torch.Tensor, out: torch.Tensor,
                                 workspace: torch.Tensor,
                                 sel_counts: Optional[torch.Tensor] = None, stream=None) -> None:
    """A refresh step with l_q query tokens per head."""
    n = d.batch * d.h_q * l_q
    _need(q, n * d.head_dim, "q")
    _need(k_cache, d.batch * d.h_k * d.cache_len * d.head_dim, "k_cache")
    _need(v_cache, d.batch * d.h_v * d.cache_len * _dv(d), "v_cache")
    _need(thresholds, n, "thresholds")
    _need(out, n * _dv(d), "out")
    _need(sel_counts, n, "sel_counts")
    ws, nbytes = _ws(workspace)
    _check(library().atopn_refresh_decode_step_lq(
        ctypes.byref(d), int(l_q), int(top_n), _ptr(q, torch.bfloat16, "q"),
        _ptr(k_cache, torch.bfloat16, "k_cache"), _ptr(v_cache, torch.bfloat16, "v_cache"),
        _ptr(thresholds, torch.float32, "thresholds"), _ptr(out, torch.bfloat16, "out"),
        _ptr(sel_counts, torch.int32, "sel_counts"), ws, nbytes, _stream(stream)),
        "atopn_refresh_decode_step_lq")


def _ptr_k8(t: torch.Tensor, name: str = "k8_cache"):
    """An fp8 E4M3 (OCP) cache: torch.float8_e4m3fn, or its raw bytes as uint8."""
    if isinstance(t, torch.Tensor) and t.dtype == torch.float8_e4m3fn:
        return _ptr(t, torch.float8_e4m3fn, name)
    return _ptr(t, torch.uint8, name)


def _need_fp8k(d: SagaDims, k8_cache: torch.Tensor, k_scale: torch.Tensor):
    _need(k8_cache, d.batch * d.h_k * d.cache_len * d.head_dim, "k8_cache")
    _need(k_scale, d.batch * d.h_k, "k_scale")


def atopn_refresh_thresholds_fp8k(d: SagaDims, top_n: int, q: torch.Tensor,
                                  k8_cache: torch.Tensor, k_scale: torch.Tensor,
                                  thresholds: torch.Tensor, workspace: torch.Tensor,
                                  logits_debug: Optional[torch.Tensor] = None,
                                  stream=None) -> None:
    """Refresh thresholds with an fp8 K cache (k_scale fp32 ``[B][h_k]``)."""
    bh = d.batch * d.h_q
    _need(q, bh * d.head_dim, "q")
    _need_fp8k(d, k8_cache, k_scale)
    _need(thresholds, bh, "thresholds")
    _need(logits_debug, bh * d.ctx_len, "logits_debug")
    ws, nbytes = _ws(workspace)
    _check(library().atopn_refresh_thresholds_fp8k(
        ctypes.byref(d), int(top_n), _ptr(q, torch.bfloat16, "q"), _ptr_k8(k8_cache),
        _ptr(k_scale, torch.float32, "k_scale"), _ptr(thresholds, torch.float32, "thresholds"),
        _ptr(logits_debug, torch.float32, "logits_debug"), ws, nbytes, _stream(stream)),
        "atopn_refresh_thresholds_fp8k")


def saga_decode_step_fp8k(d: SagaDims, q: torch.Tensor, k8_cache: torch.Tensor,
                          k_scale: torch.Tensor, v_cache: torch.Tensor, thresholds: torch.Tensor,
                          out: torch.Tensor, workspace: torch.Tensor,
                          sel_counts: Optional[torch.Tensor] = None,
                          sel_bitmap_debug: Optional[torch.Tensor] = None, stream=None) -> None:
    """A decode step with an fp8 K cache and a bf16 V cache."""
    bh = d.batch * d.h_q
    _need(q, bh * d.head_dim, "q")
    _need_fp8k(d, k8_cache, k_scale)
    _need(v_cache, d.batch * d.h_v * d.cache_len * _dv(d), "v_cache")
    _need(thresholds, bh, "thresholds")
    _need(out, bh * _dv(d), "out")
    _need(sel_counts, bh, "sel_counts")
    _need(sel_bitmap_debug, bh * ((d.cache_len + 31) // 32), "sel_bitmap_debug")
    ws, nbytes = _ws(workspace)
    _check(library().saga_decode_step_fp8k(
        ctypes.byref(d), _ptr(q, torch.bfloat16, "q"), _ptr_k8(k8_cache),
        _ptr(k_scale, torch.float32, "k_scale"), _ptr(v_cache, torch.bfloat16, "v_cache"),
        _ptr(thresholds, torch.float32, "thresholds"), _ptr(out, torch.bfloat16, "out"),
        _ptr(sel_counts, torch.int32, "sel_counts"),
        _ptr(sel_bitmap_debug, torch.int32, "sel_bitmap_debug"), ws, nbytes, _stream(stream)),
        "saga_decode_step_fp8k")


def atopn_refresh_decode_step_fp8k(d: SagaDims, top_n: int, q: torch.Tensor,
                                   k8_cache: torch.Tensor, k_scale: torch.Tensor,
                                   v_cache: torch.Tensor, thresholds: torch.Tensor,
                                   out: torch.Tensor, workspace: torch.Tensor,
                                   sel_counts: Optional[torch.Tensor] = None,
                                   stream=None) -> None:
    """A refresh step with an fp8 K cache: fresh thresholds and this step's output."""
    bh = d.batch * d.h_q
    _need(q, bh * d.head_dim, "q")
    _need_fp8k(d, k8_cache, k_scale)
    _need(v_cache, d.batch * d.h_v * d.cache_len * _dv(d), "v_cache")
    _need(thresholds, bh, "thresholds")
    _need(out, bh * _dv(d), "out")
    _need(sel_counts, bh, "sel_counts")
    ws, nbytes = _ws(workspace)
    _check(library().atopn_refresh_decode_step_fp8k(
        ctypes.byref(d), int(top_n), _ptr(q, torch.bfloat16, "q"), _ptr_k8(k8_cache),
        _ptr(k_scale, torch.float32, "k_scale"), _ptr(v_cache, torch.bfloat16, "v_cache"),
        _ptr(thresholds, torch.float32, "thresholds"), _ptr(out, torch.bfloat16, "out"),
        _ptr(sel_counts, torch.int32, "sel_counts"), ws, nbytes, _stream(stream)),
        "atopn_refresh_decode_step_fp8k")


def _need_fp8v(d: SagaDims, v8_cache: torch.Tensor, v_scale: torch.Tensor):
    _need(v8_cache, d.batch * d.h_v * d.cache_len * _dv(d), "v8_cache")
    _need(v_scale, d.batch * d.h_v, "v_scale")


def saga_decode_step_fp8kv(d: SagaDims, q: torch.Tensor, k8_cache: torch.Tensor,
                           k_scale: torch.Tensor, v8_cache: torch.Tensor, v_scale: torch.Tensor,
                           thresholds: torch.Tensor, out: torch.Tensor, workspace: torch.Tensor,
                           sel_counts: Optional[torch.Tensor] = None,
                           sel_bitmap_debug: Optional[torch.Tensor] = None, stream=None) -> None:
    """A decode step with fp8 K and V caches (v_scale fp32 ``[B][h_v]``)."""
    bh = d.batch * d.h_q
    _need(q, bh * d.head_dim, "q")
    _need_fp8k(d, k8_cache, k_scale)
    _need_fp8v(d, v8_cache, v_scale)
    _need(thresholds, bh, "thresholds")
    _need(out, bh * _dv(d), "out")
    _need(sel_counts, bh, "sel_counts")
    _need(sel_bitmap_debug, bh * ((d.cache_len + 31) // 32), "sel_bitmap_debug")
    ws, nbytes = _ws(workspace)
    _check(library().saga_decode_step_fp8kv(
        ctypes.byref(d), _ptr(q, torch.bfloat16, "q"), _ptr_k8(k8_cache),
        _ptr(k_scale, torch.float32, "k_scale"), _ptr_k8(v8_cache, "v8_cache"),
        _ptr(v_scale, torch.float32, "v_scale"), _ptr(thresholds, torch.float32, "thresholds"),
        _ptr(out, torch.bfloat16, "out"), _ptr(sel_counts, torch.int32, "sel_counts"),
        _ptr(sel_bitmap_debug, torch.int32, "sel_bitmap_debug"), ws, nbytes, _stream(stream)),
        "saga_decode_step_fp8kv")


def atopn_refresh_decode_step_fp8kv(d: SagaDims, top_n: int, q: torch.Tensor,
                                    k8_cache: torch.Tensor, k_scale: torch.Tensor,
                                    v8_cache: torch.Tensor, v_scale: torch.Tensor,
                                    thresholds: torch.Tensor, out: torch.Tensor,
                                    workspace: torch.Tensor,
                                    sel_counts: Optional[torch.Tensor] = None,
                                    stream=None) -> None:
    """A refresh step with fp8 K and V caches: fresh thresholds and this step's output."""
    bh = d.batch * d.h_q
    _need(q, bh * d.head_dim, "q")
    _need_fp8k(d, k8_cache, k_scale)
    _need_fp8v(d, v8_cache, v_scale)
    _need(thresholds, bh, "thresholds")
    _need(out, bh * _dv(d), "out")
    _need(sel_counts, bh, "sel_counts")
    ws, nbytes = _ws(workspace)
    _check(library().atopn_refresh_decode_step_fp8kv(
        ctypes.byref(d), int(top_n), _ptr(q, torch.bfloat16, "q"), _ptr_k8(k8_cache),
        _ptr(k_scale, torch.float32, "k_scale"), _ptr_k8(v8_cache, "v8_cache"),
        _ptr(v_scale, torch.float32, "v_scale"), _ptr(thresholds, torch.float32, "thresholds"),
        _ptr(out, torch.bfloat16, "out"), _ptr(sel_counts, torch.int32, "sel_counts"), ws,
        nbytes, _stream(stream)),
        "atopn_refresh_decode_step_fp8kv")


def saga_full_attention(d: SagaDims, q: torch.Tensor, k_cache: torch.Tensor,
                        v_cache: torch.Tensor, out: torch.Tensor, workspace: torch.Tensor,
                        stream=None) -> None:
    """Dense decode attention over all ``ctx_len`` rows (GQA / SAGA baseline)."""
    bh = d.batch * d.h_q
    _need(q, bh * d.head_dim, "q")
    _need(k_cache, d.batch * d.h_k * d.cache_len * d.head_dim, "k_cache")
    _need(v_cache, d.batch * d.h_v * d.cache_len * _dv(d), "v_cache")
    _need(out, bh * _dv(d), "out")
    ws, nbytes = _ws(workspace)
    _check(library().saga_full_attention(
        ctypes.byref(d), _ptr(q, torch.bfloat16, "q"), _ptr(k_cache, torch.bfloat16, "k_cache"),
        _ptr(v_cache, torch.bfloat16, "v_cache"), _ptr(out, torch.bfloat16, "out"), ws, nbytes,
        _stream(stream)), "saga_full_attention")


def saga_decode_step_noalloc(d: SagaDims, q: torch.Tensor, k_cache: torch.Tensor,
                             v_cache: torch.Tensor, thresholds: torch.Tensor, out: torch.Tensor,
                             sel_counts: Optional[torch.Tensor] = None, stream=None) -> None:
    """saga_decode_step without a workspace: the library's own per-device
    scratch (NOALLOC_SCRATCH_BYTES) is used; calls on one device must not overlap."""
    bh = d.batch * d.h_q
    _need(q, bh * d.head_dim, "q")
    _need(k_cache, d.batch * d.h_k * d.cache_len * d.head_dim, "k_cache")
    _need(v_cache, d.batch * d.h_v * d.cache_len * _dv(d), "v_cache")
    _need(thresholds, bh, "thresholds")
    _need(out, bh * _dv(d), "out")
    _need(sel_counts, bh, "sel_counts")
    _check(library().saga_decode_step_noalloc(
        ctypes.byref(d), _ptr(q, torch.bfloat16, "q"), _ptr(k_cache, torch.bfloat16, "k_cache"),
        _ptr(v_cache, torch.bfloat16, "v_cache"), _ptr(thresholds, torch.float32, "thresholds"),
        _ptr(out, torch.bfloat16, "out"), _ptr(sel_counts, torch.int32, "sel_counts"),
        _stream(stream)), "saga_decode_step_noalloc")
