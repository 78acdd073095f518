"""The C-ABI library on the CPU: it loads, exports every symbol include/saga.h
declares, sizes workspaces, and rejects bad arguments before any launch.
No call here reaches a kernel, so no GPU is needed."""
import ctypes
import os
import re
import subprocess

import pytest
import torch  # noqa: F401  (load torch's HIP runtime before the library)

import sparse_decode_attention_atop_amd as saga

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "saga.h")


def header_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text,
                                 flags=re.M)))


def test_library_built():
    assert os.path.exists(saga.LIB_PATH), "run `python -m sparse_decode_attention_atop_amd.build`"


def test_exports_match_header():
    declared = header_functions()
    assert declared == sorted(saga.EXPORTED_SYMBOLS)
    out = subprocess.run(["nm", "-D", "--defined-only", saga.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted(ln.split()[-1] for ln in out.splitlines() if " T " in ln)
    assert exported == declared, "libsaga.so must export exactly the header's functions"
    lib = saga.library()
    for name in declared:
        assert hasattr(lib, name)


def test_probe_library_exports_match_its_header():
    """The HBM measurement kernels (libsaga_probe.so) export exactly the
    functions include/saga_probe.h declares."""
    from sparse_decode_attention_atop_amd import probe
    declared = header_functions(os.path.join(ROOT, "include", "saga_probe.h"))
    assert declared == sorted(probe.EXPORTED_SYMBOLS)
    out = subprocess.run(["nm", "-D", "--defined-only", probe.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted(ln.split()[-1] for ln in out.splitlines() if " T " in ln)
    assert exported == declared
    lib = probe.library()
    fake = ctypes.c_void_p(1 << 20)
    # Arguments are checked before any launch (no GPU needed for these).
    assert lib.saga_probe_read(None, 4096, 1, 1, fake, None) == 1
    assert lib.saga_probe_read(fake, 4096 * 3, 2, 1, fake, None) == 1      # not whole chunks
    assert lib.saga_probe_read(fake, 4096, 1, 3, fake, None) == 1          # depth 3
    assert lib.saga_probe_read_tiles(fake, 16384, 64, 1, 1, fake, None) == 1    # row bytes
    assert lib.saga_probe_read_tiles(fake, 16384, 128, 1, 3, fake, None) == 1   # tiles 3
    assert lib.saga_probe_read_tiles(fake, 8192, 128, 1, 1, fake, None) == 1    # not whole chunks
    assert lib.saga_probe_rows(fake, 1 << 20, 96, 10, 0, 1, 2, fake, None) == 1
    assert lib.saga_probe_rows(fake, 1 << 20, 128, 0, 0, 1, 2, fake, None) == 1


def test_status_strings_and_version():
    assert saga.saga_status_string(0) == "ok"
    assert saga.saga_status_string(3) == "workspace too small"
    assert saga.saga_status_string(99) == "unknown status"
    assert saga.saga_version() >= 100


def good_dims(**kw):
    base = dict(batch=2, h_q=12, h_k=1, h_v=2, head_dim=128, ctx_len=1000, cache_len=1024)
    base.update(kw)
    return saga.dims(**base)


def test_workspace_sizing():
    d = good_dims()
    n = saga.saga_workspace_bytes(d, 64)
    rows = 2 * 12
    assert n >= 2 * rows * 1024 * 4          # logits + candidate buffers
    assert n % 256 == 0
    # independent of ctx_len and N
    assert saga.saga_workspace_bytes(good_dims(ctx_len=1), 1) == n
    assert saga.saga_workspace_bytes(good_dims(), 5000) == n
    for bad in (dict(batch=0), dict(h_q=12, h_k=5), dict(h_v=5), dict(ctx_len=0),
                dict(ctx_len=2000), dict(head_dim=96), dict(h_q=34, h_k=2, h_v=2)):
        assert saga.saga_workspace_bytes(good_dims(**bad), 64) == 0, bad


FAKE = ctypes.c_void_p(1 << 20)      # aligned, never dereferenced (calls fail validation first)


def call_decode(d, ws_bytes, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, tau=FAKE, out=FAKE, counts=None, bitmap=None, ws=FAKE)
    p.update(ptrs)
    return saga.library().saga_decode_step(ctypes.byref(d), p["q"], p["k"], p["v"], p["tau"],
                                           p["out"], p["counts"], p["bitmap"], p["ws"], ws_bytes,
                                           None)


def call_refresh(d, top_n, ws_bytes, **ptrs):
    p = dict(q=FAKE, k=FAKE, tau=FAKE, dbg=None, ws=FAKE)
    p.update(ptrs)
    return saga.library().atopn_refresh_thresholds(ctypes.byref(d), top_n, p["q"], p["k"],
                                                   p["tau"], p["dbg"], p["ws"], ws_bytes, None)


def call_fused(d, top_n, ws_bytes, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, tau=FAKE, out=FAKE, counts=None, ws=FAKE)
    p.update(ptrs)
    return saga.library().atopn_refresh_decode_step(ctypes.byref(d), top_n, p["q"], p["k"],
                                                    p["v"], p["tau"], p["out"], p["counts"],
                                                    p["ws"], ws_bytes, None)


def call_full(d, ws_bytes, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, ws=FAKE)
    p.update(ptrs)
    return saga.library().saga_full_attention(ctypes.byref(d), p["q"], p["k"], p["v"], p["out"],
                                              p["ws"], ws_bytes, None)


INVALID, UNSUPPORTED, SMALL = 1, 2, 3


@pytest.mark.parametrize("bad,code", [
    (dict(batch=0), INVALID), (dict(h_q=0), INVALID), (dict(h_k=5), INVALID),
    (dict(h_v=7), INVALID), (dict(ctx_len=0), INVALID), (dict(ctx_len=1025), INVALID),
    (dict(cache_len=1 << 27, ctx_len=10), INVALID), (dict(head_dim=96), UNSUPPORTED),
    (dict(h_q=34, h_k=2, h_v=2), UNSUPPORTED),
    (dict(batch=1 << 14, h_q=8, h_k=4, h_v=4), UNSUPPORTED),          # batch * h_k > 65535
    (dict(batch=1 << 14, h_q=16, h_k=1, h_v=1, cache_len=(1 << 22) + 64, ctx_len=10),
     UNSUPPORTED),                                                    # batch * h_q * cache_len > 2^40
])
def test_dims_errors_every_entry_point(bad, code):
    d = good_dims(**bad)
    assert call_decode(d, 1 << 40) == code
    assert call_refresh(d, 8, 1 << 40) == code
    assert call_fused(d, 8, 1 << 40) == code
    assert call_full(d, 1 << 40) == code


def test_reserved_fields_and_scale():
    d = good_dims()
    d.reserved2 = 1.0
    assert call_decode(d, 1 << 40) == INVALID
    d = good_dims()
    d.scale = float("nan")
    assert call_refresh(d, 8, 1 << 40) == INVALID


@pytest.mark.parametrize("name", ["q", "k", "v", "tau", "out", "ws"])
def test_decode_null_pointers(name):
    assert call_decode(good_dims(), 1 << 40, **{name: None}) == INVALID


@pytest.mark.parametrize("name", ["q", "k", "tau", "ws"])
def test_refresh_null_pointers(name):
    assert call_refresh(good_dims(), 8, 1 << 40, **{name: None}) == INVALID


@pytest.mark.parametrize("name", ["q", "k", "v", "tau", "out", "ws"])
def test_fused_null_pointers(name):
    assert call_fused(good_dims(), 8, 1 << 40, **{name: None}) == INVALID


@pytest.mark.parametrize("name", ["q", "k", "v", "out", "ws"])
def test_full_null_pointers(name):
    assert call_full(good_dims(), 1 << 40, **{name: None}) == INVALID


def test_misaligned_pointers():
    odd = ctypes.c_void_p((1 << 20) + 8)
    assert call_decode(good_dims(), 1 << 40, k=odd) == INVALID
    assert call_refresh(good_dims(), 8, 1 << 40, q=odd) == INVALID
    assert call_full(good_dims(), 1 << 40, v=odd) == INVALID
    assert call_fused(good_dims(), 8, 1 << 40, v=odd) == INVALID
    assert call_decode(good_dims(), 1 << 40, counts=ctypes.c_void_p((1 << 20) + 2)) == INVALID


def test_key_and_value_head_dims():
    # d_k and d_v are independent: 32, 64 or 128 each; 0 means d_v = d_k.
    for dk in (32, 64, 128):
        for dv in (0, 32, 64, 128):
            d = good_dims(head_dim=dk, head_dim_v=dv)
            assert saga.saga_workspace_bytes(d, 8) > 0, (dk, dv)
            assert call_decode(d, 8) == SMALL, (dk, dv)        # valid dims: stops at the workspace
            assert call_full(d, 8) == SMALL, (dk, dv)
    assert call_decode(good_dims(head_dim_v=-1), 1 << 40) == INVALID
    assert call_decode(good_dims(head_dim_v=96), 1 << 40) == UNSUPPORTED
    assert call_refresh(good_dims(head_dim=48), 8, 1 << 40) == UNSUPPORTED
    # partials are sized by d_v: a larger value dimension needs a larger workspace
    small = saga.saga_workspace_bytes(good_dims(head_dim=128, head_dim_v=32), 8)
    large = saga.saga_workspace_bytes(good_dims(head_dim=32, head_dim_v=128), 8)
    assert large > small
    # one head must stay under 2 GiB for the larger of the two dimensions
    assert call_decode(good_dims(head_dim=32, head_dim_v=128, cache_len=1 << 23, ctx_len=10),
                       1 << 40) == UNSUPPORTED


def test_top_n_and_workspace_errors():
    d = good_dims()
    assert call_refresh(d, 0, 1 << 40) == INVALID
    assert call_refresh(d, -5, 1 << 40) == INVALID
    assert call_fused(d, 0, 1 << 40) == INVALID
    need = saga.saga_workspace_bytes(d, 8)
    assert call_decode(d, need - 1) == SMALL
    assert call_refresh(d, 8, need - 1) == SMALL
    assert call_fused(d, 8, need - 1) == SMALL
    assert call_full(d, need - 1) == SMALL


def test_full_attention_unsupported_head_maps():
    # 32 query heads per value head exceeds the dense kernel's per-value-head slots.
    d = good_dims(h_q=32, h_k=2, h_v=1, head_dim=64)
    assert call_full(d, 1 << 40) == UNSUPPORTED


# ---- paged caches -----------------------------------------------------------

def good_paged(**kw):
    base = dict(block_table_dev=(1 << 20), ctx_lens_dev=(1 << 21), page_rows=256, max_pages=4,
                num_pages=16, reserved=0)
    base.update(kw)
    return saga.SagaPaged(**base)


def call_paged(kind, d, p, ws_bytes, top_n=8):
    lib = saga.library()
    pp = ctypes.byref(p) if p is not None else None
    if kind == "refresh":
        return lib.atopn_refresh_thresholds_paged(ctypes.byref(d), pp, top_n, FAKE, FAKE, FAKE,
                                                  FAKE, ws_bytes, None)
    if kind == "decode":
        return lib.saga_decode_step_paged(ctypes.byref(d), pp, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                          FAKE, ws_bytes, None)
    return lib.atopn_refresh_decode_step_paged(ctypes.byref(d), pp, top_n, FAKE, FAKE, FAKE, FAKE,
                                               FAKE, None, FAKE, ws_bytes, None)


@pytest.mark.parametrize("kind", ["refresh", "decode", "fused"])
def test_paged_argument_checks(kind):
    d = good_dims(cache_len=1024, ctx_len=1000)         # 4 pages of 256 rows
    need = saga.saga_workspace_bytes(d, 8)
    assert call_paged(kind, d, None, 1 << 40) == INVALID
    assert call_paged(kind, d, good_paged(page_rows=128, max_pages=8), 1 << 40) == INVALID
    assert call_paged(kind, d, good_paged(page_rows=300), 1 << 40) == INVALID
    assert call_paged(kind, d, good_paged(max_pages=3), 1 << 40) == INVALID   # != cache_len
    assert call_paged(kind, d, good_paged(num_pages=0), 1 << 40) == INVALID
    assert call_paged(kind, d, good_paged(reserved=1), 1 << 40) == INVALID
    assert call_paged(kind, d, good_paged(block_table_dev=None), 1 << 40) == INVALID
    assert call_paged(kind, d, good_paged(ctx_lens_dev=(1 << 21) + 2), 1 << 40) == INVALID
    # a consistent description passes validation and stops at the workspace size
    assert call_paged(kind, d, good_paged(), need - 1) == SMALL
    assert call_paged(kind, good_dims(cache_len=1024, head_dim=96), good_paged(), 1 << 40) == UNSUPPORTED


# ---- several query tokens per step ------------------------------------------

def call_lq(kind, d, l_q, ws_bytes, top_n=8):
    lib = saga.library()
    if kind == "refresh":
        return lib.atopn_refresh_thresholds_lq(ctypes.byref(d), l_q, top_n, FAKE, FAKE, FAKE, FAKE,
                                               ws_bytes, None)
    if kind == "decode":
        return lib.saga_decode_step_lq(ctypes.byref(d), l_q, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                       FAKE, ws_bytes, None)
    return lib.atopn_refresh_decode_step_lq(ctypes.byref(d), l_q, top_n, FAKE, FAKE, FAKE, FAKE,
                                            FAKE, None, FAKE, ws_bytes, None)


@pytest.mark.parametrize("kind", ["refresh", "decode", "fused"])
def test_lq_argument_checks(kind):
    d = good_dims(h_q=8, h_k=2, h_v=4, ctx_len=1000)   # 4 query heads per key head
    assert call_lq(kind, d, 0, 1 << 40) == INVALID
    assert call_lq(kind, d, 1001, 1 << 40) == INVALID   # more tokens than rows
    assert call_lq(kind, d, 5, 1 << 40) == UNSUPPORTED  # 4 x 5 > 16 query slots
    need = saga.saga_workspace_bytes(saga.dims(2, 8 * 4, 2, 4, 128, 1000, 1024), 8)
    assert call_lq(kind, d, 4, need - 1) == SMALL       # workspace of h_q * l_q heads
    assert call_lq(kind, good_dims(h_q=8, h_k=2, h_v=3), 2, 1 << 40) == INVALID


# ---- fp8 E4M3 K cache --------------------------------------------------------

def call_fp8k(kind, d, ws_bytes, top_n=8, **ptrs):
    p = dict(q=FAKE, k8=FAKE, ks=FAKE, v=FAKE, tau=FAKE, out=FAKE, ws=FAKE)
    p.update(ptrs)
    lib = saga.library()
    if kind == "refresh":
        return lib.atopn_refresh_thresholds_fp8k(ctypes.byref(d), top_n, p["q"], p["k8"], p["ks"],
                                                 p["tau"], None, p["ws"], ws_bytes, None)
    if kind == "decode":
        return lib.saga_decode_step_fp8k(ctypes.byref(d), p["q"], p["k8"], p["ks"], p["v"],
                                         p["tau"], p["out"], None, None, p["ws"], ws_bytes, None)
    return lib.atopn_refresh_decode_step_fp8k(ctypes.byref(d), top_n, p["q"], p["k8"], p["ks"],
                                              p["v"], p["tau"], p["out"], None, p["ws"], ws_bytes,
                                              None)


@pytest.mark.parametrize("kind", ["refresh", "decode", "fused"])
def test_fp8k_argument_checks(kind):
    d = good_dims()
    need = saga.saga_workspace_bytes(d, 8)
    assert call_fp8k(kind, d, 1 << 40, ks=None) == INVALID
    assert call_fp8k(kind, d, 1 << 40, ks=ctypes.c_void_p((1 << 20) + 2)) == INVALID
    assert call_fp8k(kind, d, 1 << 40, k8=None) == INVALID
    assert call_fp8k(kind, d, 1 << 40, q=None) == INVALID
    assert call_fp8k(kind, d, 1 << 40, k8=ctypes.c_void_p((1 << 20) + 8)) == INVALID
    assert call_fp8k(kind, good_dims(ctx_len=0), 1 << 40) == INVALID
    assert call_fp8k(kind, good_dims(head_dim=96), 1 << 40) == UNSUPPORTED
    assert call_fp8k(kind, good_dims(head_dim=32), 1 << 40) == UNSUPPORTED   # fp8 needs d_k >= 64
    assert call_fp8k(kind, d, need - 1) == SMALL         # same workspace as the bf16 calls
    if kind != "decode":
        assert call_fp8k(kind, d, 1 << 40, top_n=0) == INVALID


def call_fp8kv(kind, d, ws_bytes, top_n=8, **ptrs):
    p = dict(q=FAKE, k8=FAKE, ks=FAKE, v8=FAKE, vs=FAKE, tau=FAKE, out=FAKE, ws=FAKE)
    p.update(ptrs)
    lib = saga.library()
    if kind == "decode":
        return lib.saga_decode_step_fp8kv(ctypes.byref(d), p["q"], p["k8"], p["ks"], p["v8"],
                                          p["vs"], p["tau"], p["out"], None, None, p["ws"],
                                          ws_bytes, None)
    return lib.atopn_refresh_decode_step_fp8kv(ctypes.byref(d), top_n, p["q"], p["k8"], p["ks"],
                                               p["v8"], p["vs"], p["tau"], p["out"], None,
                                               p["ws"], ws_bytes, None)


@pytest.mark.parametrize("kind", ["decode", "fused"])
def test_fp8kv_argument_checks(kind):
    d = good_dims()
    need = saga.saga_workspace_bytes(d, 8)
    assert call_fp8kv(kind, d, 1 << 40, vs=None) == INVALID
    assert call_fp8kv(kind, d, 1 << 40, vs=ctypes.c_void_p((1 << 20) + 2)) == INVALID
    assert call_fp8kv(kind, d, 1 << 40, ks=None) == INVALID
    assert call_fp8kv(kind, d, 1 << 40, v8=None) == INVALID
    assert call_fp8kv(kind, d, 1 << 40, v8=ctypes.c_void_p((1 << 20) + 8)) == INVALID
    assert call_fp8kv(kind, good_dims(head_dim=32), 1 << 40) == UNSUPPORTED
    assert call_fp8kv(kind, good_dims(head_dim_v=96), 1 << 40) == UNSUPPORTED
    assert call_fp8kv(kind, d, need - 1) == SMALL        # same workspace as the bf16 calls
    if kind == "fused":
        assert call_fp8kv(kind, d, 1 << 40, top_n=0) == INVALID


def test_fp8k_binding_rejects_wrong_dtypes():
    d = good_dims()
    k8 = torch.zeros(4, dtype=torch.bfloat16)
    with pytest.raises((TypeError, ValueError)):
        saga.atopn_refresh_thresholds_fp8k(d, 8, k8, k8, k8, k8, k8)
