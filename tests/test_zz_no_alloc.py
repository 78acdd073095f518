"""saga_decode_step_noalloc (include/saga.h): the decode step whose workspace
is the library's own per-device scratch array, for callers that cannot
allocate.  Through the C ABI it must give bit-identical outputs and counts to
saga_decode_step with a caller workspace, on two calls in a row, the second
with a smaller input (the scratch then holds the first call's data), and must
refuse shapes whose workspace exceeds the array.  Runs last (file name), and
alone in a fresh process as well."""
import numpy as np
import pytest
import torch

import saga_workload as wl
import sparse_decode_attention_atop_amd as saga
from gpu_helpers import Guards, make_inputs

pytestmark = pytest.mark.gpu


def compare(q, K, V, ctx, N):
    B, hq, d = q.shape
    hk, rows, hv, dv = K.shape[1], K.shape[2], V.shape[1], V.shape[3]
    dm = saga.dims(B, hq, hk, hv, d, ctx, rows, head_dim_v=0 if dv == d else dv)
    g = Guards()
    ws = g.workspace(dm, N)
    tau = g.empty((B, hq), torch.float32, "tau")
    saga.atopn_refresh_thresholds(dm, N, q, K, tau, ws)
    ref_out = g.empty((B, hq, dv), torch.bfloat16, "out (workspace)")
    ref_cnt = g.empty((B, hq), torch.int32, "counts (workspace)")
    saga.saga_decode_step(dm, q, K, V, tau, ref_out, ws, sel_counts=ref_cnt)
    out = g.empty((B, hq, dv), torch.bfloat16, "out (no alloc)")
    cnt = g.empty((B, hq), torch.int32, "counts (no alloc)")
    saga.saga_decode_step_noalloc(dm, q, K, V, tau, out, sel_counts=cnt)
    torch.cuda.synchronize()
    g.check("after the no-alloc call")
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    assert torch.equal(cnt, ref_cnt)
    assert (cnt >= min(N, ctx)).all()


def test_no_alloc_matches_workspace_call_twice():
    # First call: the Llama-like 8K layer (one sequence, 32 query heads).
    w = wl.LLAMA_8K
    x = wl.make_layer(w, 0, device="cuda")
    print("[no-alloc] llama_like_8k, then a smaller Qwen-like shape", flush=True)
    compare(x["q"][0], x["K"], x["V"], w.L, w.top_n)
    # Second call, smaller: two sequences of 3000 rows, 12 query heads, d = 128.
    q, K, V = make_inputs(2, 12, 1, 2, 128, 3005, 1, seed=61)
    compare(q[0], K, V, 3000, 100)


def test_no_alloc_on_the_tail_gather():
    """Four sequences of Llama-like heads at 8K rows: 768 K-stream workgroups,
    which gather the value rows in their tails, on the library's scratch."""
    q, K, V = make_inputs(4, 32, 4, 8, 64, 8200, 1, seed=62)
    print("[no-alloc] llama-like heads, B=4, 8K rows (tail gather)", flush=True)
    compare(q[0], K, V, 8192, 512)


@pytest.mark.parametrize("name", ["qwen_like_128k_b1", "sweep_llama_L131072_N2048_B1"])
def test_no_alloc_at_long_context(name):
    """Batch 1 at 128K context: Qwen-like heads (27 MiB of scratch) and
    Llama-like heads (69 MiB)."""
    w = {x.name: x for x in [wl.QWEN_128K_B1, *wl.sweep()]}[name]
    x = wl.make_layer(w, 0, device="cuda", steps=1)
    print(f"[no-alloc] {name}", flush=True)
    compare(x["q"][0], x["K"], x["V"], w.L, w.top_n)


def test_no_alloc_refuses_shapes_beyond_the_scratch():
    w = wl.LLAMA_128K_B16
    dm = saga.dims(w.batch, w.h_q, w.h_k, w.h_v, w.head_dim, w.L, w.rows)
    assert saga.saga_workspace_bytes(dm, w.top_n) > saga.NOALLOC_SCRATCH_BYTES
    small = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    f32 = torch.empty(w.batch * w.h_q, dtype=torch.float32, device="cuda")
    # Pointers are only validated, never read: the call fails before any launch.
    rc = saga.library().saga_decode_step_noalloc(
        saga.ctypes.byref(dm), saga.ctypes.c_void_p(small.data_ptr()),
        saga.ctypes.c_void_p(small.data_ptr()), saga.ctypes.c_void_p(small.data_ptr()),
        saga.ctypes.c_void_p(f32.data_ptr()), saga.ctypes.c_void_p(small.data_ptr()), None, None)
    assert rc == saga.SAGA_ERR_WORKSPACE_TOO_SMALL
    bad = saga.dims(1, 12, 5, 2, 128, 100, 100)        # h_q not a multiple of h_k
    assert saga.library().saga_decode_step_noalloc(
        saga.ctypes.byref(bad), None, None, None, None, None, None, None) == \
        saga.SAGA_ERR_INVALID_ARGUMENT
