"""The small-batch decode path (fused.hip: K stream, mask, compaction and value
gather in one kernel, then a combine over many chunks), taken by
saga_decode_step when there are few (batch row, key head) groups.

Its LDS holds every entry a chunk can select, so the worst case, every row
selected for every query head, must still be exact: with thresholds of -inf
(N >= ctx) the output is full attention (checked against oracle_full) and
every count is ctx; with all logits tied (K = 0) every row is kept and the
output is the mean of the value rows.  Both at shapes whose plans use one and
two 16-row groups per wave tile and head groups of 4, 8, 12 and 16.  The
ordinary selections of this path are checked against the oracle by
test_gpu_parity.py and test_gpu_fullsize.py (their batch-1 shapes run it)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_decode_attention_atop_amd as saga
from gpu_helpers import Guards, make_inputs, to_np_bits

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-2

SHAPES = {
    # name: (B, hq, hk, hv, d, ctx) -- at most 4 (b, key head) groups
    "qwen_like_long": (1, 12, 1, 2, 128, 40000),
    "llama_like": (1, 32, 4, 8, 64, 30000),
    "group16_two_rows": (2, 16, 1, 4, 64, 9000),
    "group4_short": (1, 4, 1, 2, 128, 700),
}


def decode_with_tau(q, K, V, ctx, tau_value):
    B, hq, d = q.shape
    hk, rows, hv = K.shape[1], K.shape[2], V.shape[1]
    dm = saga.dims(B, hq, hk, hv, d, ctx, rows)
    g = Guards()
    ws = g.workspace(dm, 1)
    tau = g.empty((B, hq), torch.float32, "tau")
    tau.fill_(tau_value)
    out = g.empty((B, hq, d), torch.bfloat16, "out")
    cnt = g.empty((B, hq), torch.int32, "sel_counts")
    saga.saga_decode_step(dm, q, K, V, tau, out, ws, sel_counts=cnt)
    torch.cuda.synchronize()
    g.check()
    return out.float().cpu().numpy(), cnt.cpu().numpy()


@pytest.mark.parametrize("name", list(SHAPES))
def test_every_row_selected_is_full_attention(name):
    B, hq, hk, hv, d, ctx = SHAPES[name]
    q, K, V = make_inputs(B, hq, hk, hv, d, ctx + 3, 1, seed=200 + len(name))
    print(f"[fused all-selected {name}] ctx={ctx}", flush=True)
    out, cnt = decode_with_tau(q[0], K, V, ctx, float("-inf"))
    assert (cnt == ctx).all()
    ref = oracle.full(to_np_bits(q[0]), to_np_bits(K), to_np_bits(V), ctx)
    err = np.abs(out - ref).max()
    assert err <= OUT_TOL, f"{name}: {err:.3e}"


@pytest.mark.parametrize("name", ["qwen_like_long", "llama_like"])
def test_all_logits_tied_keeps_every_row(name):
    B, hq, hk, hv, d, ctx = SHAPES[name]
    q, K, V = make_inputs(B, hq, hk, hv, d, ctx + 3, 1, seed=210 + len(name))
    K.zero_()
    out, cnt = decode_with_tau(q[0], K, V, ctx, 0.0)
    assert (cnt == ctx).all()
    mean = V[:, :, :ctx].float().mean(dim=2).cpu().numpy()          # [B][hv][d]
    ref = np.repeat(mean, hq // hv, axis=1)
    assert np.abs(out - ref).max() <= OUT_TOL


def test_fused_runs_are_bit_identical():
    B, hq, hk, hv, d, ctx = SHAPES["qwen_like_long"]
    q, K, V = make_inputs(B, hq, hk, hv, d, ctx + 3, 1, seed=220)
    dm = saga.dims(B, hq, hk, hv, d, ctx, ctx + 3)
    ws = saga.alloc_workspace(dm, 500)
    tau = torch.empty(B, hq, device="cuda")
    saga.atopn_refresh_thresholds(dm, 500, q[0], K, tau, ws)
    outs = []
    for _ in range(3):
        out = torch.empty(B, hq, d, dtype=torch.bfloat16, device="cuda")
        saga.saga_decode_step(dm, q[0], K, V, tau, out, ws)
        torch.cuda.synchronize()
        outs.append(out.view(torch.int16).clone())
    assert all(torch.equal(outs[0], o) for o in outs[1:])
