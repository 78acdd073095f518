"""The small-batch decode path (fused.hip: K stream, mask, compaction and value
gather in one kernel, then a combine over many chunks), taken by
saga_decode_step when there are few (batch row, key head) groups and enough
chunks.

Its LDS holds every entry a chunk can select, so the worst case, every row
selected for every query head, must still be exact: with
thresholds of -inf (N >= ctx) the output is full attention (checked against
oracle_full) and every count is ctx; with all logits tied (K = 0) every row is
kept and the output is the mean of the value rows.  The shapes take one and
two 16-row groups per wave tile and head groups of 4, 8, 12 and 16.  A call
with a real threshold is checked against the GPU's own logits and the oracle
on its mask.  The ordinary selections of this path are also checked against
the oracle by test_gpu_parity.py and test_gpu_fullsize.py (their batch-1
shapes of 32K rows and more run it)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_decode_attention_atop_amd as saga
from gpu_helpers import Guards, make_inputs, to_np_bits

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-2

SHAPES = {
    # name: (B, hq, hk, hv, d, ctx) -- at most 4 (b, key head) groups, at least
    # 64 fused workgroups.  Plans (16-row groups per wave tile, chunks x rows):
    "qwen_like_long": (1, 12, 1, 2, 128, 40000),      # 1, 313 x 128
    "llama_like": (1, 32, 4, 8, 64, 30000),           # 2, 118 x 256
    "group16_two_rows": (2, 16, 1, 4, 64, 20000),     # 1, 157 x 128
    "group4": (1, 4, 1, 2, 128, 40000),               # 1, 313 x 128
    "llama_like_64k": (1, 32, 4, 8, 64, 65551),       # 2, 129 x 512
    "llama_like_128k": (1, 32, 4, 8, 64, 131104),     # 2, 171 x 768 (48 KB of queues)
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


@pytest.mark.parametrize("name", ["qwen_like_long", "llama_like", "llama_like_64k",
                                  "llama_like_128k"])
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


def test_refreshed_threshold_against_oracle():
    """Thresholds from a refresh (N = 2048), then a decode on the small-batch
    path: its selection bitmap equals the GPU logits >= tau, counts match it,
    and the output is within the bar of the fp64 oracle on that mask."""
    B, hq, hk, hv, d, ctx = SHAPES["llama_like_64k"]
    q, K, V = make_inputs(B, hq, hk, hv, d, ctx + 3, 1, seed=230)
    print(f"[fused refreshed threshold] ctx={ctx}", flush=True)
    dm = saga.dims(B, hq, hk, hv, d, ctx, ctx + 3)
    g = Guards()
    ws = g.workspace(dm, 2048)
    tau = g.empty((B, hq), torch.float32, "tau")
    logits = g.empty((B, hq, ctx), torch.float32, "logits")
    saga.atopn_refresh_thresholds(dm, 2048, q[0], K, tau, ws, logits_debug=logits)
    words = (ctx + 3 + 31) // 32
    bm = g.empty((B, hq, words), torch.int32, "bitmap")
    out = g.empty((B, hq, d), torch.bfloat16, "out")
    cnt = g.empty((B, hq), torch.int32, "sel_counts")
    saga.saga_decode_step(dm, q[0], K, V, tau, out, ws, sel_counts=cnt, sel_bitmap_debug=bm)
    torch.cuda.synchronize()
    g.check()
    lg = logits.cpu().numpy()
    tg = tau.cpu().numpy()
    bm_np = bm.cpu().numpy().view(np.uint32)
    sel = np.unpackbits(bm_np.view(np.uint8), axis=-1, bitorder="little")[..., :ctx].astype(bool)
    assert np.array_equal(sel, lg >= tg[..., None])
    assert np.array_equal(cnt.cpu().numpy(), sel.sum(axis=-1))
    ref, _ = oracle.masked(to_np_bits(q[0]), to_np_bits(K), to_np_bits(V), ctx, bm_np)
    err = np.abs(out.float().cpu().numpy() - ref).max()
    assert err <= OUT_TOL, f"{err:.3e}"
