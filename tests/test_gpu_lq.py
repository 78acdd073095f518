"""Several query tokens per head and step (the *_lq calls) on the GPU.

Token j of a step with l_q tokens attends rows 0 .. ctx - l_q + j and keeps a
threshold of its own.  Per token the calls must equal the one-token calls run
with that token's queries at ctx - (l_q - 1 - j): thresholds bit-equal, counts
equal, and outputs within the output bar of the fp64 oracle on that mask.  The
thresholds and selections are also checked against the oracle's Atop-N run of
that token's sub-problem (tau within 1e-4; sets equal away from 1e-3 of tau).
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_decode_attention_atop_amd as saga
from gpu_helpers import Guards, bitmap_to_bool, make_inputs, to_np_bits

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-2
NEAR_TAU = 1e-3

LQ_SHAPES = {
    # name: (B, hq, hk, hv, d, L, T, N, n, l_q)
    "llama_like_lq2": (2, 32, 4, 8, 64, 3000, 4, 128, 2, 2),
    "group4_lq4_d128": (2, 8, 2, 4, 128, 2000, 3, 100, 2, 4),
    "mha_lq16": (1, 4, 4, 4, 64, 900, 3, 40, 3, 16),
    "short_context_lq4": (1, 8, 2, 4, 64, 60, 3, 64, 2, 4),        # N >= ctx for every token
    "small_batch_path_lq4": (1, 8, 2, 4, 128, 40000, 3, 500, 2, 4),  # >= 64 fused workgroups
    "tail_gather_lq4_d128": (32, 8, 2, 4, 128, 16400, 2, 200, 2, 4),  # 512 workgroups, 16 slots
    "tail_gather_llama_like_lq2": (4, 32, 4, 8, 64, 3000, 3, 128, 2, 2),  # 384 workgroups, 16 slots
}


def run_lq(q, K, V, ctx_steps, N, n, lq, fused=True):
    T, B, hql, d = q.shape
    hq = hql // lq
    hk, rows, hv = K.shape[1], K.shape[2], V.shape[1]
    g = Guards()
    ws = g.workspace(saga.dims(B, hq, hk, hv, d, ctx_steps[0], rows), N, lq=lq)
    tau = g.empty((B, hq, lq), torch.float32, "tau")
    res = []
    for t, ctx in enumerate(ctx_steps):
        dm = saga.dims(B, hq, hk, hv, d, ctx, rows)
        out = g.empty((B, hq, lq, d), torch.bfloat16, "out")
        cnt = g.empty((B, hq, lq), torch.int32, "sel_counts")
        if t % n == 0 and fused:
            saga.atopn_refresh_decode_step_lq(dm, lq, N, q[t], K, V, tau, out, ws, sel_counts=cnt)
        else:
            if t % n == 0:
                saga.atopn_refresh_thresholds_lq(dm, lq, N, q[t], K, tau, ws)
            saga.saga_decode_step_lq(dm, lq, q[t], K, V, tau, out, ws, sel_counts=cnt)
        torch.cuda.synchronize()
        g.check(f"at step {t}")
        g.bufs = g.bufs[:2]
        res.append((tau.clone(), cnt.clone(), out.clone()))
    return res


def run_one_token(q, K, V, ctx_steps, N, n):
    """The one-token calls; also the selection bitmap of every step."""
    T, B, hq, d = q.shape
    hk, rows, hv = K.shape[1], K.shape[2], V.shape[1]
    g = Guards()
    ws = g.workspace(saga.dims(B, hq, hk, hv, d, ctx_steps[0], rows), N)
    tau = g.empty((B, hq), torch.float32, "tau")
    res = []
    for t, ctx in enumerate(ctx_steps):
        dm = saga.dims(B, hq, hk, hv, d, ctx, rows)
        if t % n == 0:
            saga.atopn_refresh_thresholds(dm, N, q[t], K, tau, ws)
        out = g.empty((B, hq, d), torch.bfloat16, "out")
        cnt = g.empty((B, hq), torch.int32, "sel_counts")
        bm = g.empty((B, hq, (rows + 31) // 32), torch.int32, "sel_bitmap")
        saga.saga_decode_step(dm, q[t], K, V, tau, out, ws, sel_counts=cnt, sel_bitmap_debug=bm)
        torch.cuda.synchronize()
        g.check(f"at step {t}")
        g.bufs = g.bufs[:2]
        res.append((tau.clone(), cnt.clone(), out.clone(), bm.cpu().numpy().view(np.uint32)))
    return res


def f32_bits(t):
    return t.cpu().contiguous().view(torch.int32).numpy()


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("name", list(LQ_SHAPES))
def test_each_token_equals_the_one_token_path(name, fused):
    B, hq, hk, hv, d, L, T, N, n, lq = LQ_SHAPES[name]
    rows = L + lq * T
    # Virtual heads: q[t][b][i * lq + j] is token j of query head i.
    q, K, V = make_inputs(B, hq * lq, hk, hv, d, rows, T, seed=100 + len(name))
    ctx = [L + lq * (t + 1) for t in range(T)]                    # the step's tokens included
    print(f"[lq {name}] l_q={lq} ctx={ctx}", flush=True)
    got = run_lq(q, K, V, ctx, N, n, lq, fused=fused)
    qb, Kb, Vb = to_np_bits(q), to_np_bits(K), to_np_bits(V)
    for j in range(lq):
        qj = q[:, :, j::lq].contiguous()                             # [T][B][hq][d]
        ctx_j = [c - (lq - 1 - j) for c in ctx]
        ref = run_one_token(qj, K, V, ctx_j, N, n)
        orc = oracle.atopn_run(to_np_bits(qj), Kb, Vb, ctx_j, N, n, want_sel=True,
                               want_logits=True)
        for t in range(T):
            tau_r, cnt_r, _, bm = ref[t]
            tau_g, cnt_g, out_g = got[t]
            assert np.array_equal(f32_bits(tau_r), f32_bits(tau_g[:, :, j])), (j, t)
            assert np.array_equal(cnt_r.cpu().numpy(), cnt_g[:, :, j].cpu().numpy()), (j, t)
            if N >= ctx_j[t]:
                assert torch.isneginf(tau_g[:, :, j]).all()
            ref_o, cnt_o = oracle.masked(qb[t][:, j::lq], Kb, Vb, ctx_j[t], bm)
            assert (cnt_o == cnt_g[:, :, j].cpu().numpy()).all()
            tau_o = orc["tau"][t]
            tg = tau_g[:, :, j].cpu().numpy().astype(np.float64)
            both_inf = np.isneginf(tg) & np.isneginf(tau_o)
            diff = np.subtract(tg, tau_o, out=np.zeros_like(tg), where=~both_inf)
            assert (both_inf | (np.abs(diff) <= 1e-4)).all()
            sel = bitmap_to_bool(bm, ctx_j[t])
            s_o = orc["logits"][t, :, :, :ctx_j[t]]
            near = np.abs(s_o - tau_o[..., None]) <= NEAR_TAU
            bad = (sel != orc["sel"][t, :, :, :ctx_j[t]].astype(bool)) & ~near
            assert not bad.any(), f"token {j} step {t}: {bad.sum()} entries differ from the oracle"
            err = np.abs(out_g[:, :, j].float().cpu().numpy() - ref_o).max()
            assert err <= OUT_TOL, f"token {j} step {t}: {err:.3e}"
