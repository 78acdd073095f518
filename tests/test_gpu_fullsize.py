"""Parity at the benchmark workloads' full sizes, with the calls and the launch
configuration bench.py times: one layer runs the whole decode schedule (the
one-call refresh step atopn_refresh_decode_step when t mod n == 0,
saga_decode_step otherwise, one workspace, no debug outputs), and sampled
(batch row, query head) rows are checked at every step against the fp64
oracle, which computes each sampled row on its own (a one-head sub-problem of
that row's key and value heads):

  * thresholds within 1e-4 of the oracle's, and at refresh steps bit-equal
    to the N-th largest of the GPU's own fp32 logits (host sort);
  * the call's selection count equals #{GPU logits >= tau}, and that set
    equals the oracle's Atop-N set except entries within 1e-3 of the
    threshold;
  * outputs within 1e-2 of the oracle run on that set.
The GPU logits come from a separate refresh call with its own workspace (the
same QK routine the decode kernels run).  The same check runs at three points
of the L x N x B sweep, and the full-attention path is checked at the 128K
GQA twins that form the bench's speedup denominator, and at N = 8192, where
the threshold select works on candidate lists above its staging size.  Bars
as in test_gpu_parity.py."""
import numpy as np
import pytest
import torch

import oracle
import saga_workload as wl
import sparse_decode_attention_atop_amd as saga
from gpu_helpers import (Guards, logit_tolerance, mask_to_bitmap, nth_largest_f32,
                         run_bench_schedule)

pytestmark = pytest.mark.gpu

SAMPLES = 5
OUT_TOL = 1e-2
NEAR_TAU = 1e-3
SWEEP_POINTS = ("sweep_llama_L8192_N2048_B16", "sweep_qwen_L32768_N512_B1",
                "sweep_llama_L65536_N1024_B1")


def sampled_rows(w, rng):
    rows = {(0, 0), (w.batch - 1, w.h_q - 1)}
    while len(rows) < SAMPLES:
        rows.add((int(rng.integers(w.batch)), int(rng.integers(w.h_q))))
    return sorted(rows)


def workload(name):
    if name in wl.WORKLOADS:
        return wl.WORKLOADS[name]
    return {w.name: w for w in wl.sweep()}[name]


def check_schedule(w, layer):
    print(f"[fullsize {w.name} layer {layer}]", flush=True)
    x = wl.make_layer(w, layer, device="cuda")
    q, K, V = x["q"], x["K"], x["V"]
    Gk, Gv = w.h_q // w.h_k, w.h_q // w.h_v
    rows = sampled_rows(w, np.random.default_rng(len(w.name)))
    ctx_steps = [w.ctx(t) for t in range(w.steps)]
    gpu = run_bench_schedule(q, K, V, ctx_steps, w.top_n, w.refresh_n, rows, w.scale)
    for r, (b, i) in enumerate(rows):
        Kb = wl.bits(K[b, i // Gk][None, None])
        Vb = wl.bits(V[b, i // Gv][None, None])
        qb = wl.bits(q[:, b, i][:, None, None])
        ref = oracle.atopn_run(qb, Kb, Vb, ctx_steps, w.top_n, w.refresh_n, w.scale,
                               want_sel=True, want_logits=True)
        for t, ctx in enumerate(ctx_steps):
            lg, tau = gpu["logits"][t][r], gpu["tau"][t][r]
            s = ref["logits"][t, 0, 0, :ctx]
            tol = logit_tolerance(qb[t], Kb, ctx, w.scale)[0, 0]
            assert (np.abs(lg - s) <= tol).all(), f"(b={b}, i={i}) step {t}: logits"
            if t % w.refresh_n == 0:
                assert tau == nth_largest_f32(lg, w.top_n), (b, i, t)
            assert abs(float(tau) - ref["tau"][t, 0, 0]) <= 1e-4 or \
                (np.isneginf(tau) and np.isneginf(ref["tau"][t, 0, 0])), (b, i, t)
            sel = lg >= tau
            assert gpu["counts"][t][r] == sel.sum(), f"(b={b}, i={i}) step {t}: count"
            near = np.abs(s - ref["tau"][t, 0, 0]) <= NEAR_TAU
            bad = (sel != ref["sel"][t, 0, 0, :ctx].astype(bool)) & ~near
            assert not bad.any(), f"(b={b}, i={i}) step {t}: {bad.sum()} entries differ"
            bm = mask_to_bitmap(sel[None, None], Kb.shape[2])
            mo, mc = oracle.masked(qb[t], Kb, Vb, ctx, bm, w.scale)
            assert mc[0, 0] == gpu["counts"][t][r]
            err = np.abs(gpu["out"][t][r] - mo[0, 0]).max()
            assert err <= OUT_TOL, f"(b={b}, i={i}) step {t}: {err:.3e}"
    del x, q, K, V
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["llama_like_128k_b16", "qwen_like_128k_b1", "qwen_like_128k_b16"])
def test_bench_schedule_full_size(name):
    w = wl.WORKLOADS[name]
    check_schedule(w, w.layers - 1)


@pytest.mark.parametrize("name", SWEEP_POINTS)
def test_bench_schedule_sweep_points(name):
    check_schedule(workload(name), 0)


def test_bench_schedule_large_n():
    """The benchmark's Llama-like 128K B=16 layer at N = 8192 (bench.py
    --top-n 8192): the refresh's candidate lists then hold more than the 8192
    entries the register select stages, and it selects among them in place."""
    w = wl.WORKLOADS["llama_like_128k_b16"]
    check_schedule(w.with_(name=w.name + "_n8192", top_n=8192), 0)


@pytest.mark.parametrize("name", ["llama_like_128k_b16", "qwen_like_128k_b16"])
def test_full_attention_at_gqa_twin(name):
    """saga_full_attention on the h_k = h_v twin the bench divides by, at the
    first and last step of the run, on sampled rows against oracle_full."""
    hkv = wl.GQA_HKV["llama" if "llama" in name else "qwen"]
    w = wl.WORKLOADS[name].gqa(hkv)
    print(f"[fullsize {w.name}] h_k = h_v = {hkv}", flush=True)
    x = wl.make_layer(w, 0, device="cuda")
    q, K, V = x["q"], x["K"], x["V"]
    G = w.h_q // hkv
    rows = sampled_rows(w, np.random.default_rng(7 + len(name)))
    g = Guards()
    ws = g.workspace(saga.dims(w.batch, w.h_q, w.h_k, w.h_v, w.head_dim, w.L, w.rows), 1)
    out = g.empty((w.batch, w.h_q, w.head_dim), torch.bfloat16, "out")
    for t in (0, w.steps - 1):
        ctx = w.ctx(t)
        saga.saga_full_attention(saga.dims(w.batch, w.h_q, w.h_k, w.h_v, w.head_dim, ctx, w.rows),
                                 q[t], K, V, out, ws)
        torch.cuda.synchronize()
        g.check(f"at step {t}")
        for b, i in rows:
            Kb = wl.bits(K[b, i // G][None, None])
            Vb = wl.bits(V[b, i // G][None, None])
            ref = oracle.full(wl.bits(q[t, b, i][None, None]), Kb, Vb, ctx)
            err = np.abs(out[b, i].float().cpu().numpy() - ref[0, 0]).max()
            assert err <= OUT_TOL, f"(b={b}, i={i}) step {t}: {err:.3e}"
    del x, q, K, V, ws
    torch.cuda.empty_cache()


def test_graph_replay_matches_eager():
    """A decode step captured in a HIP graph and replayed several times, with eager
    work in between, gives bit-identical outputs to the eager call."""
    w = wl.LLAMA_8K
    x = wl.make_layer(w, 0, device="cuda")
    q, K, V = x["q"], x["K"], x["V"]
    B, hq, hk, hv, d = w.batch, w.h_q, w.h_k, w.h_v, w.head_dim
    dm = saga.dims(B, hq, hk, hv, d, w.L, w.rows)
    ws = saga.alloc_workspace(dm, w.top_n)
    tau = torch.empty(B, hq, device="cuda")
    out = torch.empty(B, hq, d, dtype=torch.bfloat16, device="cuda")
    cnt = torch.empty(B, hq, dtype=torch.int32, device="cuda")

    def step():
        saga.atopn_refresh_thresholds(dm, w.top_n, q[0], K, tau, ws)
        saga.saga_decode_step(dm, q[0], K, V, tau, out, ws, sel_counts=cnt)

    step()
    torch.cuda.synchronize()
    ref_out, ref_tau, ref_cnt = out.clone(), tau.clone(), cnt.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        out.zero_()
        tau.zero_()
        saga.saga_decode_step(saga.dims(B, hq, hk, hv, d, w.L + 3, w.rows), q[3], K, V,
                              torch.full_like(tau, 0.5), torch.empty_like(out), ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(tau, ref_tau) and torch.equal(cnt, ref_cnt), rep
