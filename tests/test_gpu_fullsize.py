"""Parity at the benchmark workloads' full sizes, in the launch configuration
bench.py times: every decode step of one layer runs on the GPU through the C
ABI (refresh when t mod n == 0), and sampled (batch row, query head) outputs,
thresholds and selections are checked against the fp64 oracle, which computes
each sampled row on its own (a one-head sub-problem of that row's key and
value heads).  Bars as in test_gpu_parity.py."""
import numpy as np
import pytest
import torch

import oracle
import saga_workload as wl
import sparse_decode_attention_atop_amd as saga
from gpu_helpers import bitmap_to_bool, nth_largest_f32

pytestmark = pytest.mark.gpu

SAMPLES = 5


def sampled_rows(w, rng):
    rows = {(0, 0), (w.batch - 1, w.h_q - 1)}
    while len(rows) < SAMPLES:
        rows.add((int(rng.integers(w.batch)), int(rng.integers(w.h_q))))
    return sorted(rows)


@pytest.mark.parametrize("name", ["llama_like_128k_b16", "qwen_like_128k_b1", "qwen_like_128k_b16"])
def test_full_size_sampled_rows(name):
    w = wl.WORKLOADS[name]
    layer = w.layers - 1
    print(f"[fullsize {name} layer {layer}]", flush=True)
    x = wl.make_layer(w, layer, device="cuda")
    q, K, V = x["q"], x["K"], x["V"]
    B, hq, hk, hv, d = w.batch, w.h_q, w.h_k, w.h_v, w.head_dim
    Gk, Gv = hq // hk, hq // hv
    rows = sampled_rows(w, np.random.default_rng(len(name)))
    ws = saga.alloc_workspace(saga.dims(B, hq, hk, hv, d, w.L, w.rows), w.top_n)
    tau = torch.empty(B, hq, dtype=torch.float32, device="cuda")
    words = (w.rows + 31) // 32
    per_step = []
    for t in range(w.steps):
        ctx = w.ctx(t)
        dm = saga.dims(B, hq, hk, hv, d, ctx, w.rows)
        lg = None
        if t % w.refresh_n == 0:
            lg = torch.empty(B, hq, ctx, dtype=torch.float32, device="cuda")
            saga.atopn_refresh_thresholds(dm, w.top_n, q[t], K, tau, ws, logits_debug=lg)
        out = torch.empty(B, hq, d, dtype=torch.bfloat16, device="cuda")
        cnt = torch.empty(B, hq, dtype=torch.int32, device="cuda")
        bm = torch.empty(B, hq, words, dtype=torch.int32, device="cuda")
        saga.saga_decode_step(dm, q[t], K, V, tau, out, ws, sel_counts=cnt, sel_bitmap_debug=bm)
        torch.cuda.synchronize()
        idx = torch.tensor(rows, device="cuda")
        per_step.append(dict(
            tau=tau[idx[:, 0], idx[:, 1]].cpu().numpy(),
            out=out[idx[:, 0], idx[:, 1]].float().cpu().numpy(),
            cnt=cnt[idx[:, 0], idx[:, 1]].cpu().numpy(),
            bm=bm[idx[:, 0], idx[:, 1]].cpu().numpy().view(np.uint32),
            lg=None if lg is None else lg[idx[:, 0], idx[:, 1]].cpu().numpy()))
    ctx_steps = [w.ctx(t) for t in range(w.steps)]
    for r, (b, i) in enumerate(rows):
        Kb = wl.bits(K[b, i // Gk][None, None])
        Vb = wl.bits(V[b, i // Gv][None, None])
        qb = wl.bits(q[:, b, i][:, None, None])
        ref = oracle.atopn_run(qb, Kb, Vb, ctx_steps, w.top_n, w.refresh_n, want_sel=True,
                               want_logits=True)
        for t, ctx in enumerate(ctx_steps):
            g = per_step[t]
            if g["lg"] is not None:
                assert g["tau"][r] == nth_largest_f32(g["lg"][r], w.top_n), (b, i, t)
                assert abs(g["tau"][r] - ref["tau"][t, 0, 0]) <= 1e-4
            sel = bitmap_to_bool(g["bm"][r], ctx)
            assert g["cnt"][r] == sel.sum()
            s = ref["logits"][t, 0, 0, :ctx]
            near = np.abs(s - ref["tau"][t, 0, 0]) <= 1e-3
            bad = (sel != ref["sel"][t, 0, 0, :ctx].astype(bool)) & ~near
            assert not bad.any(), f"(b={b}, i={i}) step {t}: {bad.sum()} entries differ"
            mo, mc = oracle.masked(qb[t], Kb, Vb, ctx, g["bm"][r][None, None])
            assert mc[0, 0] == g["cnt"][r]
            err = np.abs(g["out"][r] - mo[0, 0]).max()
            assert err <= 1e-2, f"(b={b}, i={i}) step {t}: {err:.3e}"
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
