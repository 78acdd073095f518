"""The largest cache the library accepts: one cache head just under 2 GiB.

A cache head is addressed with 32-bit byte offsets, so the boundary allows
cache_len * max(d_k, d_v) * 2 < 2^31: 2^23 - 1 rows at d = 128 and 2^24 - 1 at
d = 64 (ragged: not a multiple of any tile).  Two decode steps of Atop-N (refresh at
the first) run on the GPU through the C ABI; two (batch row, query head) rows
are checked against the fp64 oracle on their one-head sub-problem.  Checks:
the GPU logits over the whole row (including its last rows, whose offsets sit
next to the limit) within the fp32 bar of the oracle's, the threshold
bit-equal to the N-th largest GPU logit, the selection against the oracle's
away from the threshold, and the outputs within 1e-2 of the oracle on the GPU's
mask.
"""
import numpy as np
import pytest
import torch

import oracle
import saga_workload as wl
import sparse_decode_attention_atop_amd as saga
from gpu_helpers import bitmap_to_bool, make_inputs, nth_largest_f32

pytestmark = pytest.mark.gpu

N, REFRESH = 1024, 2


@pytest.mark.parametrize("d", [128, 64])
def test_largest_cache_head(d):
    B, hq, hk, hv = 1, 4, 1, 2
    ROWS = (1 << 31) // (2 * d) - 1
    assert ROWS * d * 2 < (1 << 31) <= (ROWS + 1) * d * 2
    print(f"[maxsize] rows={ROWS} d={d}: drawing inputs", flush=True)
    q, K, V = make_inputs(B, hq, hk, hv, d, ROWS, 2, seed=81)
    ctx_steps = [ROWS - 1, ROWS]
    ws = saga.alloc_workspace(saga.dims(B, hq, hk, hv, d, ctx_steps[0], ROWS), N)
    tau = torch.empty(B, hq, dtype=torch.float32, device="cuda")
    words = (ROWS + 31) // 32
    steps = []
    for t, ctx in enumerate(ctx_steps):
        print(f"[maxsize] step {t} ctx={ctx}", flush=True)
        dm = saga.dims(B, hq, hk, hv, d, ctx, ROWS)
        lg = None
        if t % REFRESH == 0:
            lg = torch.empty(B, hq, ctx, dtype=torch.float32, device="cuda")
            saga.atopn_refresh_thresholds(dm, N, q[t], K, tau, ws, logits_debug=lg)
        out = torch.empty(B, hq, d, dtype=torch.bfloat16, device="cuda")
        cnt = torch.empty(B, hq, dtype=torch.int32, device="cuda")
        bm = torch.empty(B, hq, words, dtype=torch.int32, device="cuda")
        saga.saga_decode_step(dm, q[t], K, V, tau, out, ws, sel_counts=cnt, sel_bitmap_debug=bm)
        torch.cuda.synchronize()
        steps.append(dict(tau=tau.cpu().numpy().copy(), out=out.float().cpu().numpy(),
                          cnt=cnt.cpu().numpy(), bm=bm.cpu().numpy().view(np.uint32),
                          lg=None if lg is None else lg.cpu().numpy()))
    Gk, Gv = hq // hk, hq // hv
    for b, i in [(0, 0), (0, hq - 1)]:
        print(f"[maxsize] oracle for (b={b}, i={i})", flush=True)
        Kb = wl.bits(K[b, i // Gk][None, None])
        Vb = wl.bits(V[b, i // Gv][None, None])
        qb = wl.bits(q[:, b, i][:, None, None])
        ref = oracle.atopn_run(qb, Kb, Vb, ctx_steps, N, REFRESH, want_sel=True, want_logits=True)
        for t, ctx in enumerate(ctx_steps):
            g = steps[t]
            if g["lg"] is not None:
                s = g["lg"][b, i]
                err = np.abs(s.astype(np.float64) - ref["logits"][t, 0, 0, :ctx])
                # The logit bar of the other parity tests, 1e-5 * sum_c |q_c k_c| + 1e-6,
                # with the magnitude sum taken on the GPU (fp32 is ample for a bound).
                mag = (K[b, i // Gk, :ctx].float().abs() @ q[t, b, i].float().abs()).cpu().numpy()
                tol = 1e-5 * mag.astype(np.float64) + 1e-6
                assert (err <= tol).all(), f"step {t}: logits beyond the bar at rows {np.nonzero(err > tol)[0][:5]}"
                assert g["tau"][b, i] == nth_largest_f32(s, N), (b, i, t)
            sel = bitmap_to_bool(g["bm"][b, i], ctx)
            assert g["cnt"][b, i] == sel.sum()
            sr = ref["logits"][t, 0, 0, :ctx]
            near = np.abs(sr - ref["tau"][t, 0, 0]) <= 1e-3
            bad = (sel != ref["sel"][t, 0, 0, :ctx].astype(bool)) & ~near
            assert not bad.any(), f"(b={b}, i={i}) step {t}: {bad.sum()} entries differ"
            mo, mc = oracle.masked(qb[t], Kb, Vb, ctx, g["bm"][b, i][None, None])
            assert mc[0, 0] == g["cnt"][b, i]
            err = np.abs(g["out"][b, i] - mo[0, 0]).max()
            assert err <= 1e-2, f"(b={b}, i={i}) step {t}: {err:.3e}"
    del q, K, V, ws
    torch.cuda.empty_cache()


def test_more_query_rows_than_a_grid_dimension():
    """B*h_q above 65535 (the limit of a launch grid's y dimension); B*h_k stays
    under the library's own limit.  Every row: tau bit-equal to the N-th largest
    GPU logit, counts, and outputs within 1e-2 of the oracle on the GPU's mask."""
    from gpu_helpers import run_atopn, to_np_bits
    B, hq, hk, hv, d, N = 2100, 32, 4, 8, 64, 16
    assert B * hq > 65535 and B * hk <= 65535
    print(f"[maxsize] B*h_q = {B * hq}", flush=True)
    q, K, V = make_inputs(B, hq, hk, hv, d, 130, 2, seed=82, heavy=False)
    ctx_steps = [128, 129]
    gpu = run_atopn(q, K, V, ctx_steps, N, 2)
    qb, Kb, Vb = to_np_bits(q), to_np_bits(K), to_np_bits(V)
    lg, tau = gpu["logits"][0], gpu["tau"][0]
    nth = np.sort(lg.astype(np.float32), axis=-1)[..., ::-1][..., N - 1]
    assert np.array_equal(tau.view(np.uint32), nth.view(np.uint32))
    for t, ctx in enumerate(ctx_steps):
        ref, cnt = oracle.masked(qb[t], Kb, Vb, ctx, gpu["bitmap"][t])
        assert (cnt == gpu["counts"][t]).all(), t
        err = np.abs(gpu["out"][t] - ref).max()
        assert err <= 1e-2, f"step {t}: max abs err {err:.3e}"
