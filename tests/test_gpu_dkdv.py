"""Key and value head dimensions that differ (saga_dims.head_dim_v) on the GPU.

The pages weigh head count against head dimension with a Sigma-style
(h_k, d_k) = (2, 32) next to SAGA's (1, 64), both at h_v = 8, d_v = 64
("More Value per Key", ai.info summary, Main Findings).  The K side (stream,
refresh) runs at d_k and the V side (gather, combine) at d_v; every bar of the
main parity tests applies: logits within the fp32 bar of the fp64 oracle,
thresholds bit-exact against a host sort of the GPU logits, selection an exact
filter of the GPU logits and equal to the oracle's away from the threshold,
outputs within 1e-2 of the oracle on the GPU's mask.  Also the one-call refresh
step, the dense path, and paged caches.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_decode_attention_atop_amd as saga
from gpu_helpers import (bitmap_to_bool, logit_tolerance, make_inputs, nth_largest_f32,
                         run_atopn, run_fused, to_np_bits)

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-2
NEAR_TAU = 1e-3

SHAPES = {
    # name: (B, hq, hk, hv, d_k, d_v, L, T, N, n)
    "sigma_like_dk32_dv64": (2, 16, 2, 8, 32, 64, 3000, 4, 100, 2),
    "dk64_dv128": (2, 12, 1, 2, 64, 128, 2000, 3, 64, 2),
    "dk128_dv32": (1, 8, 2, 4, 128, 32, 1500, 3, 50, 2),
    "dk32_dv32": (1, 4, 1, 2, 32, 32, 900, 3, 20, 3),
    "dk32_dv128": (2, 8, 2, 4, 32, 128, 1200, 3, 40, 2),
    # Long single sequences: enough workgroups for the small-batch path (the
    # value gather inside the K-stream kernel); the shapes above take the list path.
    "dk64_dv128_long": (1, 12, 1, 2, 64, 128, 40000, 3, 500, 2),
    "sigma_like_dk32_dv64_long": (1, 16, 2, 8, 32, 64, 30000, 3, 300, 2),
}

_cache = {}


def inputs(name, seed_base=300):
    B, hq, hk, hv, dk, dv, L, T, N, n = SHAPES[name]
    q, K, V = make_inputs(B, hq, hk, hv, dk, L + T, T, seed=seed_base + len(name), dv=dv)
    assert K.shape[-1] == dk and V.shape[-1] == dv
    return q, K, V, [L + t for t in range(T)], N, n


def case(name):
    if name not in _cache:
        q, K, V, ctx, N, n = inputs(name)
        print(f"[dkdv {name}] q{tuple(q.shape)} K{tuple(K.shape)} V{tuple(V.shape)}", flush=True)
        gpu = run_atopn(q, K, V, ctx, N, n)
        qb, Kb, Vb = to_np_bits(q), to_np_bits(K), to_np_bits(V)
        ref = oracle.atopn_run(qb, Kb, Vb, ctx, N, n, want_sel=True, want_logits=True)
        _cache[name] = dict(q=qb, K=Kb, V=Vb, ctx=ctx, N=N, n=n, gpu=gpu, ref=ref)
    return _cache[name]


@pytest.mark.parametrize("name", list(SHAPES))
def test_logits_thresholds_and_selection(name):
    c = case(name)
    for t, ctx in enumerate(c["ctx"]):
        lg, tau = c["gpu"]["logits"][t], c["gpu"]["tau"][t]
        err = np.abs(lg.astype(np.float64) - c["ref"]["logits"][t][..., :ctx])
        tol = logit_tolerance(c["q"][t], c["K"], ctx)
        assert (err <= tol).all(), f"step {t}: logits off by {(err - tol).max():.3e} beyond the bar"
        if t % c["n"] == 0:
            for b in range(lg.shape[0]):
                for i in range(lg.shape[1]):
                    assert tau[b, i] == nth_largest_f32(lg[b, i], c["N"]), (t, b, i)
        sel = bitmap_to_bool(c["gpu"]["bitmap"][t], ctx)
        assert (sel == (lg >= tau[..., None])).all(), f"step {t}: not an exact filter"
        ref = c["ref"]["sel"][t][..., :ctx].astype(bool)
        near = np.abs(c["ref"]["logits"][t][..., :ctx] - c["ref"]["tau"][t][..., None]) <= NEAR_TAU
        assert not ((sel != ref) & ~near).any(), f"step {t}: selection differs off threshold"


@pytest.mark.parametrize("name", list(SHAPES))
def test_outputs_match_oracle_on_gpu_mask(name):
    c = case(name)
    for t, ctx in enumerate(c["ctx"]):
        ref, cnt = oracle.masked(c["q"][t], c["K"], c["V"], ctx, c["gpu"]["bitmap"][t])
        assert ref.shape[-1] == c["V"].shape[-1]
        assert (cnt == c["gpu"]["counts"][t]).all()
        err = np.abs(c["gpu"]["out"][t] - ref).max()
        assert err <= OUT_TOL, f"step {t}: max abs err {err:.3e}"


@pytest.mark.parametrize("name", list(SHAPES))
def test_fused_refresh_step_matches_separate_calls(name):
    q, K, V, ctx, N, n = inputs(name, seed_base=310)
    sep = run_atopn(q, K, V, ctx, N, n, logits_every_step=False)
    fus = run_fused(q, K, V, ctx, N, n)
    qb, Kb, Vb = to_np_bits(q), to_np_bits(K), to_np_bits(V)
    for t, c in enumerate(ctx):
        assert np.array_equal(fus["tau"][t].view(np.uint32), sep["tau"][t].view(np.uint32)), t
        assert np.array_equal(fus["counts"][t], sep["counts"][t]), t
        ref, _ = oracle.masked(qb[t], Kb, Vb, c, sep["bitmap"][t])
        assert np.abs(fus["out"][t] - ref).max() <= OUT_TOL, t


@pytest.mark.parametrize("name", list(SHAPES))
def test_full_attention_matches_oracle(name):
    B, hq, hk, hv, dk, dv, L, T, N, n = SHAPES[name]
    q, K, V, ctx, _, _ = inputs(name, seed_base=320)
    rows = K.shape[2]
    dm = saga.dims(B, hq, hk, hv, dk, ctx[-1], rows, head_dim_v=dv)
    ws = saga.alloc_workspace(dm, 1)
    out = torch.empty(B, hq, dv, dtype=torch.bfloat16, device="cuda")
    saga.saga_full_attention(dm, q[-1], K, V, out, ws)
    torch.cuda.synchronize()
    ref = oracle.full(to_np_bits(q)[-1], to_np_bits(K), to_np_bits(V), ctx[-1])
    err = np.abs(out.float().cpu().numpy() - ref).max()
    assert err <= OUT_TOL, f"{name}: {err:.3e}"


def test_paged_sigma_like_equals_contiguous():
    """Pools of d_k-wide K pages and d_v-wide V pages, shuffled: thresholds,
    counts and outputs bit-identical to the contiguous calls."""
    B, hq, hk, hv, dk, dv, P, maxp, N, n = 2, 16, 2, 8, 32, 64, 256, 6, 80, 2
    rows, T = maxp * P, 3
    q, K, V = make_inputs(B, hq, hk, hv, dk, rows, T, seed=330, dv=dv)
    ctx = [rows - 200 + 7 * t for t in range(T)]
    ref = run_fused(q, K, V, ctx, N, n)
    npages = B * maxp + 2
    perm = torch.from_numpy(np.random.default_rng(5).permutation(npages)[: B * maxp].astype(np.int32))
    table = perm.view(B, maxp).cuda()
    kp = torch.zeros(npages, hk, P, dk, dtype=K.dtype, device="cuda")
    vp = torch.zeros(npages, hv, P, dv, dtype=V.dtype, device="cuda")
    for b in range(B):
        for p in range(maxp):
            kp[table[b, p]] = K[b, :, p * P:(p + 1) * P]
            vp[table[b, p]] = V[b, :, p * P:(p + 1) * P]
    lens = torch.empty(B, dtype=torch.int32, device="cuda")
    pg = saga.paged(table, lens, P, npages)
    ws = saga.alloc_workspace(saga.dims(B, hq, hk, hv, dk, ctx[0], rows, head_dim_v=dv), N)
    tau = torch.empty(B, hq, device="cuda")
    for t, c in enumerate(ctx):
        lens.fill_(c)
        dm = saga.dims(B, hq, hk, hv, dk, c, rows, head_dim_v=dv)
        out = torch.empty(B, hq, dv, dtype=torch.bfloat16, device="cuda")
        cnt = torch.empty(B, hq, dtype=torch.int32, device="cuda")
        if t % n == 0:
            saga.atopn_refresh_decode_step_paged(dm, pg, N, q[t], kp, vp, tau, out, ws,
                                                 sel_counts=cnt)
        else:
            saga.saga_decode_step_paged(dm, pg, q[t], kp, vp, tau, out, ws, sel_counts=cnt)
        torch.cuda.synchronize()
        assert np.array_equal(tau.cpu().numpy().view(np.uint32), ref["tau"][t].view(np.uint32)), t
        assert np.array_equal(cnt.cpu().numpy(), ref["counts"][t]), t
        assert np.array_equal(out.float().cpu().numpy(), ref["out"][t]), t
