"""Edge cases of the threshold select and of the gather's entry staging.

Each input is built so that a given path runs, and the test checks on the host
(from the GPU's own debug logits and the sampling rule) that it does:
- a candidate set of more than 6144 entries per row, which fills nearly every
  register slot of the final select but stays under the 8192-entry staging cap;
- a candidate set above that cap, which the select reads from the lists in
  place (three radix passes over the entries) instead of recomputing logits;
- a candidate set in which every logit is equal (the select's zero-range case);
- selected rows in two far-apart bands, so the gather's walk over the list
  offsets crosses long runs of empty lists.
Bars as in the main parity tests: thresholds bit-equal to the N-th largest GPU
logit, counts equal to the number of logits >= tau, outputs within 1e-2 of the
fp64 oracle on the GPU's mask.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (make_inputs, nth_largest_f32, run_atopn, run_fused, sampled_rows,
                         to_np_bits)

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-2
STAGE = 8192          # candidates the final select stages per row


def candidates(logits_row: np.ndarray, N: int, ctx: int) -> int:
    """Entries at or above the sample pivot: the k-th largest sampled logit with
    k = ceil(mu + 5 sqrt(mu) + 5), mu = N * m / ctx (m sampled rows)."""
    rows = sampled_rows(ctx)
    m = rows.size
    mu = N * m / ctx
    k = min(int(math.ceil(mu + 5.0 * math.sqrt(mu) + 5.0)), m)
    sample = np.sort(logits_row[rows])[::-1]
    return int((logits_row >= sample[k - 1]).sum())


def check_exact(q, K, V, ctx, N):
    gpu = run_atopn(q, K, V, [ctx], N, 1)
    lg, tau, cnt = gpu["logits"][0], gpu["tau"][0], gpu["counts"][0]
    for b in range(lg.shape[0]):
        for i in range(lg.shape[1]):
            assert tau[b, i] == nth_largest_f32(lg[b, i], N), (b, i)
            assert cnt[b, i] == (lg[b, i] >= tau[b, i]).sum(), (b, i)
    ref, _ = oracle.masked(to_np_bits(q)[0], to_np_bits(K), to_np_bits(V), ctx, gpu["bitmap"][0])
    err = np.abs(gpu["out"][0] - ref).max()
    assert err <= OUT_TOL, f"max abs err {err:.3e}"
    return gpu


def test_select_with_candidates_near_the_staging_cap():
    ctx, N = 40000, 5500
    q, K, V = make_inputs(2, 8, 2, 4, 64, ctx, 1, seed=71, heavy=False)
    print(f"[refresh paths] near cap: q{tuple(q.shape)} ctx={ctx} N={N}", flush=True)
    gpu = check_exact(q, K, V, ctx, N)
    lg = gpu["logits"][0]
    counts = [candidates(lg[b, i], N, ctx) for b in range(lg.shape[0]) for i in range(lg.shape[1])]
    assert any(6144 < c <= STAGE for c in counts), counts


def test_select_with_candidates_above_the_staging_cap():
    ctx, N = 40000, 7000
    q, K, V = make_inputs(2, 8, 2, 4, 64, ctx, 1, seed=73, heavy=False)
    print(f"[refresh paths] above cap: q{tuple(q.shape)} ctx={ctx} N={N}", flush=True)
    gpu = check_exact(q, K, V, ctx, N)
    lg = gpu["logits"][0]
    counts = [candidates(lg[b, i], N, ctx) for b in range(lg.shape[0]) for i in range(lg.shape[1])]
    assert any(c > STAGE for c in counts), counts
    # The one-call refresh step on the same inputs: the same thresholds, and its
    # gather reads the long candidate lists filtered by tau.
    fz = run_fused(q, K, V, [ctx], N, 1)
    assert np.array_equal(fz["tau"][0].view(np.uint32), gpu["tau"][0].view(np.uint32))
    assert np.array_equal(fz["counts"][0], gpu["counts"][0])
    ref, _ = oracle.masked(to_np_bits(q)[0], to_np_bits(K), to_np_bits(V), ctx, gpu["bitmap"][0])
    assert np.abs(fz["out"][0] - ref).max() <= OUT_TOL


def test_select_when_every_candidate_ties():
    ctx, N = 40000, 1000
    q, K, V = make_inputs(1, 4, 1, 2, 64, ctx, 1, seed=72, heavy=False)
    print(f"[refresh paths] ties: q{tuple(q.shape)} ctx={ctx} N={N}", flush=True)
    K.mul_(0.05)
    tied = torch.arange(0, ctx, 8, device=K.device)       # 5000 identical rows
    K[:, :, tied, :] = 1.0
    q.fill_(0.1)
    gpu = check_exact(q, K, V, ctx, N)
    lg, tau, cnt = gpu["logits"][0], gpu["tau"][0], gpu["counts"][0]
    top = lg[0, 0, 0]
    assert (lg[:, :, tied.cpu().numpy()] == top).all()
    assert (tau == top).all() and (cnt == tied.numel()).all()
    for i in range(lg.shape[1]):
        assert candidates(lg[0, i], N, ctx) == tied.numel()   # all tied, under the cap


@pytest.mark.parametrize("fused", [False, True])
def test_gather_walks_over_empty_lists(fused):
    ctx, N, n = 30000, 300, 2
    q, K, V = make_inputs(1, 8, 2, 4, 64, ctx + 2, 2, seed=73, heavy=False)
    print(f"[refresh paths] empty lists (fused={fused}): q{tuple(q.shape)} ctx={ctx}", flush=True)
    band = torch.zeros(ctx + 2, dtype=torch.bool, device=K.device)
    band[:400] = True
    band[21000:21400] = True
    K[:, :, ~band, :] *= 0.01
    steps = [ctx, ctx + 1]
    if fused:
        res = run_fused(q, K, V, steps, N, n)
        sep = run_atopn(q, K, V, steps, N, n, logits_every_step=False)
        for t in range(2):
            assert np.array_equal(res["counts"][t], sep["counts"][t]), t
        masks = sep["bitmap"]
    else:
        res = run_atopn(q, K, V, steps, N, n)
        masks = res["bitmap"]
        lg = res["logits"][0]
        sel = lg >= res["tau"][0][..., None]
        outside = ~band[:ctx].cpu().numpy()
        assert not sel[..., outside].any()                  # both bands only
        assert sel[..., :400].any() and sel[..., 21000:21400].any()
    qb, Kb, Vb = to_np_bits(q), to_np_bits(K), to_np_bits(V)
    for t, c in enumerate(steps):
        ref, cnt = oracle.masked(qb[t], Kb, Vb, c, masks[t])
        assert (cnt == res["counts"][t]).all(), t
        err = np.abs(res["out"][t] - ref).max()
        assert err <= OUT_TOL, f"step {t}: max abs err {err:.3e}"
