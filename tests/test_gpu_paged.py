"""Paged caches with per-sequence lengths (the *_paged calls) on the GPU.

* Same caches, paged: the contiguous caches scattered over page pools in a
  shuffled order give bit-identical thresholds, counts and outputs to the
  contiguous calls (the work split is the same), also with garbage in the
  unused page-table slots.
* Per-sequence lengths: every sequence matches the contiguous path run on that
  sequence alone at its own length (thresholds bit-equal, counts equal,
  outputs within the output bar of the fp64 oracle on that mask), including a
  sequence with N >= its length (tau = -inf, full attention).
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


def to_pages(K, V, P, seed, extra=3):
    """Scatter [B][h][rows][d] caches over pools of pages of P rows, in a
    shuffled page order with `extra` unused pages; returns the pools and the
    block table [B][rows/P]."""
    B, hk, rows, d = K.shape
    hv = V.shape[1]
    maxp = rows // P
    n = B * maxp + extra
    perm = torch.from_numpy(np.random.default_rng(seed).permutation(n)[: B * maxp].astype(np.int32))
    table = perm.view(B, maxp).cuda()
    kp = torch.zeros(n, hk, P, d, dtype=K.dtype, device="cuda")
    vp = torch.zeros(n, hv, P, d, dtype=V.dtype, device="cuda")
    for b in range(B):
        for p in range(maxp):
            kp[table[b, p]] = K[b, :, p * P:(p + 1) * P]
            vp[table[b, p]] = V[b, :, p * P:(p + 1) * P]
    return kp, vp, table, n


def run_contiguous(q, K, V, ctx_steps, N, n):
    """Refresh at t % n == 0 (one call), decode otherwise; per-step results."""
    T, B, hq, d = q.shape
    hk, rows, hv = K.shape[1], K.shape[2], V.shape[1]
    g = Guards()
    ws = g.workspace(saga.dims(B, hq, hk, hv, d, ctx_steps[0], rows), N)
    tau = g.empty((B, hq), torch.float32, "tau")
    res = []
    for t, ctx in enumerate(ctx_steps):
        dm = saga.dims(B, hq, hk, hv, d, ctx, rows)
        out = g.empty((B, hq, d), torch.bfloat16, "out")
        cnt = g.empty((B, hq), torch.int32, "sel_counts")
        if t % n == 0:
            saga.atopn_refresh_decode_step(dm, N, q[t], K, V, tau, out, ws, sel_counts=cnt)
        else:
            saga.saga_decode_step(dm, q[t], K, V, tau, out, ws, sel_counts=cnt)
        torch.cuda.synchronize()
        g.check(f"at step {t}")
        g.bufs = g.bufs[:2]
        res.append((tau.clone(), cnt.clone(), out.clone()))
    return res


def run_paged(q, kp, vp, table, npages, P, rows, ctx_lens_steps, N, n, fused=True):
    T, B, hq, d = q.shape
    hk, hv = kp.shape[1], vp.shape[1]
    g = Guards()
    ctx_lens = torch.empty(B, dtype=torch.int32, device="cuda")
    pg = saga.paged(table, ctx_lens, P, npages)
    ws = g.workspace(saga.dims(B, hq, hk, hv, d, max(ctx_lens_steps[0]), rows), N)
    tau = g.empty((B, hq), torch.float32, "tau")
    res = []
    for t, lens in enumerate(ctx_lens_steps):
        ctx_lens.copy_(torch.tensor(lens, dtype=torch.int32))
        dm = saga.dims(B, hq, hk, hv, d, max(lens), rows)
        out = g.empty((B, hq, d), torch.bfloat16, "out")
        cnt = g.empty((B, hq), torch.int32, "sel_counts")
        if t % n == 0 and fused:
            saga.atopn_refresh_decode_step_paged(dm, pg, N, q[t], kp, vp, tau, out, ws,
                                                 sel_counts=cnt)
        else:
            if t % n == 0:
                saga.atopn_refresh_thresholds_paged(dm, pg, N, q[t], kp, tau, ws)
            saga.saga_decode_step_paged(dm, pg, q[t], kp, vp, tau, out, ws, sel_counts=cnt)
        torch.cuda.synchronize()
        g.check(f"at step {t}")
        g.bufs = g.bufs[:2]
        res.append((tau.clone(), cnt.clone(), out.clone()))
    return res


def bits(t):
    return t.cpu().contiguous().view(torch.int32).numpy() if t.dtype == torch.float32 \
        else t.cpu().contiguous().view(torch.int16).numpy()


PAGED_SHAPES = {
    # name: (B, hq, hk, hv, d, P, pages per sequence, N, n)
    "qwen_like_d128": (2, 12, 1, 2, 128, 256, 14, 128, 2),
    "llama_like_d64": (2, 32, 4, 8, 64, 512, 8, 256, 2),
    "group16_big_pages": (1, 16, 1, 4, 64, 1024, 5, 100, 3),
    # long enough for the small-batch path (at least 64 fused workgroups)
    "qwen_like_small_batch_path": (1, 12, 1, 2, 128, 256, 160, 512, 2),
    "group16_small_batch_path": (2, 16, 1, 4, 64, 1024, 40, 200, 3),
}


@pytest.mark.parametrize("name", list(PAGED_SHAPES))
def test_paged_equals_contiguous_bit_for_bit(name):
    B, hq, hk, hv, d, P, maxp, N, n = PAGED_SHAPES[name]
    rows, T = maxp * P, 4
    q, K, V = make_inputs(B, hq, hk, hv, d, rows, T, seed=80 + len(name))
    ctx = [rows - 3 * P // 2 + 37 * t for t in range(T)]          # ragged, inside the table
    print(f"[paged {name}] B={B} rows={rows} P={P} ctx={ctx}", flush=True)
    ref = run_contiguous(q, K, V, ctx, N, n)
    kp, vp, table, npages = to_pages(K, V, P, seed=1)
    got = run_paged(q, kp, vp, table, npages, P, rows, [[c] * B for c in ctx], N, n)
    for t in range(T):
        for a, b in zip(ref[t], got[t]):
            assert np.array_equal(bits(a), bits(b)), f"step {t}"


def test_paged_ignores_unused_table_slots():
    B, hq, hk, hv, d, P, maxp, N, n = PAGED_SHAPES["qwen_like_d128"]
    rows, T = maxp * P, 2
    q, K, V = make_inputs(B, hq, hk, hv, d, rows, T, seed=90)
    ctx = [6 * P + 11, 6 * P + 12]                                  # 7 of 14 pages in use
    kp, vp, table, npages = to_pages(K, V, P, seed=2)
    clean = run_paged(q, kp, vp, table, npages, P, rows, [[c] * B for c in ctx], N, n)
    junk = table.clone()
    junk[:, 8:] = torch.tensor([-1, 1 << 30, -(1 << 30), npages, 5, 0], dtype=torch.int32,
                               device="cuda").repeat(B)[: B * (maxp - 8)].view(B, maxp - 8)
    dirty = run_paged(q, kp, vp, junk, npages, P, rows, [[c] * B for c in ctx], N, n)
    for t in range(T):
        for a, b in zip(clean[t], dirty[t]):
            assert np.array_equal(bits(a), bits(b))


@pytest.mark.parametrize("fused", [True, False])
def test_per_sequence_lengths_match_each_sequence_alone(fused):
    B, hq, hk, hv, d, P = 3, 12, 1, 2, 128, 256
    maxp, N, n, T = 12, 200, 2, 3
    rows = maxp * P
    q, K, V = make_inputs(B, hq, hk, hv, d, rows, T, seed=91)
    lens = [[2900 + t, 700 + 5 * t, 150 + t] for t in range(T)]   # the last: N >= ctx
    kp, vp, table, npages = to_pages(K, V, P, seed=3)
    got = run_paged(q, kp, vp, table, npages, P, rows, lens, N, n, fused=fused)
    for b in range(B):
        ctx_b = [lens[t][b] for t in range(T)]
        print(f"[paged varlen b={b}] ctx={ctx_b}", flush=True)
        qb = q[:, b:b + 1].contiguous()
        Kb, Vb = K[b:b + 1].contiguous(), V[b:b + 1].contiguous()
        ref = run_contiguous(qb, Kb, Vb, ctx_b, N, n)
        # The oracle on this sequence alone at its own lengths.
        orc = oracle.atopn_run(to_np_bits(qb), to_np_bits(Kb), to_np_bits(Vb), ctx_b, N, n,
                               want_sel=True, want_logits=True)
        for t in range(T):
            tau_r, cnt_r, _ = ref[t]
            tau_g, cnt_g, out_g = got[t]
            assert np.array_equal(bits(tau_r[0]), bits(tau_g[b])), (b, t)
            assert np.array_equal(cnt_r[0].cpu().numpy(), cnt_g[b].cpu().numpy()), (b, t)
            if N >= ctx_b[t]:
                assert torch.isneginf(tau_g[b]).all() and (cnt_g[b] == ctx_b[t]).all()
            # outputs against the fp64 oracle on the selection of this step
            dm = saga.dims(1, hq, hk, hv, d, ctx_b[t], rows)
            ws = saga.alloc_workspace(dm, 1)
            bm = torch.empty(1, hq, (rows + 31) // 32, dtype=torch.int32, device="cuda")
            o1 = torch.empty(1, hq, d, dtype=torch.bfloat16, device="cuda")
            saga.saga_decode_step(dm, qb[t], Kb, Vb, tau_g[b:b + 1].contiguous(), o1, ws,
                                  sel_bitmap_debug=bm)
            torch.cuda.synchronize()
            bm_np = bm.cpu().numpy().view(np.uint32)
            ref_o, cnt_o = oracle.masked(to_np_bits(qb[t]), to_np_bits(Kb), to_np_bits(Vb),
                                         ctx_b[t], bm_np)
            assert (cnt_o[0] == cnt_g[b].cpu().numpy()).all()
            # Thresholds and selection against the oracle's Atop-N run.
            tau_o = orc["tau"][t, 0]
            tg = tau_g[b].cpu().numpy().astype(np.float64)
            both_inf = np.isneginf(tg) & np.isneginf(tau_o)
            diff = np.subtract(tg, tau_o, out=np.zeros_like(tg), where=~both_inf)
            assert (both_inf | (np.abs(diff) <= 1e-4)).all()
            sel = bitmap_to_bool(bm_np[0], ctx_b[t])
            s = orc["logits"][t, 0, :, :ctx_b[t]]
            near = np.abs(s - tau_o[:, None]) <= NEAR_TAU
            bad = (sel != orc["sel"][t, 0, :, :ctx_b[t]].astype(bool)) & ~near
            assert not bad.any(), f"b={b} t={t}: {bad.sum()} entries differ from the oracle"
            err = np.abs(out_g[b].float().cpu().numpy() - ref_o[0]).max()
            assert err <= OUT_TOL, f"b={b} t={t}: {err:.3e}"


# Larger batches of mixed lengths (many K-stream workgroups per call): (B, hq,
# hk, hv, d, P, pages per sequence, N, n, T, sequences checked).
LARGE_PAGED = {
    "llama_like_d64": (8, 32, 4, 8, 64, 256, 12, 100, 2, 3, None),
    "qwen_like_d128": (64, 12, 1, 2, 128, 256, 66, 300, 2, 2, [0, 1, 17, 40, 63]),
}


@pytest.mark.parametrize("name", list(LARGE_PAGED))
def test_large_batch_paged_per_sequence_lengths(name):
    """Paged calls with mixed lengths at larger batches: per sequence,
    thresholds and counts bit-equal to that sequence's own contiguous calls,
    and outputs within the bar of the oracle on that step's selection (the
    single-sequence calls take another path, so the summation order differs)."""
    B, hq, hk, hv, d, P, maxp, N, n, T, check = LARGE_PAGED[name]
    rows = maxp * P
    q, K, V = make_inputs(B, hq, hk, hv, d, rows, T, seed=95 + len(name))
    rng = np.random.default_rng(7)
    base = rng.integers(rows // 8, rows - T, size=B)
    base[0], base[-1] = rows - T, 40                             # the longest; N >= ctx
    lens = [[int(x) + t for x in base] for t in range(T)]
    kp, vp, table, npages = to_pages(K, V, P, seed=4)
    got = run_paged(q, kp, vp, table, npages, P, rows, lens, N, n)
    for b in (check if check is not None else range(B)):
        ctx_b = [lens[t][b] for t in range(T)]
        qb = q[:, b:b + 1].contiguous()
        Kb, Vb = K[b:b + 1].contiguous(), V[b:b + 1].contiguous()
        ref = run_contiguous(qb, Kb, Vb, ctx_b, N, n)
        print(f"[paged large {name} b={b}] ctx={ctx_b}", flush=True)
        for t in range(T):
            tau_r, cnt_r, _ = ref[t]
            tau_g, cnt_g, out_g = got[t]
            assert np.array_equal(bits(tau_r[0]), bits(tau_g[b])), (b, t)
            assert np.array_equal(cnt_r[0].cpu().numpy(), cnt_g[b].cpu().numpy()), (b, t)
            dm = saga.dims(1, hq, hk, hv, d, ctx_b[t], rows)
            ws = saga.alloc_workspace(dm, 1)
            bm = torch.empty(1, hq, (rows + 31) // 32, dtype=torch.int32, device="cuda")
            o1 = torch.empty(1, hq, d, dtype=torch.bfloat16, device="cuda")
            saga.saga_decode_step(dm, qb[t], Kb, Vb, tau_g[b:b + 1].contiguous(), o1, ws,
                                  sel_bitmap_debug=bm)
            torch.cuda.synchronize()
            ref_o, cnt_o = oracle.masked(to_np_bits(qb[t]), to_np_bits(Kb), to_np_bits(Vb),
                                         ctx_b[t], bm.cpu().numpy().view(np.uint32))
            assert (cnt_o[0] == cnt_g[b].cpu().numpy()).all(), (b, t)
            err = np.abs(out_g[b].float().cpu().numpy() - ref_o[0]).max()
            assert err <= OUT_TOL, f"b={b} t={t}: {err:.3e}"


@pytest.mark.parametrize("B", [80, 264])
def test_many_sequences_work_split(B):
    """More sequences than one wave (80) and than one workgroup (264) holds:
    the K stream's work split from the lengths then takes its workgroup-wide
    forms (a candidate search over lengths held in LDS; with more than 256
    sequences, several passes and a bisection).  Lengths are mixed, a few are
    0 and a few below N.  Every sequence's thresholds and counts must equal
    that sequence run alone on contiguous caches (bit for bit), empty
    sequences select nothing and output zeros, and sampled sequences' outputs
    are checked against the fp64 oracle on the GPU's selection."""
    hq, hk, hv, d, P = 4, 1, 2, 64, 256
    maxp, N, n, T = 6, 64, 2, 2
    rows = maxp * P
    q, K, V = make_inputs(B, hq, hk, hv, d, rows, T, seed=93 + B)
    rng = np.random.default_rng(B)
    base = rng.integers(1, rows - T, size=B)
    base[:3] = 0                                   # empty sequences
    base[3:6] = [5, 30, 63]                        # N >= ctx
    lens = [[int(x) + t if x else 0 for x in base] for t in range(T)]
    print(f"[paged many sequences] B={B}", flush=True)
    kp, vp, table, npages = to_pages(K, V, P, seed=4)
    got = run_paged(q, kp, vp, table, npages, P, rows, lens, N, n)
    for b in range(B):
        ctx_b = [lens[t][b] for t in range(T)]
        if ctx_b[0] == 0:
            for t in range(T):
                tau_g, cnt_g, out_g = got[t]
                assert torch.isneginf(tau_g[b]).all() and (cnt_g[b] == 0).all()
                assert (out_g[b].float() == 0).all()
            continue
        qb = q[:, b:b + 1].contiguous()
        Kb, Vb = K[b:b + 1].contiguous(), V[b:b + 1].contiguous()
        ref = run_contiguous(qb, Kb, Vb, ctx_b, N, n)
        for t in range(T):
            tau_r, cnt_r, out_r = ref[t]
            tau_g, cnt_g, out_g = got[t]
            assert np.array_equal(bits(tau_r[0]), bits(tau_g[b])), (b, t)
            assert np.array_equal(cnt_r[0].cpu().numpy(), cnt_g[b].cpu().numpy()), (b, t)
        if b % 37 == 3:                            # sampled: outputs against the oracle
            t = T - 1
            dm = saga.dims(1, hq, hk, hv, d, ctx_b[t], rows)
            ws = saga.alloc_workspace(dm, 1)
            bm = torch.empty(1, hq, (rows + 31) // 32, dtype=torch.int32, device="cuda")
            o1 = torch.empty(1, hq, d, dtype=torch.bfloat16, device="cuda")
            saga.saga_decode_step(dm, qb[t], Kb, Vb, got[t][0][b:b + 1].contiguous(), o1, ws,
                                  sel_bitmap_debug=bm)
            torch.cuda.synchronize()
            ref_o, _ = oracle.masked(to_np_bits(qb[t]), to_np_bits(Kb), to_np_bits(Vb),
                                     ctx_b[t], bm.cpu().numpy().view(np.uint32))
            err = np.abs(got[t][2][b].float().cpu().numpy() - ref_o[0]).max()
            assert err <= OUT_TOL, f"b={b}: {err:.3e}"


def test_paged_pool_beyond_4gib():
    """A V pool over 4 GiB takes the 64-bit address path of the gather; the
    data pages sit at the top of the pools."""
    B, hq, hk, hv, d, P, maxp, N, n = 2, 12, 1, 2, 128, 256, 6, 128, 2
    rows, T = maxp * P, 2
    q, K, V = make_inputs(B, hq, hk, hv, d, rows, T, seed=92)
    ctx = [rows - 100, rows - 99]
    ref = run_contiguous(q, K, V, ctx, N, n)
    page_bytes_v = hv * P * d * 2
    npages = (1 << 32) // page_bytes_v + 64                        # V pool > 4 GiB
    print(f"[paged >4GiB] V pool {npages * page_bytes_v / 2**30:.2f} GiB", flush=True)
    top = torch.arange(npages - B * maxp, npages, dtype=torch.int32)
    perm = top[torch.from_numpy(np.random.default_rng(4).permutation(B * maxp))]
    table = perm.view(B, maxp).cuda()
    kp = torch.zeros(npages, hk, P, d, dtype=K.dtype, device="cuda")
    vp = torch.zeros(npages, hv, P, d, dtype=V.dtype, device="cuda")
    for b in range(B):
        for p in range(maxp):
            kp[table[b, p]] = K[b, :, p * P:(p + 1) * P]
            vp[table[b, p]] = V[b, :, p * P:(p + 1) * P]
    got = run_paged(q, kp, vp, table, npages, P, rows, [[c] * B for c in ctx], N, n)
    del kp, vp
    torch.cuda.empty_cache()
    for t in range(T):
        for a, b in zip(ref[t], got[t]):
            assert np.array_equal(bits(a), bits(b)), f"step {t}"
