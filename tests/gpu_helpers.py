"""Helpers for the GPU parity tests: drive the C-ABI library over decode steps
with its debug outputs switched on, and bring the results to the host."""
from __future__ import annotations

import numpy as np
import torch

import sparse_decode_attention_atop_amd as saga
import saga_workload as wl


def to_np_bits(t: torch.Tensor) -> np.ndarray:
    return wl.bits(t)


def bf16_to_f32(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def make_inputs(B, hq, hk, hv, d, rows, T, seed, device="cuda", q_scale=None, heavy=True, dv=0):
    """Seeded inputs via the workload generator (random shape, not a named config);
    dv: value head dimension (0: same as d)."""
    w = wl.Workload("adhoc", 900 + seed, B, hq, hk, hv, d, rows - T, 1, 1, T, 1, head_dim_v=dv)
    x = wl.make_layer(w, 0, device=device, heavy_hitters=heavy)
    return x["q"], x["K"], x["V"]


def run_atopn(q, K, V, ctx_steps, top_n, refresh_n, scale=1.0, logits_every_step=True):
    """Run Atop-N on the GPU over len(ctx_steps) steps with every debug output.

    Returns per-step lists: tau (float32 [B][hq], the threshold in force),
    logits (float32 [B][hq][ctx] or None), counts (int32 [B][hq]),
    bitmap (uint32 [B][hq][words]), out (float32 of the bf16 output).
    """
    T, B, hq, d = q.shape
    hk, rows = K.shape[1], K.shape[2]
    hv, dv = V.shape[1], V.shape[3]
    dvx = 0 if dv == d else dv
    dev = q.device
    dims0 = saga.dims(B, hq, hk, hv, d, ctx_steps[0], rows, scale, head_dim_v=dvx)
    ws = saga.alloc_workspace(dims0, top_n, dev)
    tau = torch.empty(B, hq, dtype=torch.float32, device=dev)
    tau_scratch = torch.empty_like(tau)
    words = (rows + 31) // 32
    res = {"tau": [], "logits": [], "counts": [], "bitmap": [], "out": []}
    for t, ctx in enumerate(ctx_steps):
        dm = saga.dims(B, hq, hk, hv, d, ctx, rows, scale, head_dim_v=dvx)
        lg = torch.empty(B, hq, ctx, dtype=torch.float32, device=dev)
        if t % refresh_n == 0:
            saga.atopn_refresh_thresholds(dm, top_n, q[t], K, tau, ws, logits_debug=lg)
        elif logits_every_step:
            # Logits of a plain step, for checking; the kept thresholds are untouched.
            saga.atopn_refresh_thresholds(dm, top_n, q[t], K, tau_scratch, ws, logits_debug=lg)
        out = torch.empty(B, hq, dv, dtype=torch.bfloat16, device=dev)
        cnt = torch.empty(B, hq, dtype=torch.int32, device=dev)
        bm = torch.empty(B, hq, words, dtype=torch.int32, device=dev)
        saga.saga_decode_step(dm, q[t], K, V, tau, out, ws, sel_counts=cnt, sel_bitmap_debug=bm)
        torch.cuda.synchronize()
        res["tau"].append(tau.cpu().numpy().copy())
        res["logits"].append(lg.cpu().numpy() if (t % refresh_n == 0 or logits_every_step) else None)
        res["counts"].append(cnt.cpu().numpy())
        res["bitmap"].append(bm.cpu().numpy().view(np.uint32))
        res["out"].append(bf16_to_f32(out))
    return res


def run_fused(q, K, V, ctx_steps, top_n, refresh_n, scale=1.0):
    """Atop-N over len(ctx_steps) steps with the one-call refresh step
    (atopn_refresh_decode_step) at t mod n == 0 and saga_decode_step between.

    Returns per-step lists: tau (float32 [B][hq]), counts, out (float32).
    """
    T, B, hq, d = q.shape
    hk, rows = K.shape[1], K.shape[2]
    hv, dv = V.shape[1], V.shape[3]
    dvx = 0 if dv == d else dv
    dev = q.device
    ws = saga.alloc_workspace(saga.dims(B, hq, hk, hv, d, ctx_steps[0], rows, scale, head_dim_v=dvx),
                              top_n, dev)
    tau = torch.empty(B, hq, dtype=torch.float32, device=dev)
    res = {"tau": [], "counts": [], "out": []}
    for t, ctx in enumerate(ctx_steps):
        dm = saga.dims(B, hq, hk, hv, d, ctx, rows, scale, head_dim_v=dvx)
        out = torch.empty(B, hq, dv, dtype=torch.bfloat16, device=dev)
        cnt = torch.empty(B, hq, dtype=torch.int32, device=dev)
        if t % refresh_n == 0:
            saga.atopn_refresh_decode_step(dm, top_n, q[t], K, V, tau, out, ws, sel_counts=cnt)
        else:
            saga.saga_decode_step(dm, q[t], K, V, tau, out, ws, sel_counts=cnt)
        torch.cuda.synchronize()
        res["tau"].append(tau.cpu().numpy().copy())
        res["counts"].append(cnt.cpu().numpy())
        res["out"].append(bf16_to_f32(out))
    return res


def sampled_rows(ctx: int) -> np.ndarray:
    """Rows the threshold refresh reads to place its pivot: 16-row blocks, one
    every `stride` rows (a multiple of 16), at most 128 blocks."""
    if ctx <= 2048:
        return np.arange(ctx)
    stride = -(-(ctx // 16) // 128) * 16
    starts = np.arange(ctx // stride) * stride
    return (starts[:, None] + np.arange(16)[None, :]).ravel()


def bitmap_to_bool(bm: np.ndarray, ctx: int) -> np.ndarray:
    """[..., words] uint32 -> [..., ctx] bool."""
    bits = np.unpackbits(bm.view(np.uint8), axis=-1, bitorder="little")
    return bits[..., :ctx].astype(bool)


def nth_largest_f32(row: np.ndarray, N: int) -> np.float32:
    """Host N-th largest of float32 values (sort), -inf when N >= len."""
    if N >= row.size:
        return np.float32(-np.inf)
    return np.sort(row.astype(np.float32))[::-1][N - 1]


def logit_tolerance(q_bits, K_bits, ctx, scale=1.0):
    """|s_gpu - s_exact| bound: fp32 accumulation of d bf16 products, relative
    to sum_c |q_c k_c| (1e-5 of it) plus a small absolute floor."""
    import oracle_pins as op
    qt = op.f64(q_bits).abs()
    Kt = op.f64(K_bits)[:, :, :ctx].abs()
    Kt = Kt.repeat_interleave(qt.shape[1] // Kt.shape[1], dim=1)
    mag = torch.matmul(Kt, qt[..., None])[..., 0].numpy() * abs(scale)
    return 1e-5 * mag + 1e-6
