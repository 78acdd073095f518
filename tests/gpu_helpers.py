"""Helpers for the GPU parity tests: drive the C-ABI library over decode steps
with its debug outputs switched on, and bring the results to the host.

Every buffer a call writes (out, thresholds, counts, bitmap, logits and the
workspace) is allocated by ``Guards`` between two canary-filled bands, and the
bands are checked after every call: a kernel that writes one byte before or
after its buffer fails the test that ran it."""
from __future__ import annotations

import math

import numpy as np
import torch

import sparse_decode_attention_atop_amd as saga
import saga_workload as wl

GUARD_BYTES = 4096          # canary band on each side (keeps 256-byte alignment)
CANARY = 0xA5


class Guards:
    """Device buffers with a canary band before and after each of them."""

    def __init__(self, device="cuda"):
        self.device = device
        self.bufs = []

    def empty(self, shape, dtype, name="buffer"):
        shape = tuple(int(x) for x in shape)
        n = math.prod(shape) * torch.empty((), dtype=dtype).element_size()
        raw = torch.empty(n + 2 * GUARD_BYTES, dtype=torch.uint8, device=self.device)
        raw[:GUARD_BYTES].fill_(CANARY)
        raw[GUARD_BYTES + n:].fill_(CANARY)
        self.bufs.append((raw, n, name))
        return raw[GUARD_BYTES:GUARD_BYTES + n].view(dtype).view(shape)

    def workspace(self, dims, top_n, lq=0):
        n = (saga.saga_workspace_bytes(saga._lq_dims(dims, lq), top_n) if lq
             else saga.saga_workspace_bytes(dims, top_n))
        assert n > 0, "saga_workspace_bytes rejected the dims"
        return self.empty((n,), torch.uint8, "workspace")

    def check(self, where=""):
        for raw, n, name in self.bufs:
            lo = raw[:GUARD_BYTES] != CANARY
            hi = raw[GUARD_BYTES + n:] != CANARY
            if bool(lo.any()) or bool(hi.any()):
                raise AssertionError(
                    f"{name}: {int(lo.sum())} bytes before and {int(hi.sum())} bytes after "
                    f"the buffer were overwritten {where}")


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
    g = Guards(q.device)
    dims0 = saga.dims(B, hq, hk, hv, d, ctx_steps[0], rows, scale, head_dim_v=dvx)
    ws = g.workspace(dims0, top_n)
    tau = g.empty((B, hq), torch.float32, "tau")
    tau_scratch = g.empty((B, hq), torch.float32, "tau_scratch")
    words = (rows + 31) // 32
    res = {"tau": [], "logits": [], "counts": [], "bitmap": [], "out": []}
    for t, ctx in enumerate(ctx_steps):
        dm = saga.dims(B, hq, hk, hv, d, ctx, rows, scale, head_dim_v=dvx)
        lg = g.empty((B, hq, ctx), torch.float32, f"logits[{t}]")
        if t % refresh_n == 0:
            saga.atopn_refresh_thresholds(dm, top_n, q[t], K, tau, ws, logits_debug=lg)
        elif logits_every_step:
            # Logits of a plain step, for checking; the kept thresholds are untouched.
            saga.atopn_refresh_thresholds(dm, top_n, q[t], K, tau_scratch, ws, logits_debug=lg)
        out = g.empty((B, hq, dv), torch.bfloat16, f"out[{t}]")
        cnt = g.empty((B, hq), torch.int32, f"sel_counts[{t}]")
        bm = g.empty((B, hq, words), torch.int32, f"sel_bitmap[{t}]")
        saga.saga_decode_step(dm, q[t], K, V, tau, out, ws, sel_counts=cnt, sel_bitmap_debug=bm)
        torch.cuda.synchronize()
        g.check(f"at step {t}")
        res["tau"].append(tau.cpu().numpy().copy())
        res["logits"].append(lg.cpu().numpy() if (t % refresh_n == 0 or logits_every_step) else None)
        res["counts"].append(cnt.cpu().numpy())
        res["bitmap"].append(bm.cpu().numpy().view(np.uint32))
        res["out"].append(bf16_to_f32(out))
        g.bufs = [x for x in g.bufs if not x[2].endswith(f"[{t}]")]
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
    g = Guards(dev)
    ws = g.workspace(saga.dims(B, hq, hk, hv, d, ctx_steps[0], rows, scale, head_dim_v=dvx),
                     top_n)
    tau = g.empty((B, hq), torch.float32, "tau")
    res = {"tau": [], "counts": [], "out": []}
    for t, ctx in enumerate(ctx_steps):
        dm = saga.dims(B, hq, hk, hv, d, ctx, rows, scale, head_dim_v=dvx)
        out = g.empty((B, hq, dv), torch.bfloat16, f"out[{t}]")
        cnt = g.empty((B, hq), torch.int32, f"sel_counts[{t}]")
        if t % refresh_n == 0:
            saga.atopn_refresh_decode_step(dm, top_n, q[t], K, V, tau, out, ws, sel_counts=cnt)
        else:
            saga.saga_decode_step(dm, q[t], K, V, tau, out, ws, sel_counts=cnt)
        torch.cuda.synchronize()
        g.check(f"at step {t}")
        res["tau"].append(tau.cpu().numpy().copy())
        res["counts"].append(cnt.cpu().numpy())
        res["out"].append(bf16_to_f32(out))
        g.bufs = [x for x in g.bufs if not x[2].endswith(f"[{t}]")]
    return res


def mask_to_bitmap(mask: np.ndarray, rows: int) -> np.ndarray:
    """[..., ctx] bool -> [..., ceil(rows/32)] uint32 (bit j of word w: row 32w + j)."""
    words = (rows + 31) // 32
    full = np.zeros(mask.shape[:-1] + (words * 32,), dtype=bool)
    full[..., :mask.shape[-1]] = mask
    return np.packbits(full, axis=-1, bitorder="little").view(np.uint32)


def run_bench_schedule(q, K, V, ctx_steps, top_n, refresh_n, rows_idx, scale=1.0):
    """The decode schedule exactly as bench.py runs it on one layer: one
    workspace for every step, atopn_refresh_decode_step when t mod n == 0 and
    saga_decode_step otherwise, no debug outputs.  After each call the sampled
    (b, i) rows' thresholds, counts and outputs are kept, and the same step's
    fp32 logits of those rows are read from a separate refresh call (its own
    workspace and scratch thresholds) so the call's selection {s >= tau} can be
    rebuilt on the host.

    Returns per-step lists: tau [R], counts [R], out [R][dv] (float32),
    logits [R][ctx] (float32) for the R sampled rows."""
    T, B, hq, d = q.shape
    hk, rows = K.shape[1], K.shape[2]
    hv, dv = V.shape[1], V.shape[3]
    dvx = 0 if dv == d else dv
    dev = q.device
    g = Guards(dev)
    dims0 = saga.dims(B, hq, hk, hv, d, ctx_steps[0], rows, scale, head_dim_v=dvx)
    ws = g.workspace(dims0, top_n)
    tau = g.empty((B, hq), torch.float32, "tau")
    out = g.empty((B, hq, dv), torch.bfloat16, "out")
    cnt = g.empty((B, hq), torch.int32, "sel_counts")
    ws_dbg = saga.alloc_workspace(dims0, top_n, dev)
    tau_dbg = torch.empty(B, hq, dtype=torch.float32, device=dev)
    idx = torch.tensor(rows_idx, device=dev)
    res = {"tau": [], "counts": [], "out": [], "logits": []}
    for t, ctx in enumerate(ctx_steps):
        dm = saga.dims(B, hq, hk, hv, d, ctx, rows, scale, head_dim_v=dvx)
        if t % refresh_n == 0:
            saga.atopn_refresh_decode_step(dm, top_n, q[t], K, V, tau, out, ws, sel_counts=cnt)
        else:
            saga.saga_decode_step(dm, q[t], K, V, tau, out, ws, sel_counts=cnt)
        torch.cuda.synchronize()
        g.check(f"at step {t}")
        lg = torch.empty(B, hq, ctx, dtype=torch.float32, device=dev)
        saga.atopn_refresh_thresholds(dm, top_n, q[t], K, tau_dbg, ws_dbg, logits_debug=lg)
        torch.cuda.synchronize()
        res["tau"].append(tau[idx[:, 0], idx[:, 1]].cpu().numpy())
        res["counts"].append(cnt[idx[:, 0], idx[:, 1]].cpu().numpy())
        res["out"].append(out[idx[:, 0], idx[:, 1]].float().cpu().numpy())
        res["logits"].append(lg[idx[:, 0], idx[:, 1]].cpu().numpy())
        del lg
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
