"""fp8 E4M3 K and V caches (the *_fp8kv calls) on the GPU.

* Power-of-two V scales: scale * decode(code) is exact in bf16, and scaling a
  sum by a power of two commutes with fp32 rounding, so the fp8 K/V calls must
  match the fp8 K calls run on the dequantized V cache: thresholds, counts and
  selection bitmaps bit for bit (the K side is the same), outputs equal or one
  bf16 step apart (the fp8 gather holds 16 elements per lane where the bf16
  one holds 8, so its slots sum the entries in another order).  Also at the
  Llama-like 128K batch-16 shape the benchmark times.
* General scales (amax / 448 per head): outputs within 1e-2 of the fp64 oracle
  on the E4M3 K and V caches with the GPU's mask, counts equal; the one-call
  refresh step against the separate calls.
"""
import numpy as np
import pytest
import torch

import oracle
import saga_workload as wl
import sparse_decode_attention_atop_amd as saga
from gpu_helpers import make_inputs, to_np_bits
from test_gpu_fp8k import SHAPES, match, run_fp8

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-2


def dequant_v(V8, vs):
    x = V8.view(torch.float8_e4m3fn).to(torch.float32) * vs[:, :, None, None]
    Vb = x.to(torch.bfloat16)
    assert torch.equal(Vb.to(torch.float32), x), "dequantized V is not exact in bf16"
    return Vb.contiguous()


def run_fp8kv(q, K8, ks, V8, vs, ctx_steps, N, n, fused=False):
    """The fp8 K/V calls over len(ctx_steps) steps (thresholds from the fp8 K
    refresh, or the one-call refresh step when fused)."""
    T, B, hq, d = q.shape
    hk, rows, hv, dv = K8.shape[1], K8.shape[2], V8.shape[1], V8.shape[3]
    dvx = 0 if dv == d else dv
    ws = saga.alloc_workspace(saga.dims(B, hq, hk, hv, d, ctx_steps[0], rows, head_dim_v=dvx), N)
    tau = torch.empty(B, hq, device="cuda")
    words = (rows + 31) // 32
    res = {"tau": [], "counts": [], "bitmap": [], "out": []}
    for t, ctx in enumerate(ctx_steps):
        dm = saga.dims(B, hq, hk, hv, d, ctx, rows, head_dim_v=dvx)
        out = torch.empty(B, hq, dv, dtype=torch.bfloat16, device="cuda")
        cnt = torch.empty(B, hq, dtype=torch.int32, device="cuda")
        bm = None
        if fused and t % n == 0:
            saga.atopn_refresh_decode_step_fp8kv(dm, N, q[t], K8, ks, V8, vs, tau, out, ws,
                                                 sel_counts=cnt)
        else:
            if t % n == 0:
                saga.atopn_refresh_thresholds_fp8k(dm, N, q[t], K8, ks, tau, ws)
            bm = torch.empty(B, hq, words, dtype=torch.int32, device="cuda")
            saga.saga_decode_step_fp8kv(dm, q[t], K8, ks, V8, vs, tau, out, ws, sel_counts=cnt,
                                        sel_bitmap_debug=bm)
        torch.cuda.synchronize()
        res["tau"].append(tau.cpu().numpy().copy())
        res["counts"].append(cnt.cpu().numpy())
        res["bitmap"].append(None if bm is None else bm.cpu().numpy().view(np.uint32))
        res["out"].append(out.float().cpu().numpy())
    return res


def inputs(name, seed, pow2):
    B, hq, hk, hv, d, L, T, N, n = SHAPES[name]
    q, K, V = make_inputs(B, hq, hk, hv, d, L + T, T, seed=seed)
    K8, ks = wl.quantize_k_e4m3(K, pow2_scales=pow2)
    V8, vs = wl.quantize_k_e4m3(V, pow2_scales=pow2)
    return q, K8, ks, V8, vs, [L + t for t in range(T)], N, n


@pytest.mark.parametrize("name", list(SHAPES))
def test_pow2_value_scales_match_fp8k_on_dequantized_v(name):
    q, K8, ks, V8, vs, ctx, N, n = inputs(name, 400 + len(name), pow2=True)
    print(f"[fp8kv pow2 {name}] V8{tuple(V8.shape)} ctx={ctx}", flush=True)
    got = run_fp8kv(q, K8, ks, V8, vs, ctx, N, n)
    ref = run_fp8(q, K8, ks, dequant_v(V8, vs), ctx, N, n)
    for k in ("tau", "counts", "bitmap", "out"):
        for t in range(len(ctx)):
            assert match(k, got[k][t], ref[k][t]), f"{k} differs at step {t}"


@pytest.mark.parametrize("name", ["qwen_like_small", "llama_like_small", "short_ctx"])
def test_pow2_value_scales_fused_refresh_step(name):
    q, K8, ks, V8, vs, ctx, N, n = inputs(name, 410 + len(name), pow2=True)
    got = run_fp8kv(q, K8, ks, V8, vs, ctx, N, n, fused=True)
    ref = run_fp8(q, K8, ks, dequant_v(V8, vs), ctx, N, n, fused=True, debug=False)
    for k in ("tau", "counts", "out"):
        for t in range(len(ctx)):
            assert match(k, got[k][t], ref[k][t]), f"{k} differs at step {t}"


def test_pow2_value_scales_at_the_benchmark_shape():
    """Llama-like heads, 128K context, batch 16, N = 2048: a refresh step then a
    plain step, fp8 K/V calls against fp8 K calls on the dequantized V cache."""
    w = wl.LLAMA_128K_B16
    x = wl.make_layer(w, 0, device="cuda", steps=2)
    q, K, V = x["q"], x["K"], x["V"]
    K8, ks = wl.quantize_k_e4m3(K, pow2_scales=True)
    V8, vs = wl.quantize_k_e4m3(V, pow2_scales=True)
    Vd = dequant_v(V8, vs)
    del K, V, x
    ctx = [w.ctx(0), w.ctx(1)]
    print(f"[fp8kv full] {w.name} ctx={ctx}", flush=True)
    got = run_fp8kv(q, K8, ks, V8, vs, ctx, w.top_n, 2, fused=True)
    ref = run_fp8(q, K8, ks, Vd, ctx, w.top_n, 2, fused=True, debug=False)
    for k in ("tau", "counts", "out"):
        for t in range(2):
            assert match(k, got[k][t], ref[k][t]), f"{k} differs at step {t}"


@pytest.mark.parametrize("name", ["qwen_like_small", "llama_like_small", "mha_d128", "short_ctx"])
def test_general_scales_outputs_match_oracle_on_gpu_mask(name):
    q, K8, ks, V8, vs, ctx, N, n = inputs(name, 420 + len(name), pow2=False)
    print(f"[fp8kv general {name}] v scales {vs.flatten()[:3].tolist()}", flush=True)
    gpu = run_fp8kv(q, K8, ks, V8, vs, ctx, N, n)
    qb, K8n, ksn, V8n, vsn = (to_np_bits(q), K8.cpu().numpy(), ks.cpu().numpy(),
                              V8.cpu().numpy(), vs.cpu().numpy())
    for t, c in enumerate(ctx):
        ref, cnt = oracle.masked_e4m3kv(qb[t], K8n, ksn, V8n, vsn, c, gpu["bitmap"][t])
        assert (cnt == gpu["counts"][t]).all(), t
        err = np.abs(gpu["out"][t] - ref).max()
        assert err <= OUT_TOL, f"step {t}: max abs err {err:.3e}"


@pytest.mark.parametrize("name", ["qwen_like_small", "llama_like_small"])
def test_general_scales_fused_refresh_step_matches_separate_calls(name):
    q, K8, ks, V8, vs, ctx, N, n = inputs(name, 430 + len(name), pow2=False)
    sep = run_fp8kv(q, K8, ks, V8, vs, ctx, N, n)
    fus = run_fp8kv(q, K8, ks, V8, vs, ctx, N, n, fused=True)
    qb, K8n, ksn, V8n, vsn = (to_np_bits(q), K8.cpu().numpy(), ks.cpu().numpy(),
                              V8.cpu().numpy(), vs.cpu().numpy())
    for t, c in enumerate(ctx):
        assert np.array_equal(fus["tau"][t].view(np.uint32), sep["tau"][t].view(np.uint32)), t
        assert np.array_equal(fus["counts"][t], sep["counts"][t]), t
        ref, _ = oracle.masked_e4m3kv(qb[t], K8n, ksn, V8n, vsn, c, sep["bitmap"][t])
        assert np.abs(fus["out"][t] - ref).max() <= OUT_TOL, t


@pytest.mark.parametrize("dk,dv", [(64, 32), (128, 64), (64, 128)])
def test_general_scales_key_and_value_dims_differ(dk, dv):
    """fp8 K at d_k and fp8 V at d_v (every value-row width the fp8 gather has)."""
    B, hq, hk, hv, L, T, N, n = 2, 8, 2, 4, 1800, 3, 40, 2
    q, K, V = make_inputs(B, hq, hk, hv, dk, L + T, T, seed=440 + dk + dv, dv=dv)
    K8, ks = wl.quantize_k_e4m3(K)
    V8, vs = wl.quantize_k_e4m3(V)
    ctx = [L + t for t in range(T)]
    print(f"[fp8kv dk={dk} dv={dv}] V8{tuple(V8.shape)}", flush=True)
    gpu = run_fp8kv(q, K8, ks, V8, vs, ctx, N, n)
    qb, K8n, ksn, V8n, vsn = (to_np_bits(q), K8.cpu().numpy(), ks.cpu().numpy(),
                              V8.cpu().numpy(), vs.cpu().numpy())
    for t, c in enumerate(ctx):
        ref, cnt = oracle.masked_e4m3kv(qb[t], K8n, ksn, V8n, vsn, c, gpu["bitmap"][t])
        assert ref.shape[-1] == dv
        assert (cnt == gpu["counts"][t]).all(), t
        err = np.abs(gpu["out"][t] - ref).max()
        assert err <= OUT_TOL, f"step {t}: max abs err {err:.3e}"
