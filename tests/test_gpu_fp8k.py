"""An fp8 E4M3 K cache (the *_fp8k calls) on the GPU.

* Power-of-two scales: scale * decode(code) is then exact in bf16, the kernels
  widen the codes exactly and fold the scale into the logit scale.  They sum
  the head dimension in another order than the bf16 kernels (16-byte loads
  that span two MFMA slabs); reordering the head dimension of q and K alike
  leaves attention unchanged and makes the bf16 calls sum in that order.  So
  logits, thresholds, counts and selection bitmaps must be bit-identical to
  the bf16 calls run on the dequantized cache with q and K so reordered --
  and the bf16 parity tests tie those to the oracle.  The fp8 stream's tile
  and launch sizes are tuned on their own (they may differ from bf16's), so
  the selected entries can reach the gather in another order and its fp32
  sums round differently: outputs must be equal or one bf16 step apart.  Also at
  the Llama-like 128K batch-16 shape the benchmark times, and on the
  recompute path of the refresh.
* General scales (amax / 448 per head): logits within the logit bar of the
  fp64 oracle on the E4M3 cache, thresholds bit-exact against a host sort of
  the GPU logits, selection equal to the oracle's away from the threshold,
  outputs within the output bar of the oracle on the GPU's mask.
* The short shapes take the list path (select lists, then a gather launch);
  the 40K single-sequence shape takes the small-batch path.
"""
import numpy as np
import pytest
import torch

import oracle
import saga_workload as wl
import sparse_decode_attention_atop_amd as saga
from gpu_helpers import (bitmap_to_bool, make_inputs, nth_largest_f32, run_atopn, run_fused,
                         sampled_rows, to_np_bits)

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-2
NEAR_TAU = 1e-3


def dequant_bf16(K8, ks):
    """bf16 cache holding scale * decode(code); exact for power-of-two scales."""
    x = K8.view(torch.float8_e4m3fn).to(torch.float32) * ks[:, :, None, None]
    Kb = x.to(torch.bfloat16)
    assert torch.equal(Kb.to(torch.float32), x), "dequantized cache is not exact in bf16"
    return Kb.contiguous()


def fp8_order(d):
    """Head-dim positions as the fp8 kernels sum them: MFMA slab m, lane group
    g, element e is head-dim index 64*(m//2) + 16*g + 8*(m%2) + e, where the
    bf16 kernels use 32*m + 8*g + e."""
    idx = [64 * (m // 2) + 16 * g + 8 * (m % 2) + e
           for m in range(d // 32) for g in range(4) for e in range(8)]
    assert sorted(idx) == list(range(d))
    return torch.tensor(idx, device="cuda")


def bf16_twin(q, K8, ks):
    """q and the dequantized cache, head dimension in the fp8 kernels' order."""
    idx = fp8_order(q.shape[-1])
    return q[..., idx].contiguous(), dequant_bf16(K8, ks)[..., idx].contiguous()


def run_fp8(q, K8, ks, V, ctx_steps, N, n, fused=False, debug=True):
    """The fp8k calls over len(ctx_steps) steps; same result layout as run_atopn
    (logits and bitmap are None at fused refresh steps)."""
    T, B, hq, d = q.shape
    hk, rows, hv = K8.shape[1], K8.shape[2], V.shape[1]
    ws = saga.alloc_workspace(saga.dims(B, hq, hk, hv, d, ctx_steps[0], rows), N)
    tau = torch.empty(B, hq, device="cuda")
    tau_scratch = torch.empty_like(tau)
    words = (rows + 31) // 32
    res = {"tau": [], "logits": [], "counts": [], "bitmap": [], "out": []}
    for t, ctx in enumerate(ctx_steps):
        dm = saga.dims(B, hq, hk, hv, d, ctx, rows)
        out = torch.empty(B, hq, d, dtype=torch.bfloat16, device="cuda")
        cnt = torch.empty(B, hq, dtype=torch.int32, device="cuda")
        lg = bm = None
        if fused and t % n == 0:
            saga.atopn_refresh_decode_step_fp8k(dm, N, q[t], K8, ks, V, tau, out, ws,
                                                sel_counts=cnt)
        else:
            if debug:
                lg = torch.empty(B, hq, ctx, device="cuda")
                saga.atopn_refresh_thresholds_fp8k(dm, N, q[t], K8, ks,
                                                   tau if t % n == 0 else tau_scratch, ws,
                                                   logits_debug=lg)
            elif t % n == 0:
                saga.atopn_refresh_thresholds_fp8k(dm, N, q[t], K8, ks, tau, ws)
            bm = torch.empty(B, hq, words, dtype=torch.int32, device="cuda")
            saga.saga_decode_step_fp8k(dm, q[t], K8, ks, V, tau, out, ws, sel_counts=cnt,
                                       sel_bitmap_debug=bm)
        torch.cuda.synchronize()
        res["tau"].append(tau.cpu().numpy().copy())
        res["logits"].append(None if lg is None else lg.cpu().numpy())
        res["counts"].append(cnt.cpu().numpy())
        res["bitmap"].append(None if bm is None else bm.cpu().numpy().view(np.uint32))
        res["out"].append(out.float().cpu().numpy())
    return res


def same_bits(a, b):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    return a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


def bf16_step_apart(a, b):
    """Two bf16 outputs (as float32) equal or one bf16 rounding step apart
    (plus 1e-6 for values near zero, where fp32 sums carry absolute error)."""
    m = np.maximum(np.abs(a), np.abs(b))
    ulp = np.exp2(np.floor(np.log2(np.where(m > 0, m, 1.0))) - 7)
    return a.shape == b.shape and bool((np.abs(a - b) <= np.where(m > 0, ulp, 0) + 1e-6).all())


def match(key, a, b):
    return bf16_step_apart(a, b) if key == "out" else same_bits(a, b)


SHAPES = {
    # name: (B, hq, hk, hv, d, L, T, N, n)
    "qwen_like_small": (2, 12, 1, 2, 128, 3000, 5, 100, 3),
    "llama_like_small": (2, 32, 4, 8, 64, 2500, 4, 64, 2),
    "group16_d64": (3, 16, 1, 4, 64, 1500, 4, 40, 2),
    "mha_d128": (2, 8, 8, 8, 128, 700, 3, 33, 2),
    "short_ctx": (1, 4, 2, 4, 64, 17, 3, 5, 2),
    # 320 workgroups: the K stream gathers the (bf16) value rows in its tail
    "tail_llama_like": (4, 32, 4, 8, 64, 2500, 3, 64, 2),
    # One sequence, one key head, 40K rows: enough workgroups for the
    # small-batch path (the value gather inside the K-stream kernel).
    "qwen_like_long": (1, 12, 1, 2, 128, 40000, 3, 500, 2),
}


def inputs(name, seed, pow2):
    B, hq, hk, hv, d, L, T, N, n = SHAPES[name]
    q, K, V = make_inputs(B, hq, hk, hv, d, L + T, T, seed=seed)
    K8, ks = wl.quantize_k_e4m3(K, pow2_scales=pow2)
    return q, K8, ks, V, [L + t for t in range(T)], N, n


@pytest.mark.parametrize("name", list(SHAPES))
def test_pow2_scales_bit_identical_to_bf16_calls(name):
    q, K8, ks, V, ctx, N, n = inputs(name, 200 + len(name), pow2=True)
    print(f"[fp8k pow2 {name}] K8{tuple(K8.shape)} ctx={ctx} N={N} n={n}", flush=True)
    got = run_fp8(q, K8, ks, V, ctx, N, n)
    ref = run_atopn(*bf16_twin(q, K8, ks), V, ctx, N, n)
    for k in ("tau", "logits", "counts", "bitmap", "out"):
        for t in range(len(ctx)):
            assert match(k, got[k][t], ref[k][t]), f"{k} differs at step {t}"


@pytest.mark.parametrize("name", ["qwen_like_small", "llama_like_small", "short_ctx",
                                  "qwen_like_long"])
def test_pow2_scales_fused_refresh_step_bit_identical(name):
    q, K8, ks, V, ctx, N, n = inputs(name, 210 + len(name), pow2=True)
    got = run_fp8(q, K8, ks, V, ctx, N, n, fused=True, debug=False)
    ref = run_fused(*bf16_twin(q, K8, ks), V, ctx, N, n)
    for k in ("tau", "counts", "out"):
        for t in range(len(ctx)):
            assert match(k, got[k][t], ref[k][t]), f"{k} differs at step {t}"


def test_pow2_scales_recompute_path_bit_identical():
    """The pivot sample sees only the highest logits, so the refresh takes its
    exact recompute path (and the fused step re-streams the group)."""
    ctx, N = 40000, 5000
    q, K, V = make_inputs(1, 4, 1, 2, 64, ctx, 1, seed=220, heavy=False)
    rows = sampled_rows(ctx)
    assert rows.size < N
    K.mul_(0.05)
    K[:, :, torch.from_numpy(rows).cuda(), :] = 1.0
    q.fill_(0.1)
    K8, ks = wl.quantize_k_e4m3(K, pow2_scales=True)
    qd, Kd = bf16_twin(q, K8, ks)
    for fused in (False, True):
        got = run_fp8(q, K8, ks, V, [ctx], N, 1, fused=fused, debug=not fused)
        ref = (run_fused if fused else run_atopn)(qd, Kd, V, [ctx], N, 1)
        assert (got["counts"][0] >= N).all()
        for k in ("tau", "counts", "out"):
            assert match(k, got[k][0], ref[k][0]), (fused, k)


def test_pow2_scales_at_the_benchmark_shape():
    """Llama-like heads, 128K context, batch 16, N = 2048: a refresh step then a
    plain step, fp8 calls against bf16 calls on the dequantized cache."""
    w = wl.LLAMA_128K_B16
    x = wl.make_layer(w, 0, device="cuda", steps=2)
    q, K, V = x["q"], x["K"], x["V"]
    K8, ks = wl.quantize_k_e4m3(K, pow2_scales=True)
    qd, Kd = bf16_twin(q, K8, ks)
    del K, x
    ctx = [w.ctx(0), w.ctx(1)]
    print(f"[fp8k full] {w.name} ctx={ctx}", flush=True)
    got = run_fp8(q, K8, ks, V, ctx, w.top_n, 2, fused=True, debug=False)
    ref = run_fused(qd, Kd, V, ctx, w.top_n, 2)
    for k in ("tau", "counts", "out"):
        for t in range(2):
            assert match(k, got[k][t], ref[k][t]), f"{k} differs at step {t}"


_cache = {}


def general(name):
    if name not in _cache:
        q, K8, ks, V, ctx, N, n = inputs(name, 230 + len(name), pow2=False)
        print(f"[fp8k general {name}] scales {ks.flatten()[:4].tolist()}", flush=True)
        gpu = run_fp8(q, K8, ks, V, ctx, N, n)
        qb, K8n, ksn, Vb = to_np_bits(q), K8.cpu().numpy(), ks.cpu().numpy(), to_np_bits(V)
        ref = oracle.atopn_run_e4m3k(qb, K8n, ksn, Vb, ctx, N, n, want_sel=True,
                                     want_logits=True)
        kval = K8.view(torch.float8_e4m3fn).to(torch.float64).cpu() * ks.double().cpu()[:, :, None, None]
        _cache[name] = dict(q=qb, K8=K8n, ks=ksn, V=Vb, kval=kval.numpy(), ctx=ctx, N=N, n=n,
                            gpu=gpu, ref=ref)
    return _cache[name]


def tolerance(qbits, kval, ctx):
    """1e-5 * sum_c |q_c k_c| + 1e-6 per logit (fp32 accumulation bar)."""
    qf = torch.from_numpy(qbits.astype(np.uint32) << 16).view(torch.float32).double().abs()
    kf = torch.from_numpy(np.abs(kval[:, :, :ctx]))
    kf = kf.repeat_interleave(qf.shape[1] // kf.shape[1], dim=1)
    return (1e-5 * torch.matmul(kf, qf[..., None])[..., 0] + 1e-6).numpy()


GENERAL = ["qwen_like_small", "llama_like_small", "mha_d128", "qwen_like_long"]


@pytest.mark.parametrize("name", GENERAL)
def test_general_scales_logits_match_oracle(name):
    c = general(name)
    for t, ctx in enumerate(c["ctx"]):
        err = np.abs(c["gpu"]["logits"][t].astype(np.float64) - c["ref"]["logits"][t][..., :ctx])
        tol = tolerance(c["q"][t], c["kval"], ctx)
        assert (err <= tol).all(), f"step {t}: worst excess {(err - tol).max():.3e}"


@pytest.mark.parametrize("name", GENERAL)
def test_general_scales_thresholds_and_selection(name):
    c = general(name)
    N = c["N"]
    for t, ctx in enumerate(c["ctx"]):
        lg, tau = c["gpu"]["logits"][t], c["gpu"]["tau"][t]
        if t % c["n"] == 0:
            for b in range(lg.shape[0]):
                for i in range(lg.shape[1]):
                    assert tau[b, i] == nth_largest_f32(lg[b, i], N), (t, b, i)
        sel = bitmap_to_bool(c["gpu"]["bitmap"][t], ctx)
        assert (sel == (lg >= tau[..., None])).all(), f"step {t}: not an exact filter"
        ref = c["ref"]["sel"][t][..., :ctx].astype(bool)
        near = np.abs(c["ref"]["logits"][t][..., :ctx] - c["ref"]["tau"][t][..., None]) <= NEAR_TAU
        assert not ((sel != ref) & ~near).any(), f"step {t}: selection differs off threshold"


@pytest.mark.parametrize("name", GENERAL)
def test_general_scales_outputs_match_oracle_on_gpu_mask(name):
    c = general(name)
    for t, ctx in enumerate(c["ctx"]):
        ref, cnt = oracle.masked_e4m3k(c["q"][t], c["K8"], c["ks"], c["V"], ctx,
                                       c["gpu"]["bitmap"][t])
        assert (cnt == c["gpu"]["counts"][t]).all()
        err = np.abs(c["gpu"]["out"][t] - ref).max()
        assert err <= OUT_TOL, f"step {t}: max abs err {err:.3e}"
