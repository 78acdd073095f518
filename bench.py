#!/usr/bin/env python3
"""Decode-attention benchmark of SAGA + Atop-N on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A *step* is one decode step of the whole hot path for every layer of the
workload and every batch row: for each layer, the exact top-N threshold
refresh when t mod n == 0 (QK logits + radix select) and the fused Atop-N
decode (K stream, threshold mask, ballot compaction, masked online softmax,
sparse V gather, split-sequence combine).  Step t attends ctx_t = L + t rows
and t cycles through the workload's T = 32 decode steps, so K = 320 steps is
the pages' protocol of 10 runs x 32 generated tokens.  Each step (all layers)
is captured once into a HIP graph and replayed; inputs are resident in HBM
before the timed region.

Printed: one JSON line with steps/s (value), tokens/s, the roofline of the
dominant kernel (the decode call: algorithmic bytes per call over its
duration in graph replays of the plain decode steps, timed by events on the
replay stream; the eager per-call figure is reported beside it), the same
library's full-attention GQA baseline on
the GQA twin of the shape (h_k = h_v), and the CPU oracle timed on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
KERNEL_SOURCES = ("decode.hip", "device.hpp", "kernels.hpp", "tuning.hpp")


def kernel_sources_hash() -> str:
    """sha256 over the decode kernels' sources: a traffic figure measured with
    rocprofv3 counters applies only while this hash is unchanged."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_decode_attention_atop_amd", "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(path, workload):
    """HBM bytes per decode call from a committed rocprofv3 summary (a JSON block
    in a markdown file), or None when absent, for another workload, or stale."""
    if not path or not os.path.exists(path):
        return None
    text = open(path).read()
    start = text.find("```json")
    if start < 0:
        return None
    end = text.find("```", start + 7)
    try:
        tr = json.loads(text[start + 7:end])
    except ValueError:
        return None
    if tr.get("workload") != workload or tr.get("kernel_sources") != kernel_sources_hash():
        return None
    return tr.get("bytes_per_call")
DEFAULT_WORKLOAD = "llama_like_128k_b16"
GQA_TWIN = {"llama_like_128k_b16": 8, "qwen_like_128k_b1": 2, "qwen_like_128k_b16": 2,
            "llama_like_8k": 8, "tiny": 2}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--decompose", action="store_true",
                   help="time GQA full, SAGA full, Atop-N at GQA heads and SAGA + Atop-N")
    p.add_argument("--steps", type=int, default=320)
    p.add_argument("--warmup", type=int, default=32)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--no-gqa", action="store_true", help="skip the full-attention GQA baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--traffic", default=None,
                   help="markdown summary holding rocprofv3-measured HBM bytes per decode call "
                        "(default: profiles/traffic_<workload>.md)")
    p.add_argument("--calibrate", action="store_true",
                   help="measured HBM ceilings: sequential read and random-row probe kernels, "
                        "and a 4 GiB device copy (the known-size kernel that scales rocprofv3 "
                        "byte counters)")
    p.add_argument("--eager-only", action="store_true",
                   help="one eager pass over the decode steps, no timing (for counter runs)")
    p.add_argument("--paged", type=int, default=0,
                   help="time the schedule on paged caches with pages of this many rows")
    p.add_argument("--varlen", action="store_true",
                   help="with --paged: per-sequence lengths drawn from [L/4, L]")
    p.add_argument("--top-n", type=int, default=0,
                   help="main schedule with this N instead of the workload's (the workload is "
                        "then reported as <name>_n<N>)")
    p.add_argument("--lq", type=int, default=0,
                   help="time the schedule with this many query tokens per head and step")
    p.add_argument("--fp8k", action="store_true",
                   help="store the K cache as fp8 E4M3 (the *_fp8k calls)")
    p.add_argument("--fp8kv", action="store_true",
                   help="store the K and V caches as fp8 E4M3 (the *_fp8kv calls)")
    p.add_argument("--sigma", action="store_true",
                   help="Sigma-style heads: twice the key heads at half the key head dimension "
                        "(same K bytes), value heads unchanged; main schedule only")
    p.add_argument("--sweep", action="store_true",
                   help="Llama-like and Qwen-like shapes over L x N x B: SAGA Atop-N vs the "
                        "full-attention GQA path, one JSON line per point")
    return p.parse_args()


def calibrate(torch):
    """Measured HBM ceilings for the decode step's two access patterns, from
    the committed probe kernels (libsaga_probe.so): a sequential read of
    contiguous per-workgroup chunks (the K stream) and reads of pseudo-random
    64/128/256-byte rows of an 8 GiB buffer with fresh rows every launch (the
    value gather), each swept over workgroup counts and loads in flight; plus
    torch's 4 GiB device copy, the known-size kernel that scales rocprofv3's
    byte counters.  Prints one JSON line."""
    from sparse_decode_attention_atop_amd import probe

    def timed(fn, reps=10):
        fn(0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for r in range(reps):
            fn(r + 1)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps / 1e3

    sink = torch.empty(1 << 20, dtype=torch.int32, device="cuda")
    seq = []
    buf = torch.ones(4 << 30, dtype=torch.uint8, device="cuda")
    for total in (1 << 30, 4 << 30):
        for wg in (256, 512, 768, 1024, 1536, 2048):
            nbytes = total // (wg * 4096) * (wg * 4096)
            for depth in (1, 2, 4):
                sec = timed(lambda r: probe.probe_read(buf, nbytes, wg, depth, sink))
                seq.append({"bytes": nbytes, "workgroups": wg, "depth": depth,
                            "us": round(sec * 1e6, 2), "gbs": round(nbytes / sec / 1e9, 1)})
                log(f"read {nbytes >> 20} MiB wg={wg} depth={depth}: {seq[-1]['gbs']} GB/s")
    tiles = []
    for rb in (128, 256):
        for wg in (512, 768, 1024):
            nbytes = (1 << 30) // (wg * 16384) * (wg * 16384)
            for nt in (1, 2):
                sec = timed(lambda r: probe.probe_read_tiles(buf, nbytes, rb, wg, nt, sink))
                tiles.append({"bytes": nbytes, "row_bytes": rb, "workgroups": wg, "tiles": nt,
                              "us": round(sec * 1e6, 2), "gbs": round(nbytes / sec / 1e9, 1)})
                log(f"tiles {rb} B rows {nbytes >> 20} MiB wg={wg} tiles={nt}: "
                    f"{tiles[-1]['gbs']} GB/s")
    del buf
    torch.cuda.empty_cache()
    rows_res = {}
    big = torch.ones(8 << 30, dtype=torch.uint8, device="cuda")
    gather_bytes = 148 << 20                 # about one Llama-like 128K B=16 gather
    for rb in (64, 128, 256):
        pts = []
        n = gather_bytes // rb
        for wg in (1024, 2048, 4096):
            for depth in (2, 4, 8):
                sec = timed(lambda r: probe.probe_rows(big, rb, n, 1000 * r + wg + depth, wg,
                                                       depth, sink))
                pts.append({"rows": n, "workgroups": wg, "depth": depth,
                            "us": round(sec * 1e6, 2), "gbs": round(n * rb / sec / 1e9, 1)})
                log(f"rows {rb} B x {n} wg={wg} depth={depth}: {pts[-1]['gbs']} GB/s")
        best = max(pts, key=lambda p: p["gbs"])
        rows_res[str(rb)] = {"best_gbs": best["gbs"], "best": best, "table": pts}
    del big
    torch.cuda.empty_cache()
    n = 4 << 30
    src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    t_copy = timed(lambda r: dst.copy_(src))
    best_seq = {tot: max((p for p in seq if p["bytes"] > tot // 2 and p["bytes"] <= tot),
                         key=lambda p: p["gbs"]) for tot in (1 << 30, 4 << 30)}
    print(json.dumps({
        "calibration": "HBM ceilings of the decode step's access patterns (probe kernels)",
        "peak_gbs": HBM_PEAK_GBS,
        "sequential_read": {"best_1gib": best_seq[1 << 30], "best_4gib": best_seq[4 << 30],
                            "table": seq},
        "sequential_read_stream_lanes": {"best": max(tiles, key=lambda p: p["gbs"]),
                                         "table": tiles},
        "random_rows": rows_res,
        "torch_copy_4gib": {"bytes_read": n, "bytes_written": n,
                            "gbs_read_plus_written": round(2 * n / t_copy / 1e9, 1)}}), flush=True)


def layer_inputs(torch, wl, w, layer):
    x = wl.make_layer(w, layer, device="cuda")
    return x["K"], x["V"], x["q"]


def decode_algorithmic_bytes(w, ctx, sel_total, k_bytes=2, v_bytes=2):
    """Bytes the fused decode launch must move: K once per (b, key head)
    (k_bytes per element: 2 for bf16, 1 for fp8), the selected V rows (v_bytes
    per element), q, out and the thresholds."""
    d, dv = w.head_dim, w.head_dim_v or w.head_dim
    return (w.batch * w.h_k * ctx * d * k_bytes + sel_total * dv * v_bytes
            + w.batch * w.h_q * (d + dv) * 2 + w.batch * w.h_q * 4)


def full_algorithmic_bytes(w, ctx):
    d, dv = w.head_dim, w.head_dim_v or w.head_dim
    return w.batch * ctx * (w.h_k * d + w.h_v * dv) * 2 + w.batch * w.h_q * (d + dv) * 2


def time_graphs(torch, graphs, steps, warmup):
    T = len(graphs)
    for k in range(warmup):
        graphs[k % T].replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for k in range(steps):
        graphs[(warmup + k) % T].replay()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / 1e3, wall


def run_saga(torch, saga, wl, w, args):
    T, L = w.steps, w.L
    layers = []
    log(f"generating {w.layers} layers of {w.name} ({w.kv_bytes() / 1e9:.1f} GB of KV cache)")
    for layer in range(w.layers):
        K, V, q = layer_inputs(torch, wl, w, layer)
        log(f"  layer {layer} ready")
        layers.append(dict(K=K, V=V, q=q,
                           tau=torch.empty(w.batch, w.h_q, dtype=torch.float32, device="cuda"),
                           out=torch.empty(w.batch, w.h_q, w.head_dim_v or w.head_dim,
                                           dtype=torch.bfloat16, device="cuda"),
                           cnt=torch.empty(w.batch, w.h_q, dtype=torch.int32, device="cuda")))
    torch.cuda.synchronize()
    d0 = saga.dims(w.batch, w.h_q, w.h_k, w.h_v, w.head_dim, L, w.rows, w.scale,
                   head_dim_v=w.head_dim_v)
    ws = saga.alloc_workspace(d0, w.top_n)

    def step(t, events=None):
        dm = saga.dims(w.batch, w.h_q, w.h_k, w.h_v, w.head_dim, L + t, w.rows, w.scale,
                       head_dim_v=w.head_dim_v)
        for li, x in enumerate(layers):
            if events is not None:
                events[li][0].record()
            if t % w.refresh_n == 0:
                # Refresh step: fresh thresholds and this step's output in one call.
                saga.atopn_refresh_decode_step(dm, w.top_n, x["q"][t], x["K"], x["V"], x["tau"],
                                               x["out"], ws, sel_counts=x["cnt"])
            else:
                saga.saga_decode_step(dm, x["q"][t], x["K"], x["V"], x["tau"], x["out"], ws,
                                      sel_counts=x["cnt"])
            if events is not None:
                events[li][1].record()

    # Eager pass over one full run, then a second one with per-call timing by
    # events on the stream the calls run on, and the selected count of each.
    log("eager pass (per-call timing)")
    for t in range(T):
        step(t)
    torch.cuda.synchronize()
    if args.eager_only:
        log("eager pass done")
        return None
    launches, refreshes = [], []
    for t in range(T):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in layers]
        step(t, ev)
        torch.cuda.synchronize()
        for li, x in enumerate(layers):
            ms = ev[li][0].elapsed_time(ev[li][1])
            sel = int(x["cnt"].sum().item())
            rec = (t, li, ms, decode_algorithmic_bytes(w, L + t, sel), sel)
            (refreshes if t % w.refresh_n == 0 else launches).append(rec)

    log("capturing one HIP graph per decode step")
    graphs = []
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for t in range(T):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                step(t)
            graphs.append(g)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps after {args.warmup} warmup steps")
    sec, wall = time_graphs(torch, graphs, args.steps, args.warmup)
    # The plain decode call as the timed schedule runs it: three passes over
    # the step graphs that hold only saga_decode_step calls (t mod n != 0),
    # timed by events on the replay stream; per call = elapsed / calls.  The
    # eager per-call events above also count the host's launch gaps inside
    # each call.
    plain = [g for t, g in enumerate(graphs) if t % w.refresh_n != 0]
    graph_call_ms = None
    if plain:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(3):
            for g in plain:
                g.replay()
        e1.record()
        torch.cuda.synchronize()
        graph_call_ms = e0.elapsed_time(e1) / (3 * len(plain) * len(layers))
    return dict(layers=layers, launches=launches, refreshes=refreshes, sec=sec, wall=wall,
                ws=ws, graphs=graphs, graph_call_ms=graph_call_ms)


def to_pages(torch, X, P, perm):
    """[B][h][rows][d] cache -> pool [pages][h][P][d] (zero-padded last page),
    sequence b's page p stored at pool page perm[b * max_pages + p]."""
    B, h, rows, d = X.shape
    maxp = -(-rows // P)
    Xp = torch.zeros(B, h, maxp * P, d, dtype=X.dtype, device=X.device)
    Xp[:, :, :rows] = X
    Y = Xp.view(B, h, maxp, P, d).permute(0, 2, 1, 3, 4).reshape(B * maxp, h, P, d)
    del Xp
    pool = torch.empty_like(Y)
    pool[torch.from_numpy(perm.astype("int64")).to(X.device)] = Y
    return pool


def run_saga_paged(torch, saga, wl, w, args):
    """The main schedule on paged caches (pages of args.paged rows, shuffled in
    the pools).  With args.varlen, sequence b attends L_b + t rows, L_b drawn
    (seeded) uniformly from [L/4, L]; otherwise every sequence attends L + t."""
    import numpy as np
    T, L, P = w.steps, w.L, args.paged
    maxp = -(-w.rows // P)
    cache_len = maxp * P
    rng = np.random.default_rng(7)
    Lb = (rng.integers(L // 4, L + 1, size=w.batch) if args.varlen
          else np.full(w.batch, L)).astype(np.int64)
    perm = rng.permutation(w.batch * maxp).astype(np.int32)
    table = torch.from_numpy(perm).view(w.batch, maxp).cuda()
    ctx_lens = torch.empty(w.batch, dtype=torch.int32, device="cuda")
    pg = saga.paged(table, ctx_lens, P, w.batch * maxp)
    layers = []
    log(f"generating {w.layers} paged layers of {w.name} (pages of {P} rows)")
    for layer in range(w.layers):
        K, V, q = layer_inputs(torch, wl, w, layer)
        kp, vp = to_pages(torch, K, P, perm), to_pages(torch, V, P, perm)
        del K, V
        layers.append(dict(K=kp, V=vp, q=q,
                           tau=torch.empty(w.batch, w.h_q, dtype=torch.float32, device="cuda"),
                           out=torch.empty(w.batch, w.h_q, w.head_dim, dtype=torch.bfloat16,
                                           device="cuda"),
                           cnt=torch.empty(w.batch, w.h_q, dtype=torch.int32, device="cuda")))
        log(f"  layer {layer} ready")
    lens = [torch.from_numpy((Lb + t).astype(np.int32)).cuda() for t in range(T)]
    ws = saga.alloc_workspace(saga.dims(w.batch, w.h_q, w.h_k, w.h_v, w.head_dim, int(Lb.max()),
                                        cache_len, w.scale), w.top_n)

    def step(t):
        ctx_lens.copy_(lens[t])
        dm = saga.dims(w.batch, w.h_q, w.h_k, w.h_v, w.head_dim, int(Lb.max()) + t, cache_len,
                       w.scale)
        for x in layers:
            if t % w.refresh_n == 0:
                saga.atopn_refresh_decode_step_paged(dm, pg, w.top_n, x["q"][t], x["K"], x["V"],
                                                     x["tau"], x["out"], ws, sel_counts=x["cnt"])
            else:
                saga.saga_decode_step_paged(dm, pg, x["q"][t], x["K"], x["V"], x["tau"],
                                            x["out"], ws, sel_counts=x["cnt"])

    sel = 0
    for t in range(T):
        step(t)
        torch.cuda.synchronize()
        sel += sum(int(x["cnt"].sum().item()) for x in layers)
    graphs = []
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for t in range(T):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                step(t)
            graphs.append(g)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    log(f"timing {args.steps} paged steps after {args.warmup} warmup steps")
    sec, _ = time_graphs(torch, graphs, args.steps, args.warmup)
    d = w.head_dim
    k_bytes = w.layers * w.h_k * d * 2 * sum(int((Lb + t).sum()) for t in range(T)) / T
    step_bytes = (k_bytes + sel * d * 2 / T
                  + w.layers * (2 * w.batch * w.h_q * d * 2 + w.batch * w.h_q * 4))
    return dict(sec=sec, step_bytes=step_bytes, ctx=Lb.tolist())


def run_saga_lq(torch, saga, wl, w, args):
    """The main schedule with args.lq query tokens per head and step (token j
    of step t attends L + lq*t + j + 1 rows), through the *_lq calls."""
    lq, T = args.lq, w.steps
    w2 = w.with_(h_q=w.h_q * lq, L=w.L + (lq - 1) * T)            # rows = L + lq*T
    layers = []
    log(f"generating {w.layers} layers of {w.name} with {lq} query tokens per step")
    for layer in range(w.layers):
        K, V, q = layer_inputs(torch, wl, w2, layer)
        layers.append(dict(K=K, V=V, q=q,
                           tau=torch.empty(w.batch, w.h_q, lq, device="cuda"),
                           out=torch.empty(w.batch, w.h_q, lq, w.head_dim, dtype=torch.bfloat16,
                                           device="cuda"),
                           cnt=torch.empty(w.batch, w.h_q, lq, dtype=torch.int32, device="cuda")))
        log(f"  layer {layer} ready")
    ctx = [w.L + lq * (t + 1) for t in range(T)]
    ws = saga.alloc_workspace_lq(saga.dims(w.batch, w.h_q, w.h_k, w.h_v, w.head_dim, ctx[0],
                                           w2.rows, w.scale), lq, w.top_n)

    def step(t):
        dm = saga.dims(w.batch, w.h_q, w.h_k, w.h_v, w.head_dim, ctx[t], w2.rows, w.scale)
        for x in layers:
            if t % w.refresh_n == 0:
                saga.atopn_refresh_decode_step_lq(dm, lq, w.top_n, x["q"][t], x["K"], x["V"],
                                                  x["tau"], x["out"], ws, sel_counts=x["cnt"])
            else:
                saga.saga_decode_step_lq(dm, lq, x["q"][t], x["K"], x["V"], x["tau"], x["out"],
                                         ws, sel_counts=x["cnt"])

    sel = 0
    for t in range(T):
        step(t)
        torch.cuda.synchronize()
        sel += sum(int(x["cnt"].sum().item()) for x in layers)
    graphs = []
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for t in range(T):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                step(t)
            graphs.append(g)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps of {lq} tokens after {args.warmup} warmup steps")
    sec, _ = time_graphs(torch, graphs, args.steps, args.warmup)
    d = w.head_dim
    step_bytes = (w.layers * w.batch * w.h_k * d * 2 * sum(ctx) / T + sel * d * 2 / T
                  + w.layers * (2 * w.batch * w.h_q * lq * d * 2 + w.batch * w.h_q * lq * 4))
    return dict(sec=sec, step_bytes=step_bytes)


def run_saga_fp8k(torch, saga, wl, w, args, v8=False):
    """The main schedule with the K cache stored as fp8 E4M3 (one scale per
    sequence and key head, amax / 448) and V in bf16, through the *_fp8k calls;
    with v8 the V cache too (one scale per sequence and value head), through
    the *_fp8kv calls (thresholds from atopn_refresh_thresholds_fp8k)."""
    T, L = w.steps, w.L
    layers = []
    log(f"generating {w.layers} layers of {w.name} with an fp8 K{'/V' if v8 else ''} cache")
    for layer in range(w.layers):
        K, V, q = layer_inputs(torch, wl, w, layer)
        K8, ks = wl.quantize_k_e4m3(K)
        del K
        vs = None
        if v8:
            V, vs = wl.quantize_k_e4m3(V)
        layers.append(dict(K8=K8, ks=ks, V=V, vs=vs, q=q,
                           tau=torch.empty(w.batch, w.h_q, device="cuda"),
                           out=torch.empty(w.batch, w.h_q, w.head_dim, dtype=torch.bfloat16,
                                           device="cuda"),
                           cnt=torch.empty(w.batch, w.h_q, dtype=torch.int32, device="cuda")))
        log(f"  layer {layer} ready")
    torch.cuda.empty_cache()
    ws = saga.alloc_workspace(saga.dims(w.batch, w.h_q, w.h_k, w.h_v, w.head_dim, L, w.rows,
                                        w.scale), w.top_n)

    def step(t, events=None):
        dm = saga.dims(w.batch, w.h_q, w.h_k, w.h_v, w.head_dim, L + t, w.rows, w.scale)
        for li, x in enumerate(layers):
            if events is not None:
                events[li][0].record()
            if v8 and t % w.refresh_n == 0:
                saga.atopn_refresh_decode_step_fp8kv(dm, w.top_n, x["q"][t], x["K8"], x["ks"],
                                                     x["V"], x["vs"], x["tau"], x["out"], ws,
                                                     sel_counts=x["cnt"])
            elif v8:
                saga.saga_decode_step_fp8kv(dm, x["q"][t], x["K8"], x["ks"], x["V"], x["vs"],
                                            x["tau"], x["out"], ws, sel_counts=x["cnt"])
            elif t % w.refresh_n == 0:
                saga.atopn_refresh_decode_step_fp8k(dm, w.top_n, x["q"][t], x["K8"], x["ks"],
                                                    x["V"], x["tau"], x["out"], ws,
                                                    sel_counts=x["cnt"])
            else:
                saga.saga_decode_step_fp8k(dm, x["q"][t], x["K8"], x["ks"], x["V"], x["tau"],
                                           x["out"], ws, sel_counts=x["cnt"])
            if events is not None:
                events[li][1].record()

    for t in range(T):
        step(t)
    torch.cuda.synchronize()
    sel, launches = 0, []
    for t in range(T):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in layers]
        step(t, ev)
        torch.cuda.synchronize()
        for li, x in enumerate(layers):
            n_sel = int(x["cnt"].sum().item())
            sel += n_sel
            if t % w.refresh_n:
                launches.append((ev[li][0].elapsed_time(ev[li][1]),
                                 decode_algorithmic_bytes(w, L + t, n_sel, k_bytes=1,
                                                          v_bytes=1 if v8 else 2)))
    graphs = []
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for t in range(T):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                step(t)
            graphs.append(g)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    log(f"timing {args.steps} fp8 steps after {args.warmup} warmup steps")
    sec, _ = time_graphs(torch, graphs, args.steps, args.warmup)
    vb = 1 if v8 else 2
    step_bytes = sum(decode_algorithmic_bytes(w, L + t, 0, k_bytes=1, v_bytes=vb)
                     for t in range(T)) * w.layers / T + sel * w.head_dim * vb / T
    call_ms = sum(ms for ms, _ in launches) / len(launches)
    call_gbs = sum(b for _, b in launches) / len(launches) / (call_ms / 1e3) / 1e9
    return dict(sec=sec, step_bytes=step_bytes, call_ms=call_ms, call_gbs=call_gbs)


def run_gqa(torch, saga, wl, w, hkv, args):
    return run_full(torch, saga, wl, w.gqa(hkv), args) | {"hkv": hkv}


def run_full(torch, saga, wl, g, args):
    """Dense attention (saga_full_attention) over every layer of workload g."""
    T, L = g.steps, g.L
    layers = []
    log(f"generating {g.name}: h_k={g.h_k}, h_v={g.h_v} ({g.kv_bytes() / 1e9:.1f} GB)")
    for layer in range(g.layers):
        K, V, q = layer_inputs(torch, wl, g, layer)
        log(f"  layer {layer} ready")
        layers.append(dict(K=K, V=V, q=q, out=torch.empty(g.batch, g.h_q, g.head_dim_v or g.head_dim,
                                                          dtype=torch.bfloat16, device="cuda")))
    d0 = saga.dims(g.batch, g.h_q, g.h_k, g.h_v, g.head_dim, L, g.rows, g.scale,
                   head_dim_v=g.head_dim_v)
    ws = saga.alloc_workspace(d0, 1)

    def step(t):
        dm = saga.dims(g.batch, g.h_q, g.h_k, g.h_v, g.head_dim, L + t, g.rows, g.scale,
                       head_dim_v=g.head_dim_v)
        for x in layers:
            saga.saga_full_attention(dm, x["q"][t], x["K"], x["V"], x["out"], ws)

    for t in range(T):
        step(t)
    torch.cuda.synchronize()
    graphs = []
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for t in range(T):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=s):
                step(t)
            graphs.append(gr)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    sec, _ = time_graphs(torch, graphs, args.steps, args.warmup)
    per_step_bytes = sum(full_algorithmic_bytes(g, L + (k % T)) for k in range(args.steps))
    per_step_bytes *= g.layers / args.steps
    del layers, graphs
    torch.cuda.empty_cache()
    return dict(sec=sec, bytes_per_step=per_step_bytes)


def cpu_baseline(torch, wl, w, layers, n_layers=2):
    """The fp64 oracle on a bounded sample of the same workload: the whole
    decode run (all w.steps steps, refreshes every w.refresh_n) of the first
    n_layers layers, every batch row and query head; scaled to steps/s of all
    w.layers layers."""
    import oracle
    cores = oracle.max_threads()
    sample = layers[:n_layers]
    total = 0.0
    for x in sample:
        K, V, q = wl.bits(x["K"]), wl.bits(x["V"]), wl.bits(x["q"])
        t0 = time.perf_counter()
        oracle.atopn_run(q, K, V, [w.L + s for s in range(w.steps)], w.top_n, w.refresh_n)
        total += time.perf_counter() - t0
        del K, V, q
    per_layer_step = total / (len(sample) * w.steps)
    per_step = per_layer_step * w.layers
    return {"value": 1.0 / per_step, "unit": "steps/s", "cores": cores, "kind": "oracle",
            "sample": (f"layers 0-{len(sample) - 1} of {w.name}: the full run of {w.steps} decode "
                       f"steps (exact refresh every {w.refresh_n}) over all {w.batch}x{w.h_q} "
                       f"(batch row, query head) pairs, {total:.1f} s; scaled to {w.layers} "
                       f"layers per step"),
            "sample_seconds": round(total, 2)}


def atopn_recall(wl, w, layer_x, b=0):
    """Informational: how much of the exact top-N set the Atop-N selection
    keeps at each step (stale thresholds between refreshes), from the oracle
    on layer 0, batch row b, every query head, the whole decode run."""
    import numpy as np
    import oracle
    q = wl.bits(layer_x["q"][:, b:b + 1])
    K, V = wl.bits(layer_x["K"][b:b + 1]), wl.bits(layer_x["V"][b:b + 1])
    ctx = [w.L + s for s in range(w.steps)]
    r = oracle.atopn_run(q, K, V, ctx, w.top_n, w.refresh_n, want_sel=True, want_logits=True)
    rec = np.empty((w.steps, w.h_q))
    for t, n in enumerate(ctx):
        for i in range(w.h_q):
            s = r["logits"][t, 0, i, :n]
            top = np.argpartition(-s, w.top_n - 1)[:w.top_n]       # exact top-N (no ties)
            rec[t, i] = r["sel"][t, 0, i, top].mean()
    refresh = [t for t in range(w.steps) if t % w.refresh_n == 0]
    stale = [t for t in range(w.steps) if t % w.refresh_n]
    return {"mean": round(float(rec.mean()), 5), "min": round(float(rec.min()), 5),
            "at_refresh_steps": round(float(rec[refresh].mean()), 5),
            "between_refreshes": round(float(rec[stale].mean()), 5) if stale else None,
            "mean_selected_per_head": round(float(r["count"].mean()), 1),
            "sample": f"oracle, layer 0 of {w.name}, batch row {b}, all {w.h_q} query heads, "
                      f"{w.steps} steps"}


def torch_rates(torch):
    """Streaming rates of torch's own device kernels (copy_, sum) over 2 GiB,
    measured in the same run: a reference point next to the 8 TB/s spec peak,
    not a ceiling (torch's reduction reads slower than the library's K stream)."""
    n = 1 << 29                                         # fp32 elements: 2 GiB
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)

    def rate(fn, bytes_per_call, reps=10):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return bytes_per_call * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9

    copy = rate(lambda: b.copy_(a), 2 * 4 * n)
    read = rate(lambda: a.sum(), 4 * n)
    del a, b
    torch.cuda.empty_cache()
    return {"copy_gbs": round(copy, 1), "sum_gbs": round(read, 1),
            "how": "torch copy_ (bytes read + written) and sum (bytes read) over 2 GiB fp32"}


MALL_BYTES = 256 << 20


def sweep(torch, saga, wl, args):
    """Per point: enough layers that one step streams >= 4x the 256 MB Infinity
    Cache (capped at the family's layer count), 64 timed steps (two 32-token
    runs) after 8 warmup; reports per-layer latency of both paths."""
    fam_hkv = {"llama": 8, "qwen": 2}
    args.steps, args.warmup, args.eager_only = 64, 8, False
    for w0 in wl.sweep():
        fam = "llama" if "llama" in w0.name else "qwen"
        per_layer = w0.batch * (w0.h_k + w0.h_v) * w0.rows * w0.head_dim * 2
        layers = max(2, min(w0.layers, -(-4 * MALL_BYTES // per_layer)))
        w = w0.with_(layers=layers)
        res = run_saga(torch, saga, wl, w, args)
        sec = res["sec"]
        step_bytes = sum(x[3] for x in res["launches"] + res["refreshes"]) / w.steps
        del res
        torch.cuda.empty_cache()
        gq = run_gqa(torch, saga, wl, w, fam_hkv[fam], args)
        torch.cuda.empty_cache()
        saga_ms = 1e3 * sec / args.steps / layers
        gqa_ms = 1e3 * gq["sec"] / args.steps / layers
        print(json.dumps({
            "point": w0.name, "family": fam, "L": w0.L, "top_n": w0.top_n, "batch": w0.batch,
            "layers_timed": layers, "saga_atopn_ms_per_layer": round(saga_ms, 4),
            "gqa_full_ms_per_layer": round(gqa_ms, 4), "speedup": round(gqa_ms / saga_ms, 3),
            "saga_hbm_gbs": round(step_bytes / layers / (saga_ms * 1e-3) / 1e9, 1),
            "gqa_hbm_gbs": round(gq["bytes_per_step"] / layers / (gqa_ms * 1e-3) / 1e9, 1),
            "cache_resident": per_layer * layers < 2 * MALL_BYTES}), flush=True)


def decompose(torch, saga, wl, args):
    """The pages' decomposition of the speedup on one shape: full-attention GQA,
    SAGA full attention (merged key heads, no sparsity), Atop-N at the GQA head
    counts (sparsity, no merging) and SAGA + Atop-N, each on its own seeded
    inputs, per layer and step (refresh steps included)."""
    w0 = wl.WORKLOADS[args.workload]
    hkv = GQA_TWIN[w0.name]
    per_layer = w0.batch * (w0.h_k + w0.h_v) * w0.rows * w0.head_dim * 2
    layers = max(2, min(w0.layers, -(-4 * MALL_BYTES // per_layer)))
    w = w0.with_(layers=layers)
    args.eager_only = False
    rows = []
    for label, kind, x in (("GQA full attention", "full", w.gqa(hkv)),
                           ("SAGA full attention (merging alone)", "full", w),
                           ("Atop-N at GQA heads (sparsity alone)", "atopn", w.gqa(hkv)),
                           ("SAGA + Atop-N", "atopn", w)):
        if kind == "full":
            res = run_full(torch, saga, wl, x, args)
        else:
            res = run_saga(torch, saga, wl, x, args)
            del res["graphs"], res["layers"]
        torch.cuda.empty_cache()
        ms = 1e3 * res["sec"] / args.steps / layers
        rows.append((label, x, ms))
    base = rows[0][2]
    for label, x, ms in rows:
        print(json.dumps({"decomposition": label, "workload": w0.name, "h_k": x.h_k, "h_v": x.h_v,
                          "top_n": x.top_n if "Atop-N" in label else None,
                          "layers_timed": layers, "ms_per_layer": round(ms, 4),
                          "speedup_vs_gqa_full": round(base / ms, 3)}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the pages evaluate on one GPU; sharding is a design note only).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import sparse_decode_attention_atop_amd as saga
    import saga_workload as wl

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    saga.library()          # fail loudly now if the HIP library is missing
    if args.calibrate:
        calibrate(torch)
        return
    if args.sweep:
        sweep(torch, saga, wl, args)
        return
    if args.decompose:
        decompose(torch, saga, wl, args)
        return
    if args.lq:
        w = wl.WORKLOADS[args.workload]
        res = run_saga_lq(torch, saga, wl, w, args)
        sps = args.steps / res["sec"]
        gbs = res["step_bytes"] / (res["sec"] / args.steps) / 1e9
        print(json.dumps({"metric": "decode-attn steps/s, several query tokens per step",
                          "value": round(sps, 3), "unit": "steps/s",
                          "tokens_per_s": round(sps * w.batch * args.lq, 2),
                          "ms_per_step": round(1e3 * res["sec"] / args.steps, 4),
                          "steps": args.steps, "warmup": args.warmup,
                          "hbm_gbs_step": round(gbs, 1), "hbm_frac_step": round(gbs / HBM_PEAK_GBS, 4),
                          "config": {"workload": w.name, "l_q": args.lq}}), flush=True)
        return
    if args.fp8k or args.fp8kv:
        w = wl.WORKLOADS[args.workload]
        res = run_saga_fp8k(torch, saga, wl, w, args, v8=args.fp8kv)
        sps = args.steps / res["sec"]
        gbs = res["step_bytes"] / (res["sec"] / args.steps) / 1e9
        kv = "fp8 K and V caches" if args.fp8kv else "an fp8 K cache"
        print(json.dumps({"metric": f"decode-attn steps/s with {kv}",
                          "value": round(sps, 3), "unit": "steps/s",
                          "ms_per_step": round(1e3 * res["sec"] / args.steps, 4),
                          "steps": args.steps, "warmup": args.warmup,
                          "dtype": "fp8e4m3 K, fp8e4m3 V" if args.fp8kv else "fp8e4m3 K, bf16 V",
                          "hbm_gbs_step": round(gbs, 1), "hbm_frac_step": round(gbs / HBM_PEAK_GBS, 4),
                          "decode_call_us_eager": round(1e3 * res["call_ms"], 2),
                          "decode_call_gbs_eager": round(res["call_gbs"], 1),
                          "config": {"workload": w.name, "k_cache": "fp8 e4m3, per-head scale",
                                     "v_cache": ("fp8 e4m3, per-head scale" if args.fp8kv
                                                 else "bf16")}}),
              flush=True)
        return
    if args.paged:
        w = wl.WORKLOADS[args.workload]
        res = run_saga_paged(torch, saga, wl, w, args)
        sps = args.steps / res["sec"]
        gbs = res["step_bytes"] / (res["sec"] / args.steps) / 1e9
        print(json.dumps({"metric": "decode-attn steps/s on paged caches", "value": round(sps, 3),
                          "unit": "steps/s", "ms_per_step": round(1e3 * res["sec"] / args.steps, 4),
                          "steps": args.steps, "warmup": args.warmup,
                          "hbm_gbs_step": round(gbs, 1), "hbm_frac_step": round(gbs / HBM_PEAK_GBS, 4),
                          "config": {"workload": w.name, "page_rows": args.paged,
                                     "varlen": bool(args.varlen), "ctx_lens_at_t0": res["ctx"]}}),
              flush=True)
        return
    w = wl.WORKLOADS[args.workload]
    if args.top_n:
        w = w.with_(name=f"{w.name}_n{args.top_n}", top_n=args.top_n)
    if args.sigma:
        # The pages' Sigma-style alternative: (2 h_k, d_k / 2) instead of (h_k, d_k), d_v kept.
        w = w.with_(name=w.name + "_sigma", h_k=2 * w.h_k, head_dim=w.head_dim // 2,
                    head_dim_v=w.head_dim)
    res = run_saga(torch, saga, wl, w, args)
    if res is None:
        return
    T = w.steps
    sec = res["sec"]
    steps_per_s = args.steps / sec
    ms_per_step = 1e3 * sec / args.steps

    launches = res["launches"] or res["refreshes"]    # n = 1: every step refreshes
    eager_ms = sum(x[2] for x in launches) / len(launches)
    avg_ms = res["graph_call_ms"] or eager_ms
    avg_bytes = sum(x[3] for x in launches) / len(launches)
    achieved = avg_bytes / (avg_ms * 1e-3) / 1e9
    avg_sel = sum(x[4] for x in launches) / len(launches) / (w.batch * w.h_q)
    refreshes = res["refreshes"]
    step_bytes = (sum(x[3] for x in launches) + sum(x[3] for x in refreshes)) / T
    ref_ms = sum(x[2] for x in refreshes) / len(refreshes)
    traffic = measured_traffic(args.traffic or os.path.join(ROOT, "profiles",
                                                            f"traffic_{w.name}.md"), w.name)

    extra = {}
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(torch, wl, w, res["layers"])
        log("Atop-N recall against exact top-N (oracle, informational)")
        extra["atopn_recall"] = atopn_recall(wl, w, res["layers"][0])
    if not args.no_gqa and w.name in GQA_TWIN:
        del res["graphs"]
        for x in res["layers"]:
            x.clear()
        res["layers"] = None
        torch.cuda.empty_cache()
        gq = run_gqa(torch, saga, wl, w, GQA_TWIN[w.name], args)
        gqa_sps = args.steps / gq["sec"]
        extra["gqa_full_attention"] = {
            "h_kv": gq["hkv"], "steps_per_s": round(gqa_sps, 3),
            "ms_per_step": round(1e3 * gq["sec"] / args.steps, 4),
            "hbm_gbs_algorithmic": round(gq["bytes_per_step"] / (gq["sec"] / args.steps) / 1e9, 1)}
        extra["speedup_vs_gqa_full"] = round(steps_per_s / gqa_sps, 3)
    extra["torch_reference_rates"] = torch_rates(torch)

    line = {
        "metric": "decode-attn steps/s (B x layers) + HBM GB/s % peak, SAGA Atop-N @128K",
        "value": round(steps_per_s, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; shapes of the pages' Llama/Qwen decode setups, no weights)",
        "config": {"workload": w.name, "batch": w.batch, "h_q": w.h_q, "h_k": w.h_k,
                   "h_v": w.h_v, "head_dim": w.head_dim, "head_dim_v": w.head_dim_v or w.head_dim,
                   "L": w.L, "top_n": w.top_n,
                   "refresh_n": w.refresh_n, "decode_steps": w.steps, "layers": w.layers},
        "tokens_per_s": round(steps_per_s * w.batch, 2),
        "hbm_gbs_step": round(step_bytes / (sec / args.steps) / 1e9, 1),
        "hbm_frac_step": round(step_bytes / (sec / args.steps) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm",
                     "kernel": "saga_decode_step (one plain call: K stream, selection, value gather, combine)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "avg_launch_ms": round(avg_ms, 5),
                     "timed_as": ("graph replays of the plain decode steps"
                                  if res["graph_call_ms"] else "eager calls"),
                     "eager_call_ms": round(eager_ms, 5),
                     "algorithmic_bytes_per_launch": int(avg_bytes),
                     "mean_selected_per_head": round(avg_sel, 1)},
        "refresh_step": {"call": "atopn_refresh_decode_step", "avg_call_ms": round(ref_ms, 5),
                         "calls_per_step": round(len(refreshes) / T, 3)},
        "cpu_baseline": cpu,
    }
    line.update(extra)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
