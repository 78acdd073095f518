"""Pins that tie the CPU oracle to something other than itself.

Each ``pin_*`` function raises ``AssertionError`` when the oracle disagrees
with a fact fixed by the pages or by mathematics: a library routine it must
reduce to (torch's scaled-dot-product attention, matmul, topk, softmax), a
closed form, an invariant, or brute force on tiny inputs.  They are called by
``test_oracle_pins.py`` and, against deliberately broken builds of the oracle,
by ``test_oracle_mutants.py`` (every planted mistake must trip at least one).

Sources: "More Value per Key: Asymmetric Sparse Attention for Faster LLM
Decoding" -- ai.info AI summary (Key Contributions 2 and 3, Main Findings,
Methodology, Why This Matters: combinable with cache quantization) and
atlas.scime.ai AI summary (Approach, Experimental setup: exact top-N and
full-attention GQA are listed baselines); the OCP 8-bit floating point
specification for the E4M3 key-cache format.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ------------------------------------------------------------------ inputs
def rand_case(seed, B, hq, hk, hv, d, rows, T=1, scale=1.0):
    """Random bf16 q/K/V (as uint16 bits) with continuous values (ties improbable)."""
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn(T, B, hq, d, generator=g) * scale).to(torch.bfloat16)
    K = torch.randn(B, hk, rows, d, generator=g).to(torch.bfloat16)
    V = torch.randn(B, hv, rows, d, generator=g).to(torch.bfloat16)
    u = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return u(q), u(K), u(V)


def f64(bits):
    """uint16 bf16 bits -> float64 torch tensor (exact)."""
    a = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return torch.from_numpy(a.view(np.float32).astype(np.float64))


def to_bits(x: torch.Tensor):
    return x.to(torch.bfloat16).contiguous().view(torch.int16).numpy().view(np.uint16)


def sdpa_ref(q, K, V, ctx, scale, mask=None):
    """Library attention (float64) with contiguous head grouping made explicit.

    q [B][hq][d], K [B][hk][rows][d], V [B][hv][rows][d]; mask [B][hq][ctx] bool.
    """
    qt, Kt, Vt = f64(q), f64(K)[:, :, :ctx], f64(V)[:, :, :ctx]
    hq, hk, hv = qt.shape[1], Kt.shape[1], Vt.shape[1]
    Kt = Kt.repeat_interleave(hq // hk, dim=1)
    Vt = Vt.repeat_interleave(hq // hv, dim=1)
    am = None if mask is None else torch.as_tensor(mask)[:, :, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(
        qt[:, :, None, :], Kt, Vt, attn_mask=am, scale=scale)
    return o[:, :, 0, :].numpy()


def lib_logits(q, K, ctx, scale):
    """Logits by torch float64 matmul (head map repeat_interleave)."""
    qt, Kt = f64(q), f64(K)[:, :, :ctx]
    Kt = Kt.repeat_interleave(qt.shape[1] // Kt.shape[1], dim=1)
    return (scale * torch.matmul(Kt, qt[..., None])[..., 0]).numpy()


def topk_mask(s, N):
    """Boolean top-N mask per row via torch.topk (library)."""
    st = torch.from_numpy(np.ascontiguousarray(s))
    k = min(N, st.shape[-1])
    idx = torch.topk(st, k, dim=-1).indices
    m = torch.zeros_like(st, dtype=torch.bool)
    m.scatter_(-1, idx, True)
    return m.numpy()


def count_rule_selection(s, N):
    """Brute-force selection: keep j iff fewer than N entries are strictly larger.

    Equivalent to s_j >= (N-th largest) with ties kept, but computed by
    pairwise counting, with no sort and no threshold.
    """
    s = np.asarray(s)
    greater = (s[None, :] > s[:, None]).sum(axis=1)
    return greater < N


def rand_case_dkdv(seed, B, hq, hk, hv, dk, dv, rows, T=1):
    """Random bf16 q/K/V bits with key dimension dk and value dimension dv."""
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(T, B, hq, dk, generator=g).to(torch.bfloat16)
    K = torch.randn(B, hk, rows, dk, generator=g).to(torch.bfloat16)
    V = torch.randn(B, hv, rows, dv, generator=g).to(torch.bfloat16)
    u = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return u(q), u(K), u(V)


def mask_bitmap(mask, rows):
    """bool [..][ctx] -> uint32 [..][ceil(rows/32)], bit j%32 of word j/32 = mask[j]."""
    words = (rows + 31) // 32
    full = np.zeros(mask.shape[:-1] + (words * 32,), dtype=np.uint8)
    full[..., :mask.shape[-1]] = mask
    return np.packbits(full, axis=-1, bitorder="little").view(np.uint32)


def rand_e4m3(seed, B, hk, rows, d, pow2_scales):
    """Random E4M3 codes (never the NaN codes) and per-(b, key head) scales:
    distinct powers of two, or arbitrary positive values."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(B, hk, rows, d), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] ^= 0x01                       # 0x7F/0xFF -> 0x7E/0xFE
    if pow2_scales:
        ks = np.array([[2.0 ** (((b * hk + g) % 7) - 3) for g in range(hk)] for b in range(B)])
    else:
        ks = rng.uniform(0.01, 0.3, size=(B, hk))
    return codes, ks.astype(np.float32)


def lib_e4m3(codes):
    """float64 values of E4M3 codes via torch's float8_e4m3fn dtype (library)."""
    t = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def assert_close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0
    assert err <= tol, f"{what}: max abs diff {err:.3e} > {tol:.1e}"


# -------------------------------------------------------------------- pins
def pin_logits_vs_matmul():
    q, K, _ = rand_case(1, 2, 6, 2, 3, 32, 40)
    for scale in (1.0, 0.125):
        s = oracle.logits(q[0], K, 37, scale)
        assert_close(s, lib_logits(q[0], K, 37, scale), 1e-12, "logits vs matmul")


def pin_nth_largest_definition():
    rng = np.random.default_rng(7)
    for n, N in ((1, 1), (9, 3), (50, 50), (50, 51), (64, 1), (100, 37)):
        s = rng.standard_normal(n)
        t = oracle.nth_largest(s, N)
        if N >= n:
            assert t == -math.inf, "N >= n must give -inf"
            continue
        assert (s > t).sum() < N <= (s >= t).sum(), "N-th largest violates its definition"
    s = np.array([3.0, 1.0, 3.0, 2.0, 3.0, 0.0])           # ties at the top
    assert oracle.nth_largest(s, 2) == 3.0 and oracle.nth_largest(s, 4) == 2.0


def pin_exact_topn_vs_library():
    """Exact top-N = library attention restricted to torch.topk's set (SAGA maps)."""
    for (B, hq, hk, hv, d, rows, N) in ((2, 8, 2, 4, 16, 48, 5), (1, 6, 1, 2, 64, 70, 9)):
        q, K, V = rand_case(11 + hq, B, hq, hk, hv, d, rows)
        ctx = rows - 3
        o = oracle.exact_topn(q[0], K, V, ctx, N)
        m = topk_mask(lib_logits(q[0], K, ctx, 1.0), N)
        assert_close(o, sdpa_ref(q[0], K, V, ctx, 1.0, m), 1e-12, "exact top-N vs sdpa+topk")


def pin_refresh_every_step_is_exact_topn():
    """n = 1: Atop-N equals exact top-N attention at every step."""
    T = 5
    q, K, V = rand_case(21, 2, 8, 2, 4, 32, 60, T=T)
    ctx = [50 + t for t in range(T)]
    r = oracle.atopn_run(q, K, V, ctx, top_n=7, refresh_n=1)
    for t in range(T):
        assert_close(r["out"][t], oracle.exact_topn(q[t], K, V, ctx[t], 7), 1e-12,
                     f"n=1 step {t} vs exact top-N")
        assert (r["count"][t] == 7).all(), "exact thresholds must select exactly N"


def pin_full_when_n_covers_context():
    """N >= ctx: Atop-N is full attention (library sdpa; GQA via enable_gqa too)."""
    T = 3
    q, K, V = rand_case(31, 2, 8, 2, 4, 32, 40, T=T)
    ctx = [38, 39, 40]
    r = oracle.atopn_run(q, K, V, ctx, top_n=40, refresh_n=2)
    for t in range(T):
        ref = sdpa_ref(q[t], K, V, ctx[t], 1.0)
        assert_close(r["out"][t], ref, 1e-12, "N>=ctx vs sdpa")
        assert_close(oracle.full(q[t], K, V, ctx[t]), ref, 1e-12, "full vs sdpa")
        assert (r["count"][t] == ctx[t]).all() and np.isneginf(r["tau"][t]).all()
    # h_k == h_v: the library's own GQA expansion.
    q, K, V = rand_case(32, 1, 8, 2, 2, 16, 30)
    ref = torch.nn.functional.scaled_dot_product_attention(
        f64(q[0])[:, :, None, :], f64(K)[:, :, :30], f64(V)[:, :, :30], scale=1.0,
        enable_gqa=True)[:, :, 0, :].numpy()
    assert_close(oracle.full(q[0], K, V, 30), ref, 1e-12, "GQA full vs sdpa(enable_gqa)")
    r = oracle.atopn_run(q, K, V, [30], top_n=64, refresh_n=1)
    assert_close(r["out"][0], ref, 1e-12, "GQA Atop-N (N>=ctx) vs sdpa(enable_gqa)")


def pin_gqa_and_mha_special_cases():
    """h_k == h_v is standard GQA top-N; h_q == h_k == h_v is multi-head attention."""
    for (hq, hk, hv) in ((8, 2, 2), (4, 4, 4)):
        q, K, V = rand_case(41 + hk, 2, hq, hk, hv, 32, 64)
        s = lib_logits(q[0], K, 64, 1.0)
        m = topk_mask(s, 6)
        qt = f64(q[0])[:, :, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, f64(K), f64(V), attn_mask=torch.from_numpy(m)[:, :, None, :], scale=1.0,
            enable_gqa=(hq != hk))[:, :, 0, :].numpy()
        r = oracle.atopn_run(q, K, V, [64], top_n=6, refresh_n=3)
        assert_close(r["out"][0], ref, 1e-12, f"(hq,hk,hv)={(hq, hk, hv)} vs sdpa")


def pin_stale_threshold_schedule():
    """Refresh at t % n == 0; in between, S = {s >= tau of the last refresh}.

    tau is recomputed here by pairwise counting (no sort) on library logits,
    and each step's output must equal library attention over that set.
    """
    T, n, N = 10, 4, 5
    q, K, V = rand_case(51, 1, 4, 1, 2, 16, 48, T=T)
    ctx = [36 + t for t in range(T)]
    r = oracle.atopn_run(q, K, V, ctx, top_n=N, refresh_n=n, want_sel=True)
    tau = None
    for t in range(T):
        s = lib_logits(q[t], K, ctx[t], 1.0)[0]              # [hq][ctx]
        if t % n == 0:
            tau = np.array([s[i][count_rule_selection(s[i], N)].min() for i in range(4)])
        assert_close(r["tau"][t][0], tau, 1e-12, f"tau at step {t}")
        sel = s >= tau[:, None]
        assert (r["sel"][t][0][:, :ctx[t]] == sel).all(), f"selection at step {t}"
        assert (r["count"][t][0] == sel.sum(axis=1)).all()
        ref = sdpa_ref(q[t], K, V, ctx[t], 1.0, sel[None])
        assert_close(r["out"][t], ref, 1e-12, f"output at step {t}")


def pin_tiny_bruteforce_subsets():
    """Tiny rows: the selected set is the size-N subset with the largest logit sum."""
    for seed in range(6):
        q, K, V = rand_case(60 + seed, 1, 2, 1, 1, 8, 9)
        N = 1 + seed % 4
        r = oracle.atopn_run(q, K, V, [9], top_n=N, refresh_n=1, want_sel=True)
        s = lib_logits(q[0], K, 9, 1.0)[0]
        for i in range(2):
            best = max(itertools.combinations(range(9), N), key=lambda c: s[i][list(c)].sum())
            want = np.zeros(9, dtype=bool)
            want[list(best)] = True
            assert (r["sel"][0][0][i].astype(bool) == want).all(), "brute-force subset"


def pin_weights_sum_to_one():
    q, K, _ = rand_case(71, 1, 4, 1, 2, 16, 40, T=4)
    V = to_bits(torch.ones(1, 2, 40, 16))
    r = oracle.atopn_run(q, K, V, [30, 31, 32, 33], top_n=5, refresh_n=2)
    assert_close(r["out"], np.ones_like(r["out"]), 1e-14, "V = 1 must give 1")


def pin_identity_values_give_probabilities():
    """V rows = unit vectors (ctx <= d): out is the probability vector itself."""
    d, ctx, N = 32, 24, 6
    q, K, _ = rand_case(81, 1, 4, 2, 2, d, ctx)
    V = to_bits(torch.eye(d)[:ctx].expand(1, 2, ctx, d))
    r = oracle.atopn_run(q, K, V, [ctx], top_n=N, refresh_n=1)
    s = torch.from_numpy(lib_logits(q[0], K, ctx, 1.0))
    m = torch.from_numpy(topk_mask(s.numpy(), N))
    p = torch.softmax(s.masked_fill(~m, -math.inf), dim=-1).numpy()
    assert_close(r["out"][0][..., :ctx], p, 1e-12, "identity V")
    assert_close(r["out"][0][..., ctx:], 0.0, 0.0, "identity V tail")


def pin_single_selection_copies_row():
    """N = 1: the output is the value row of the arg-max logit, exactly."""
    q, K, V = rand_case(91, 2, 6, 3, 2, 16, 33)
    r = oracle.atopn_run(q, K, V, [33], top_n=1, refresh_n=1)
    s = torch.from_numpy(lib_logits(q[0], K, 33, 1.0))
    j = torch.argmax(s, dim=-1).numpy()
    Vf = f64(V).numpy()
    for b in range(2):
        for i in range(6):
            assert (r["out"][0][b][i] == Vf[b][i // 3][j[b][i]]).all(), "N=1 copies the row"


def pin_zero_keys_keep_all_ties():
    """K = 0: every logit ties at 0, tau = 0 and the whole context is kept (mean of V)."""
    q, _, V = rand_case(101, 1, 4, 1, 2, 16, 20)
    K = to_bits(torch.zeros(1, 1, 20, 16))
    r = oracle.atopn_run(q, K, V, [17], top_n=3, refresh_n=1)
    assert (r["count"][0] == 17).all() and (r["tau"][0] == 0.0).all()
    mean = f64(V)[:, :, :17].mean(dim=2).numpy()              # [1][hv][d]
    assert_close(r["out"][0], mean.repeat(2, axis=1), 1e-14, "uniform average")


def pin_masked_mode():
    """Caller-given masks: empty gives zeros, a topk mask gives library attention."""
    q, K, V = rand_case(111, 2, 8, 2, 4, 32, 50)
    words = (50 + 31) // 32
    out, cnt = oracle.masked(q[0], K, V, 45, np.zeros((2, 8, words), np.uint32))
    assert (out == 0).all() and (cnt == 0).all()
    m = topk_mask(lib_logits(q[0], K, 45, 1.0), 7)
    bm = np.zeros((2, 8, words), np.uint32)
    for j in range(45):
        bm[..., j // 32] |= (m[..., j].astype(np.uint32) << np.uint32(j % 32))
    out, cnt = oracle.masked(q[0], K, V, 45, bm)
    assert (cnt == 7).all()
    assert_close(out, sdpa_ref(q[0], K, V, 45, 1.0, m), 1e-12, "masked vs sdpa")


def pin_golden_hand_worked():
    """Hand-worked two-step example with closed-form outputs (tests/golden)."""
    with open(os.path.join(GOLDEN, "hand_worked_atopn.json")) as f:
        g = json.load(f)
    q = to_bits(torch.tensor(g["q"], dtype=torch.float32))
    K = to_bits(torch.tensor(g["K"], dtype=torch.float32))
    V = to_bits(torch.tensor(g["V"], dtype=torch.float32))
    r = oracle.atopn_run(q, K, V, g["ctx"], top_n=g["top_n"], refresh_n=g["refresh_n"],
                         scale=g["scale"], want_sel=True)
    for t, step in enumerate(g["expect"]):
        assert_close(r["out"][t][0], step["out"], 1e-12, f"golden out step {t}")
        assert_close(r["tau"][t][0], step["tau"], 0.0, f"golden tau step {t}")
        sel = r["sel"][t][0][:, :g["ctx"][t]].astype(int).tolist()
        assert sel == step["sel"], f"golden selection step {t}"


def pin_e4m3_decode_vs_library_and_format():
    codes = np.arange(256, dtype=np.uint8)
    got, lib = oracle.e4m3_decode(codes), lib_e4m3(codes)
    nan = np.isnan(got)
    assert nan.tolist() == np.isnan(lib).tolist(), "E4M3 NaN codes"
    assert sorted(np.flatnonzero(nan).tolist()) == [0x7F, 0xFF], "E4M3 has exactly two NaNs"
    assert np.array_equal(got[~nan], lib[~nan]), "E4M3 decode vs torch float8_e4m3fn"
    # Landmarks of the format: largest normal, smallest normal and subnormal, one, signed zero.
    marks = {0x7E: 448.0, 0xFE: -448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9,
             0x38: 1.0, 0x3C: 1.5, 0x00: 0.0}
    for c, v in marks.items():
        assert got[c] == v, f"E4M3 code {c:#04x}"
    assert math.copysign(1.0, got[0x80]) == -1.0 and got[0x80] == 0.0, "E4M3 negative zero"


def pin_e4m3k_logits_vs_matmul():
    """Logits with an E4M3 key cache = float64 matmul against scale * decode."""
    B, hq, hk, d, rows, ctx = 2, 8, 2, 32, 50, 47
    q, _, _ = rand_case(31, B, hq, hk, hk, d, rows)
    K8, ks = rand_e4m3(32, B, hk, rows, d, pow2_scales=False)
    Kf = torch.from_numpy(lib_e4m3(K8) * ks.astype(np.float64)[:, :, None, None])[:, :, :ctx]
    qt = f64(q[0])
    ref = torch.matmul(Kf.repeat_interleave(hq // hk, dim=1), qt[..., None])[..., 0] * 0.25
    got = oracle.logits_e4m3k(q[0], K8, ks, ctx, 0.25)
    assert_close(got / np.abs(ref.numpy()).max(), ref.numpy() / np.abs(ref.numpy()).max(),
                 1e-13, "E4M3 logits vs matmul")


def pin_e4m3k_reduces_to_bf16_cache():
    """Power-of-two scales make scale * decode(code) exact in bf16: the E4M3
    runs must then equal the bf16 runs on those values, bit for bit."""
    T, B, hq, hk, hv, d, rows = 4, 2, 8, 2, 4, 32, 70
    q, _, V = rand_case(33, B, hq, hk, hv, d, rows, T=T)
    K8, ks = rand_e4m3(34, B, hk, rows, d, pow2_scales=True)
    Kb = to_bits(torch.from_numpy(lib_e4m3(K8) * ks.astype(np.float64)[:, :, None, None]))
    assert np.array_equal(f64(Kb).numpy(), lib_e4m3(K8) * ks[:, :, None, None]), "not exact"
    ctx = [60 + t for t in range(T)]
    a = oracle.atopn_run_e4m3k(q, K8, ks, V, ctx, 9, 2, 0.5, want_sel=True, want_logits=True)
    b = oracle.atopn_run(q, Kb, V, ctx, 9, 2, 0.5, want_sel=True, want_logits=True)
    for k in ("out", "tau", "count", "sel", "logits"):
        assert np.array_equal(a[k], b[k]), f"E4M3 run differs from bf16 run in {k}"
    bm = np.packbits(b["sel"][1].astype(np.uint8), axis=-1, bitorder="little")
    bm = np.pad(bm, ((0, 0), (0, 0), (0, (-bm.shape[-1]) % 4))).view(np.uint32)
    m8 = oracle.masked_e4m3k(q[1], K8, ks, V, ctx[1], bm, 0.5)
    mb = oracle.masked(q[1], Kb, V, ctx[1], bm, 0.5)
    assert np.array_equal(m8[0], mb[0]) and np.array_equal(m8[1], mb[1]), "E4M3 masked"
    assert np.array_equal(m8[1], b["count"][1]), "masked count vs run count"


def pin_e4m3kv_reduces_to_bf16_caches():
    """E4M3 key and value caches with power-of-two scales: every scale * decode(code)
    is exact in bf16, so the E4M3 K/V runs must equal the bf16 runs on the values
    that torch's float8_e4m3fn decode gives, bit for bit (separate V decoding path)."""
    T, B, hq, hk, hv, d, rows = 4, 2, 8, 2, 4, 32, 70
    q, _, _ = rand_case(35, B, hq, hk, hv, d, rows, T=T)
    K8, ks = rand_e4m3(36, B, hk, rows, d, pow2_scales=True)
    V8, vs = rand_e4m3(37, B, hv, rows, d, pow2_scales=True)
    deq = lambda c, sc: lib_e4m3(c) * sc.astype(np.float64)[:, :, None, None]
    Kb, Vb = to_bits(torch.from_numpy(deq(K8, ks))), to_bits(torch.from_numpy(deq(V8, vs)))
    assert np.array_equal(f64(Vb).numpy(), deq(V8, vs)), "not exact"
    ctx = [60 + t for t in range(T)]
    a = oracle.atopn_run_e4m3kv(q, K8, ks, V8, vs, ctx, 9, 2, 0.5, want_sel=True, want_logits=True)
    b = oracle.atopn_run(q, Kb, Vb, ctx, 9, 2, 0.5, want_sel=True, want_logits=True)
    for k in ("out", "tau", "count", "sel", "logits"):
        assert np.array_equal(a[k], b[k]), f"E4M3 K/V run differs from bf16 run in {k}"
    bm = mask_bitmap(b["sel"][1][..., :ctx[1]].astype(bool), rows)
    m8 = oracle.masked_e4m3kv(q[1], K8, ks, V8, vs, ctx[1], bm, 0.5)
    mb = oracle.masked(q[1], Kb, Vb, ctx[1], bm, 0.5)
    assert np.array_equal(m8[0], mb[0]) and np.array_equal(m8[1], mb[1]), "E4M3 K/V masked"


def pin_e4m3kv_full_vs_library_attention():
    """Arbitrary (not power-of-two) scales: with N covering the context the E4M3
    K/V run is full attention over v_scale * decode(code), equal to torch's
    scaled-dot-product attention on torch-decoded float64 caches."""
    B, hq, hk, hv, d, rows = 2, 8, 2, 4, 32, 50
    q, _, _ = rand_case(38, B, hq, hk, hv, d, rows, T=1)
    K8, ks = rand_e4m3(39, B, hk, rows, d, pow2_scales=False)
    V8, vs = rand_e4m3(40, B, hv, rows, d, pow2_scales=False)
    ctx = rows - 3
    Kt = torch.from_numpy(lib_e4m3(K8) * ks.astype(np.float64)[:, :, None, None])[:, :, :ctx]
    Vt = torch.from_numpy(lib_e4m3(V8) * vs.astype(np.float64)[:, :, None, None])[:, :, :ctx]
    want = torch.nn.functional.scaled_dot_product_attention(
        f64(q[0])[:, :, None, :], Kt.repeat_interleave(hq // hk, dim=1),
        Vt.repeat_interleave(hq // hv, dim=1), scale=0.25)[:, :, 0, :].numpy()
    r = oracle.atopn_run_e4m3kv(q, K8, ks, V8, vs, [ctx], rows, 1, 0.25)
    assert (r["count"][0] == ctx).all()
    assert_close(r["out"][0], want, 1e-12, "E4M3 K/V full attention vs torch")


def pin_key_and_value_dims_independent():
    """d_k != d_v (the pages' Sigma-style (h_k, d_k) = (2, 32) against d_v = 64, and
    the reverse): full, exact top-N, Atop-N at n = 1 and masked mode against torch's
    scaled-dot-product attention, which takes separate key and value dimensions."""
    for (B, hq, hk, hv, dk, dv, rows, N) in ((2, 8, 2, 4, 32, 64, 48, 6),
                                             (1, 6, 1, 2, 64, 16, 70, 9)):
        q, K, V = rand_case_dkdv(40 + dk, B, hq, hk, hv, dk, dv, rows, T=2)
        ctx = rows - 5
        full = oracle.full(q[0], K, V, ctx, 0.5)
        assert full.shape == (B, hq, dv)
        assert_close(full, sdpa_ref(q[0], K, V, ctx, 0.5), 1e-12, "full, d_k != d_v")
        m = topk_mask(lib_logits(q[0], K, ctx, 0.5), N)
        want = sdpa_ref(q[0], K, V, ctx, 0.5, m)
        assert_close(oracle.exact_topn(q[0], K, V, ctx, N, 0.5), want, 1e-12, "exact top-N, d_k != d_v")
        r = oracle.atopn_run(q, K, V, [ctx, ctx + 1], N, 1, 0.5, want_sel=True)
        assert_close(r["out"][0], want, 1e-12, "Atop-N n=1, d_k != d_v")
        m1 = topk_mask(lib_logits(q[1], K, ctx + 1, 0.5), N)
        assert_close(r["out"][1], sdpa_ref(q[1], K, V, ctx + 1, 0.5, m1), 1e-12, "step 1")
        o, cnt = oracle.masked(q[0], K, V, ctx, mask_bitmap(m, rows), 0.5)
        assert_close(o, want, 1e-12, "masked, d_k != d_v")
        assert (cnt == N).all()


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]


def run_all():
    for p in ALL_PINS:
        p()


if __name__ == "__main__":
    run_all()
    print("all pins hold")
