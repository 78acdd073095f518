"""Plant plausible mistakes in the CPU oracle and check that a pin catches each.

Every mutant is a one-line textual change to ``oracle/oracle.c`` (a wrong
index, sign, head map, comparison, schedule or dropped term).  It is compiled
into a temporary library and the whole pin suite runs against it in a child
process; the test passes only if that run fails.  This shows the pins are
strong enough that the oracle cannot be subtly wrong and still pass them.
Runs on the CPU only.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, original text, mutated text) -- each original must occur exactly once.
MUTANTS = [
    ("key_operand_index", "elem_at(Kh, j * d + c);\n        s[j]",
     "elem_at(Kh, j * d + (d - 1 - c));\n        s[j]"),
    ("dropped_scale", "s[j] = scale * acc;", "s[j] = acc;"),
    ("key_head_map", "const kv_head Kh = head_of(K, b, hk, i / Gk, cache_len, d);\n"
     "        const kv_head Vh = head_of(V, b, hv, i / Gv, cache_len, dv);\n"
     "        double* s = (double*)malloc(sizeof(double) * (size_t)cache_len);",
     "const kv_head Kh = head_of(K, b, hk, i % hk, cache_len, d);\n"
     "        const kv_head Vh = head_of(V, b, hv, i / Gv, cache_len, dv);\n"
     "        double* s = (double*)malloc(sizeof(double) * (size_t)cache_len);"),
    ("value_head_map", "const kv_head Vh = head_of(V, b, hv, i / Gv, cache_len, dv);\n"
     "        double* s = (double*)malloc(sizeof(double) * (size_t)cache_len);",
     "const kv_head Vh = head_of(V, b, hv, i / Gk % hv, cache_len, dv);\n"
     "        double* s = (double*)malloc(sizeof(double) * (size_t)cache_len);"),
    ("value_head_stride_is_key_dim", "const kv_head Vh = head_of(V, b, hv, i / Gv, cache_len, dv);\n"
     "        double* s = (double*)malloc(sizeof(double) * (size_t)cache_len);",
     "const kv_head Vh = head_of(V, b, hv, i / Gv, cache_len, d);\n"
     "        double* s = (double*)malloc(sizeof(double) * (size_t)cache_len);"),
    ("output_stride_is_key_dim", "count[row] = attend_selected(s, S, n, &Vh, dv, out + row * dv);",
     "count[row] = attend_selected(s, S, n, &Vh, dv, out + row * d);"),
    ("threshold_rank_off_by_one", "double t = tmp[N - 1];", "double t = tmp[N];"),
    ("sort_ascending", "return (x < y) - (x > y);", "return (x > y) - (x < y);"),
    ("strict_comparison", "S[j] = (s[j] >= threshold);", "S[j] = (s[j] > threshold);"),
    ("refresh_phase", "if (t % refresh_n == 0) threshold", "if ((t + 1) % refresh_n == 0) threshold"),
    ("refresh_never", "if (t % refresh_n == 0) threshold", "if (t == 0) threshold"),
    ("softmax_sign", "double w = exp(s[j] - m);\n        denom += w;\n        for (int c = 0; c < dv; ++c) out[c]",
     "double w = exp(m - s[j]);\n        denom += w;\n        for (int c = 0; c < dv; ++c) out[c]"),
    ("dropped_normalisation", "for (int c = 0; c < dv; ++c) out[c] /= denom;\n    return count;",
     "for (int c = 0; c < dv; ++c) out[c] /= 1.0;\n    return count;"),
    ("value_row_index", "out[c] += w * elem_at(Vh, j * dv + c);\n    }\n    for (int c = 0; c < dv; ++c) out[c] /= denom;\n    return count;",
     "out[c] += w * elem_at(Vh, (ctx - 1 - j) * dv + c);\n    }\n    for (int c = 0; c < dv; ++c) out[c] /= denom;\n    return count;"),
    ("empty_selection_not_zero", "if (count == 0) return 0;", "if (count == 0) { out[0] = 1.0; return 0; }"),
    ("exact_topn_keeps_one_more", "const int64_t keep = top_n < ctx ? top_n : ctx;",
     "const int64_t keep = top_n < ctx ? top_n + 1 : ctx;"),
    ("e4m3_exponent_bias", "ldexp(1.0 + (double)m / 8.0, e - 7)", "ldexp(1.0 + (double)m / 8.0, e - 8)"),
    ("e4m3_subnormal_as_normal", "e == 0 ? ldexp((double)m / 8.0, -6)", "e == 0 ? ldexp(1.0 + (double)m / 8.0, -6)"),
    ("e4m3_no_nan", "if (e == 15 && m == 7) return NAN;", "if (e == 16) return NAN;"),
    ("e4m3_sign_dropped", "return sign ? -mag : mag;", "return mag;"),
    ("e4m3_scale_index", "r.scale = (double)kc->scale[(int64_t)b * H + h];",
     "r.scale = (double)kc->scale[h];"),
    ("e4m3_value_scale_is_key_scale",
     "vc = {NULL, V8, v_scale};\n    return atopn_run_impl",
     "vc = {NULL, V8, k_scale};\n    return atopn_run_impl"),
    ("e4m3_value_codes_read_as_bf16",
     "vc = {NULL, V8, v_scale};\n    return masked_impl",
     "vc = {(const uint16_t*)V8, NULL, NULL};\n    return masked_impl"),
    ("e4m3_scale_dropped", "if (k->e4m3) return k->scale * e4m3_to_double", "if (k->e4m3) return e4m3_to_double"),
    ("full_softmax_drops_max_row", "for (int64_t j = 0; j < ctx; ++j) if (s[j] > m) m = s[j];\n        double* o",
     "for (int64_t j = 0; j < ctx; ++j) if (s[j] > m) m = s[j];\n        s[0] = -INFINITY;\n        double* o"),
]


def _run_mutant(name, old, new, workdir):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutant {name}: anchor text not found exactly once"
    src = os.path.join(workdir, f"{name}.c")
    lib = os.path.join(workdir, f"lib{name}.so")
    with open(src, "w") as f:
        f.write(text.replace(old, new))
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", lib, src,
                    "-lm"], check=True)
    env = dict(os.environ, SAGA_ORACLE_LIBRARY=lib, OMP_NUM_THREADS="1")
    code = ("import sys; sys.path[:0] = [%r, %r]; import oracle_pins; oracle_pins.run_all()"
            % (ROOT, os.path.join(ROOT, "tests")))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=300)
    return r.returncode, (r.stderr or "")[-400:]


def test_every_planted_mistake_is_caught():
    with tempfile.TemporaryDirectory() as wd:
        with ThreadPoolExecutor(max_workers=4) as ex:
            futs = {m[0]: ex.submit(_run_mutant, *m, wd) for m in MUTANTS}
            survivors = [name for name, f in futs.items() if f.result()[0] == 0]
    assert not survivors, f"mutants not caught by any pin: {survivors}"


def test_unmutated_oracle_passes_in_child():
    """Control: the same child-process harness passes on the real oracle."""
    code = ("import sys; sys.path[:0] = [%r, %r]; import oracle_pins; oracle_pins.run_all()"
            % (ROOT, os.path.join(ROOT, "tests")))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-800:]
