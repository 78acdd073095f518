"""Summaries of rocprofv3 output for the profiles kept with the library.

    python -m sparse_decode_attention_atop_amd.profsum trace DIR [TOP]
        per-kernel calls / total / average / min / max (us) from a
        ``rocprofv3 --kernel-trace --stats`` run (its *_results.db).

    python -m sparse_decode_attention_atop_amd.profsum traffic WORKLOAD FETCH_DIR WRITE_DIR \\
            CAL_FETCH_DIR CAL_WRITE_DIR
        HBM bytes per plain decode call (stream + gather + combine) from
        ``rocprofv3 --pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs written as CSV,
        each scaled by what the same counter reads on the plain 4 GiB device
        copy of ``bench.py --calibrate``; prints a markdown table and the JSON
        block that ``bench.py`` reads.

    python -m sparse_decode_attention_atop_amd.profsum sweep FILE
        the markdown table of a ``bench.py --sweep`` run (its JSON lines).

    python -m sparse_decode_attention_atop_amd.profsum util DIR
        MFMA and VALU use per kernel of a plain decode call from a
        ``rocprofv3 --pmc MfmaUtil VALUBusy MfmaFlopsBF16`` run written as CSV
        (rocprofv3's own derived counters, one value per dispatch).

Launches are classified by order: a stream-select launch right after the
pivot kernel is a refresh step's candidate pass, one right after the final
select is its repair pass, any other starts a plain decode call; a gather and
combine belong to the stream launch before them.
"""
from __future__ import annotations

import csv
import glob
import json
import os
import re
import sqlite3
import sys

# This library's kernels (not torch's vectorized_gather_kernel and the like).
OURS = re.compile(r"(?<![A-Za-z_])(select_stream|gather_kernel|combine_kernel|refresh_final|"
                  r"pivot_kernel|sample_logits|full_attn|fill_u32)")


def short(name: str) -> str:
    n = name.replace("saga::(anonymous namespace)::", "").replace("void ", "")
    n = re.sub(r"\((saga::)?\w+Args\)|\(saga::Partials.*\)", "", n)
    return n[:60]


def trace(d: str, top: int = 25) -> str:
    dbs = glob.glob(os.path.join(d, "**", "*_results.db"), recursive=True)
    if not dbs:
        raise SystemExit(f"no *_results.db under {d}")
    rows = sqlite3.connect(dbs[0]).execute(
        "select name, count(*), sum(duration), avg(duration), min(duration), max(duration) "
        "from kernels group by name order by sum(duration) desc").fetchall()
    tot = sum(r[2] for r in rows)
    out = [f"| kernel | calls | total (us) | avg (us) | min (us) | max (us) | % |",
           "|---|---|---|---|---|---|---|"]
    for n, k, s, a, mn, mx in rows[:top]:
        out.append(f"| `{short(n)}` | {k} | {s / 1e3:.1f} | {a / 1e3:.2f} | {mn / 1e3:.2f} | "
                   f"{mx / 1e3:.2f} | {100 * s / tot:.2f} |")
    return "\n".join(out)


def _counter(d: str, name: str):
    """{dispatch_id: (kernel, value summed over dimensions)} for one counter."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter CSV under {d}")
    acc = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != name:
                continue
            key = int(r["Dispatch_Id"])
            k, v = acc.get(key, (r["Kernel_Name"], 0.0))
            acc[key] = (k, v + float(r["Counter_Value"]))
    return acc


def _calibration(d: str, name: str) -> float:
    """Counter reading (KiB) of the largest dispatch of a calibration run."""
    vals = [v for _, v in _counter(d, name).values()]
    return max(vals)


def _decode_calls(disp):
    """Group dispatches (sorted by id) into plain decode calls: a K stream, then
    a gather and a combine, or (the K stream gathering in its tail) only a
    combine."""
    calls, cur, prev = [], None, ""
    for i in sorted(disp):
        k, v = disp[i]
        if not OURS.search(k):
            continue
        if "select_stream" in k:
            if "pivot_kernel" in prev or "refresh_final" in prev:
                cur = None                                  # part of a refresh step
            else:
                cur = {"select_stream": v}
                calls.append(cur)
        elif cur is not None and ("gather_kernel" in k or "combine_kernel" in k):
            cur[k.split("<")[0].split("::")[-1].split()[-1]] = v
        prev = k
    return [c for c in calls if "combine_kernel" in c]


def traffic(workload, fdir, wdir, cfdir, cwdir):
    ff = 4.0 * 2 ** 20 / _calibration(cfdir, "FETCH_SIZE")     # 4 GiB read, KiB counter
    wf = 4.0 * 2 ** 20 / _calibration(cwdir, "WRITE_SIZE")
    fetch = _decode_calls(_counter(fdir, "FETCH_SIZE"))
    write = _decode_calls(_counter(wdir, "WRITE_SIZE"))
    n = min(len(fetch), len(write))
    kinds = [k for k in ("select_stream", "gather_kernel", "combine_kernel")
             if any(k in c for c in fetch[:n])]
    mean = lambda calls, k: sum(c.get(k, 0.0) for c in calls[:n]) / n * 1024.0
    lines = [f"Plain decode calls measured: {n}; scale factors fetch {ff:.4f}, write {wf:.4f}.", "",
             "| kernel | fetch raw (MiB) | fetch scaled (MiB) | write scaled (MiB) |",
             "|---|---|---|---|"]
    fb = wb = 0.0
    for k in kinds:
        fr, wr = mean(fetch, k), mean(write, k)
        fb += fr * ff
        wb += wr * wf
        lines.append(f"| `{k}` | {fr / 2**20:.1f} | {fr * ff / 2**20:.1f} | {wr * wf / 2**20:.2f} |")
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    blob = {"workload": workload, "kernel_sources": bench.kernel_sources_hash(),
            "bytes_per_call": int(fb + wb), "fetch_bytes_per_call": int(fb),
            "write_bytes_per_call": int(wb), "fetch_factor": round(ff, 4),
            "write_factor": round(wf, 4), "decode_calls": n}
    return "\n".join(lines) + "\n\n```json\n" + json.dumps(blob, indent=1) + "\n```\n"


def sweep(path):
    """Markdown table of bench.py --sweep's JSON lines (other lines skipped)."""
    pts = []
    for ln in open(path):
        ln = ln.strip()
        if ln.startswith("{") and '"point"' in ln:
            pts.append(json.loads(ln))
    out = ["| family | L | N | B | layers | saga (ms/layer) | gqa (ms/layer) | speedup | "
           "saga GB/s | gqa GB/s |", "|---|---|---|---|---|---|---|---|---|---|"]
    for p in pts:
        out.append(f"| {p['family']} | {p['L']} | {p['top_n']} | {p['batch']} | "
                   f"{p['layers_timed']} | {p['saga_atopn_ms_per_layer']:.4f} | "
                   f"{p['gqa_full_ms_per_layer']:.4f} | {p['speedup']:.2f} | "
                   f"{p['saga_hbm_gbs']:.0f} | {p['gqa_hbm_gbs']:.0f} |")
    return "\n".join(out)


def util(d):
    names = ["MfmaUtil", "VALUBusy", "MfmaFlopsBF16"]
    per = {nm: _decode_calls(_counter(d, nm)) for nm in names}
    n = min(len(c) for c in per.values())
    kinds = [k for k in ("select_stream", "gather_kernel", "combine_kernel")
             if any(k in c for c in per[names[0]][:n])]
    mean = lambda nm, k: sum(c.get(k, 0.0) for c in per[nm][:n]) / n
    lines = [f"Plain decode calls measured: {n}.", "",
             "| kernel | MFMA busy (% of SIMD cycles) | VALU busy (%) | bf16 MFMA GFLOP per launch |",
             "|---|---|---|---|"]
    for k in kinds:
        lines.append(f"| `{k}` | {mean('MfmaUtil', k):.2f} | {mean('VALUBusy', k):.2f} | "
                     f"{mean('MfmaFlopsBF16', k) / 1e9:.3f} |")
    return "\n".join(lines)


def main(argv):
    if len(argv) >= 2 and argv[0] == "trace":
        print(trace(argv[1], int(argv[2]) if len(argv) > 2 else 25))
    elif len(argv) == 6 and argv[0] == "traffic":
        print(traffic(*argv[1:]))
    elif len(argv) == 2 and argv[0] == "sweep":
        print(sweep(argv[1]))
    elif len(argv) == 2 and argv[0] == "util":
        print(util(argv[1]))
    else:
        print(__doc__, file=sys.stderr)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
