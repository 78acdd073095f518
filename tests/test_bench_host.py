"""Host-side parts of bench.py (no GPU): the one-GPU refusal and the rule that
a committed HBM-traffic figure is reported only for its own workload and only
while the decode kernels' sources are the ones it was measured on."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""                      # no JSON line


def write_summary(path, **blob):
    path.write_text("# summary\n\n```json\n" + json.dumps(blob) + "\n```\n")
    return str(path)


def test_traffic_for_the_current_sources_and_workload(tmp_path):
    p = write_summary(tmp_path / "t.md", workload="w", kernel_sources=bench.kernel_sources_hash(),
                      bytes_per_call=1234)
    assert bench.measured_traffic(p, "w") == 1234


def test_traffic_is_withheld_when_stale_or_for_another_workload(tmp_path):
    h = bench.kernel_sources_hash()
    stale = write_summary(tmp_path / "s.md", workload="w", kernel_sources="0" * 16,
                          bytes_per_call=1)
    other = write_summary(tmp_path / "o.md", workload="other", kernel_sources=h, bytes_per_call=1)
    assert bench.measured_traffic(stale, "w") is None
    assert bench.measured_traffic(other, "w") is None
    assert bench.measured_traffic(str(tmp_path / "missing.md"), "w") is None
    (tmp_path / "bad.md").write_text("```json\n{not json\n```\n")
    assert bench.measured_traffic(str(tmp_path / "bad.md"), "w") is None

