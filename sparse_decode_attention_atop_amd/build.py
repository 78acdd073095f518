"""Build libsaga.so (HIP, gfx950) in-tree with hipcc.

    python -m sparse_decode_attention_atop_amd.build

Each ``csrc/*.hip`` file is compiled to an object for gfx950 and the objects
are linked into ``sparse_decode_attention_atop_amd/libsaga.so``.  Only the
symbols declared in ``include/saga.h`` are exported.  The HBM measurement
kernels in ``probe/*.hip`` are linked into ``libsaga_probe.so`` (symbols of
``include/saga_probe.h``); the decode library does not use them.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsaga.so")
PROBE_LIB = os.path.join(PKG, "libsaga_probe.so")
PROBE_SRC = os.path.join(PKG, "probe")
BUILD_DIR = os.path.join(PKG, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-result",
    # Keep the compiler from forming packed fp32 instructions (v_pk_*_f32).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def sources(folder=CSRC):
    return sorted(glob.glob(os.path.join(folder, "*.hip")))


def _compile(src: str, extra=(), build_dir=BUILD_DIR) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    # The host pass does not know the gfx-only feature flag; that note is noise.
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in r.stderr.splitlines() if ln.strip() and noise not in ln]
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False, extra_flags=(), out: str = LIB) -> str:
    """Compile every HIP source and link libsaga.so; returns the library path.
    The default build also links libsaga_probe.so.

    ``extra_flags`` (e.g. ``-DSAGA_STREAM_U64=4``) and ``out`` build a variant
    with other tuning constants somewhere else."""
    build_dir = BUILD_DIR if out == LIB else out + ".objs"
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    probe_srcs = sources(PROBE_SRC) if out == LIB else []
    with ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(probe_srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, tuple(extra_flags), build_dir), srcs))
        probe_objs = list(ex.map(lambda s: _compile(s, (), build_dir), probe_srcs))
    _link(objs, out)
    if probe_objs:
        _link(probe_objs, PROBE_LIB)
    if verbose:
        print(f"built {out}" + (f" and {PROBE_LIB}" if probe_objs else ""))
    return out


if __name__ == "__main__":
    build(verbose=True)
