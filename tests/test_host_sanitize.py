"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The C-ABI host code (``csrc/api.hip``: argument validation, chunk plans,
  workspace layout, dispatch) is compiled for the CPU with both sanitizers and
  linked with ``host_check/launch_stubs.cpp``, which stands in for the kernel
  launchers and touches the extreme elements every kernel would index.
  ``host_check/abi_driver.cpp`` then calls every entry point on a table of
  shapes with exact-size host buffers, and walks the error paths.  Overruns of
  a buffer are sanitizer reports; overruns between regions of the one
  workspace allocation are caught by the region-overlap check.
* The fp64 oracle is built with both sanitizers and the whole pin suite runs
  against that build in a child process.
Planted mistakes (an undersized workspace region, an out-of-bounds write in
the oracle) must make each check fail, which shows the checks are live.
"""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_decode_attention_atop_amd", "csrc")
CHECK = os.path.join(ROOT, "tests", "host_check")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"
# Host-only compiles; the sanitizers apply to host code (there is no device code).
HOST_FLAGS = ["-x", "hip", "--offload-host-only", "-O1", "-g", "-fno-omit-frame-pointer",
              "-std=c++17", "-Xarch_host", "-fsanitize=address,undefined",
              "-Xarch_host", "-fno-sanitize-recover=undefined",
              f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")

needs_rocm = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                                reason="ROCm compilers not installed")


def _compile(src, obj):
    r = subprocess.run([HIPCC, *HOST_FLAGS, "-c", src, "-o", obj], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def _build_check(tmp, api_src):
    objs = []
    for name, src in (("api", api_src), ("stubs", os.path.join(CHECK, "launch_stubs.cpp")),
                      ("driver", os.path.join(CHECK, "abi_driver.cpp"))):
        obj = os.path.join(tmp, name + ".o")
        if not os.path.exists(obj) or name == "api":
            _compile(src, obj)
        objs.append(obj)
    exe = os.path.join(tmp, "abi_check")
    r = subprocess.run([CLANG, "-fsanitize=address,undefined", *objs, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


@needs_rocm
def test_abi_host_code_under_sanitizers(tmp_path):
    exe = _build_check(str(tmp_path), os.path.join(CSRC, "api.hip"))
    r = subprocess.run([exe, "--big"], capture_output=True, text=True, env=ENV, timeout=600)
    print(r.stderr[-3000:])
    assert r.returncode == 0, r.stderr[-5000:]
    assert re.search(r"\d+ checks, 0 failures", r.stderr)


# One-line mistakes in the workspace plan; each must fail the host check.
LAYOUT_MUTANTS = [
    ("list maxima region halved",
     "L.lmax = take(rows * L.max_chunks * kWavesPerBlock * 4);",
     "L.lmax = take(rows * L.max_chunks * kWavesPerBlock * 2);"),
    ("no slack for the last chunk's rounding",
     "L.entry_rows = d->cache_len + top_rows;", "L.entry_rows = d->cache_len;"),
    ("partials sized for one chunk", "L.pm = take(rows * L.max_chunks * 4);",
     "L.pm = take(rows * 4);"),
    ("sample region one row short", "L.sample = take(rows * kSampleMax * 4);",
     "L.sample = take((rows - 1) * kSampleMax * 4);"),
]


@needs_rocm
@pytest.mark.parametrize("name,old,new", LAYOUT_MUTANTS, ids=[m[0] for m in LAYOUT_MUTANTS])
def test_planted_layout_mistake_is_caught(tmp_path, name, old, new):
    src = open(os.path.join(CSRC, "api.hip")).read()
    assert src.count(old) == 1, f"mutant anchor not found: {old}"
    mut = os.path.join(str(tmp_path), "api_mutant.hip")
    with open(mut, "w") as f:
        f.write(src.replace(old, new))
    exe = _build_check(str(tmp_path), mut)
    r = subprocess.run([exe, "--big"], capture_output=True, text=True, env=ENV, timeout=600)
    assert r.returncode != 0, f"planted mistake not caught: {name}"


def _sanitized_oracle(tmp, src):
    lib = os.path.join(tmp, "liboracle_asan.so")
    r = subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer",
                        "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                        "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-o", lib, src, "-lm"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return lib


def _libasan():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = os.path.realpath(r.stdout.strip())
    return path if os.path.exists(path) else None


def _run_pins(lib):
    env = dict(ENV, LD_PRELOAD=_libasan(), SAGA_ORACLE_LIBRARY=lib)
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                          capture_output=True, text=True, env=env, cwd=ROOT, timeout=900)


@pytest.mark.skipif(shutil.which("gcc") is None or _libasan() is None,
                    reason="gcc's AddressSanitizer runtime not installed")
def test_oracle_pins_under_sanitizers(tmp_path):
    lib = _sanitized_oracle(str(tmp_path), os.path.join(ROOT, "oracle", "oracle.c"))
    r = _run_pins(lib)
    assert r.returncode == 0, (r.stdout + r.stderr)[-5000:]
    assert "passed" in r.stdout

    # A planted out-of-bounds write (one element past the threshold sort's
    # scratch array) must be reported.
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    anchor = "double t = tmp[N - 1];"
    assert src.count(anchor) == 1
    bad = os.path.join(str(tmp_path), "oracle_oob.c")
    with open(bad, "w") as f:
        f.write(src.replace(anchor, "tmp[n] = 0.0;\n    " + anchor))
    r = _run_pins(_sanitized_oracle(str(tmp_path), bad))
    assert r.returncode != 0 and "AddressSanitizer" in (r.stdout + r.stderr)
