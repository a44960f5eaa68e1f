"""Build the gfx950 shared libraries in-tree with hipcc.

``libdspark.so`` is the verification library: every HIP source of the path
under ``csrc/`` in one hipcc invocation, its C ABI declared in
``include/dspark.h`` at the repository root.  ``libdspark_bench.so`` is the
benchmark's measurement library (``csrc/probe.hip``, C ABI in
``include/dspark_bench.h``); the verification library does not contain it."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ["api.hip", "schedule.hip", "verify.hip", "calib.hip", "markov.hip"]
LIB = os.path.join(HERE, "libdspark.so")
BENCH_SOURCES = ["probe.hip"]
BENCH_LIB = os.path.join(HERE, "libdspark_bench.so")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
    # exact control of rounding: no implicit contraction into FMA
    "-ffp-contract=off",
    # only the C ABI is exported
    "-fvisibility=hidden",
    # never emit packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False, out: str = LIB, defines=(), sources=SOURCES) -> str:
    """Compile ``sources`` (under csrc/) to ``out``; ``defines`` are extra -D
    tuning knobs."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    srcs = [os.path.join(HERE, "csrc", s) for s in sources]
    tmp = out + ".tmp"
    cmd = [hipcc, *FLAGS, *[f"-D{d}" for d in defines], "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(HERE, "csrc"), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


def build_all(verbose: bool = False) -> list:
    """Both libraries: the verification library and the benchmark's."""
    return [build(verbose=verbose),
            build(verbose=verbose, out=BENCH_LIB, sources=BENCH_SOURCES)]


if __name__ == "__main__":
    for p in build_all(verbose=True):
        print(p)
