"""Build libnvfp4.so (the HIP kernels and the C ABI) in-tree for gfx950, and
the test-only conversion probe library (tests/gpu_probe/libnvfp4_probe.so).

Each source compiles to its own object in parallel (no device code crosses a
translation unit), then the objects link into the shared library.

Usage: python -m block_scaled_fp4_nibble_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libnvfp4.so")
SOURCES = ["api.hip", "quantize.hip", "gemm.hip", "gemv.hip", "combine.hip", "w4a4.hip"]
PROBE_SRC = os.path.join(ROOT, "tests", "gpu_probe", "conv_probe.hip")
PROBE_LIB = os.path.join(ROOT, "tests", "gpu_probe", "libnvfp4_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # every FP32 step is rounded on its own (the encoder must match the
    # definition bit for bit); no fused multiply-add contraction
    "-ffp-contract=off",
    # keep the compiler from forming packed FP32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

# the host pass does not know the packed-fp32 target feature and says so
_NOISE = "'-packed-fp32-ops' is not a recognized feature"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if _NOISE not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if msgs and verbose:
        print("\n".join(msgs))


def _link(objs, out, verbose):
    tmp = out + ".tmp%d" % os.getpid()
    try:
        _run([HIPCC] + FLAGS + ["-shared"] + objs + ["-o", tmp], verbose)
        os.replace(tmp, out)
    finally:
        if os.path.exists(tmp):
            os.remove(tmp)
    return out


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile libnvfp4.so and the test probe library; returns the former's path."""
    jobs = jobs or min(8, len(SOURCES) + 1)
    with tempfile.TemporaryDirectory(prefix="nvfp4_build_") as tmpdir:
        units = [(os.path.join(CSRC, s), os.path.join(tmpdir, s + ".o")) for s in SOURCES]
        probe_obj = os.path.join(tmpdir, "conv_probe.o")
        work = units + [(PROBE_SRC, probe_obj)]
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            futs = [ex.submit(_run, [HIPCC] + FLAGS + ["-c", src, "-o", obj], verbose)
                    for src, obj in work]
            for f in futs:
                f.result()
        _link([obj for _, obj in units], LIB, verbose)
        _link([probe_obj], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
