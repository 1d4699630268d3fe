"""Build libw4a8.so (the C ABI library) in-tree for gfx950.

    python w4a8_gemm_amd/build.py

HIP sources are compiled by hipcc for gfx950 only; the host packer is plain
C++ compiled by g++ with -ffp-contract=off so that every fp32 step of the
quantization is a single IEEE operation.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libw4a8.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    "-ffp-contract=off",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
HOST_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-ffp-contract=off", "-pthread",
              "-Wall", "-Wextra", "-I", os.path.join(ROOT, "include")]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd[:3])} ...")
    return res


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    steps = []
    for src in ("fused.hip", "skinny.hip", "tiled.hip", "quant_act.hip", "w4a16.hip",
                "probe.hip", "scratch.hip"):
        obj = os.path.join(BUILD, src + ".o")
        steps.append((obj, [HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]))
    for src in ("api.cpp", "configs.cpp"):
        obj = os.path.join(BUILD, src + ".o")
        steps.append((obj, [HIPCC, *HIP_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src),
                            "-o", obj]))
    gxx = shutil.which("g++") or "g++"
    obj = os.path.join(BUILD, "pack.cpp.o")
    steps.append((obj, [gxx, *HOST_FLAGS, "-c", os.path.join(CSRC, "pack.cpp"), "-o", obj]))
    # the compilations are independent processes: run them side by side
    workers = max(1, min(len(steps), os.cpu_count() or 1))
    with concurrent.futures.ThreadPoolExecutor(workers) as pool:
        for f in [pool.submit(_run, cmd, verbose) for _, cmd in steps]:
            f.result()
    objs = [obj for obj, _ in steps]
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs, "-pthread"], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
