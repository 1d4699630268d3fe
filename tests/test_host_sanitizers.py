"""The host side of the C ABI (packer, argument validation, kernel planning)
built with AddressSanitizer and UndefinedBehaviorSanitizer and exercised in a
child process: bit-exact packing against the oracle on awkward matrices, and
thousands of random, extreme argument sets for every entry point.

The build is host-only: the real pack.cpp, configs.cpp and api.cpp, with the
kernel launches replaced by stubs that report "no device" (host_stubs.cpp),
compiled by g++ (no GPU code is built with a sanitizer).
"""
import json
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

from oracle import ref

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "w4a8_gemm_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")


def build_sanitized(out_dir):
    gxx = shutil.which("g++")
    flags = ["-O1", "-g", "-fPIC", "-std=c++17", "-ffp-contract=off", "-pthread",
             "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__",
             "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include")]
    objs = []
    for src in (os.path.join(CSRC, "pack.cpp"), os.path.join(CSRC, "configs.cpp"),
                os.path.join(CSRC, "api.cpp"), os.path.join(HERE, "host_stubs.cpp")):
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        subprocess.run([gxx, *flags, "-x", "c++", "-c", src, "-o", obj], check=True)
        objs.append(obj)
    lib = os.path.join(out_dir, "libw4a8_host_sanitized.so")
    subprocess.run([gxx, "-shared", "-fsanitize=address,undefined", "-pthread", *objs,
                    "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                    "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", lib], check=True)
    return lib


def awkward_cases(tmp):
    """Weight matrices that stress the packer: zero rows, a single outlier per
    row, constant groups, subnormal-scale rows, heavy tails, and the mode and
    group-size corners; plus two that must be refused (NaN, fp16 overflow)."""
    rng = np.random.default_rng(11)
    cases = []

    def add(w, g, threads=0):
        path = os.path.join(tmp, f"w{len(cases)}.npy")
        np.save(path, np.ascontiguousarray(w, dtype=np.float32))
        cases.append({"w_path": path, "g": g, "threads": threads})

    for g in (32, 64, 128, 0, 1):
        w = (rng.standard_normal((48, 256)) * 0.02).astype(np.float32)
        w[0] = 0                                   # zero row
        w[1] = 0
        w[1, 77] = 3.5                             # single outlier
        w[2, :64] = 0.25                           # constant groups
        w[3] = rng.standard_normal(256).astype(np.float32) * np.float32(1e-6)   # subnormal s1
        w[4] = rng.standard_t(2, 256).astype(np.float32) * np.float32(0.05)     # heavy tail
        w[5] = -np.abs(w[5])                       # one sign only
        w[6] = np.abs(w[6])
        w[7, ::2] = 1e-38                          # denormal-range values
        add(w, g, threads=int(rng.integers(0, 5)))
    add((rng.standard_normal((16, 128)) * 1e-3).astype(np.float32), 128)
    add((rng.standard_normal((32, 384)) * 10).astype(np.float32), 128)   # K = 3 blocks
    w = rng.standard_normal((16, 256)).astype(np.float32)
    w[3, 5] = np.nan
    add(w, 128)                                    # NONFINITE
    w = rng.standard_normal((16, 256)).astype(np.float32) * np.float32(1e9)
    add(w, 128)                                    # RANGE (s1 overflows fp16)
    return cases


def test_host_abi_under_asan_and_ubsan(tmp_path):
    lib = build_sanitized(str(tmp_path))
    cases = awkward_cases(str(tmp_path))
    cases_path = os.path.join(str(tmp_path), "cases.json")
    with open(cases_path, "w") as f:
        json.dump(cases, f)
    out = os.path.join(str(tmp_path), "out.npz")
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    env = dict(os.environ, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, os.path.join(HERE, "san_driver.py"), lib, out, cases_path],
                         capture_output=True, text=True, env=env, timeout=600)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
    report = json.loads(res.stdout.strip().splitlines()[-1])
    assert report["ok"]
    # both outcomes of validation were reached (rejections and stubbed launches)
    assert "('status', 1)" in report["statuses"] and "('status', 7)" in report["statuses"]

    got = np.load(out)
    for ci, c in enumerate(cases):
        w = np.load(c["w_path"])
        st = int(got[f"status_{ci}"])
        if not np.isfinite(w).all():
            assert st == 4
            continue
        if np.abs(w).max() > 1e6:
            assert st == 5
            continue
        assert st == 0, (ci, st)
        qw = ref.quantize_weights(w, c["g"])
        assert np.array_equal(got[f"q_{ci}"], qw["q"]), ci
        assert np.array_equal(got[f"s1_{ci}"], qw["s1"].view(np.uint16)), ci
        if c["g"] != ref.NF_CODE:
            assert np.array_equal(got[f"z_{ci}"], qw["z"]), ci
            assert np.array_equal(got[f"s2_{ci}"], qw["s2"]), ci
