"""Seeded synthetic inputs for the W4A8 linear-layer workloads.

This module only draws random numbers and lists layer shapes.  It holds none
of the quantization or GEMM arithmetic, so both the CPU oracle and the GPU
path can take their inputs from it without sharing any of the method.

Weights stand in for trained Llama-3-8B / Qwen1.5-72B linear layers (the
models the QServe/QoQ abstract and the FLUTE abstract measure on); no trained
checkpoint is used.  Recipe:

* W (N x K fp32, row = output channel):  0.02 * X * u[n], with X ~ N(0, 1)
  (or Student-t with 4 degrees of freedom for the heavy-tailed sweep) and a
  per-row multiplier u[n] ~ U(0.5, 2).
* A (M x K fp16): N(0, 1) with 4 distinct columns, drawn once per matrix and
  shared by all rows, multiplied by 20 before the cast to fp16 (outlier
  channels, the situation per-token activation quantization has to absorb).
"""
from __future__ import annotations

import numpy as np

# (N, K) of the four linear layers of one transformer block.
LLAMA3_8B = {
    "qkv": (6144, 4096),
    "o": (4096, 4096),
    "gate_up": (28672, 4096),
    "down": (4096, 14336),
}
QWEN15_72B = {
    "qkv": (24576, 8192),
    "o": (8192, 8192),
    "gate_up": (49152, 8192),
    "down": (8192, 24576),
}

# Workload table.  Each run is (config, M, layer, N, K, g, weight_dist);
# g == 0 means per-channel (one scale and zero per output row, no groups).
def workloads() -> dict[str, list[tuple]]:
    runs: dict[str, list[tuple]] = {}
    runs["tiny"] = [("tiny", 16, "tiny", 256, 512, 128, "normal")]
    runs["llama3_8b_decode"] = [
        ("llama3_8b_decode", m, name, n, k, 128, "normal")
        for m in (1, 4, 16) for name, (n, k) in LLAMA3_8B.items()]
    runs["llama3_8b_batched"] = [
        ("llama3_8b_batched", m, name, n, k, 128, "normal")
        for m in (64, 256, 1024) for name, (n, k) in LLAMA3_8B.items()]
    runs["qwen15_72b_large"] = [
        ("qwen15_72b_large", m, name, n, k, 128, "normal")
        for m in (2048, 4096) for name, (n, k) in QWEN15_72B.items()]
    n, k = LLAMA3_8B["gate_up"]
    runs["group_sweep"] = [
        ("group_sweep", m, "gate_up", n, k, g, "student_t4")
        for m in (1, 32, 512) for g in (32, 64, 128, 0)]
    # the metric's whole range in one step: decode, batched serving and the
    # large-batch layers (each run keeps the seeds of the workload it comes
    # from, named in its first field)
    runs["m1_to_4096"] = (runs["llama3_8b_decode"] + runs["llama3_8b_batched"]
                          + runs["qwen15_72b_large"])
    return runs


# workloads made of the runs of others
COMPOSITE = ("m1_to_4096",)


def weight_seed(config_idx: int, shape_idx: int, g_idx: int) -> int:
    return 1000 * config_idx + 10 * shape_idx + g_idx


def act_seed(config_idx: int, shape_idx: int, m_idx: int) -> int:
    return 1000 * config_idx + 10 * shape_idx + 500 + m_idx


def weights(n: int, k: int, seed: int, dist: str = "normal",
            sigma: float = 0.02) -> np.ndarray:
    """N x K float32 weight matrix (row-major, row = output channel)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    row_mult = rng.uniform(0.5, 2.0, size=n).astype(np.float32)
    if dist == "normal":
        x = rng.standard_normal((n, k), dtype=np.float32)
    elif dist == "student_t4":
        x = rng.standard_t(4.0, size=(n, k)).astype(np.float32)
    else:
        raise ValueError(f"unknown weight distribution {dist!r}")
    x *= np.float32(sigma)
    x *= row_mult[:, None]
    return x


def activations(m: int, k: int, seed: int, n_outliers: int = 4,
                gain: float = 20.0) -> np.ndarray:
    """M x K float16 activations with a few outlier channels."""
    rng = np.random.Generator(np.random.PCG64(seed))
    a = rng.standard_normal((m, k), dtype=np.float32)
    cols = rng.choice(k, size=min(n_outliers, k), replace=False)
    a[:, cols] *= np.float32(gain)
    return a.astype(np.float16)


def raw_int8(shape, seed: int, lo: int = -127, hi: int = 127) -> np.ndarray:
    """Uniform int8 values in [lo, hi] (for kernel tests that start from A8)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(lo, hi + 1, size=shape, dtype=np.int16).astype(np.int8)
