"""GPU parity of the W4A16 comparison GEMM (same packed weights, fp16
activations, fp32 accumulation) against the oracle's exact sum.

Bar: |Y - Y_ref| <= 1 fp16 ulp + 1e-3 |Y_ref| + K * 2^-24 * sum_k |A W16^|
(ref.y16_tolerance_ok): the fp16 products are exact in fp32, so only the
fp32 summation and the final fp16 rounding separate the two."""
import numpy as np
import pytest

import synth
import w4a8_gemm_amd as w4
from gpu_util import device, log
from oracle import ref

pytestmark = pytest.mark.gpu


def _run(a_np, blob, n, k, g, **kw):
    import torch
    dev = device()
    a = torch.from_numpy(a_np).to(dev)
    y = w4.w4a16(a, w4.to_device(blob, dev), n, k, g, **kw)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("m,n,k,g,dist", [
    (1, 48, 384, 64, "normal"),
    (3, 272, 640, 32, "student_t4"),
    (16, 256, 512, 128, "normal"),
    (17, 80, 1024, 128, "normal"),
    (33, 112, 256, 0, "student_t4"),
    (64, 512, 1152, 128, "normal"),
    (5, 4112, 2688, 64, "student_t4"),
    (100, 512, 1024, 128, "normal"),          # skinny above 64 tokens: the tiled grid would be 4 tiles
    (128, 272, 640, 64, "student_t4"),
])
def test_w4a16_matches_oracle(m, n, k, g, dist):
    w = synth.weights(n, k, seed=800 + n + k, dist=dist)
    a = synth.activations(m, k, seed=900 + m)
    qw = ref.quantize_weights(w, g)
    y_ref, _, sum_abs = ref.w4a16_linear(a, qw)
    log(f"w4a16 m={m} n={n} k={k} g={g}")
    y = _run(a, w4.pack(w, g), n, k, g)
    ok = ref.y16_tolerance_ok(y, y_ref, sum_abs, k)
    assert ok.all(), np.argwhere(~ok)[:5]


@pytest.mark.parametrize("n_tiles,k_split", [(1, 1), (2, 3), (4, 8), (1, 5), (2, 8)])
def test_w4a16_every_shape(n_tiles, k_split):
    m, n, k, g = 9, 320, 2048, 32
    w = synth.weights(n, k, seed=71, dist="student_t4")
    a = synth.activations(m, k, seed=72)
    qw = ref.quantize_weights(w, g)
    y_ref, _, sum_abs = ref.w4a16_linear(a, qw)
    log(f"w4a16 n_tiles={n_tiles} k_split={k_split}")
    y = _run(a, w4.pack(w, g), n, k, g, variant=1, n_tiles=n_tiles, k_split=k_split)
    assert ref.y16_tolerance_ok(y, y_ref, sum_abs, k).all()


def test_w4a16_full_size_decode_sampled():
    """The Llama-3-8B gate+up and down layers at M = 1, 4, 16: 64 sampled
    output columns (all rows) against the oracle."""
    import torch
    dev = device()
    for (n, k) in ((28672, 4096), (4096, 14336)):
        w = synth.weights(n, k, seed=n + k)
        blob = w4.to_device(w4.pack(w, 128), dev)
        rng = np.random.default_rng(n)
        cols = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 64, replace=False)]))
        qw = ref.quantize_weights(w[cols], 128)
        del w
        for m in (1, 4, 16):
            a = synth.activations(m, k, seed=m + k)
            log(f"w4a16 full-size m={m} n={n} k={k}")
            y = w4.w4a16(torch.from_numpy(a).to(dev), blob, n, k, 128)
            torch.cuda.synchronize()
            y_s = y.cpu().numpy()[:, cols]
            y_ref, _, sum_abs = ref.w4a16_linear(a, qw)
            assert ref.y16_tolerance_ok(y_s, y_ref, sum_abs, k).all()


def test_w4a16_vs_w4a8_same_weights():
    """Same blob: W4A16 and W4A8 differ only by the per-token int8
    quantization of the activations; the GPU's gap between the two equals the
    oracle's (the outlier columns make it several percent here)."""
    import torch
    dev = device()
    m, n, k, g = 4, 512, 2048, 128
    w = synth.weights(n, k, seed=5)
    a = synth.activations(m, k, seed=6)
    blob = w4.to_device(w4.pack(w, g), dev)
    a_dev = torch.from_numpy(a).to(dev)
    log("w4a16 vs w4a8")
    y16 = w4.w4a16(a_dev, blob, n, k, g).cpu().numpy().astype(np.float64)
    y8, _, _ = w4.linear(a_dev, blob, n, k, g)
    torch.cuda.synchronize()
    y8 = y8.cpu().numpy().astype(np.float64)
    rel_gpu = np.linalg.norm(y8 - y16) / np.linalg.norm(y16)
    out = ref.linear(a, w, g)
    y16_ref, _, _ = ref.w4a16_linear(a, out["qw"])
    y16_ref = y16_ref.astype(np.float64)
    rel_ref = np.linalg.norm(out["y"].astype(np.float64) - y16_ref) / np.linalg.norm(y16_ref)
    assert abs(rel_gpu - rel_ref) < 1e-3 * max(1.0, rel_ref * 100), (rel_gpu, rel_ref)


@pytest.mark.parametrize("m,n,k,g,dist,variant", [
    (65, 144, 384, 64, "normal", 0),          # ragged rows and a workgroup with one real column tile
    (300, 256, 1024, 128, "student_t4", 0),   # two row tiles, the second ragged
    (257, 400, 640, 32, "normal", 0),
    (128, 128, 256, 0, "student_t4", 0),      # per-channel
    (1, 48, 384, 128, "normal", 2),           # the tiled kernel forced at one token
    (40, 272, 768, 64, "normal", 2),
    (512, 1024, 2048, 128, "student_t4", 0),
])
def test_w4a16_tiled_matches_oracle(m, n, k, g, dist, variant):
    """The tiled W4A16 kernel (M > 64, or forced): every output within the
    fp32 summation bound of the oracle's exact sum."""
    w = synth.weights(n, k, seed=810 + n + k, dist=dist)
    a = synth.activations(m, k, seed=910 + m)
    qw = ref.quantize_weights(w, g)
    y_ref, _, sum_abs = ref.w4a16_linear(a, qw)
    log(f"w4a16 tiled m={m} n={n} k={k} g={g} variant={variant}")
    y = _run(a, w4.pack(w, g), n, k, g, variant=variant)
    ok = ref.y16_tolerance_ok(y, y_ref, sum_abs, k)
    assert ok.all(), np.argwhere(~ok)[:5]


def test_w4a16_tiled_full_size_sampled():
    """The batched Llama-3-8B QKV and down layers at M = 256 and 1024 and the
    Qwen1.5-72B O layer at M = 2048 on the tiled kernel: 64 sampled output
    columns (plus the first and last), all rows, against the oracle."""
    import torch
    dev = device()
    for (n, k) in ((6144, 4096), (4096, 14336), (8192, 8192)):
        w = synth.weights(n, k, seed=n + k + 1)
        blob = w4.to_device(w4.pack(w, 128), dev)
        rng = np.random.default_rng(n + 1)
        cols = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 64, replace=False)]))
        qw = ref.quantize_weights(w[cols], 128)
        del w
        for m in ((256, 1024) if k != 8192 else (2048,)):
            a = synth.activations(m, k, seed=m + k + 1)
            log(f"w4a16 tiled full-size m={m} n={n} k={k}")
            y = w4.w4a16(torch.from_numpy(a).to(dev), blob, n, k, 128)
            torch.cuda.synchronize()
            y_s = y.cpu().numpy()[:, cols]
            y_ref, _, sum_abs = ref.w4a16_linear(a, qw)
            assert ref.y16_tolerance_ok(y_s, y_ref, sum_abs, k).all()
