"""Seeded random layer shapes through the automatic plans, against the oracle.

The fixed parity cases pick shapes by hand; these draw M, N, K, g and the
weight distribution from a seeded generator, spread over the plan's regimes
(fused and skinny at small M, the LDS-tiled kernels with and without a K
split, the 256 x 256 ping-pong kernel, long K), with ragged M and N.  Each
case runs the whole layer (`w4a8_linear`, the path the benchmark times) and
checks A8 and s_a bit-exact on every element, the int32 accumulators
bit-exact and Y within the fp16 tolerance on sampled columns (plus both
edges of the first, a middle and the last 16-column tile).  The method is
the W4A8 layer of the QServe/QoQ abstract: per-token int8 activations times
progressively quantized 4-bit weights, exact integer accumulation, scales
applied once at the end.
"""
import numpy as np
import pytest

import synth
import w4a8_gemm_amd as w4
from gpu_util import device, log
from oracle import ref

# (name, smallest M, largest M, K / 128 range, 16-column tiles range)
REGIMES = [
    ("decode", 1, 16, (1, 112), (1, 1023)),
    ("small", 17, 64, (1, 112), (1, 1023)),
    ("mid", 65, 700, (1, 64), (1, 1023)),
    ("large", 701, 2304, (1, 64), (1, 1023)),
    ("long_k", 1024, 1536, (96, 128), (1, 1023)),
    # 40-64 tokens, K >= 4096, 80-191 tiles of 64 x 128: split 64 x 128 tiles
    ("wide_small", 40, 64, (32, 36), (640, 1528)),
    # 129-192 tokens, 8192 <= K <= 16384, < 192 tiles of 64 x 128
    ("m129_192", 129, 192, (64, 128), (64, 504)),
    # 200-700 tokens, K >= 8192, few 128 x 256 tiles: 128 x 256 split
    ("split_mid", 200, 700, (64, 112), (64, 400)),
]
MAX_WEIGHTS = 48 * 2 ** 20      # N * K drawn at most (host memory for the fp32 weights)
MAX_ACTS = 24 * 2 ** 20         # M * K


def draw(seed):
    rng = np.random.default_rng(7919 * seed + 13)
    name, m_lo, m_hi, (kb_lo, kb_hi), (t_lo, t_hi) = REGIMES[seed % len(REGIMES)]
    m = int(rng.integers(m_lo, m_hi + 1))
    k = 128 * int(rng.integers(kb_lo, kb_hi + 1))
    n = 16 * int(rng.integers(t_lo, t_hi + 1))
    n = max(16, min(n, MAX_WEIGHTS // k // 16 * 16))
    if name == "long_k":
        # 32-223 tiles of 256 x 256 (the ping-pong kernel with K split)
        n = max(n, 16 * ((32 * 65536 // m + 15) // 16))
        n = min(n, MAX_WEIGHTS // k // 16 * 16)
    m = min(m, max(1, MAX_ACTS // k))
    g = [32, 64, 128, 0][int(rng.integers(4))]
    dist = "student_t4" if rng.random() < 0.3 else "normal"
    return name, m, n, k, g, dist


CASES = [draw(s) for s in range(40)]


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(len(CASES)))
def test_linear_random_shape(seed):
    name, m, n, k, g, dist = CASES[seed]
    import torch
    dev = device()
    w = synth.weights(n, k, seed=90000 + seed, dist=dist)
    blob = w4.pack(w, g)
    rng = np.random.default_rng(seed)
    mid = (n // 32) * 16
    edges = [0, 15, mid, mid + 15, n - 16, n - 1]
    cols = np.unique(np.concatenate([[c for c in edges if 0 <= c < n],
                                     rng.choice(n, min(n, 48), replace=False)]))
    qw = ref.quantize_weights(w[cols], g)
    del w
    a = synth.activations(m, k, seed=91000 + seed)
    launches = w4.lib.w4a8_linear_launches(m, n, k, g, None)
    log(f"random shape {seed}: {name} m={m} n={n} k={k} g={g} {dist}, {launches} launch(es)")
    wdev = w4.to_device(blob, dev)
    y, a8, s_a, acc = w4.linear(torch.from_numpy(a).to(dev), wdev, n, k, g, want_acc=True)
    torch.cuda.synchronize()
    want_a8, want_sa = ref.quant_act(a)
    assert np.array_equal(s_a.cpu().numpy().view(np.uint16), want_sa.view(np.uint16))
    assert np.array_equal(a8.cpu().numpy(), want_a8)
    acc_ref = ref.gemm_acc(want_a8, ref.decoded_weights(qw))
    assert np.array_equal(acc.cpu().numpy()[:, cols], acc_ref)
    y_ref = ref.epilogue(acc_ref, want_sa, qw["s1"])
    assert ref.y_tolerance_ok(y.cpu().numpy()[:, cols], y_ref).all()


def test_draws_cover_every_regime():
    """The draws reach each plan regime, including the split ping-pong one
    (M >= 1024, K >= 12288, 32-223 tiles of 256 x 256), and the K-split
    regimes take the split the plan is meant to choose (read through the
    workspace size: one int32 plane of M x N per slice)."""
    names = {c[0] for c in CASES}
    assert names == {r[0] for r in REGIMES}
    assert {c[4] for c in CASES} == {32, 64, 128, 0}
    for name, m, n, k, g, _ in CASES:
        t64 = ((m + 63) // 64) * ((n // 16 + 7) // 8)
        slices = w4.lib.w4a8_gemm_workspace_size(m, n, k, g, None) // (m * n * 4)
        if name == "long_k":
            tiles = ((m + 255) // 256) * ((n // 16 + 15) // 16)
            assert k >= 12288 and 32 <= tiles < 224
        if name == "wide_small":
            assert 80 <= t64 < 192 and slices == max(2, 256 // t64)
        if name == "m129_192":
            assert t64 < 192 and slices >= 2
        if name == "split_mid":
            assert slices >= 2
