"""The allocation-free GEMM entry point (w4a8_gemm_noalloc) through the C ABI,
against w4a8_gemm on the same inputs: the int32 accumulators and Y must be
identical (the same kernels and plans, the K-split partial sums in the
library's static scratch instead of a workspace), and the accumulators match
the CPU oracle on sampled columns.
"""
import numpy as np
import pytest

import synth
import w4a8_gemm_amd as w4
from gpu_util import device, log
from oracle import ref

pytestmark = pytest.mark.gpu


def _inputs(m, n, k, g, seed):
    import torch
    dev = device()
    w = synth.weights(n, k, seed=seed)
    blob = w4.to_device(w4.pack(w, g), dev)
    a8_np, s_a_np = ref.quant_act(synth.activations(m, k, seed=seed + 1))
    a8 = torch.from_numpy(a8_np).to(dev)
    s_a = torch.from_numpy(s_a_np).to(dev)
    return w, blob, a8, s_a, a8_np, s_a_np


def _both(m, n, k, g, blob, a8, s_a, slices=0):
    """w4a8_gemm (own workspace) and w4a8_gemm_noalloc on the same inputs."""
    import torch
    dev = a8.device
    y_ref, acc_ref = w4.gemm(a8, s_a, blob, n, k, g, want_acc=True, slices=slices)
    y = torch.empty((m, n), dtype=torch.float16, device=dev)
    acc = torch.empty((m, n), dtype=torch.int32, device=dev)
    w4.gemm_noalloc(a8, s_a, blob, n, k, g, y, acc, slices=slices)
    torch.cuda.synchronize()
    return y.cpu().numpy(), acc.cpu().numpy(), y_ref.cpu().numpy(), acc_ref.cpu().numpy()


def test_noalloc_matches_gemm_on_two_calls_in_a_row():
    """Two calls in a row that both split K into the scratch, the second on a
    smaller input: each equals w4a8_gemm, and the accumulators equal the
    oracle's on sampled columns."""
    g = 128
    for m, n, k, seed in ((100, 4096, 14336, 11), (48, 2048, 14336, 13)):
        assert w4.lib.w4a8_gemm_workspace_size(m, n, k, g, None) > 0, "the plan must split K"
        w, blob, a8, s_a, a8_np, s_a_np = _inputs(m, n, k, g, seed)
        log(f"gemm_noalloc m={m} n={n} k={k} g={g}")
        y, acc, y_ref, acc_ref = _both(m, n, k, g, blob, a8, s_a)
        assert np.array_equal(acc, acc_ref)
        assert np.array_equal(y.view(np.uint16), y_ref.view(np.uint16))
        cols = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(seed).choice(n, 48)]))
        qw = ref.quantize_weights(w[cols], g)
        want = ref.gemm_acc(a8_np, ref.decoded_weights(qw))
        assert np.array_equal(acc[:, cols], want)
        assert ref.y_tolerance_ok(y[:, cols], ref.epilogue(want, s_a_np, qw["s1"])).all()


def test_noalloc_narrows_a_split_that_does_not_fit():
    """1408 x 4096 x 8192: w4a8_gemm splits K three ways (69 MB of partial
    sums), more than the 64 MiB scratch; the allocation-free call takes two
    slices and gives the same results."""
    m, n, k, g = 1408, 4096, 8192, 128
    assert w4.lib.w4a8_gemm_workspace_size(m, n, k, g, None) > 64 << 20
    _, blob, a8, s_a, _, _ = _inputs(m, n, k, g, 17)
    log(f"gemm_noalloc narrowed split m={m} n={n} k={k}")
    y, acc, y_ref, acc_ref = _both(m, n, k, g, blob, a8, s_a)
    assert np.array_equal(acc, acc_ref)
    assert np.array_equal(y.view(np.uint16), y_ref.view(np.uint16))


def test_noalloc_forced_split():
    """A forced split that fits runs in the scratch; one that does not is
    rejected before anything is enqueued."""
    import torch
    m, n, k, g = 64, 4096, 8192, 128
    _, blob, a8, s_a, _, _ = _inputs(m, n, k, g, 19)
    log(f"gemm_noalloc forced slices m={m} n={n} k={k}")
    y, acc, y_ref, acc_ref = _both(m, n, k, g, blob, a8, s_a, slices=8)
    assert np.array_equal(acc, acc_ref)
    assert np.array_equal(y.view(np.uint16), y_ref.view(np.uint16))
    big_m = 4096
    a8b = torch.zeros((big_m, k), dtype=torch.int8, device=a8.device)
    s_ab = torch.zeros((big_m,), dtype=torch.float16, device=a8.device)
    yb = torch.empty((big_m, n), dtype=torch.float16, device=a8.device)
    with pytest.raises(w4.W4A8Error) as err:
        w4.gemm_noalloc(a8b, s_ab, blob, n, k, g, yb, slices=2)   # 2 x 64 MiB of partials
    assert err.value.status == 3


def test_noalloc_ping_pong_split_fills_the_scratch():
    """The Llama-3-8B down projection at M = 1024 splits K four ways on the
    256 x 256 ping-pong kernel: 1024 x 4096 x 4 slices of int32 partials fill
    the 64 MiB scratch exactly.  The allocation-free call keeps that split and
    equals w4a8_gemm; the accumulators equal the oracle's on sampled columns."""
    m, n, k, g = 1024, 4096, 14336, 128
    assert w4.lib.w4a8_gemm_workspace_size(m, n, k, g, None) == 64 << 20
    w, blob, a8, s_a, a8_np, s_a_np = _inputs(m, n, k, g, 23)
    log(f"gemm_noalloc ping-pong split m={m} n={n} k={k}")
    y, acc, y_ref, acc_ref = _both(m, n, k, g, blob, a8, s_a)
    assert np.array_equal(acc, acc_ref)
    assert np.array_equal(y.view(np.uint16), y_ref.view(np.uint16))
    cols = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(23).choice(n, 32)]))
    qw = ref.quantize_weights(w[cols], g)
    want = ref.gemm_acc(a8_np, ref.decoded_weights(qw))
    assert np.array_equal(acc[:, cols], want)


@pytest.mark.parametrize("m,n,k", [(48, 11008, 4096), (160, 4096, 11008)])
def test_noalloc_split_regimes_of_the_plan(m, n, k):
    """The K-split plans at 40-64 tokens on wide layers (two slices) and at
    129-192 tokens (towards ~384 workgroups) through the static scratch: the
    same split as w4a8_gemm's workspace, identical results, and accumulators
    equal to the oracle's on sampled columns."""
    g = 128
    need = w4.lib.w4a8_gemm_workspace_size(m, n, k, g, None)
    assert 0 < need <= 64 * 2 ** 20, "the plan must split K within the scratch"
    w, blob, a8, s_a, a8_np, s_a_np = _inputs(m, n, k, g, m + n)
    log(f"gemm_noalloc split regime m={m} n={n} k={k}")
    y, acc, y_ref, acc_ref = _both(m, n, k, g, blob, a8, s_a)
    assert np.array_equal(acc, acc_ref)
    assert np.array_equal(y.view(np.uint16), y_ref.view(np.uint16))
    cols = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(m).choice(n, 32)]))
    qw = ref.quantize_weights(w[cols], g)
    assert np.array_equal(acc[:, cols], ref.gemm_acc(a8_np, ref.decoded_weights(qw)))
