"""GPU parity of the codebook (NormalFloat-style, register-table decode)
weight mode: int32 accumulators bit-exact with the oracle on every kernel
shape, Y within the oracle tolerance."""
import numpy as np
import pytest

import synth
import w4a8_gemm_amd as w4
from gpu_util import device, log, run_gemm
from oracle import ref

pytestmark = pytest.mark.gpu
NF = ref.NF_CODE


@pytest.mark.parametrize("m,n,k", [(1, 48, 384), (3, 272, 640), (16, 256, 512), (33, 112, 2688),
                                   (64, 512, 1152), (65, 320, 512), (200, 272, 2688),
                                   (513, 4112, 640)])
def test_codebook_auto_bit_exact(m, n, k):
    w = synth.weights(n, k, seed=1000 + n + k, dist="student_t4")
    a = synth.activations(m, k, seed=1100 + m)
    out = ref.linear(a, w, NF)
    log(f"codebook auto m={m} n={n} k={k}")
    y, acc = run_gemm(out["a8"], out["s_a"], w4.pack(w, NF), n, k, NF)
    assert np.array_equal(acc, out["acc"])
    assert ref.y_tolerance_ok(y, out["y"]).all()


def test_codebook_every_kernel_shape():
    m, n, k = 130, 1040, 1152
    w = synth.weights(n, k, seed=5, dist="student_t4")
    a = synth.activations(m, k, seed=6)
    out = ref.linear(a, w, NF)
    blob = w4.pack(w, NF)
    for kw in (dict(variant=2, m_tiles=4, stages=2), dict(variant=2, m_tiles=8, stages=3),
               dict(variant=2, m_tiles=8, n_tiles=2), dict(variant=2, row_groups=2),
               dict(variant=2, m_tiles=8, k_split=2), dict(variant=2, slices=3)):
        log(f"codebook tiled {kw}")
        y, acc = run_gemm(out["a8"], out["s_a"], blob, n, k, NF, **kw)
        assert np.array_equal(acc, out["acc"]), kw
    for mm, ks, nt in ((16, 1, 1), (16, 8, 4), (40, 3, 2), (64, 5, 1)):
        log(f"codebook skinny m={mm} k_split={ks} n_tiles={nt}")
        y, acc = run_gemm(out["a8"][:mm], out["s_a"][:mm], blob, n, k, NF, variant=1,
                          k_split=ks, n_tiles=nt)
        assert np.array_equal(acc, out["acc"][:mm])


@pytest.mark.parametrize("m,launches", [(2, 1), (30, 2)])
def test_codebook_linear(m, launches):
    """w4a8_linear in the codebook mode: the fused kernel for a few tokens,
    quantizer + GEMM for more."""
    import torch
    dev = device()
    n, k = 256, 1024
    w = synth.weights(n, k, seed=8)
    a = synth.activations(m, k, seed=9)
    out = ref.linear(a, w, NF)
    assert w4.lib.w4a8_linear_launches(m, n, k, NF, None) == launches
    log(f"codebook linear m={m}")
    y, a8, s_a, acc = w4.linear(torch.from_numpy(a).to(dev), w4.to_device(w4.pack(w, NF), dev),
                                n, k, NF, want_acc=True)
    torch.cuda.synchronize()
    assert np.array_equal(a8.cpu().numpy(), out["a8"])
    assert np.array_equal(acc.cpu().numpy(), out["acc"])
    assert ref.y_tolerance_ok(y.cpu().numpy(), out["y"]).all()


@pytest.mark.parametrize("m", [1, 16, 1024])
def test_codebook_full_size_sampled(m):
    """Llama-3-8B gate+up at full size: 64 sampled columns, all rows."""
    import torch
    dev = device()
    n, k = 28672, 4096
    w = synth.weights(n, k, seed=77)
    blob = w4.to_device(w4.pack(w, NF), dev)
    rng = np.random.default_rng(m)
    cols = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 64, replace=False)]))
    qw = ref.quantize_weights(w[cols], NF)
    del w
    a = synth.activations(m, k, seed=m)
    log(f"codebook full-size m={m}")
    a8, s_a = w4.quant_act(torch.from_numpy(a).to(dev))
    y, acc = w4.gemm(a8, s_a, blob, n, k, NF, want_acc=True)
    torch.cuda.synchronize()
    idx = torch.from_numpy(cols).to(dev)
    acc_s = acc.index_select(1, idx).cpu().numpy()
    want_a8, want_sa = ref.quant_act(a)
    acc_ref = ref.gemm_acc(want_a8, ref.decoded_weights(qw))
    assert np.array_equal(acc_s, acc_ref)
    y_ref = ref.epilogue(acc_ref, want_sa, qw["s1"])
    assert ref.y_tolerance_ok(y.index_select(1, idx).cpu().numpy(), y_ref).all()
