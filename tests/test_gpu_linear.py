"""GPU parity of the whole layer (w4a8_linear): per-token quantization fused
into the small-M GEMM, against the CPU oracle and against the two-launch path.

Bar: A8, s_a and the int32 accumulators bit-exact with the oracle; Y within
the oracle tolerance and bit-identical to quantizer + GEMM."""
import numpy as np
import pytest

import synth
import w4a8_gemm_amd as w4
from gpu_util import device, log
from oracle import ref

pytestmark = pytest.mark.gpu


def _run_linear(a_np, blob, n, k, g, lda=None, lda8=None, **kw):
    import torch
    dev = device()
    m = a_np.shape[0]
    lda = lda or k
    lda8 = lda8 or k
    a_full = torch.zeros((m, lda), dtype=torch.float16, device=dev)
    a_full[:, :k] = torch.from_numpy(a_np).to(dev)
    a8_full = torch.full((m, lda8), 99, dtype=torch.int8, device=dev)
    wdev = w4.to_device(blob, dev)
    y, a8, s_a, acc = w4.linear(a_full[:, :k], wdev, n, k, g, a8=a8_full[:, :k], want_acc=True,
                                **kw)
    torch.cuda.synchronize()
    return (y.cpu().numpy(), a8_full.cpu().numpy(), s_a.cpu().numpy(), acc.cpu().numpy())


def _run_two_launch(a_np, blob, n, k, g):
    import torch
    dev = device()
    a = torch.from_numpy(a_np).to(dev)
    a8, s_a = w4.quant_act(a)
    y, acc = w4.gemm(a8, s_a, w4.to_device(blob, dev), n, k, g, want_acc=True)
    torch.cuda.synchronize()
    return y.cpu().numpy(), acc.cpu().numpy()


SHAPES = [  # n, k, g
    (256, 512, 128),
    (48, 384, 64),
    (272, 640, 32),
    (112, 256, 0),
    (96, 2688, 128),        # 21 k-blocks: ragged wave ranges
    (4112, 1152, 64),       # 257 column tiles
]


@pytest.mark.parametrize("n,k,g", SHAPES)
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8])
def test_linear_fused_matches_oracle_and_two_launches(m, n, k, g):
    w = synth.weights(n, k, seed=500 + n + k + g, dist="student_t4")
    a = synth.activations(m, k, seed=600 + m + k)
    out = ref.linear(a, w, g)
    blob = w4.pack(w, g)
    log(f"linear fused m={m} n={n} k={k} g={g}")
    y, a8, s_a, acc = _run_linear(a, blob, n, k, g, variant=3)
    assert np.array_equal(s_a.view(np.uint16), out["s_a"].view(np.uint16))
    assert np.array_equal(a8, out["a8"])
    assert np.array_equal(acc, out["acc"])
    assert ref.y_tolerance_ok(y, out["y"]).all()
    log(f"two launches m={m} n={n} k={k} g={g}")
    y2, acc2 = _run_two_launch(a, blob, n, k, g)
    assert np.array_equal(acc2, acc)
    assert np.array_equal(y2.view(np.uint16), y.view(np.uint16))


@pytest.mark.parametrize("n_tiles,k_split", [(1, 1), (1, 8), (2, 3), (4, 2), (4, 8), (2, 5)])
def test_linear_fused_every_shape(n_tiles, k_split):
    n, k, g, m = 320, 2048, 32, 4
    w = synth.weights(n, k, seed=71, dist="student_t4")
    a = synth.activations(m, k, seed=72)
    out = ref.linear(a, w, g)
    log(f"linear fused n_tiles={n_tiles} k_split={k_split}")
    y, a8, s_a, acc = _run_linear(a, w4.pack(w, g), n, k, g, variant=3, n_tiles=n_tiles,
                                  k_split=k_split)
    assert np.array_equal(a8, out["a8"])
    assert np.array_equal(acc, out["acc"])
    assert ref.y_tolerance_ok(y, out["y"]).all()


def test_linear_strided_rows_and_padding():
    n, k, g, m = 96, 640, 64, 3
    w = synth.weights(n, k, seed=81)
    a = synth.activations(m, k, seed=82)
    out = ref.linear(a, w, g)
    log("linear fused lda=648 lda8=656")
    y, a8_full, s_a, acc = _run_linear(a, w4.pack(w, g), n, k, g, lda=648, lda8=656,
                                       variant=3)
    assert np.array_equal(a8_full[:, :k], out["a8"])
    assert (a8_full[:, k:] == 99).all()                    # padding untouched
    assert np.array_equal(acc, out["acc"])


@pytest.mark.parametrize("m,n,k,g", [(16, 256, 14336, 128), (9, 64, 512, 128), (100, 272, 768, 64),
                                     (4, 64, 131072, 128)])
def test_linear_two_launch_path(m, n, k, g):
    """Where the fused kernel does not apply (more than 8 rows, or its LDS
    copy of A would not fit), the same call runs quantizer + GEMM."""
    w = synth.weights(n, k, seed=91 + m)
    a = synth.activations(m, k, seed=92 + m)
    blob = w4.pack(w, g)
    if k > 20000:   # long K: compare against the two-launch path only
        log(f"linear auto m={m} n={n} k={k} g={g}")
        y, a8, s_a, acc = _run_linear(a, blob, n, k, g)
        want_a8, want_sa = ref.quant_act(a)
        assert np.array_equal(a8, want_a8)
        y2, acc2 = _run_two_launch(a, blob, n, k, g)
        assert np.array_equal(acc, acc2)
        assert np.array_equal(y.view(np.uint16), y2.view(np.uint16))
        return
    out = ref.linear(a, w, g)
    log(f"linear auto m={m} n={n} k={k} g={g}")
    y, a8, s_a, acc = _run_linear(a, blob, n, k, g)
    assert np.array_equal(a8, out["a8"])
    assert np.array_equal(acc, out["acc"])
    assert ref.y_tolerance_ok(y, out["y"]).all()


def test_linear_zero_rows_and_extremes():
    """A zero token row (s_a = 0) and a row with one huge outlier."""
    n, k, g, m = 128, 1024, 128, 4
    w = synth.weights(n, k, seed=101)
    a = synth.activations(m, k, seed=102)
    a[1] = 0
    a[2, 5] = np.float16(60000.0)
    out = ref.linear(a, w, g)
    log("linear fused zero row + outlier")
    y, a8, s_a, acc = _run_linear(a, w4.pack(w, g), n, k, g, variant=3)
    assert np.array_equal(s_a.view(np.uint16), out["s_a"].view(np.uint16))
    assert np.array_equal(a8, out["a8"])
    assert np.array_equal(acc, out["acc"])
    assert ref.y_tolerance_ok(y, out["y"]).all()


def _decode_layers():
    items = synth.workloads()["llama3_8b_decode"]
    cfg_idx = list(synth.workloads()).index("llama3_8b_decode")
    layers = {}
    for (_, m, layer, n, k, g, dist) in items:
        layers.setdefault((layer, n, k, g, dist), []).append(m)
    return [pytest.param(cfg_idx, i, key, ms, id=key[0]) for i, (key, ms) in enumerate(layers.items())]


@pytest.mark.parametrize("cfg_idx,shape_idx,key,ms", _decode_layers())
def test_linear_full_size_decode(cfg_idx, shape_idx, key, ms):
    """The decode workload's layers at full size, M = 1, 4, 16 as the bench
    runs them: A8/s_a bit-exact with the oracle, and Y and acc identical to
    the two-launch path on every output."""
    layer, n, k, g, dist = key
    w = synth.weights(n, k, seed=synth.weight_seed(cfg_idx, shape_idx, 0), dist=dist)
    blob = w4.pack(w, g)
    del w
    for mi, m in enumerate(ms):
        a = synth.activations(m, k, seed=synth.act_seed(cfg_idx, shape_idx, mi))
        log(f"linear full-size {layer} m={m} n={n} k={k}")
        y, a8, s_a, acc = _run_linear(a, blob, n, k, g)
        want_a8, want_sa = ref.quant_act(a)
        assert np.array_equal(s_a.view(np.uint16), want_sa.view(np.uint16))
        assert np.array_equal(a8, want_a8)
        y2, acc2 = _run_two_launch(a, blob, n, k, g)
        assert np.array_equal(acc, acc2)
        assert np.array_equal(y.view(np.uint16), y2.view(np.uint16))
