"""GPU parity of the whole layer (w4a8_linear): per-token quantization fused
into the small-M GEMM, against the CPU oracle and against the two-launch path.

Bar: A8, s_a and the int32 accumulators bit-exact with the oracle; Y within
the oracle tolerance and bit-identical to quantizer + GEMM."""
import ctypes

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


def _fused_applies(m, n, k, g, **opts):
    o = w4.GemmOpts(3, opts.get("k_split", 0), opts.get("n_tiles", 0), 0, 0, 0, 0,
                    opts.get("workgroups", 0))
    return int(w4.lib.w4a8_linear_launches(m, n, k, g, ctypes.byref(o))) == 1


@pytest.mark.parametrize("n,k,g", SHAPES)
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8, 9, 12, 16])
def test_linear_fused_matches_oracle_and_two_launches(m, n, k, g):
    """Where the fused kernel applies (rows x blocks per wave within its
    register budget) it is forced; elsewhere the automatic path runs."""
    w = synth.weights(n, k, seed=500 + n + k + g, dist="student_t4")
    a = synth.activations(m, k, seed=600 + m + k)
    out = ref.linear(a, w, g)
    blob = w4.pack(w, g)
    fused = _fused_applies(m, n, k, g)
    log(f"linear {'fused' if fused else 'auto'} m={m} n={n} k={k} g={g}")
    y, a8, s_a, acc = _run_linear(a, blob, n, k, g, variant=3 if fused else 0)
    assert np.array_equal(s_a.view(np.uint16), out["s_a"].view(np.uint16))
    assert np.array_equal(a8, out["a8"])
    assert np.array_equal(acc, out["acc"])
    assert ref.y_tolerance_ok(y, out["y"]).all()
    log(f"two launches m={m} n={n} k={k} g={g}")
    y2, acc2 = _run_two_launch(a, blob, n, k, g)
    assert np.array_equal(acc2, acc)
    assert np.array_equal(y2.view(np.uint16), y.view(np.uint16))


@pytest.mark.parametrize("n_tiles,k_split,workgroups", [
    (1, 1, 0), (1, 8, 0), (2, 3, 0), (2, 5, 0), (2, 2, 0),
    (1, 8, 1), (2, 2, 3), (1, 4, 7), (2, 8, 2), (2, 1, 10), (1, 2, 64)])
def test_linear_fused_every_shape(n_tiles, k_split, workgroups):
    """Every column-tile count, K split (including waves without blocks) and
    persistent grid (one workgroup for all groups, ragged group counts per
    workgroup, more workgroups than groups) gives the oracle's result."""
    n, k, g, m = 320, 2048, 32, 4
    w = synth.weights(n, k, seed=71, dist="student_t4")
    a = synth.activations(m, k, seed=72)
    out = ref.linear(a, w, g)
    log(f"linear fused n_tiles={n_tiles} k_split={k_split} workgroups={workgroups}")
    y, a8, s_a, acc = _run_linear(a, w4.pack(w, g), n, k, g, variant=3, n_tiles=n_tiles,
                                  k_split=k_split, workgroups=workgroups)
    assert np.array_equal(a8, out["a8"])
    assert np.array_equal(acc, out["acc"])
    assert ref.y_tolerance_ok(y, out["y"]).all()


@pytest.mark.parametrize("m,n,k,g,workgroups", [
    (16, 4112, 4096, 128, 0), (16, 4112, 4096, 128, 100), (11, 1040, 4096, 64, 7),
    (4, 4096, 14336, 128, 0), (8, 2064, 8192, 128, 50), (13, 272, 2048, 1, 3),
    (2, 6144, 4096, 1, 0), (4, 528, 16384, 0, 0), (3, 1040, 8192, 64, 0)])
def test_linear_fused_up_to_16_rows(m, n, k, g, workgroups):
    """Up to 16 tokens, long wave ranges (16 blocks; per-row groups over 2048 k
    per wave, the widest partial sums), codebook weights, and persistent
    grids: A8, s_a and acc bit-exact with the oracle."""
    w = synth.weights(n, k, seed=131 + m, dist="student_t4")
    a = synth.activations(m, k, seed=132 + m)
    assert _fused_applies(m, n, k, g, workgroups=workgroups)
    out = ref.linear(a, w, g)
    log(f"linear fused m={m} n={n} k={k} g={g} workgroups={workgroups}")
    y, a8, s_a, acc = _run_linear(a, w4.pack(w, g), n, k, g, variant=3, workgroups=workgroups)
    assert np.array_equal(s_a.view(np.uint16), out["s_a"].view(np.uint16))
    assert np.array_equal(a8, out["a8"])
    assert np.array_equal(acc, out["acc"])
    assert ref.y_tolerance_ok(y, out["y"]).all()


@pytest.mark.parametrize("m,n,k,g", [(16, 16400, 4096, 128), (3, 8208, 4096, 64)])
def test_linear_auto_paired_tiles_ragged(m, n, k, g):
    """The automatic plan's two column tiles per group (layers of more than
    512 tiles above 2 tokens; 16 tokens only on 1024+ tiles) with an odd tile
    count, so the last group holds one tile: one fused launch, bit-exact
    with the oracle."""
    assert int(w4.lib.w4a8_linear_launches(m, n, k, g, None)) == 1
    w = synth.weights(n, k, seed=151 + m, dist="student_t4")
    a = synth.activations(m, k, seed=152 + m)
    out = ref.linear(a, w, g)
    log(f"linear auto paired tiles m={m} n={n} k={k} g={g}")
    y, a8, s_a, acc = _run_linear(a, w4.pack(w, g), n, k, g)
    assert np.array_equal(s_a.view(np.uint16), out["s_a"].view(np.uint16))
    assert np.array_equal(a8, out["a8"])
    assert np.array_equal(acc, out["acc"])
    assert ref.y_tolerance_ok(y, out["y"]).all()


@pytest.mark.parametrize("m,n,k,g", [(64, 4096, 14336, 128), (33, 1040, 16384, 64),
                                     (48, 2048, 8192, 0), (40, 528, 12288, 32), (96, 1040, 8192, 64)])
def test_linear_auto_small_m_k_split(m, n, k, g):
    """17..128 tokens with long K: the automatic plan splits K over
    workgroups of 64 x 128 tiles (quantizer, GEMM, reduction); ragged column
    tiles, per-row and 32-wide groups; bit-exact with the oracle."""
    assert int(w4.lib.w4a8_linear_launches(m, n, k, g, None)) == 3
    w = synth.weights(n, k, seed=171 + m, dist="student_t4")
    a = synth.activations(m, k, seed=172 + m)
    out = ref.linear(a, w, g)
    log(f"linear auto split m={m} n={n} k={k} g={g}")
    y, a8, s_a, acc = _run_linear(a, w4.pack(w, g), n, k, g)
    assert np.array_equal(a8, out["a8"])
    assert np.array_equal(acc, out["acc"])
    assert ref.y_tolerance_ok(y, out["y"]).all()


def test_linear_fused_rounding_ties():
    """Rows built so that A * (1 / s_a) lands on every half-integer and near
    the clamp: s_a = 1 (absmax 127), 2 (absmax 254) and an inexact scale."""
    n, k, g = 64, 2048, 128
    rng = np.random.default_rng(141)
    rows = []
    for amax in (127.0, 254.0, 100.0, 1000.0):
        halves = np.arange(-2 * amax, 2 * amax + 1) / 2.0            # every multiple of 0.5
        row = rng.choice(halves, size=k).astype(np.float16)
        row[rng.integers(k)] = np.float16(amax)
        rows.append(row)
    a = np.stack(rows)
    w = synth.weights(n, k, seed=142)
    out = ref.linear(a, w, g)
    log("linear fused rounding ties")
    y, a8, s_a, acc = _run_linear(a, w4.pack(w, g), n, k, g, variant=3)
    assert np.array_equal(s_a.view(np.uint16), out["s_a"].view(np.uint16))
    assert np.array_equal(a8, out["a8"])
    assert np.array_equal(acc, out["acc"])


@pytest.mark.parametrize("m", [3, 70])
def test_linear_max_depth(m):
    """The whole layer at K = W4A8_K_MAX (131072): quantizer rows of 16384
    chunks, then the skinny (M = 3) or K-split tiled (M = 70) GEMM."""
    n, k, g = 48, 131072, 64
    w = synth.weights(n, k, seed=71, dist="student_t4")
    a = synth.activations(m, k, seed=72 + m)
    out = ref.linear(a, w, g)
    blob = w4.pack(w, g)
    log(f"linear max depth m={m} k={k}")
    y, a8, s_a, acc = _run_linear(a, blob, n, k, g, variant=0)
    assert np.array_equal(s_a.view(np.uint16), out["s_a"].view(np.uint16))
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


@pytest.mark.parametrize("m,n,k,g", [(16, 256, 14336, 128), (17, 64, 512, 128), (100, 272, 768, 64),
                                     (4, 64, 131072, 128)])
def test_linear_two_launch_path(m, n, k, g):
    """Where the fused kernel does not apply (more than 16 rows, rows x
    blocks per wave beyond its register budget, or a wave range longer than
    16 blocks), the same call runs quantizer + GEMM."""
    assert not _fused_applies(m, n, k, g)
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
    runs them: A8/s_a bit-exact with the oracle, acc bit-exact and Y within
    tolerance of the oracle on 64 sampled columns (plus the first and last
    and both ends of a middle 16-column tile), and Y and acc identical to the
    two-launch path on every output."""
    layer, n, k, g, dist = key
    w = synth.weights(n, k, seed=synth.weight_seed(cfg_idx, shape_idx, 0), dist=dist)
    blob = w4.pack(w, g)
    rng = np.random.default_rng(500 + shape_idx)
    mid = (n // 32) * 16
    cols = np.unique(np.concatenate([[0, n - 1, mid, mid + 15], rng.choice(n, 64, replace=False)]))
    qw = ref.quantize_weights(w[cols], g)
    del w
    w8hat = ref.decoded_weights(qw)
    for mi, m in enumerate(ms):
        a = synth.activations(m, k, seed=synth.act_seed(cfg_idx, shape_idx, mi))
        log(f"linear full-size {layer} m={m} n={n} k={k}")
        y, a8, s_a, acc = _run_linear(a, blob, n, k, g)
        want_a8, want_sa = ref.quant_act(a)
        assert np.array_equal(s_a.view(np.uint16), want_sa.view(np.uint16))
        assert np.array_equal(a8, want_a8)
        acc_ref = ref.gemm_acc(want_a8, w8hat)
        assert np.array_equal(acc[:, cols], acc_ref)
        assert ref.y_tolerance_ok(y[:, cols], ref.epilogue(acc_ref, want_sa, qw["s1"])).all()
        y2, acc2 = _run_two_launch(a, blob, n, k, g)
        assert np.array_equal(acc, acc2)
        assert np.array_equal(y.view(np.uint16), y2.view(np.uint16))
