"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: A8, s_a and the int32 accumulators bit-exact; Y within
1e-3 * |Y_ref| + 1 fp16 ulp of the oracle's single-rounding epilogue.
"""
import numpy as np
import pytest

import synth
import w4a8_gemm_amd as w4
from gpu_util import device, log, run_gemm, run_quant_act
from oracle import ref

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------ activation quantizer
@pytest.mark.parametrize("m,k", [(1, 4096), (16, 14336), (37, 1000), (5, 8), (3, 7),
                                 (64, 4096), (2, 24576), (300, 136),
                                 (3, 16392), (4, 32768), (2, 32776),   # 16-chunk rows and past them
                                 (2, 131072)])                         # the deepest K the GEMM takes
def test_quant_act_bit_exact(m, k):
    a = synth.activations(m, k, seed=m * 7 + k)
    log(f"quant_act m={m} k={k}")
    a8, s_a = run_quant_act(a)
    want_a8, want_sa = ref.quant_act(a)
    assert np.array_equal(s_a.view(np.uint16), want_sa.view(np.uint16))
    assert np.array_equal(a8, want_a8)


def test_quant_act_exhaustive_fp16_scales():
    """Every positive finite fp16 absmax, one token each, bit-exact."""
    bits = np.arange(1, 0x7C00, dtype=np.uint16)
    alpha = bits.view(np.float16)
    rng = np.random.default_rng(3)
    frac = rng.uniform(-1, 1, size=(alpha.size, 63)).astype(np.float32)
    a = np.empty((alpha.size, 64), dtype=np.float16)
    a[:, 0] = alpha
    a[:, 1:] = (frac * alpha.astype(np.float32)[:, None]).astype(np.float16)
    log(f"quant_act exhaustive scales m={alpha.size}")
    a8, s_a = run_quant_act(a)
    want_a8, want_sa = ref.quant_act(a)
    assert np.array_equal(s_a.view(np.uint16), want_sa.view(np.uint16))
    assert np.array_equal(a8, want_a8)


def test_quant_act_every_fp16_value():
    """Every finite fp16 value quantized under five scales (s_a = 1, 2, 0.5,
    an inexact one and the largest), so that A * (1 / s_a) meets every
    half-integer tie and the clamp: A8 bit-exact."""
    vals = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16).view(np.float16)
    vals = vals[np.isfinite(vals)]
    rows = []
    for amax in (127.0, 254.0, 63.5, 100.0, 65504.0):
        row = vals[np.abs(vals.astype(np.float32)) <= amax]
        row = np.concatenate([row, [np.float16(amax)]])
        rows.append(row)
    k = max(r.size for r in rows)
    a = np.zeros((len(rows), k), dtype=np.float16)
    for i, r in enumerate(rows):
        a[i, :r.size] = r
    log(f"quant_act every fp16 value m={a.shape[0]} k={k}")
    a8, s_a = run_quant_act(a)
    want_a8, want_sa = ref.quant_act(a)
    assert np.array_equal(s_a.view(np.uint16), want_sa.view(np.uint16))
    assert np.array_equal(a8, want_a8)


def test_quant_act_zero_rows_and_ties():
    a = np.zeros((4, 256), dtype=np.float16)
    a[1, :8] = [127, 2.5, -3.5, 0.5, -0.5, 1.5, 0, -127]
    a[2, 100] = -65504.0
    a[3, :] = 1e-7
    log("quant_act zero rows and ties")
    a8, s_a = run_quant_act(a)
    want_a8, want_sa = ref.quant_act(a)
    assert np.array_equal(s_a.view(np.uint16), want_sa.view(np.uint16))
    assert np.array_equal(a8, want_a8)
    assert not a8[0].any() and float(s_a[0]) == 0


def test_quant_act_strided_rows():
    import torch
    dev = torch.device("cuda:0")
    a_full = synth.activations(9, 520, seed=5)
    a = torch.from_numpy(a_full).to(dev)[:, :512]          # lda = 520 > k
    a8 = torch.zeros((9, 528), dtype=torch.int8, device=dev)
    s_a = torch.empty(9, dtype=torch.float16, device=dev)
    log("quant_act strided lda=520 lda8=528")
    w4.quant_act(a, a8=a8[:, :512], s_a=s_a)
    torch.cuda.synchronize()
    want_a8, want_sa = ref.quant_act(a_full[:, :512])
    assert np.array_equal(a8[:, :512].cpu().numpy(), want_a8)
    assert not a8[:, 512:].cpu().numpy().any()              # padding untouched
    assert np.array_equal(s_a.cpu().numpy().view(np.uint16), want_sa.view(np.uint16))


@pytest.mark.parametrize("scale", [0.0, 6e-08, 0.001, 0.05, 3.0, 1000.0])
@pytest.mark.parametrize("m,k", [(1, 4096), (16, 14336), (37, 1000), (3, 7), (5, 8), (2, 24576)])
def test_quant_act_static_bit_exact(m, k, scale):
    """Static per-tensor scale: A8 and s_a bit-exact with the oracle, on the
    vector and the scalar path, with scales that clamp everything, nothing,
    or flush everything to 0."""
    import torch
    dev = device()
    a = synth.activations(m, k, seed=m * 7 + k)
    s = np.float16(scale)
    log(f"quant_act_static m={m} k={k} scale={float(s)!r}")
    a8, s_a = w4.quant_act_static(torch.from_numpy(a).to(dev), float(s))
    torch.cuda.synchronize()
    want_a8, want_sa = ref.quant_act_static(a, s)
    assert np.array_equal(s_a.cpu().numpy().view(np.uint16), want_sa.view(np.uint16))
    assert np.array_equal(a8.cpu().numpy(), want_a8)


def test_quant_act_static_then_gemm():
    """The GEMM consumes the static scales unchanged."""
    m, n, k, g = 24, 272, 1152, 64
    w = synth.weights(n, k, seed=31, dist="student_t4")
    a = synth.activations(m, k, seed=32)
    s = np.float16(0.125)
    qw = ref.quantize_weights(w, g)
    want_a8, want_sa = ref.quant_act_static(a, s)
    acc_ref = ref.gemm_acc(want_a8, ref.decoded_weights(qw))
    y_ref = ref.epilogue(acc_ref, want_sa, qw["s1"])
    import torch
    dev = device()
    log("quant_act_static + gemm")
    a8, s_a = w4.quant_act_static(torch.from_numpy(a).to(dev), float(s))
    y, acc = w4.gemm(a8, s_a, w4.to_device(w4.pack(w, g), dev), n, k, g, want_acc=True)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    assert ref.y_tolerance_ok(y.cpu().numpy(), y_ref).all()


# ------------------------------------------------------------ GEMM, whole outputs
SMALL = [
    # m, n, k, g, dist
    (16, 256, 512, 128, "normal"),          # the tiny workload
    (1, 48, 384, 64, "normal"),
    (3, 272, 640, 32, "student_t4"),
    (17, 80, 1024, 128, "normal"),
    (33, 112, 256, 0, "student_t4"),
    (64, 512, 1152, 128, "normal"),
    (65, 320, 512, 128, "normal"),
    (100, 1040, 768, 64, "student_t4"),
    (130, 48, 128, 32, "normal"),
    (256, 512, 1024, 0, "normal"),
]


def _layer(m, n, k, g, dist, seed):
    w = synth.weights(n, k, seed=seed, dist=dist)
    a = synth.activations(m, k, seed=seed + 1)
    return w, a, ref.linear(a, w, g)


@pytest.mark.parametrize("m,n,k,g,dist", SMALL)
def test_gemm_auto_bit_exact(m, n, k, g, dist):
    w, a, out = _layer(m, n, k, g, dist, seed=m + n + k + g)
    blob = w4.pack(w, g)
    log(f"gemm auto m={m} n={n} k={k} g={g}")
    y, acc = run_gemm(out["a8"], out["s_a"], blob, n, k, g)
    assert np.array_equal(acc, out["acc"])
    assert ref.y_tolerance_ok(y, out["y"]).all()


@pytest.mark.parametrize("k_split", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("m,n,k,g", [(16, 256, 512, 128), (5, 96, 1152, 32), (40, 64, 384, 0)])
def test_gemm_skinny_every_split_identical(m, n, k, g, k_split):
    w, a, out = _layer(m, n, k, g, "normal", seed=11 + m)
    blob = w4.pack(w, g)
    mr = 1 if m <= 16 else (2 if m <= 32 else 4)
    assert k_split * mr <= 64                      # n < 32768: one column tile per wave
    log(f"gemm skinny m={m} n={n} k={k} g={g} k_split={k_split}")
    y, acc = run_gemm(out["a8"], out["s_a"], blob, n, k, g, variant=1, k_split=k_split)
    assert np.array_equal(acc, out["acc"])
    assert ref.y_tolerance_ok(y, out["y"]).all()


@pytest.mark.parametrize("g", [32, 64, 128, 0])
@pytest.mark.parametrize("k_split", [1, 2])
@pytest.mark.parametrize("m", [1, 16, 33, 64])
def test_gemm_skinny_long_wave_ranges(m, g, k_split):
    """Each wave streams many blocks through its ring (steady state runs
    several times), for every group size: the ring's meta reuse must hold."""
    n, k = 96, 2688                                  # 21 k-blocks: ragged last group
    w, a, out = _layer(m, n, k, g, "student_t4", seed=300 + m + g)
    blob = w4.pack(w, g)
    log(f"gemm skinny long ranges m={m} n={n} k={k} g={g} k_split={k_split}")
    for nt in (1, 2, 4):
        if m > 16 and nt == 4:
            continue
        y, acc = run_gemm(out["a8"], out["s_a"], blob, n, k, g, variant=1, k_split=k_split,
                          n_tiles=nt)
        assert np.array_equal(acc, out["acc"]), f"n_tiles={nt}"
        assert ref.y_tolerance_ok(y, out["y"]).all()


@pytest.mark.parametrize("m,n,k,g", [(1, 64, 256, 128), (48, 96, 640, 64), (64, 4096, 512, 32),
                                     (200, 272, 2688, 128), (130, 1040, 1152, 0),
                                     (300, 528, 1408, 64), (513, 4112, 640, 128)])
def test_gemm_tiled_every_tile_shape(m, n, k, g):
    """Every tiled kernel shape (row tiles per wave, column tiles per wave,
    row groups per workgroup, stages) on ragged M and N edges."""
    w, a, out = _layer(m, n, k, g, "student_t4", seed=90 + m)
    blob = w4.pack(w, g)
    for mt, nt, rg, st, ks in ((0, 0, 0, 0, 0), (4, 4, 1, 2, 0), (4, 4, 1, 3, 0), (8, 4, 1, 2, 0),
                               (8, 4, 1, 3, 0), (8, 2, 1, 3, 0), (8, 4, 2, 0, 0), (8, 4, 1, 0, 2),
                               (4, 4, 1, 0, 2),
                               # deeper pipelines (more stages than k-blocks at k = 256) and
                               # 64 x 128 tiles
                               (8, 4, 1, 4, 0), (4, 4, 1, 4, 0), (4, 4, 1, 5, 0), (8, 2, 1, 2, 0),
                               (8, 2, 1, 4, 0), (8, 2, 1, 5, 0), (8, 2, 1, 6, 0), (4, 2, 1, 2, 0),
                               (4, 2, 1, 3, 0), (4, 2, 1, 4, 0), (4, 2, 1, 6, 0), (4, 2, 1, 8, 0),
                               # two k-groups on 128-column tiles
                               (8, 2, 1, 2, 2), (8, 2, 1, 3, 2), (4, 2, 1, 2, 2), (4, 2, 1, 3, 2),
                               (4, 2, 1, 4, 2)):
        log(f"gemm tiled m={m} n={n} k={k} g={g} m_tiles={mt} n_tiles={nt} row_groups={rg} "
            f"stages={st} k_split={ks}")
        y, acc = run_gemm(out["a8"], out["s_a"], blob, n, k, g, variant=2, m_tiles=mt,
                          n_tiles=nt, row_groups=rg, stages=st, k_split=ks)
        assert np.array_equal(acc, out["acc"]), (mt, nt, rg, st, ks)
        assert ref.y_tolerance_ok(y, out["y"]).all()


@pytest.mark.parametrize("m,n,k,g", [(130, 1040, 1152, 0), (300, 528, 2688, 64), (77, 256, 640, 32)])
def test_gemm_tiled_k_slices_exact(m, n, k, g):
    """K split over workgroups: int32 partials through a caller workspace that
    starts out full of garbage, ragged last slice, with and without k-groups."""
    import torch
    w, a, out = _layer(m, n, k, g, "student_t4", seed=700 + m)
    blob = w4.pack(w, g)
    dev = device()
    a8 = torch.from_numpy(out["a8"]).to(dev)
    s_a = torch.from_numpy(out["s_a"]).to(dev)
    wdev = w4.to_device(blob, dev)
    kblocks = k // 128
    for sl, mt, nt, st, ks in ((2, 8, 0, 0, 0), (3, 4, 0, 0, 0), (5, 8, 0, 0, 2),
                               (min(kblocks, 16), 4, 0, 0, 2), (16, 8, 0, 0, 0),
                               (2, 8, 2, 6, 0), (3, 4, 2, 8, 0), (4, 4, 4, 5, 0), (3, 4, 2, 4, 2)):
        ws = torch.full((16 * m * n * 4 + 64,), 0x5A, dtype=torch.uint8, device=dev)
        log(f"gemm tiled slices={sl} m={m} n={n} k={k} g={g} m_tiles={mt} n_tiles={nt} "
            f"stages={st} k_split={ks}")
        y, acc = w4.gemm(a8, s_a, wdev, n, k, g, want_acc=True, variant=2, m_tiles=mt,
                         n_tiles=nt, stages=st, k_split=ks, slices=sl, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(acc.cpu().numpy(), out["acc"]), (sl, mt, nt, st, ks)
        assert ref.y_tolerance_ok(y.cpu().numpy(), out["y"]).all()
    # the 256 x 256 ping-pong kernel with its K split over workgroups
    for sl in (2, 3, min(kblocks, 5)):
        ws = torch.full((16 * m * n * 4 + 64,), 0x5A, dtype=torch.uint8, device=dev)
        log(f"gemm ping-pong slices={sl} m={m} n={n} k={k} g={g}")
        y, acc = w4.gemm(a8, s_a, wdev, n, k, g, want_acc=True, variant=2, row_groups=2,
                         slices=sl, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(acc.cpu().numpy(), out["acc"]), ("ping-pong", sl)
        assert ref.y_tolerance_ok(y.cpu().numpy(), out["y"]).all()


def test_gemm_extreme_operands():
    """A8 = +-127 and decoded weights at the int8 extremes over the deepest K."""
    n, k, g = 32, 24576, 128
    w = np.zeros((n, k), dtype=np.float32)
    w[0::2] = 1.0                                   # W8 = 119 everywhere
    w[1::2] = -1.0
    w[2, :] = np.tile(np.array([-1.0, 1.0], np.float32), k // 2)
    blob = w4.pack(w, g)
    qw = ref.quantize_weights(w, g)
    w8hat = ref.decoded_weights(qw)
    a8 = np.full((3, k), 127, dtype=np.int8)
    a8[1] = -127
    a8[2, ::2] = -127
    s_a = np.ones(3, dtype=np.float16) * np.float16(2 ** -10)
    acc_ref = ref.gemm_acc(a8, w8hat)
    log("gemm extreme operands k=24576")
    y, acc = run_gemm(a8, s_a, blob, n, k, g)
    assert np.array_equal(acc, acc_ref)


@pytest.mark.parametrize("m", [1, 5, 80])
def test_gemm_max_depth_extremes(m):
    """K = W4A8_K_MAX (131072) with A8 = +-127 against decoded weights of
    +-120 and +-112: sums reach 127 * 120 * 131072 (about 2.0e9, just under
    2^31) and must stay exact.  M = 1 and 5 take the skinny kernel with long
    wave ranges, M = 80 the tiled kernel with K split over workgroups."""
    n, k, g = 32, 131072, 128
    w = np.ones((n, k), dtype=np.float32)        # W8 = 119 -> s2 = 8, q = 15: 120
    w[1::2] = -1.0
    w[2, 1::2] = -1.0                            # +-119 in one group: s2 = 16, z = 7: +-112
    blob = w4.pack(w, g)
    qw = ref.quantize_weights(w, g)
    w8hat = ref.decoded_weights(qw)
    assert w8hat[0].min() == 120 and w8hat[2].max() == 112 and w8hat[2].min() == -112
    a8 = np.full((m, k), 127, dtype=np.int8)
    a8[1::2] = -127
    s_a = np.full(m, 2.0 ** -14, dtype=np.float16)
    acc_ref = ref.gemm_acc(a8, w8hat)
    assert np.abs(acc_ref).max() == 127 * 120 * k
    log(f"gemm max depth m={m} k={k}")
    y, acc = run_gemm(a8, s_a, blob, n, k, g)
    assert np.array_equal(acc, acc_ref)
    assert ref.y_tolerance_ok(y, ref.epilogue(acc_ref, s_a, qw["s1"])).all()


def test_gemm_zero_token_and_strided_output():
    import torch
    m, n, k, g = 20, 160, 512, 64
    w, a, out = _layer(m, n, k, g, "normal", seed=123)
    a = a.copy()
    a[4] = 0
    out = ref.linear(a, w, g)
    blob = w4.pack(w, g)
    dev = torch.device("cuda:0")
    a8 = torch.zeros((m, k + 32), dtype=torch.int8, device=dev)
    a8[:, :k] = torch.from_numpy(out["a8"]).to(dev)
    s_a = torch.from_numpy(out["s_a"]).to(dev)
    y = torch.full((m, n + 8), -1.0, dtype=torch.float16, device=dev)
    acc = torch.zeros((m, n + 4), dtype=torch.int32, device=dev)
    wdev = w4.to_device(blob, dev)
    log("gemm strided lda8/ldy/ldacc with a zero token")
    w4.gemm(a8[:, :k], s_a, wdev, n, k, g, y=y[:, :n], acc=acc[:, :n])
    torch.cuda.synchronize()
    y_np, acc_np = y.cpu().numpy(), acc.cpu().numpy()
    assert np.array_equal(acc_np[:, :n], out["acc"])
    assert ref.y_tolerance_ok(y_np[:, :n], out["y"]).all()
    assert (y_np[:, n:] == -1.0).all() and not acc_np[:, n:].any()
    assert not y_np[4, :n].any()


def test_gemm_empty_batch_is_noop():
    import torch
    dev = torch.device("cuda:0")
    w = synth.weights(64, 256, seed=1)
    blob = w4.to_device(w4.pack(w, 128), dev)
    a8 = torch.zeros((0, 256), dtype=torch.int8, device=dev)
    s_a = torch.zeros((0,), dtype=torch.float16, device=dev)
    y = w4.gemm(a8, s_a, blob, 64, 256, 128)
    assert tuple(y.shape) == (0, 64)


# ------------------------------------------------------------ full sizes, sampled
def _full_runs():
    runs = []
    for cfg_idx, (name, items) in enumerate(synth.workloads().items()):
        if name == "tiny" or name in synth.COMPOSITE:
            continue
        layers = {}
        for (_, m, layer, n, k, g, dist) in items:
            layers.setdefault((layer, n, k, g, dist), []).append(m)
        for shape_idx, (key, ms) in enumerate(layers.items()):
            runs.append(pytest.param(cfg_idx, shape_idx, key, ms, id=f"{name}-{key[0]}-g{key[3]}"))
    return runs


@pytest.mark.parametrize("cfg_idx,shape_idx,key,ms", _full_runs())
def test_gemm_full_size_sampled(cfg_idx, shape_idx, key, ms):
    """Every full-size run: whole A8/s_a bit-exact, acc bit-exact and Y within
    tolerance on 64 sampled columns (plus the first and last), all rows."""
    import torch
    layer, n, k, g, dist = key
    dev = torch.device("cuda:0")
    w = synth.weights(n, k, seed=synth.weight_seed(cfg_idx, shape_idx, 0), dist=dist)
    blob = w4.pack(w, g)
    wdev = w4.to_device(blob, dev)
    rng = np.random.default_rng(cfg_idx * 100 + shape_idx)
    cols = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 64, replace=False)]))
    qw = ref.quantize_weights(w[cols], g)
    del w
    w8hat = ref.decoded_weights(qw)
    for mi, m in enumerate(ms):
        a = synth.activations(m, k, seed=synth.act_seed(cfg_idx, shape_idx, mi))
        log(f"full-size {layer} m={m} n={n} k={k} g={g}")
        a_dev = torch.from_numpy(a).to(dev)
        a8, s_a = w4.quant_act(a_dev)
        y, acc = w4.gemm(a8, s_a, wdev, n, k, g, want_acc=True)
        torch.cuda.synchronize()
        idx = torch.from_numpy(cols).to(dev)
        y_s = y.index_select(1, idx).cpu().numpy()
        acc_s = acc.index_select(1, idx).cpu().numpy()
        a8_np, s_a_np = a8.cpu().numpy(), s_a.cpu().numpy()
        del y, acc, a8, s_a, a_dev
        want_a8, want_sa = ref.quant_act(a)
        assert np.array_equal(s_a_np.view(np.uint16), want_sa.view(np.uint16))
        assert np.array_equal(a8_np, want_a8)
        acc_ref = ref.gemm_acc(want_a8, w8hat)
        assert np.array_equal(acc_s, acc_ref)
        y_ref = ref.epilogue(acc_ref, want_sa, qw["s1"])
        assert ref.y_tolerance_ok(y_s, y_ref).all()
