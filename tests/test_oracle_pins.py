"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each check is a function of the implementation under test, so the mutation
tests at the bottom can show that a plausible mistake planted in a copy of
the oracle fails at least one pin.
"""
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------ independent helpers
def half_of_fraction(x: Fraction) -> float:
    """IEEE binary16 round-half-even of an exact rational (independent of numpy)."""
    if x == 0:
        return 0.0
    sign = -1 if x < 0 else 1
    ax = abs(x)
    e = 0
    while ax >= Fraction(2) ** (e + 1):
        e += 1
    while ax < Fraction(2) ** e:
        e -= 1
    e = max(e, -14)                     # subnormals share the 2**-24 quantum
    quantum = Fraction(2) ** (e - 10)
    n = round(ax / quantum)             # Fraction.__round__ is half-to-even
    v = n * quantum
    if v > 65504:
        return sign * float("inf")
    return sign * float(v)


def half_bits_struct(x: float) -> int:
    """binary16 bits of a float via Python's struct (round-half-even)."""
    return struct.unpack("<H", struct.pack("<e", x))[0]


def read_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            rows.append(line)
    return rows


# ------------------------------------------------------------ rational rounding
def test_rne_ratio_matches_fraction_round():
    nums = np.arange(-300, 301)
    for den in range(1, 21):
        got = ref.rne_ratio(nums, den)
        want = [round(Fraction(int(n), den)) for n in nums]
        assert got.tolist() == want


def test_ceil_ratio():
    for num in range(-50, 260):
        for den in (1, 2, 7, 15):
            assert ref.ceil_ratio(num, den) == -((-num) // den)
            assert ref.ceil_ratio(num, den) == int(np.ceil(Fraction(num, den)))


# ------------------------------------------------------------ fp16 conversions
def test_to_f16_matches_exact_rational_rounding():
    rng = np.random.default_rng(5)
    vals = np.concatenate([
        rng.standard_normal(3000).astype(np.float32) * np.float32(10.0) ** rng.integers(-8, 5, 3000),
        np.array([1 + 2 ** -11, 1 + 3 * 2 ** -11, 2 ** -25, 3 * 2 ** -25, 65519.0, 65520.0,
                  2 ** -14 * (1 - 2 ** -11)], dtype=np.float32)])
    got = ref.to_f16(vals.astype(np.float32)).astype(np.float64)
    for v, g in zip(vals, got):
        want = half_of_fraction(Fraction(float(v)))
        assert g == want or (np.isinf(g) and np.isinf(want)), (v, g, want)


# ------------------------------------------------------------ O2 level 2
def level2_domain_check(level2, limit=119, decode=ref.decode):
    """Exhaustive over every (lo, hi, w8) with -limit <= lo <= 0 <= hi <= limit.

    A level-2 result for one element depends only on its group's lo, hi and
    on its own value, so groups [lo, hi, lo..hi] cover the whole domain.
    Returns the number of violations of: s2 in [1,16], z in [0,15],
    q in [0,15], decode in int8, and |w8 - decode| <= s2/2 (where unclamped).
    The decoded values come from `decode` (the oracle's own by default), with
    each group as one row of one group.
    """
    width = 2 * limit + 3
    los, his = np.meshgrid(np.arange(-limit, 1), np.arange(0, limit + 1), indexing="ij")
    los = los.ravel()
    his = his.ravel()
    offs = np.arange(width - 2)
    vals = los[:, None] + offs[None, :]
    vals = np.minimum(vals, his[:, None])           # pad with hi (inside the group)
    groups = np.concatenate([los[:, None], his[:, None], vals], axis=1)
    s2, z, q = level2(groups)
    s2 = s2.astype(np.int64)
    z = z.astype(np.int64)
    q = q.astype(np.int64)
    dec = np.asarray(decode(q, z[:, None], s2[:, None], groups.shape[1]), dtype=np.int64)
    bad = 0
    bad += int(np.sum((s2 < 1) | (s2 > 16)))
    bad += int(np.sum((z < 0) | (z > 15)))
    bad += int(np.sum((q < 0) | (q > 15)))
    bad += int(np.sum((dec < -128) | (dec > 127)))
    err = np.abs(groups - dec)
    # a clamp to 15 can add one extra step; otherwise the error is <= s2/2
    unclamped = q < 15
    bad += int(np.sum((2 * err > s2[:, None]) & unclamped))
    bad += int(np.sum(err > s2[:, None] + s2[:, None] // 2))
    return bad


def test_level2_exhaustive_domain():
    assert level2_domain_check(ref.level2_groups) == 0


def test_level1_range_119_is_the_widest_safe_range():
    # The +-119 reading: every decode stays in int8 at 119, not at 120.
    assert level2_domain_check(ref.level2_groups, limit=119) == 0
    assert level2_domain_check(ref.level2_groups, limit=120) > 0


def level2_golden_check(level2):
    bad = []
    for line in read_rows("level2_cases.txt"):
        lo, hi, w8, s2_w, z_w, q_w, dec_w = (int(t) for t in line.split())
        group = np.array([[lo, hi, w8]])
        s2, z, q = level2(group)
        dec = (int(q[0, 2]) - int(z[0])) * int(s2[0])
        if (int(s2[0]), int(z[0]), int(q[0, 2]), dec) != (s2_w, z_w, q_w, dec_w):
            bad.append((line, int(s2[0]), int(z[0]), int(q[0, 2]), dec))
    return bad


def test_level2_golden():
    assert level2_golden_check(ref.level2_groups) == []


def test_level2_identity_special_case():
    # W8 in [0, 15] -> s2 = 1, z = 0, q = W8: decode is the identity.
    rng = np.random.default_rng(0)
    g = rng.integers(0, 16, size=(100, 128))
    g[:, 0] = 15
    s2, z, q = ref.level2_groups(g)
    assert (s2 == 1).all() and (z == 0).all() and (q == g).all()


# ------------------------------------------------------------ decode
def decode_golden_cases():
    """Parse decode_cases.txt into [(name, g, q, z, s2, [(n, k, q, want)])]."""
    cases = []
    for line in read_rows("decode_cases.txt"):
        tok = line.split()
        if tok[0] == "case":
            g, k, n = int(tok[2]), int(tok[3]), int(tok[4])
            groups = k // g
            rows = np.arange(n)[:, None]
            cols = np.arange(k)[None, :]
            q = ((5 * cols + 3 * rows) % 16).astype(np.uint8)
            z = np.full((n, groups), 255, dtype=np.uint8)     # every row is listed
            s2 = np.zeros((n, groups), dtype=np.uint8)
            cases.append([tok[1], g, q, z, s2, []])
        elif tok[0] == "zs":
            r = int(tok[1])
            zs, s2s = " ".join(tok[2:]).split("|")
            cases[-1][3][r] = [int(t) for t in zs.split()]
            cases[-1][4][r] = [int(t) for t in s2s.split()]
        else:
            cases[-1][5].append(tuple(int(t) for t in tok))
    return cases


def decode_golden_check(decode):
    """Mismatches of decode(q, z, s2, g) against the hand-worked values."""
    bad = []
    for name, g, q, z, s2, points in decode_golden_cases():
        assert (z != 255).all(), name
        dec = np.asarray(decode(q, z, s2, g))
        assert dec.shape == q.shape, name
        for n, k, q_w, want in points:
            if int(q[n, k]) != q_w or int(dec[n, k]) != want:
                bad.append((name, n, k, int(q[n, k]), int(dec[n, k]), want))
    return bad


def test_decode_golden():
    assert decode_golden_check(ref.decode) == []


def dequant_loop_check(decode, gs=(32, 64, 128, 0)):
    """Plain Python loops over the logical arrays alone, element by element:
    W^[n][k] = s1[n] * (q[n][k] - z[n][k // g]) * s2[n][k // g], then the
    dequant-then-matmul Y[m][n] = sum_k (s_a[m] * A8[m][k]) * W^[n][k] in
    exact rationals; `decode` must give the same integers and s_a * s1 *
    (A8 @ decode^T) the same Y.  g = 0 is per-channel (one group per row).
    Returns the number of mismatching values."""
    bad = 0
    n, k, m = 6, 256, 3
    w = synth.weights(n, k, seed=41, dist="student_t4")
    a = synth.activations(m, k, seed=42)
    a8, s_a = ref.quant_act(a)
    for g in gs:
        qw = ref.quantize_weights(w, g)
        q, z, s2, s1 = qw["q"], qw["z"], qw["s2"], qw["s1"]
        geff = k if g == 0 else g
        dec = np.asarray(decode(q, z, s2, geff))
        wq = [[Fraction(float(s1[i])) * (int(q[i, t]) - int(z[i, t // geff])) * int(s2[i, t // geff])
               for t in range(k)] for i in range(n)]
        for i in range(n):
            for t in range(k):
                if Fraction(float(s1[i])) * int(dec[i, t]) != wq[i][t]:
                    bad += 1
        acc = a8.astype(np.int64) @ dec.astype(np.int64).T
        for r in range(m):
            sa = Fraction(float(s_a[r]))
            for i in range(n):
                y = sum(sa * int(a8[r, t]) * wq[i][t] for t in range(k))
                if y != sa * Fraction(float(s1[i])) * int(acc[r, i]):
                    bad += 1
    return bad


def test_dequant_loop_matches_decode():
    assert dequant_loop_check(ref.decode) == 0


def test_decoded_weights_is_decode_of_the_packed_arrays():
    w = synth.weights(8, 256, seed=43)
    for g in (32, 64, 128, 0):
        qw = ref.quantize_weights(w, g)
        geff = 256 if g == 0 else g
        assert qw["g_eff"] == geff
        assert np.array_equal(ref.decoded_weights(qw), ref.decode(qw["q"], qw["z"], qw["s2"], geff))


def _dec_mod_group(q, z, s2, g):               # group index k % G instead of k // g
    k = q.shape[1]
    j = np.arange(k) % z.shape[1]
    return (q.astype(np.int32) - z[:, j].astype(np.int32)) * s2[:, j].astype(np.int32)


def _dec_plus_s2(q, z, s2, g):                 # an extra +s2 offset
    return ref.decode(q, z, s2, g) + np.repeat(s2.astype(np.int32), g, axis=1)


def _dec_neighbour_z(q, z, s2, g):             # z taken from the next group
    zz = np.roll(z, -1, axis=1) if z.shape[1] > 1 else z.astype(np.int32) + 1
    return ref.decode(q, zz, s2, g)


def _dec_unscaled_z(q, z, s2, g):              # q * s2 - z: the zero not scaled
    zz = np.repeat(z.astype(np.int32), g, axis=1)
    ss = np.repeat(s2.astype(np.int32), g, axis=1)
    return q.astype(np.int32) * ss - zz


@pytest.mark.parametrize("mutant", [_dec_mod_group, _dec_plus_s2, _dec_neighbour_z,
                                    _dec_unscaled_z])
def test_decode_pins_catch_mutants(mutant):
    # each plausible decode mistake fails the element-wise pins, not only the
    # whole-layer norm bound
    assert decode_golden_check(mutant) != []
    assert dequant_loop_check(mutant, gs=(32, 0)) > 0
    assert level2_domain_check(ref.level2_groups, decode=mutant) > 0 or mutant is _dec_mod_group


# ------------------------------------------------------------ O1 level 1
def test_level1_golden():
    for line in read_rows("level1_cases.txt"):
        body = line.split(":", 1)[1]
        vals, s1_w, w8_w = (p.split() for p in body.split("|"))
        w = np.array([[float(v) for v in vals]], dtype=np.float32)
        s1, w8 = ref.level1_rows(w)
        assert float(s1[0]) == float(s1_w[0]), line
        assert w8[0].tolist() == [int(t) for t in w8_w], line


def level1_invariant_check(level1, w):
    """Closed-form invariants of level 1 on rows with a normal fp16 scale."""
    s1, w8 = level1(w)
    s = s1.astype(np.float64)
    alpha = np.abs(w).max(axis=1).astype(np.float64)
    problems = 0
    # scale is fp16(fp32(alpha / 119)), checked through an independent rounding
    for i in range(0, w.shape[0], max(1, w.shape[0] // 64)):
        want = half_of_fraction(Fraction(float(np.float32(alpha[i]) / np.float32(119))))
        problems += float(s1[i]) != want
    problems += int(np.sum(np.abs(w8) > 119))
    # absmax element maps to exactly +-119 (fp16 scale off by <= 2**-11 relative)
    arg = np.abs(w).argmax(axis=1)
    top = w8[np.arange(w.shape[0]), arg]
    problems += int(np.sum(np.abs(top) != 119))
    # sign agrees, and reconstruction error <= s1/2 (+ fp32 product rounding)
    recon = s[:, None] * w8
    problems += int(np.sum(np.abs(w - recon) > s[:, None] * (0.5 + 2 ** -10)))
    problems += int(np.sum(np.sign(w8) * np.sign(w) < 0))
    return problems


def test_level1_invariants_random_rows():
    w = synth.weights(512, 256, seed=11)
    assert level1_invariant_check(ref.level1_rows, w) == 0
    w = synth.weights(256, 512, seed=12, dist="student_t4")
    assert level1_invariant_check(ref.level1_rows, w) == 0


def test_level1_zero_row_and_tiny_scale():
    w = np.zeros((3, 64), dtype=np.float32)
    w[1, 3] = 1e-4                      # 1e-4/119: subnormal fp16 scale
    w[2, 5] = 1e-7                      # 1e-7/119 underflows: scale 0, row 0
    s1, w8 = ref.level1_rows(w)
    assert float(s1[0]) == 0 and not w8[0].any()
    assert 0 < float(s1[1]) < 2 ** -14 and abs(w8[1]).max() <= 119
    assert float(s1[2]) == 0 and not w8[2].any()


# ------------------------------------------------------------ O1' per channel
def test_per_channel_invariants():
    w = synth.weights(300, 256, seed=13, dist="student_t4")
    s1, q, z, s2 = ref.per_channel(w)
    assert (s2 == 1).all() and q.max() <= 15 and z.max() <= 15
    s = s1.astype(np.float64)
    dec = q.astype(np.int64) - z.astype(np.int64)
    err = np.abs(w - s[:, None] * dec)
    # unclamped elements: error <= s1/2 (+ fp32 rounding); clamped ones <= 1.5 s1
    assert (err <= s[:, None] * (1.5 + 2 ** -10)).all()
    assert np.mean(err <= s[:, None] * (0.5 + 2 ** -10)) > 0.99
    # zero representable: a zero weight decodes to exactly 0
    w2 = w.copy()
    w2[:, 7] = 0
    s1b, qb, zb, _ = ref.per_channel(w2)
    assert (qb[:, 7].astype(int) == zb[:, 0].astype(int)).all()


def test_per_channel_hand_case():
    # lo = -1.5, hi = 6: (6 + 1.5)/15 = 0.5 -> s1 = 0.5, r = 2, z = rint(3) = 3
    w = np.array([[-1.5, 6.0, 0.25, 0.75, -0.25, 0.0, 1.0, 2.0]], dtype=np.float32)
    s1, q, z, s2 = ref.per_channel(w)
    assert float(s1[0]) == 0.5 and int(z[0, 0]) == 3
    # q = rint(2w) + 3: -3+3, 12+3, rint(0.5)=0 -> 3, rint(1.5)=2 -> 5, rint(-0.5)=0 -> 3, 3, 5, 7
    assert q[0].tolist() == [0, 15, 3, 5, 3, 3, 5, 7]


# ------------------------------------------------------------ O3 activations
def test_act_golden():
    for line in read_rows("act_cases.txt"):
        body = line.split(":", 1)[1]
        vals, s_w, a8_w = (p.split() for p in body.split("|"))
        a = np.array([[float(v) for v in vals]], dtype=np.float16)
        a8, s_a = ref.quant_act(a)
        assert float(s_a[0]) == float(s_w[0]), line
        assert a8[0].tolist() == [int(t) for t in a8_w], line


def act_scale_sweep_check(quant_act):
    """Every positive finite fp16 absmax value, one token each."""
    bits = np.arange(1, 0x7C00, dtype=np.uint16)
    alpha = bits.view(np.float16)
    m = alpha.size
    a = np.zeros((m, 8), dtype=np.float16)
    a[:, 0] = alpha
    a[:, 1] = -(alpha / np.float16(3))
    a[:, 2] = alpha * np.float16(0.5)
    a8, s_a = quant_act(a)
    problems = 0
    # independent scale: fp16 of the fp32 quotient, through struct
    q32 = alpha.astype(np.float32) / np.float32(127)
    want_bits = np.array([half_bits_struct(float(v)) for v in q32], dtype=np.uint16)
    problems += int(np.sum(s_a.view(np.uint16) != want_bits))
    problems += int(np.sum(np.abs(a8.astype(int)) > 127))
    normal = s_a.astype(np.float32) >= np.float32(2 ** -14)
    problems += int(np.sum(a8[normal, 0] != 127))
    # symmetry: quantizing -A gives -A8
    a8n, _ = quant_act(-a)
    problems += int(np.sum(a8n.astype(int) != -a8.astype(int)))
    return problems


def test_act_exhaustive_fp16_scale_sweep():
    assert act_scale_sweep_check(ref.quant_act) == 0


def test_act_reconstruction_bound():
    a = synth.activations(64, 512, seed=3)
    a8, s_a = ref.quant_act(a)
    s = s_a.astype(np.float64)
    err = np.abs(a.astype(np.float64) - s[:, None] * a8)
    assert (err <= s[:, None] * (0.5 + 2 ** -10)).all()


# ------------------------------------------------------------ O4 GEMM
def brute_acc(a8, w8hat):
    m, k = a8.shape
    n = w8hat.shape[0]
    out = np.zeros((m, n), dtype=np.int64)
    for i in range(m):
        for j in range(n):
            s = 0
            for t in range(k):
                s += int(a8[i, t]) * int(w8hat[j, t])
            out[i, j] = s
    return out


def gemm_brute_check(gemm):
    rng = np.random.default_rng(7)
    a8 = rng.integers(-127, 128, size=(3, 67)).astype(np.int8)
    w8 = rng.integers(-128, 128, size=(5, 67)).astype(np.int32)
    return np.array_equal(gemm(a8, w8), brute_acc(a8, w8))


def test_gemm_brute_force():
    assert gemm_brute_check(ref.gemm_acc)


def test_gemm_extremes_exact():
    k = 24576                                   # deepest layer of the workloads
    a8 = np.full((2, k), 127, dtype=np.int8)
    a8[1] = -127
    w8 = np.full((3, k), -128, dtype=np.int32)
    w8[1] = 127
    acc = ref.gemm_acc(a8, w8)
    assert acc[0, 0] == 127 * -128 * k and acc[1, 1] == -127 * 127 * k


def test_dequant_then_matmul_matches_scaled_acc():
    # float dequant-then-matmul equals s_a * s1 * acc up to fp64 rounding
    w = synth.weights(48, 256, seed=21)
    a = synth.activations(5, 256, seed=22)
    out = ref.linear(a, w, 64)
    wd = out["qw"]["s1"].astype(np.float64)[:, None] * out["w8hat"]
    ad = out["s_a"].astype(np.float64)[:, None] * out["a8"].astype(np.float64)
    y_float = ad @ wd.T
    y_int = (out["acc"] * out["s_a"].astype(np.float64)[:, None]
             * out["qw"]["s1"].astype(np.float64)[None, :])
    assert np.allclose(y_float, y_int, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------ O5 epilogue
def test_epilogue_single_rounding():
    rng = np.random.default_rng(9)
    acc = rng.integers(-3 * 10 ** 8, 3 * 10 ** 8, size=(20, 30))
    s_a = (rng.random(20) * 0.05 + 1e-4).astype(np.float16)
    s1 = (rng.random(30) * 0.001 + 1e-5).astype(np.float16)
    y = ref.epilogue(acc, s_a, s1)
    for i in range(0, 20, 3):
        for j in range(0, 30, 4):
            exact = Fraction(int(acc[i, j])) * Fraction(float(s_a[i])) * Fraction(float(s1[j]))
            assert float(y[i, j]) == half_of_fraction(exact)


def test_tolerance_rule():
    y_ref = np.array([1.0, 100.0, 0.0, -3.0], dtype=np.float16)
    assert ref.y_tolerance_ok(y_ref, y_ref).all()
    one_ulp = np.nextafter(y_ref, np.float16(np.inf))
    assert ref.y_tolerance_ok(one_ulp, y_ref).all()
    far = y_ref + np.float16(1.0)
    assert not ref.y_tolerance_ok(far, y_ref)[[0, 2, 3]].any()


def test_whole_layer_smoke_bound():
    # model accuracy is not pinned (needs trained weights); keep a loose bound
    w = synth.weights(256, 512, seed=1)
    a = synth.activations(16, 512, seed=2)
    out = ref.linear(a, w, 128)
    y_fp = a.astype(np.float64) @ w.astype(np.float64).T
    rel = np.linalg.norm(out["y"].astype(np.float64) - y_fp) / np.linalg.norm(y_fp)
    assert rel < 0.15


# ------------------------------------------------------------ mutation tests
def _mut_round_not_ceil(w8):
    w8 = np.asarray(w8, dtype=np.int64)
    lo = np.minimum(0, w8.min(axis=-1))
    hi = np.maximum(0, w8.max(axis=-1))
    s2 = np.maximum(1, ref.rne_ratio(hi - lo, 15))
    z = ref.rne_ratio(-lo, s2)
    q = ref.rne_ratio(w8, s2[..., None]) + z[..., None]
    return s2, z, np.clip(q, 0, 15)


def _mut_no_zero_in_range(w8):
    w8 = np.asarray(w8, dtype=np.int64)
    lo = w8.min(axis=-1)
    hi = w8.max(axis=-1)
    s2 = np.maximum(1, ref.ceil_ratio(hi - lo, 15))
    z = ref.rne_ratio(-lo, s2)
    q = ref.rne_ratio(w8, s2[..., None]) + z[..., None]
    return s2, z, np.clip(q, 0, 15)


def _mut_zero_sign(w8):
    s2, z, q = ref.level2_groups(w8)
    q2 = ref.rne_ratio(np.asarray(w8, np.int64), s2[..., None].astype(np.int64)) - z[..., None]
    return s2, z, np.clip(q2, 0, 15)


def _mut_floor_div(w8):
    w8 = np.asarray(w8, dtype=np.int64)
    lo = np.minimum(0, w8.min(axis=-1))
    hi = np.maximum(0, w8.max(axis=-1))
    s2 = np.maximum(1, ref.ceil_ratio(hi - lo, 15))
    z = ref.rne_ratio(-lo, s2)
    q = w8 // s2[..., None] + z[..., None]
    return s2, z, np.clip(q, 0, 15)


@pytest.mark.parametrize("mutant", [_mut_round_not_ceil, _mut_no_zero_in_range,
                                    _mut_zero_sign, _mut_floor_div])
def test_level2_pins_catch_mutants(mutant):
    caught = level2_domain_check(mutant) > 0 or level2_golden_check(mutant) != []
    assert caught


def test_level1_pins_catch_mutants():
    w = synth.weights(128, 256, seed=31)

    def wrong_limit(x):                       # 127 instead of 119
        x = np.asarray(x, np.float32)
        s1 = ref.to_f16(np.abs(x).max(axis=1) / np.float32(127))
        r = np.float32(1) / s1.astype(np.float32)
        return s1, np.clip(np.rint(x * r[:, None]), -127, 127).astype(np.int32)

    def truncating(x):                        # trunc instead of rint
        s1, _ = ref.level1_rows(x)
        r = np.float32(1) / s1.astype(np.float32)
        return s1, np.clip(np.trunc(np.asarray(x, np.float32) * r[:, None]), -119, 119).astype(np.int32)

    def f32_scale(x):                         # scale left in fp32, not fp16
        x = np.asarray(x, np.float32)
        s = np.abs(x).max(axis=1) / np.float32(119)
        r = np.float32(1) / s
        return s, np.clip(np.rint(x * r[:, None]), -119, 119).astype(np.int32)

    for mutant in (wrong_limit, truncating, f32_scale):
        assert level1_invariant_check(mutant, w) > 0, mutant.__name__


def test_act_pins_catch_mutants():
    def floor_round(a):
        a32 = np.asarray(a, np.float16).astype(np.float32)
        s_a = ref.to_f16(np.abs(a32).max(axis=1) / np.float32(127))
        r = np.zeros_like(s_a, dtype=np.float32)
        nz = s_a != 0
        r[nz] = np.float32(1) / s_a[nz].astype(np.float32)
        return np.clip(np.floor(a32 * r[:, None] + 0.5), -127, 127).astype(np.int8), s_a

    def divide_by_128(a):
        a32 = np.asarray(a, np.float16).astype(np.float32)
        s_a = ref.to_f16(np.abs(a32).max(axis=1) / np.float32(128))
        r = np.zeros_like(s_a, dtype=np.float32)
        nz = s_a != 0
        r[nz] = np.float32(1) / s_a[nz].astype(np.float32)
        return np.clip(np.rint(a32 * r[:, None]), -127, 127).astype(np.int8), s_a

    assert act_scale_sweep_check(floor_round) > 0
    assert act_scale_sweep_check(divide_by_128) > 0


def test_gemm_pins_catch_mutants():
    def transposed_k(a8, w8):                 # reversed k order on one operand
        return ref.gemm_acc(a8, w8[:, ::-1])

    def int16_wrap(a8, w8):                   # accumulator wrapped to int16
        s = ref.gemm_acc(a8, w8)
        return (s + 2 ** 15) % 2 ** 16 - 2 ** 15

    assert not gemm_brute_check(transposed_k)
    assert not gemm_brute_check(int16_wrap)


# ------------------------------------------------------------ O3' static scale
def _rne_fraction(x: Fraction) -> int:
    f = x.numerator // x.denominator
    r = x - f
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return f


def act_static_golden_check(fn):
    """Hand-worked cases (tests/golden/act_static_cases.txt); returns mismatches."""
    bad = []
    with open(os.path.join(GOLDEN, "act_static_cases.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            sc, av, ex = (x.strip() for x in line.split("|"))
            a = np.array([[float(v) for v in av.split()]], dtype=np.float16)
            want = np.array([[int(v) for v in ex.split()]], dtype=np.int8)
            a8, s_a = fn(a, np.float16(float(sc)))
            if not np.array_equal(a8, want) or s_a[0] != np.float16(float(sc)):
                bad.append(line.strip())
    return bad


def act_static_exhaustive_check(fn, exponents=(-14, -3, 0, 5)):
    """Every finite fp16 input at power-of-two scales, where A * (1/s) is exact:
    the result must be the exact rational A / s rounded half-to-even and
    clamped to +-127.  Returns the number of mismatches."""
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16)
    vals = vals[np.isfinite(vals)]
    bad = 0
    for e in exponents:
        s = np.float16(2.0 ** e)
        a8, _ = fn(vals[None, :], s)
        want = np.array([max(-127, min(127, _rne_fraction(Fraction(float(v)) / Fraction(2) ** e)))
                         for v in vals], dtype=np.int64)
        bad += int(np.sum(a8[0].astype(np.int64) != want))
    return bad


def test_act_static_golden():
    assert act_static_golden_check(ref.quant_act_static) == []


def test_act_static_exhaustive_power_of_two_scales():
    assert act_static_exhaustive_check(ref.quant_act_static) == 0


def test_act_static_invariants():
    a = synth.activations(7, 300, seed=41)
    for s in (np.float16(0.01), np.float16(0.3), np.float16(7.0)):
        a8, s_a = ref.quant_act_static(a, s)
        assert (s_a == s).all() and s_a.dtype == np.float16
        assert np.abs(a8.astype(np.int64)).max() <= 127
        nz = a8 != 0
        assert (np.sign(a8[nz]) == np.sign(a[nz].astype(np.float32))).all()
    a8, s_a = ref.quant_act_static(a, np.float16(0.0))
    assert not a8.any() and not s_a.astype(np.float32).any()


def test_act_static_pins_catch_mutants():
    def round_half_up(a, s):
        a32 = np.asarray(a, np.float16).astype(np.float32)
        r = np.float32(1) / np.float32(s) if float(s) else np.float32(0)
        a8 = np.clip(np.floor(a32 * r + np.float32(0.5)), -127, 127).astype(np.int8)
        return a8, np.full(a32.shape[0], s, np.float16)

    def clamp_128(a, s):
        a32 = np.asarray(a, np.float16).astype(np.float32)
        r = np.float32(1) / np.float32(s) if float(s) else np.float32(0)
        a8 = np.clip(np.rint(a32 * r), -128, 127).astype(np.int8)
        return a8, np.full(a32.shape[0], s, np.float16)

    for mutant in (round_half_up, clamp_128):
        assert act_static_golden_check(mutant) or act_static_exhaustive_check(mutant, (0,)) > 0


# ------------------------------------------------------------ W4A16 comparison path
def w16_exact_check(fn, w, g):
    """W16^ against the exact rational s1 * W8^ rounded half-to-even by
    half_of_fraction (no numpy rounding involved); returns mismatches."""
    qw = ref.quantize_weights(w, g)
    got = fn(qw).astype(np.float64)
    w8 = ref.decoded_weights(qw)
    bad = 0
    for n in range(w8.shape[0]):
        s1 = Fraction(float(qw["s1"][n]))
        for kk in range(w8.shape[1]):
            if got[n, kk] != half_of_fraction(s1 * int(w8[n, kk])):
                bad += 1
    return bad


def test_w16_weights_single_rounding_of_exact_product():
    w = synth.weights(24, 256, seed=61, dist="student_t4")
    for g in (32, 128, 0):
        assert w16_exact_check(ref.w16_weights, w, g) == 0


def w4a16_brute_check(fn):
    """Y16 on a tiny case against an exact rational sum rounded once."""
    rng = np.random.default_rng(62)
    w = synth.weights(8, 128, seed=63)
    a = (rng.standard_normal((3, 128)) * 2).astype(np.float16)
    qw = ref.quantize_weights(w, 64)
    y, w16, sum_abs = fn(a, qw)
    bad = 0
    for m in range(3):
        for n in range(8):
            exact = sum(Fraction(float(a[m, kk])) * Fraction(float(w16[n, kk])) for kk in range(128))
            if float(y[m, n]) != half_of_fraction(exact):
                bad += 1
            if abs(sum_abs[m, n] - float(sum(abs(Fraction(float(a[m, kk])) * Fraction(float(w16[n, kk])))
                                              for kk in range(128)))) > 1e-9 * max(1.0, sum_abs[m, n]):
                bad += 1
    return bad


def test_w4a16_brute_force():
    assert w4a16_brute_check(ref.w4a16_linear) == 0


def test_w4a16_tolerance_rule():
    y_ref = np.array([1.0, -2.0, 1000.0], np.float16)
    s = np.array([1.0, 1.0, 1.0])
    assert ref.y16_tolerance_ok(y_ref, y_ref, s, 4096).all()
    # one ulp off passes; far off fails
    assert ref.y16_tolerance_ok(np.nextafter(y_ref, np.float16(np.inf)), y_ref, s, 4096).all()
    assert not ref.y16_tolerance_ok(y_ref * np.float16(1.01), y_ref, s, 4096).any()
    # the accumulation term scales with K and sum |A W|
    assert ref.y16_tolerance_ok(np.float16(1.0) + np.float16(0.03), np.float16(1.0),
                                np.float64(2 ** 14), 2 ** 9)


def test_w4a16_pins_catch_mutants():
    def w16_truncating(qw):
        w8 = ref.decoded_weights(qw).astype(np.float64)
        v = qw["s1"].astype(np.float64)[:, None] * w8
        # round toward zero in fp16
        f = v.astype(np.float16)
        over = np.abs(f.astype(np.float64)) > np.abs(v)
        f[over] = np.nextafter(f[over], np.float16(0))
        return f
    w = synth.weights(24, 256, seed=61, dist="student_t4")
    assert w16_exact_check(w16_truncating, w, 128) > 0

    def y_fp16_accumulate(a, qw):               # accumulating in fp16 loses the sum
        y, w16, sa = ref.w4a16_linear(a, qw)
        acc = np.zeros((a.shape[0], w16.shape[0]), np.float16)
        for kk in range(a.shape[1]):
            acc = (acc + (a[:, kk:kk + 1].astype(np.float16) * w16[:, kk][None, :]).astype(np.float16))
        return acc, w16, sa
    assert w4a16_brute_check(y_fp16_accumulate) > 0


# ------------------------------------------------------------ O1'' codebook mode
def _inv_normal_cdf(p: float) -> float:
    """Standard-normal quantile by bisection on math.erf (independent of scipy)."""
    import math
    lo, hi = -10.0, 10.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if 0.5 * (1.0 + math.erf(mid / math.sqrt(2.0))) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def test_nf_codebook_from_its_definition():
    lut = ref.nf_codebook()
    z = [_inv_normal_cdf((i + 0.5) / 16) for i in range(16)]
    want = [int(round(119.0 * v / z[-1])) for v in z]      # no exact .5 ties occur
    assert lut.tolist() == want
    assert (np.diff(lut) > 0).all() and (lut == -lut[::-1]).all() and lut[-1] == 119


def nf_nearest_check(fn):
    """Exhaustive over every level-1 value: the chosen level is a nearest one,
    and the lowest index among equally near ones.  Returns violations."""
    lut = [int(v) for v in ref.nf_codebook()]
    w8 = np.arange(-119, 120)
    q = fn(w8, np.array(lut))
    bad = 0
    for v, j in zip(w8.tolist(), q.tolist()):
        dist = [abs(level - v) for level in lut]
        best = min(dist)
        if dist[j] != best or j != dist.index(best):
            bad += 1
    return bad


def test_nf_nearest_exhaustive():
    assert nf_nearest_check(ref.nf_nearest) == 0


def nf_golden_check(fn):
    bad = []
    lut = ref.nf_codebook()
    with open(os.path.join(GOLDEN, "nf_cases.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            w8, idx, dec = (int(x) for x in line.split("|"))
            j = int(fn(np.array([w8]), lut)[0])
            if j != idx or int(lut[j]) != dec:
                bad.append(line.strip())
    return bad


def test_nf_golden():
    assert nf_golden_check(ref.nf_nearest) == []


def test_nf_whole_rows():
    """Codebook mode on rows: decoded weights are codebook levels, s1 is the
    level-1 scale, and the GEMM of the decoded weights matches brute force."""
    w = synth.weights(16, 256, seed=77, dist="student_t4")
    qw = ref.quantize_weights(w, ref.NF_CODE)
    s1, w8 = ref.level1_rows(np.asarray(w, np.float32))
    assert np.array_equal(qw["s1"].view(np.uint16), s1.view(np.uint16))
    dec = ref.decoded_weights(qw)
    assert set(np.unique(dec).tolist()) <= set(ref.nf_codebook().tolist())
    assert (np.abs(dec - w8) <= 17).all()        # half the widest level gap (119 - 84 = 35)
    a8 = np.random.default_rng(3).integers(-127, 128, (3, 256))
    acc = ref.gemm_acc(a8, dec)
    brute = np.array([[sum(int(a8[m, kk]) * int(dec[n, kk]) for kk in range(256))
                       for n in range(16)] for m in range(3)])
    assert np.array_equal(acc, brute)


def test_nf_pins_catch_mutants():
    def ties_up(w8, lut):
        d = np.abs(np.asarray(w8, np.int64)[..., None] - lut.astype(np.int64))
        return (15 - np.argmin(d[..., ::-1], axis=-1)).astype(np.uint8)

    def truncate_toward_zero(w8, lut):
        w8 = np.asarray(w8, np.int64)
        out = np.zeros(w8.shape, np.uint8)
        for i, v in enumerate(w8.ravel()):
            cands = [j for j in range(16) if abs(int(lut[j])) <= abs(v) and np.sign(lut[j]) == np.sign(v)]
            out.ravel()[i] = cands[-1] if v > 0 and cands else (cands[0] if cands else 7)
        return out

    for mutant in (ties_up, truncate_toward_zero):
        assert nf_nearest_check(mutant) > 0 or nf_golden_check(mutant), mutant.__name__
