"""Property-based check of the weight packer against the oracle.

Hypothesis draws small weight matrices built row by row from awkward kinds
(zero rows, one outlier, constant rows and groups, ramps, rows whose fp16
scale is subnormal, heavy tails, one sign only, integer values, values at
the fp16 scale's upper end) and every group mode, and the C packer must
give the oracle's codes, zero points, group scales and row scales bit for
bit (the progressive scheme of the QServe paper, "QoQ" section: int8 per
output channel, then 4-bit per group with integer scale and zero point)."""
import numpy as np
import pytest
from hypothesis import HealthCheck, event, given, settings
from hypothesis import strategies as st

import w4a8_gemm_amd as w4
from oracle import ref

ROW_KINDS = ("normal", "zero", "outlier", "constant", "ramp", "tiny", "heavy", "one_sign",
             "integers", "group_constant", "huge", "two_values")


def make_row(kind, k, rng, scale):
    if kind == "zero":
        return np.zeros(k)
    if kind == "outlier":
        r = rng.standard_normal(k) * 1e-3 * scale
        r[rng.integers(k)] = 10 * scale * (1 if rng.random() < 0.5 else -1)
        return r
    if kind == "constant":
        return np.full(k, scale * (1 if rng.random() < 0.5 else -1))
    if kind == "ramp":
        return np.linspace(-scale, scale, k)
    if kind == "tiny":
        # max |w| / 119 below fp16's smallest normal (6.1e-5): a subnormal s1
        return rng.standard_normal(k) * 1e-6
    if kind == "heavy":
        return rng.standard_t(1.5, k) * scale
    if kind == "one_sign":
        return np.abs(rng.standard_normal(k)) * scale * (1 if rng.random() < 0.5 else -1)
    if kind == "integers":
        return rng.integers(-8, 9, k).astype(np.float64)
    if kind == "group_constant":
        r = np.repeat(rng.standard_normal(k // 32), 32) * scale
        return r
    if kind == "huge":
        # row maxima on both sides of the largest scale fp16 holds: about
        # 4.9e5 in per-channel mode (span / 15), 7.8e6 with groups (max / 119)
        r = rng.standard_normal(k)
        return r / np.abs(r).max() * rng.uniform(1e5, 7.9e6)
    if kind == "two_values":
        return np.where(rng.random(k) < 0.5, -scale, 0.5 * scale)
    return rng.standard_normal(k) * scale


@st.composite
def weight_cases(draw):
    n = draw(st.sampled_from([16, 32]))
    k = draw(st.sampled_from([128, 256, 384]))
    g = draw(st.sampled_from([32, 64, 128, 0, ref.NF_CODE]))
    if g not in (0, ref.NF_CODE) and k % g:
        g = 0
    seed = draw(st.integers(0, 2 ** 32 - 1))
    kinds = draw(st.lists(st.sampled_from(ROW_KINDS), min_size=n, max_size=n))
    log_scale = draw(st.floats(-6.0, 3.0))
    rng = np.random.default_rng(seed)
    w = np.stack([make_row(kind, k, rng, 10.0 ** log_scale) for kind in kinds])
    return w.astype(np.float32), g


@settings(max_examples=120, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.too_slow])
@given(weight_cases())
def test_pack_equals_oracle_on_drawn_matrices(case):
    w, g = case
    assert np.isfinite(w).all()
    with np.errstate(over="ignore", invalid="ignore"):
        want = ref.quantize_weights(w, g)
    if not np.isfinite(want["s1"].astype(np.float32)).all():
        # a row scale that overflows fp16 is refused, never wrapped or clamped
        event("refused: scale overflows fp16")
        with pytest.raises(w4.W4A8Error) as err:
            w4.pack(w, g)
        assert err.value.status == 5        # W4A8_ERR_RANGE
        return
    event(f"packed, g={g}")
    bits = want["s1"].view(np.uint16)
    if (((bits & 0x7C00) == 0) & ((bits & 0x03FF) != 0)).any():
        event("packed with a subnormal row scale")
    blob = w4.pack(w, g, n_threads=int(np.abs(w).sum() * 7) % 3)
    got = w4.unpack(blob)
    assert np.array_equal(got["q"], want["q"])
    assert np.array_equal(got["s1"].view(np.uint16), want["s1"].view(np.uint16))
    if g == ref.NF_CODE:
        assert np.array_equal(got["levels"], want["lut"])
    else:
        assert np.array_equal(got["z"], want["z"])
        assert np.array_equal(got["s2"], want["s2"])
        assert got["q"].max() <= 15 and got["z"].max() <= 15
    # the decoded level-2 weights stay inside the int8 range of level 1
    w8hat = ref.decoded_weights(want)
    assert np.abs(w8hat).max() <= 127


@settings(max_examples=40, deadline=None, derandomize=True)
@given(st.integers(0, 2 ** 32 - 1), st.sampled_from([32, 64, 128, 0]))
def test_pack_is_row_local(seed, g):
    """Packing rows separately gives the rows of packing them together: no
    state crosses output channels (each row has its own s1 and groups)."""
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((32, 256)) * 0.05).astype(np.float32)
    whole = w4.unpack(w4.pack(w, g))
    top = w4.unpack(w4.pack(np.ascontiguousarray(w[:16]), g))
    bottom = w4.unpack(w4.pack(np.ascontiguousarray(w[16:]), g))
    for key in ("q", "z", "s2", "s1"):
        assert np.array_equal(whole[key], np.concatenate([top[key], bottom[key]]))
