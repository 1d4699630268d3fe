"""CPU oracle for the W4A8 linear layer.  TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The library (C ABI + HIP kernels) never calls it, and it
shares no code, table or helper with the library.

What is computed, and where it comes from
-----------------------------------------
The QServe/QoQ abstract (page "[Feature] Support W4A8KV4 Quantization
(QServe/QoQ)", the quoted abstract) names the method: 4-bit weights, 8-bit
activations, and a *progressive* weight quantization whose decode to the
8-bit GEMM operand is cheap, so that the GEMM runs on 8-bit integer units
with no dequantization of partial sums.  The pages print no formula, so the
steps below are the plainest reading of that description:

  O1  level 1, per output row n:   symmetric int8 with an fp16 scale s1[n]
  O2  level 2, per group of g consecutive k of row n: asymmetric uint4 with an
      integer step s2 and an integer zero z, applied to the int8 values, so
      the decode  W8^ = (q - z) * s2  is integer multiply-subtract only and
      must land in int8 (the LiquidGEMM digest, section "Метод", also asks
      the decode to be overflow-free)
  O1' per-channel mode (no level-2 groups): one fp16 scale and one uint4 zero
      per row, s2 = 1
  O3  per-token symmetric int8 activations with an fp16 scale s_a[m]
      (per-token dynamic quantization is the usual practice the PrefixQuant
      page contrasts against, section "Key Findings")
  O3' the static alternative: one fp16 scale for the whole tensor
  O4  acc[m, n] = sum_k A8[m, k] * W8^[n, k]   (exact integer)
  O5  Y[m, n]   = fp16(acc * s_a[m] * s1[n])   (the scale epilogue)

Every rounding is pinned: fp32 operations are single IEEE operations
(numpy float32 arithmetic, no fused multiply-add), fp16(x) is IEEE binary16
round-to-nearest-even, rint is round-half-to-even.  Integer divisions that
the definition states as exact rationals are done in integers.

Parity pins for every function live in tests/test_oracle_pins.py.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
W8_LIMIT = 119   # level-1 symmetric range (see level1_rows)
A8_LIMIT = 127   # activation symmetric range
Q_MAX = 15       # uint4


# ---------------------------------------------------------------- helpers
def to_f16(x) -> np.ndarray:
    """IEEE binary16, round-to-nearest-even (numpy's conversion is RNE)."""
    with np.errstate(over="ignore"):
        return np.asarray(x).astype(np.float16)


def rne_ratio(num, den) -> np.ndarray:
    """round-half-to-even of the exact rational num/den (den > 0), in integers."""
    num = np.asarray(num, dtype=np.int64)
    den = np.asarray(den, dtype=np.int64)
    fl, rem = np.divmod(num, den)             # floor, 0 <= rem < den
    twice = 2 * rem
    up = (twice > den) | ((twice == den) & (fl % 2 == 1))
    return fl + up.astype(np.int64)


def ceil_ratio(num, den) -> np.ndarray:
    num = np.asarray(num, dtype=np.int64)
    den = np.asarray(den, dtype=np.int64)
    return -((-num) // den)


def _safe_recip(scale_f16: np.ndarray) -> np.ndarray:
    """fp32(1 / fp32(scale)), and 0 where the scale is 0 (never computes 1/0)."""
    s = scale_f16.astype(F32)
    out = np.zeros_like(s)
    nz = s != 0
    out[nz] = F32(1.0) / s[nz]
    return out


# ---------------------------------------------------------------- O1
def level1_rows(w: np.ndarray):
    """O1: per-row symmetric int8 with an fp16 scale.

    alpha = max_k |W[n,k]|;  s1 = fp16(fp32(alpha / 119));
    W8 = clamp(rint(fp32(W * fp32(1/s1))), -119, 119), and W8 = 0 where s1 = 0.

    Reading: the range is +-119 rather than +-127 because it is the widest
    symmetric int8 range for which every level-2 decode (q - z) * s2 of O2
    stays inside int8 (a level-2 step of up to 16 rounds by up to 8).
    Returns (s1 float16[N], W8 int32[N, K]).
    """
    w = np.ascontiguousarray(w, dtype=F32)
    alpha = np.max(np.abs(w), axis=1)
    s1 = to_f16(alpha / F32(W8_LIMIT))
    r = _safe_recip(s1)
    w8 = np.rint(w * r[:, None])
    w8 = np.clip(w8, -W8_LIMIT, W8_LIMIT).astype(np.int32)
    return s1, w8


# ---------------------------------------------------------------- O2
def level2_groups(w8: np.ndarray):
    """O2 on a batch of groups: w8 is (..., g) int; returns (s2, z, q).

    lo = min(0, min w8);  hi = max(0, max w8)       (zero always representable)
    s2 = max(1, ceil((hi - lo) / 15))                in [1, 16]
    z  = rne(-lo / s2)                               in [0, 15]
    q  = clamp(rne(w8 / s2) + z, 0, 15)
    Reading: s2 uses the ceiling, because with round-to-nearest the zero can
    reach 16 and no longer fit four bits.
    """
    w8 = np.asarray(w8, dtype=np.int64)
    lo = np.minimum(0, w8.min(axis=-1))
    hi = np.maximum(0, w8.max(axis=-1))
    s2 = np.maximum(1, ceil_ratio(hi - lo, Q_MAX))
    z = rne_ratio(-lo, s2)
    q = rne_ratio(w8, s2[..., None]) + z[..., None]
    q = np.clip(q, 0, Q_MAX)
    return s2.astype(np.uint8), z.astype(np.uint8), q.astype(np.uint8)


def decode(q: np.ndarray, z: np.ndarray, s2: np.ndarray, g: int) -> np.ndarray:
    """W8^[n, k] = (q[n, k] - z[n, k // g]) * s2[n, k // g]  (int32)."""
    zz = np.repeat(z.astype(np.int32), g, axis=1)
    ss = np.repeat(s2.astype(np.int32), g, axis=1)
    return (q.astype(np.int32) - zz) * ss


# ---------------------------------------------------------------- O1'
def per_channel(w: np.ndarray):
    """O1' (g = K, no level-2 groups): uint4 per row with an fp16 scale.

    lo = min(0, min_k W), hi = max(0, max_k W) (fp32);  s1 = fp16(fp32((hi-lo)/15));
    r = fp32(1/s1);  z = clamp(rint(fp32(-lo * r)), 0, 15);
    q = clamp(rint(fp32(W * r)) + z, 0, 15);  q = z = 0 where s1 = 0; s2 = 1.
    Returns (s1 float16[N], q uint8[N, K], z uint8[N, 1], s2 uint8[N, 1]).
    """
    w = np.ascontiguousarray(w, dtype=F32)
    lo = np.minimum(F32(0), w.min(axis=1))
    hi = np.maximum(F32(0), w.max(axis=1))
    s1 = to_f16((hi - lo) / F32(Q_MAX))
    r = _safe_recip(s1)
    z = np.clip(np.rint(-lo * r), 0, Q_MAX)
    q = np.clip(np.rint(w * r[:, None]) + z[:, None], 0, Q_MAX)
    zero = s1.astype(F32) == 0
    q[zero, :] = 0
    z[zero] = 0
    n = w.shape[0]
    return (s1, q.astype(np.uint8), z.astype(np.uint8).reshape(n, 1),
            np.ones((n, 1), dtype=np.uint8))


# ---------------------------------------------------------------- O1'' codebook
NF_CODE = 1   # the "group size" value that selects the codebook mode


def nf_codebook() -> np.ndarray:
    """The 16 int8 levels of the non-uniform (NormalFloat-style) 4-bit code,
    FLUTE page, section 方法详解 (LUT-quantized weights, NormalFloat).  The
    page prints no levels; reading: the standard-normal quantiles at the 16
    probabilities (i + 1/2) / 16, scaled so the largest is 119 (the level-1
    int8 range) and rounded half-to-even to integers."""
    from scipy.stats import norm
    z = norm.ppf((np.arange(16) + 0.5) / 16.0)
    return np.rint(119.0 * z / z[-1]).astype(np.int32)


def nf_nearest(w8: np.ndarray, lut: np.ndarray) -> np.ndarray:
    """Index of the codebook level nearest to each int8 value; ties go to the
    lower index."""
    d = np.abs(np.asarray(w8, np.int64)[..., None] - lut.astype(np.int64))
    return np.argmin(d, axis=-1).astype(np.uint8)    # argmin keeps the first minimum


def quantize_weights_nf(w: np.ndarray):
    """O1'' codebook mode, per output row: the level-1 int8 quantization O1
    (s1 = fp16(absmax / 119)), then each int8 value replaced by the nearest
    level of nf_codebook(); the decoded weight is LUT[q]."""
    w = np.ascontiguousarray(w, dtype=F32)
    s1, w8 = level1_rows(w)
    lut = nf_codebook()
    return {"q": nf_nearest(w8, lut), "s1": s1, "lut": lut, "g_eff": NF_CODE}


# ---------------------------------------------------------------- O1 + O2
def quantize_weights(w: np.ndarray, g: int):
    """Progressive quantization of W (N x K fp32); g = 0 or g = K is per-channel,
    g = NF_CODE the codebook mode.

    Returns a dict with q uint8[N,K], z uint8[N,G], s2 uint8[N,G],
    s1 float16[N] and g_eff (the group length used by decode); the codebook
    mode returns q, s1 and the lut instead of z and s2.
    """
    if g == NF_CODE:
        return quantize_weights_nf(w)
    w = np.ascontiguousarray(w, dtype=F32)
    n, k = w.shape
    if g == 0 or g == k:
        s1, q, z, s2 = per_channel(w)
        return {"q": q, "z": z, "s2": s2, "s1": s1, "g_eff": k}
    if k % g:
        raise ValueError("K must be a multiple of g")
    s1, w8 = level1_rows(w)
    s2, z, q = level2_groups(w8.reshape(n, k // g, g))
    return {"q": q.reshape(n, k), "z": z, "s2": s2, "s1": s1, "g_eff": g}


def decoded_weights(qw: dict) -> np.ndarray:
    if "lut" in qw:
        return qw["lut"][qw["q"].astype(np.int64)].astype(np.int32)
    return decode(qw["q"], qw["z"], qw["s2"], qw["g_eff"])


# ---------------------------------------------------------------- O3
def quant_act(a: np.ndarray):
    """O3: per-token symmetric int8.

    alpha = max_k |A[m,k]| (fp16 -> fp32 is exact);  s_a = fp16(fp32(alpha/127));
    A8 = clamp(rint(fp32(A * fp32(1/s_a))), -127, 127), and 0 where s_a = 0.
    Returns (A8 int8[M, K], s_a float16[M]).
    """
    a32 = np.asarray(a, dtype=np.float16).astype(F32)
    alpha = np.max(np.abs(a32), axis=1)
    s_a = to_f16(alpha / F32(A8_LIMIT))
    r = _safe_recip(s_a)
    a8 = np.clip(np.rint(a32 * r[:, None]), -A8_LIMIT, A8_LIMIT)
    return a8.astype(np.int8), s_a


def quant_act_static(a: np.ndarray, scale_f16) -> tuple:
    """O3' (static per-tensor activation scale): one fp16 scale s fixed
    ahead of time for the whole tensor, so no per-token reduction runs (the
    static alternative the PrefixQuant page sets against per-token dynamic
    quantization, section "Key Findings").

    A8 = clamp(rint(fp32(A * fp32(1/s))), -127, 127), and 0 where s = 0;
    s_a[m] = s for every row, so the GEMM epilogue is unchanged.
    Returns (A8 int8[M, K], s_a float16[M]).
    """
    a32 = np.asarray(a, dtype=np.float16).astype(F32)
    s = to_f16(np.asarray(scale_f16, dtype=np.float16).reshape(()))
    r = _safe_recip(s.reshape(1))[0]
    a8 = np.clip(np.rint(a32 * r), -A8_LIMIT, A8_LIMIT)
    s_a = np.full(a32.shape[0], s, dtype=np.float16)
    return a8.astype(np.int8), s_a


# ---------------------------------------------------------------- O4
def gemm_acc(a8: np.ndarray, w8hat: np.ndarray) -> np.ndarray:
    """O4: acc[m, n] = sum_k A8[m, k] * W8^[n, k], exactly.

    The product is formed by a float64 matrix product of integer-valued
    matrices: every partial sum is an integer below 2**53 (|A8| <= 127,
    |W8^| <= 128, K < 2**38), so every summation order gives the exact sum.
    """
    a = np.asarray(a8, dtype=np.float64)
    w = np.asarray(w8hat, dtype=np.float64)
    if a.shape[1] and 127 * 128 * a.shape[1] >= 2 ** 53:
        raise ValueError("K too large for an exact float64 product")
    acc = a @ w.T
    out = acc.astype(np.int64)
    if out.size and np.abs(out).max() >= 2 ** 31:
        raise OverflowError("accumulator leaves int32")
    return out


# ---------------------------------------------------------------- O5
def epilogue(acc: np.ndarray, s_a: np.ndarray, s1: np.ndarray) -> np.ndarray:
    """O5: Y = fp16(fp64(acc) * fp64(s_a[m]) * fp64(s1[n])) (one rounding)."""
    y = (np.asarray(acc, dtype=np.float64)
         * np.asarray(s_a, dtype=np.float64)[:, None]
         * np.asarray(s1, dtype=np.float64)[None, :])
    return to_f16(y)


def y_tolerance_ok(y, y_ref) -> np.ndarray:
    """|Y - Y_ref| <= 1e-3 |Y_ref| + one fp16 ulp at Y_ref (elementwise)."""
    y = np.asarray(y, dtype=np.float16)
    y_ref = np.asarray(y_ref, dtype=np.float16)
    ulp = np.spacing(np.abs(y_ref)).astype(np.float64)
    diff = np.abs(y.astype(np.float64) - y_ref.astype(np.float64))
    return diff <= 1e-3 * np.abs(y_ref.astype(np.float64)) + ulp


# ---------------------------------------------------------------- W4A16
# The comparison path (the W4A16 kernels the pages measure against: the
# AWQ-style weight-only baseline of the QServe/QoQ abstract, QUICK's and
# FLUTE's mixed-precision GEMMs): the same 4-bit weights, decoded to fp16
# and multiplied with fp16 activations in fp32.  Reading: the fp16 weight is
# the level-1 dequantization of the decoded int8 weight, rounded once,
#     W16^[n, k] = fp16(s1[n] * W8^[n, k])
# (s1 * W8^ is exact in float64), and
#     Y16[m, n] = fp16(sum_k A[m, k] * W16^[n, k])  (exact sum, one rounding).
def w16_weights(qw: dict) -> np.ndarray:
    """W16^ = fp16(s1 * W8^): one rounding of the exact product."""
    w8 = decoded_weights(qw).astype(np.float64)
    return to_f16(qw["s1"].astype(np.float64)[:, None] * w8)


def w4a16_linear(a: np.ndarray, qw: dict):
    """Y16 = fp16(A @ W16^.T) with the sum taken in float64.  Returns
    (Y16 float16[M, N], W16^ float16[N, K], sum_abs float64[M, N]) where
    sum_abs = sum_k |A * W16^| bounds any accumulation error."""
    w16 = w16_weights(qw).astype(np.float64)
    a64 = np.asarray(a, dtype=np.float16).astype(np.float64)
    y = a64 @ w16.T
    sum_abs = np.abs(a64) @ np.abs(w16).T
    return to_f16(y), w16.astype(np.float16), sum_abs


def y16_tolerance_ok(y, y_ref, sum_abs, k: int) -> np.ndarray:
    """Bar for an fp32-accumulated fp16 GEMM: one fp16 ulp at Y_ref, plus
    1e-3 |Y_ref|, plus the first-order fp32 summation bound K * 2^-24 *
    sum_k |A * W16^| (products of two fp16 values are exact in fp32)."""
    y = np.asarray(y, dtype=np.float16).astype(np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float16)
    ulp = np.spacing(np.abs(y_ref)).astype(np.float64)
    yr = y_ref.astype(np.float64)
    bound = ulp + 1e-3 * np.abs(yr) + k * 2.0 ** -24 * np.asarray(sum_abs, np.float64)
    return np.abs(y - yr) <= bound


# ---------------------------------------------------------------- whole layer
def linear(a: np.ndarray, w: np.ndarray, g: int):
    """The whole layer on the CPU: returns every intermediate, for tests."""
    qw = quantize_weights(w, g)
    a8, s_a = quant_act(a)
    w8hat = decoded_weights(qw)
    acc = gemm_acc(a8, w8hat)
    y = epilogue(acc, s_a, qw["s1"])
    return {"qw": qw, "a8": a8, "s_a": s_a, "w8hat": w8hat, "acc": acc, "y": y}
