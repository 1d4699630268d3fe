"""CPU tests of the C ABI library: exports, argument validation, and the host
packer against the oracle (no GPU needed; no compute call touches HIP)."""
import ctypes
import subprocess

import numpy as np
import torch
import pytest

import synth
import w4a8_gemm_amd as w4
from oracle import ref


def test_library_exports_every_header_function():
    names = w4.header_functions()
    assert len(names) >= 8
    out = subprocess.run(["nm", "-D", "--defined-only", w4.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = [n for n in names if n not in exported]
    assert missing == []
    for n in names:
        assert hasattr(w4.lib, n)


def test_status_strings():
    for code in range(8):
        assert w4.status_string(code)
    assert w4.status_string(0) == "ok"


@pytest.mark.parametrize("n,k,g,ok", [
    (256, 512, 128, True), (256, 512, 64, True), (256, 512, 32, True),
    (256, 512, 0, True), (256, 512, 512, True),
    (250, 512, 128, False),   # n % 16
    (256, 500, 128, False),   # k % 128
    (256, 512, 256, False),   # g not supported
    (256, 512, 96, False),
    (16, 131072, 128, True), (16, 131200, 128, False),   # K limit
    (0, 512, 128, False), (256, 0, 128, False),
])
def test_packed_size_shapes(n, k, g, ok):
    size = w4.packed_size(n, k, g)
    assert (size > 0) == ok
    if ok:
        groups = 1 if g in (0, k) else k // g
        assert size >= 256 + n * k // 2 + n * ((groups + 3) // 4 * 4) + 2 * n


def _compare_with_oracle(w, g):
    blob = w4.pack(w, g)
    got = w4.unpack(blob)
    want = ref.quantize_weights(w, g)
    assert np.array_equal(got["q"], want["q"])
    assert np.array_equal(got["z"], want["z"])
    assert np.array_equal(got["s2"], want["s2"])
    assert np.array_equal(got["s1"].view(np.uint16), want["s1"].view(np.uint16))
    return blob


@pytest.mark.parametrize("dist", ["normal", "student_t4"])
@pytest.mark.parametrize("g", [32, 64, 128, 0])
def test_pack_matches_oracle(dist, g):
    w = synth.weights(128, 1024, seed=40 + g, dist=dist)
    _compare_with_oracle(w, g)


@pytest.mark.parametrize("dist", ["normal", "student_t4"])
def test_pack_codebook_matches_oracle(dist):
    """Codebook mode: codes, s1 and the level table in the header equal the
    oracle's (its levels derived from the normal quantiles)."""
    w = synth.weights(128, 1024, seed=90, dist=dist)
    blob = w4.pack(w, w4.CODEBOOK_NF)
    got = w4.unpack(blob)
    want = ref.quantize_weights(w, ref.NF_CODE)
    assert got["g"] == w4.CODEBOOK_NF and got["z"].shape == (128, 0)
    assert np.array_equal(got["q"], want["q"])
    assert np.array_equal(got["s1"].view(np.uint16), want["s1"].view(np.uint16))
    assert np.array_equal(got["levels"], want["lut"])
    assert w4.packed_size(128, 1024, w4.CODEBOOK_NF) == 256 + 128 * 1024 // 2 + 256
    # the independent layout reader sees the same codes
    assert np.array_equal(_decode_layout(blob)[0], want["q"])


def test_pack_matches_oracle_special_rows():
    w = synth.weights(64, 512, seed=77)
    w[0] = 0.0                                  # zero row
    w[1] = 0.0
    w[1, 5] = 3.0                               # single outlier
    w[2] = 0.01                                 # constant positive row
    w[3] = -0.02                                # constant negative row
    w[4, :] = np.linspace(-1, 1, 512)           # ramp
    w[5, :128] = 0.0                            # zero group
    w[6] = 1e-4                                 # subnormal fp16 scale
    w[7] = 60000.0 * 119 / 119                  # large but finite scale
    for g in (32, 64, 128, 0):
        _compare_with_oracle(w, g)


def _decode_layout(blob):
    """Independent reader of the documented layout v1 (test-side)."""
    n, k, g = w4.blob_info(blob)
    groups = 1 if g == 0 else (0 if g == w4.CODEBOOK_NF else k // g)
    qsec = blob[256:256 + n * k // 2]
    kb = k // 128
    # reshape to [tile][kblock][lane][16 bytes]
    chunk = qsec.reshape(n // 16, kb, 64, 16)
    q = np.zeros((n, k), dtype=np.uint8)
    for lane in range(64):
        r, quarter = lane % 16, lane // 16
        for h in range(2):
            for j in range(16):
                dword = 2 * h + j // 8
                jj = j % 8
                byte = chunk[:, :, lane, dword * 4 + jj % 4]
                nib = (byte >> (4 * (jj // 4))) & 15
                kk = np.arange(kb) * 128 + 64 * h + 16 * quarter + j
                q[r::16, :][:, kk] = nib
    meta_off = 256 + ((n * k // 2 + 255) // 256) * 256
    g4 = (groups + 3) // 4 * 4
    meta = blob[meta_off:meta_off + n * g4].reshape(n, g4)
    assert not meta[:, groups:].any()           # padding is zero
    meta = meta[:, :groups]
    s1_off = meta_off + ((n * g4 + 255) // 256) * 256
    s1 = blob[s1_off:s1_off + 2 * n].view(np.float16)
    return q, meta & 15, (meta >> 4) + 1, s1


@pytest.mark.parametrize("g", [32, 128, 0])
def test_blob_bytes_follow_documented_layout(g):
    w = synth.weights(48, 384, seed=5)
    blob = w4.pack(w, g)
    q, z, s2, s1 = _decode_layout(blob)
    want = ref.quantize_weights(w, g)
    assert np.array_equal(q, want["q"])
    assert np.array_equal(z, want["z"])
    assert np.array_equal(s2, want["s2"])
    assert np.array_equal(s1.view(np.uint16), want["s1"].view(np.uint16))


def test_pack_deterministic_across_threads():
    w = synth.weights(512, 1024, seed=8, dist="student_t4")
    b1 = w4.pack(w, 64, n_threads=1)
    b3 = w4.pack(w, 64, n_threads=3)
    b0 = w4.pack(w, 64, n_threads=0)
    assert np.array_equal(b1, b3) and np.array_equal(b1, b0)


def test_pack_errors():
    w = synth.weights(32, 256, seed=1)
    bad = w.copy()
    bad[3, 7] = np.nan
    with pytest.raises(w4.W4A8Error) as e:
        w4.pack(bad, 128)
    assert e.value.status == 4
    bad[3, 7] = np.inf
    with pytest.raises(w4.W4A8Error) as e:
        w4.pack(bad, 128)
    assert e.value.status == 4
    big = w.copy()
    big[0, 0] = 3.0e38                           # absmax/119 overflows fp16
    with pytest.raises(w4.W4A8Error) as e:
        w4.pack(big, 128)
    assert e.value.status == 5
    size = w4.packed_size(32, 256, 128)
    blob = np.empty(size, dtype=np.uint8)
    st = w4.lib.w4a8_pack(w.ctypes.data, 32, 256, 256, 128, blob.ctypes.data, size - 1, 0)
    assert st == 3
    st = w4.lib.w4a8_pack(None, 32, 256, 256, 128, blob.ctypes.data, size, 0)
    assert st == 1
    st = w4.lib.w4a8_pack(w.ctypes.data, 32, 256, 255, 128, blob.ctypes.data, size, 0)
    assert st == 1


def test_unpack_rejects_bad_header():
    w = synth.weights(32, 256, seed=1)
    blob = w4.pack(w, 128)
    broken = blob.copy()
    broken[0] ^= 0xFF
    with pytest.raises(w4.W4A8Error) as e:
        w4.unpack(broken)
    assert e.value.status == 6
    with pytest.raises(w4.W4A8Error):
        w4.unpack(blob[:100].copy())


def test_gpu_entry_points_validate_before_any_hip_call():
    """Every rejected argument returns its status without touching HIP."""
    L = w4.lib
    fake = ctypes.c_void_p(4096)          # never dereferenced: rejected first
    # quant_act
    assert L.w4a8_quant_act(fake, 4, 0, 8, fake, 8, fake, None) == 1      # k <= 0
    assert L.w4a8_quant_act(fake, -1, 8, 8, fake, 8, fake, None) == 1     # m < 0
    assert L.w4a8_quant_act(fake, 4, 8, 7, fake, 8, fake, None) == 1      # lda < k
    assert L.w4a8_quant_act(None, 4, 8, 8, fake, 8, fake, None) == 1      # null
    assert L.w4a8_quant_act(None, 0, 8, 8, None, 8, None, None) == 0      # m == 0: no-op
    # static scale: finite and >= 0 (fp16 bits), else rejected
    one = 0x3C00
    for bad in (0xBC00, 0x7C00, 0xFC00, 0x7E00, 0x8001):              # -1, +inf, -inf, NaN, -tiny
        assert L.w4a8_quant_act_static(fake, 4, 8, 8, bad, fake, 8, fake, None) == 1, hex(bad)
    assert L.w4a8_quant_act_static(fake, 4, 8, 7, one, fake, 8, fake, None) == 1  # lda < k
    assert L.w4a8_quant_act_static(fake, 4, 8, 8, one, None, 8, fake, None) == 1  # null
    assert L.w4a8_quant_act_static(None, 0, 8, 8, one, None, 8, None, None) == 0  # m == 0
    # gemm: (a8, lda8, s_a, m, blob, n, k, g, y, ldy, acc, ldacc, ws, ws_bytes, opts, stream)
    args = [fake, 512, fake, 4, fake, 256, 512, 128, fake, 256, None, 0, None, 0, None, None]

    def call(**kw):
        a = list(args)
        names = ["a8", "lda8", "s_a", "m", "blob", "n", "k", "g", "y", "ldy", "acc", "ldacc",
                 "ws", "wsb", "opts", "stream"]
        for key, v in kw.items():
            a[names.index(key)] = v
        return L.w4a8_gemm(*a)

    assert call(n=250) == 2
    assert call(k=500) == 2
    assert call(g=96) == 2
    assert call(k=131200, lda8=131200) == 2
    assert call(m=-1) == 1
    assert call(a8=None) == 1
    assert call(blob=None) == 1
    assert call(y=None) == 1
    assert call(lda8=500) == 1
    assert call(lda8=520) == 1                      # not a multiple of 16
    assert call(ldy=100) == 1
    assert call(acc=fake, ldacc=10) == 1
    assert call(a8=ctypes.c_void_p(4104)) == 1      # misaligned
    assert call(m=0, a8=None, s_a=None, y=None, blob=None) == 0   # empty batch
    opts = w4.GemmOpts(7, 0)
    assert call(opts=ctypes.byref(opts)) == 1
    opts = w4.GemmOpts(1, 9)                         # unsupported split (> 8 waves)
    assert call(opts=ctypes.byref(opts)) == 1
    opts = w4.GemmOpts(1, 0)
    assert call(m=100, lda8=512, opts=ctypes.byref(opts)) == 2   # skinny is M <= 64
    # tiled shapes that do not exist: 8-wave tiles only as 8 x 4 tiles per
    # wave with 3 stages (row groups) or 2 stages (k-groups), never both;
    # row groups and k-groups 1 or 2; four-wave tiles only to the pipeline
    # depth that fits LDS (8 x 4: 4, 4 x 4: 5, 8 x 2: 6, 4 x 2: 8, not 5 or 7)
    for v, ks, nt, mt, st, rg in ((2, 0, 0, 4, 0, 2), (2, 0, 0, 8, 2, 2), (2, 0, 2, 8, 3, 2),
                                  (2, 0, 0, 0, 0, 3), (2, 0, 0, 8, 5, 1), (2, 0, 0, 6, 0, 1),
                                  (2, 0, 4, 4, 6, 1), (2, 0, 2, 8, 7, 1), (2, 0, 2, 4, 5, 1),
                                  (2, 0, 2, 4, 9, 1), (2, 0, 2, 4, 1, 1),
                                  (2, 3, 0, 0, 0, 0), (2, 2, 2, 8, 4, 0), (2, 2, 0, 8, 3, 0),
                                  (2, 2, 2, 4, 5, 0), (2, 2, 0, 8, 0, 2)):
        opts = w4.GemmOpts(v, ks, nt, mt, st, rg)
        assert call(m=100, lda8=512, opts=ctypes.byref(opts)) == 1, (mt, st, rg)
    # K split over workgroups: at most 16 slices; the workspace must hold
    # slices * m * n * 4 bytes and be 16-byte aligned
    opts = w4.GemmOpts(2, 0, 0, 0, 0, 0, 17)
    assert call(m=100, lda8=512, opts=ctypes.byref(opts)) == 1
    opts = w4.GemmOpts(2, 0, 0, 0, 0, 0, 2)
    assert call(m=100, lda8=512, opts=ctypes.byref(opts)) == 3          # no workspace
    need = 2 * 100 * 256 * 4                          # m = 100, n = 256
    assert call(m=100, lda8=512, ws=ctypes.c_void_p(4096), wsb=need - 1,
                opts=ctypes.byref(opts)) == 3
    assert call(m=100, lda8=512, ws=ctypes.c_void_p(4104), wsb=need,
                opts=ctypes.byref(opts)) == 1                             # misaligned


def test_gemm_workspace_size():
    """Workspace bytes follow the same plan as w4a8_gemm (host only)."""
    L = w4.lib
    assert L.w4a8_gemm_workspace_size(16, 4096, 4096, 128, None) == 0       # skinny: none
    assert L.w4a8_gemm_workspace_size(4096, 8192, 8192, 128, None) == 0     # big grid: none
    # few 128 x 256 tiles and long K: K split over workgroups, int32 partials
    need = L.w4a8_gemm_workspace_size(256, 4096, 14336, 128, None)
    assert need > 0 and need % (256 * 4096 * 4) == 0 and need // (256 * 4096 * 4) in range(2, 9)
    opts = w4.GemmOpts(2, 0, 0, 0, 0, 0, 3)
    assert L.w4a8_gemm_workspace_size(100, 256, 1024, 64, ctypes.byref(opts)) == 3 * 100 * 256 * 4
    opts = w4.GemmOpts(2, 0, 0, 8, 2, 0, 0)                  # forced shape: no automatic split
    assert L.w4a8_gemm_workspace_size(256, 4096, 14336, 128, ctypes.byref(opts)) == 0
    opts = w4.GemmOpts(2, 0, 0, 0, 0, 0, 12)                 # more slices than k-blocks: one each
    assert L.w4a8_gemm_workspace_size(100, 256, 1024, 128, ctypes.byref(opts)) == 8 * 100 * 256 * 4
    opts = w4.GemmOpts(2, 0, 0, 0, 0, 0, 17)                 # beyond 16 slices: invalid, none
    assert L.w4a8_gemm_workspace_size(100, 256, 4096, 128, ctypes.byref(opts)) == 0
    assert L.w4a8_gemm_workspace_size(256, 4096, 14336, 96, None) == 0     # unsupported g


def test_plan_splits_follow_the_measured_regimes():
    """The automatic plan's K splits, read through the workspace size (one
    int32 plane of M x N per slice): the skinny kernel (no split) up to 32
    tokens on wide layers and up to 64 tiles of 64 x 128 at any M <= 64;
    64 x 128 tiles split in two from 40 tokens on 80-191 such tiles; at
    129-192 tokens 64 x 128 tiles split towards ~384 workgroups; none on
    grids that fill the GPU."""
    L = w4.lib
    plane = lambda m, n: m * n * 4
    assert L.w4a8_gemm_workspace_size(32, 11008, 4096, 128, None) == 0        # skinny
    assert L.w4a8_gemm_workspace_size(64, 6144, 4096, 128, None) == 0         # skinny (48 tiles)
    assert L.w4a8_gemm_workspace_size(48, 11008, 4096, 128, None) == 2 * plane(48, 11008)
    assert L.w4a8_gemm_workspace_size(64, 16384, 4096, 128, None) == 2 * plane(64, 16384)
    assert L.w4a8_gemm_workspace_size(48, 11008, 2048, 128, None) == 0        # K < 4096: skinny
    # 160 tokens, 96 tiles of 64 x 128: ceil(384 / 96) = 4 slices
    assert L.w4a8_gemm_workspace_size(160, 4096, 11008, 128, None) == 4 * plane(160, 4096)
    # 192 tokens, 120 tiles: ceil(384 / 120) = 4, at most K / 2048 = 6
    assert L.w4a8_gemm_workspace_size(192, 5120, 13824, 128, None) == 4 * plane(192, 5120)
    assert L.w4a8_gemm_workspace_size(1536, 11008, 4096, 128, None) == 0      # full grid
    assert L.w4a8_gemm_workspace_size(1536, 8192, 8192, 128, None) == 0
    assert L.w4a8_gemm_workspace_size(0, 4096, 14336, 128, None) == 0


def test_linear_validates_before_any_hip_call():
    L = w4.lib
    fake = ctypes.c_void_p(4096)
    # (a, lda, m, k, blob, n, g, y, ldy, a8, lda8, s_a, acc, ldacc, ws, ws_bytes, opts, stream)
    args = [fake, 512, 4, 512, fake, 256, 128, fake, 256, fake, 512, fake, None, 0, None, 0,
            None, None]
    names = ["a", "lda", "m", "k", "blob", "n", "g", "y", "ldy", "a8", "lda8", "s_a", "acc",
             "ldacc", "ws", "wsb", "opts", "stream"]

    def call(**kw):
        a = list(args)
        for key, v in kw.items():
            a[names.index(key)] = v
        return L.w4a8_linear(*a)

    assert call(n=250) == 2
    assert call(g=96) == 2
    assert call(m=-1) == 1
    assert call(m=0, a=None, a8=None, s_a=None, y=None, blob=None) == 0
    for key in ("a", "blob", "y", "a8", "s_a"):
        assert call(**{key: None}) == 1, key
    assert call(lda=500) == 1                          # lda < k
    assert call(lda=516) == 1                          # lda % 8
    assert call(lda8=520) == 1                         # lda8 % 16
    assert call(a=ctypes.c_void_p(4104)) == 1          # misaligned activations
    assert call(a8=ctypes.c_void_p(4104)) == 1         # misaligned A8
    opts = w4.GemmOpts(4)
    assert call(opts=ctypes.byref(opts)) == 1          # no such variant
    opts = w4.GemmOpts(3)
    assert call(m=17, opts=ctypes.byref(opts)) == 2    # fused: at most 16 rows
    assert call(m=8, k=14336, lda=14336, lda8=14336, opts=ctypes.byref(opts)) == 2  # rows x K range
    opts = w4.GemmOpts(3, 0, 0, 0, 0, 0, 0, -1)
    assert call(opts=ctypes.byref(opts)) == 1          # negative workgroup count
    opts = w4.GemmOpts(3)
    assert call(m=4, k=131072, lda=131072, lda8=131072, opts=ctypes.byref(opts)) == 2  # long K


@pytest.mark.skipif(torch.cuda.device_count() > 0,
                    reason="passes fake device pointers: host-only check")
def test_linear_checks_the_gemm_before_the_quantizer():
    """w4a8_linear on the two-launch path rejects what w4a8_gemm would reject
    before it enqueues the quantizer: the fake pointers are never used."""
    L = w4.lib
    fake = ctypes.c_void_p(4096)
    m, n, k, g = 100, 4096, 14336, 128
    assert L.w4a8_linear_launches(m, n, k, g, None) == 3           # K split: needs a workspace
    need = L.w4a8_gemm_workspace_size(m, n, k, g, None)
    assert need > 0
    # (a, lda, m, k, blob, n, g, y, ldy, a8, lda8, s_a, acc, ldacc, ws, ws_bytes, opts, stream)
    assert L.w4a8_linear(fake, k, m, k, fake, n, g, fake, n, fake, k, fake, None, 0, None, 0,
                         None, None) == 3                           # no workspace
    assert L.w4a8_linear(fake, k, m, k, fake, n, g, fake, n, fake, k, fake, None, 0, fake,
                         need - 16, None, None) == 3                # workspace too small
    assert L.w4a8_linear(fake, k, m, k, fake, n, g, fake, n, fake, k, fake, None, 0,
                         ctypes.c_void_p(4104), need, None, None) == 1   # misaligned workspace
    opts = w4.GemmOpts(1)
    assert L.w4a8_linear(fake, k, m, k, fake, n, g, fake, n, fake, k, fake, None, 0, None, 0,
                         ctypes.byref(opts), None) == 2             # skinny: at most 64 rows
    opts = w4.GemmOpts(2, 0, 0, 0, 0, 0, 17)
    assert L.w4a8_linear(fake, k, m, k, fake, n, g, fake, n, fake, k, fake, None, 0, None, 0,
                         ctypes.byref(opts), None) == 1             # more slices than allowed
    opts = w4.GemmOpts(2, 0, 0, 7)
    assert L.w4a8_linear(fake, k, m, k, fake, n, g, fake, n, fake, k, fake, None, 0, None, 0,
                         ctypes.byref(opts), None) == 1             # no such row-tile count


def test_linear_launch_plan():
    """w4a8_linear_launches: one fused launch up to 57344 activations
    (M x K), 65536 on layers of 16384 columns or more, where the fused
    kernel applies, two otherwise, three when the
    GEMM splits K over workgroups; forced, the fused kernel takes up to 16
    tokens (rows x k-blocks per wave within its budget, wave ranges of at
    most 16 blocks)."""
    L = w4.lib
    assert L.w4a8_linear_launches(1, 4096, 4096, 128, None) == 1
    assert L.w4a8_linear_launches(2, 28672, 4096, 32, None) == 1
    assert L.w4a8_linear_launches(1, 4096, 14336, 0, None) == 1
    assert L.w4a8_linear_launches(4, 4096, 4096, 128, None) == 1
    assert L.w4a8_linear_launches(2, 4096, 14336, 128, None) == 1
    assert L.w4a8_linear_launches(2, 256, 1024, 1, None) == 1         # codebook weights
    assert L.w4a8_linear_launches(8, 4096, 4096, 128, None) == 1
    assert L.w4a8_linear_launches(14, 4096, 4096, 128, None) == 1     # 57344 activations
    assert L.w4a8_linear_launches(15, 4096, 4096, 128, None) == 2
    assert L.w4a8_linear_launches(4, 4096, 14336, 128, None) == 1
    assert L.w4a8_linear_launches(16, 4096, 4096, 128, None) == 2
    assert L.w4a8_linear_launches(16, 16384, 4096, 128, None) == 1    # wide: 65536 activations
    assert L.w4a8_linear_launches(16, 16368, 4096, 128, None) == 2
    assert L.w4a8_linear_launches(17, 4096, 4096, 128, None) == 2
    assert L.w4a8_linear_launches(256, 4096, 14336, 128, None) == 3
    assert L.w4a8_linear_launches(64, 4096, 14336, 128, None) == 3    # 17..64 tokens, long K
    assert L.w4a8_linear_launches(24, 4096, 14336, 128, None) == 2    # below 393216 activations
    assert L.w4a8_linear_launches(1, 4096, 131072, 128, None) == 2    # K range too long to fuse
    opts = w4.GemmOpts(3)
    assert L.w4a8_linear_launches(16, 4096, 4096, 128, ctypes.byref(opts)) == 1
    assert L.w4a8_linear_launches(4, 4096, 14336, 128, ctypes.byref(opts)) == 1
    assert L.w4a8_linear_launches(5, 4096, 14336, 128, ctypes.byref(opts)) == 0  # 8 rows x 16 blocks
    assert L.w4a8_linear_launches(17, 4096, 4096, 128, ctypes.byref(opts)) == 0
    opts = w4.GemmOpts(3, 0, 4)
    assert L.w4a8_linear_launches(1, 4096, 4096, 128, ctypes.byref(opts)) == 0  # 1 or 2 tiles
    opts = w4.GemmOpts(3, 0, 0, 0, 0, 0, 0, -1)
    assert L.w4a8_linear_launches(1, 4096, 4096, 128, ctypes.byref(opts)) == 0
    assert L.w4a8_linear_launches(1, 4008, 4096, 128, None) == 0      # n % 16


def test_w4a16_validates_before_any_hip_call():
    L = w4.lib
    fake = ctypes.c_void_p(4096)
    # (a, lda, m, k, blob, n, g, y, ldy, opts, stream)
    assert L.w4a16_gemm(fake, 512, 4, 512, fake, 250, 128, fake, 256, None, None) == 2   # n % 16
    opts = w4.GemmOpts(1)
    assert L.w4a16_gemm(fake, 512, 129, 512, fake, 256, 128, fake, 256, ctypes.byref(opts),
                        None) == 2                                                    # skinny, m > 128
    assert L.w4a16_gemm(fake, 512, 65, 512, fake, 256, 1, fake, 256, None, None) == 2    # codebook
    assert L.w4a16_gemm(fake, 516, 4, 512, fake, 256, 128, fake, 256, None, None) == 1   # lda % 8
    assert L.w4a16_gemm(fake, 500, 4, 512, fake, 256, 128, fake, 256, None, None) == 1   # lda < k
    assert L.w4a16_gemm(None, 512, 4, 512, fake, 256, 128, fake, 256, None, None) == 1
    assert L.w4a16_gemm(ctypes.c_void_p(4104), 512, 4, 512, fake, 256, 128, fake, 256, None,
                        None) == 1                                                    # misaligned
    opts = w4.GemmOpts(3)
    assert L.w4a16_gemm(fake, 512, 4, 512, fake, 256, 128, fake, 256, ctypes.byref(opts),
                        None) == 1                                                    # no variant 3
    opts = w4.GemmOpts(1, 9)
    assert L.w4a16_gemm(fake, 512, 4, 512, fake, 256, 128, fake, 256, ctypes.byref(opts),
                        None) == 1                                                    # > 8 waves
    assert L.w4a16_gemm(None, 512, 0, 512, None, 256, 128, None, 256, None, None) == 0



def test_row_strides_are_bounded():
    """Activation row strides above W4A8_LD_MAX are refused before any HIP
    call (the tiled kernels address 256 rows through one 32-bit buffer range)."""
    L = w4.lib
    fake = ctypes.c_void_p(4096)
    big = (1 << 22) + 16
    ws = ctypes.c_void_p(8192)
    # w4a8_gemm(a8, lda8, s_a, m, blob, n, k, g, y, ldy, acc, ldacc, ws, ws_bytes, opts, stream)
    assert L.w4a8_gemm(fake, big, fake, 4, fake, 256, 512, 128, fake, 256, None, 0, ws, 1 << 20,
                       None, None) == 1
    assert L.w4a8_gemm_noalloc(fake, big, fake, 4, fake, 256, 512, 128, fake, 256, None, 0,
                               None, None) == 1
    # w4a8_linear(a, lda, m, k, blob, n, g, y, ldy, a8, lda8, s_a, acc, ldacc, ws, ws_bytes, opts, stream)
    assert L.w4a8_linear(fake, big, 4, 512, fake, 256, 128, fake, 256, fake, 512, fake, None, 0,
                         ws, 1 << 20, None, None) == 1
    assert L.w4a8_linear(fake, 512, 4, 512, fake, 256, 128, fake, 256, fake, big, fake, None, 0,
                         ws, 1 << 20, None, None) == 1
    assert L.w4a16_gemm(fake, big, 4, 512, fake, 256, 128, fake, 256, None, None) == 1


def test_read_probe_validates_before_any_hip_call():
    L = w4.lib
    fake = ctypes.c_void_p(4096)
    assert L.w4a8_read_probe(fake, 0, 256, fake, None) == 0          # nothing to read
    assert L.w4a8_read_probe(None, 4096, 256, fake, None) == 1
    assert L.w4a8_read_probe(fake, 4096, 256, None, None) == 1
    assert L.w4a8_read_probe(fake, 4104, 256, fake, None) == 1       # not a multiple of 16
    assert L.w4a8_read_probe(ctypes.c_void_p(4104), 4096, 256, fake, None) == 1   # misaligned
    assert L.w4a8_read_probe(fake, 4096, 0, fake, None) == 1
    assert L.w4a8_read_probe(fake, 4096, 65537, fake, None) == 1


def test_gemm_noalloc_validates_before_any_hip_call():
    """The allocation-free GEMM checks its arguments, and that a forced K
    split fits the static scratch, before any HIP call."""
    L = w4.lib
    fake = ctypes.c_void_p(4096)
    # (a8, lda8, s_a, m, blob, n, k, g, y, ldy, acc, ldacc, opts, stream)
    assert L.w4a8_gemm_noalloc(None, 512, None, 0, None, 256, 512, 128, None, 256, None, 0,
                               None, None) == 0                                  # m == 0
    assert L.w4a8_gemm_noalloc(fake, 512, fake, 4, fake, 250, 512, 128, fake, 256, None, 0,
                               None, None) == 2                                  # n % 16
    assert L.w4a8_gemm_noalloc(None, 512, fake, 4, fake, 256, 512, 128, fake, 256, None, 0,
                               None, None) == 1
    assert L.w4a8_gemm_noalloc(fake, 520, fake, 4, fake, 256, 512, 128, fake, 256, None, 0,
                               None, None) == 1                                  # lda8 % 16
    opts = w4.GemmOpts(0, 0, 0, 0, 0, 0, 2)
    assert L.w4a8_gemm_noalloc(fake, 8192, fake, 4096, fake, 4096, 8192, 128, fake, 4096, None,
                               0, ctypes.byref(opts), None) == 3    # 2 x 64 MiB of partial sums
    opts = w4.GemmOpts(1)
    assert L.w4a8_gemm_noalloc(fake, 8192, fake, 100, fake, 4096, 8192, 128, fake, 4096, None,
                               0, ctypes.byref(opts), None) == 2    # skinny: at most 64 rows
