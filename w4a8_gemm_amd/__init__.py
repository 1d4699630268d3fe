"""Python binding of libw4a8.so (the MI355X W4A8 linear layer).

This module only marshals arguments: numpy arrays for the host packer,
torch tensors for device memory, and torch's current HIP stream.  Every
step of the layer runs inside the C ABI library; there is no fallback.  If
the library has not been built, importing this module raises.

    blob  = pack(w, g)                       # host, offline
    wdev  = to_device(blob)                  # one copy to HBM
    a8, s_a = quant_act(a)                   # per-token int8 (GPU)
    y     = gemm(a8, s_a, wdev, n, k, g)     # W4A8 GEMM (GPU)
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4a8.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "w4a8.h")

GROUP_PER_CHANNEL = 0
K_QUANTUM = 128
N_QUANTUM = 16
K_MAX = 131072

STATUS = {
    0: "W4A8_OK",
    1: "W4A8_ERR_INVALID_ARGUMENT",
    2: "W4A8_ERR_UNSUPPORTED",
    3: "W4A8_ERR_BUFFER_TOO_SMALL",
    4: "W4A8_ERR_NONFINITE",
    5: "W4A8_ERR_RANGE",
    6: "W4A8_ERR_LAYOUT",
    7: "W4A8_ERR_DEVICE",
}


class W4A8Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


class GemmOpts(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int), ("k_split", ctypes.c_int),
                ("n_tiles", ctypes.c_int), ("m_tiles", ctypes.c_int),
                ("stages", ctypes.c_int), ("row_groups", ctypes.c_int),
                ("slices", ctypes.c_int), ("workgroups", ctypes.c_int)]


def _load():
    # torch is imported first on purpose: it carries its own HIP runtime
    # (same soname as the system one).  Loading it first makes the library's
    # libamdhip64 dependency resolve to that already-loaded runtime, so torch
    # allocations, torch streams and this library's kernels share one HIP
    # runtime in the process.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python w4a8_gemm_amd/build.py` (or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    sig = {
        "w4a8_status_string": (ctypes.c_char_p, [I]),
        "w4a8_last_device_error": (ctypes.c_char_p, []),
        "w4a8_packed_size": (Z, [I, I, I]),
        "w4a8_pack": (I, [P, I, I, I, I, P, Z, I]),
        "w4a8_blob_info": (I, [P, Z, P, P, P]),
        "w4a8_unpack": (I, [P, Z, P, P, P, P]),
        "w4a8_quant_act": (I, [P, I, I, I, P, I, P, P]),
        "w4a8_quant_act_static": (I, [P, I, I, I, ctypes.c_uint16, P, I, P, P]),
        "w4a8_gemm_workspace_size": (Z, [I, I, I, I, P]),
        "w4a8_gemm": (I, [P, I, P, I, P, I, I, I, P, I, P, I, P, Z, P, P]),
        "w4a8_linear": (I, [P, I, I, I, P, I, I, P, I, P, I, P, P, I, P, Z, P, P]),
        "w4a8_linear_launches": (I, [I, I, I, I, P]),
        "w4a16_gemm": (I, [P, I, I, I, P, I, I, P, I, P, P]),
        "w4a8_read_probe": (I, [P, Z, I, P, P]),
        "w4a8_gemm_noalloc": (I, [P, I, P, I, P, I, I, I, P, I, P, I, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def header_functions() -> list[str]:
    """Names of the functions declared in include/w4a8.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(w4a8_[a-z0-9_]+)\s*\(", text)))


def _check(status: int, where: str):
    if status != 0:
        if status == 7:
            where = f"{where} ({lib.w4a8_last_device_error().decode()})"
        raise W4A8Error(status, where)


def status_string(status: int) -> str:
    return lib.w4a8_status_string(status).decode()


# ------------------------------------------------------------------ host side
GROUP_PER_CHANNEL = 0
CODEBOOK_NF = 1      # g value of the non-uniform codebook mode


def packed_size(n: int, k: int, g: int) -> int:
    return int(lib.w4a8_packed_size(n, k, g))


def pack(w: np.ndarray, g: int, n_threads: int = 0) -> np.ndarray:
    """Quantize and pack an N x K float32 weight matrix; returns the blob (uint8)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    size = packed_size(n, k, g)
    if size == 0:
        raise W4A8Error(2, "w4a8_packed_size")
    blob = np.empty(size, dtype=np.uint8)
    _check(lib.w4a8_pack(w.ctypes.data, n, k, k, g, blob.ctypes.data, size, n_threads),
           "w4a8_pack")
    return blob


def blob_info(blob: np.ndarray) -> tuple[int, int, int]:
    n, k, g = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(lib.w4a8_blob_info(blob.ctypes.data, blob.nbytes, ctypes.byref(n), ctypes.byref(k),
                              ctypes.byref(g)), "w4a8_blob_info")
    return n.value, k.value, g.value


def unpack(blob: np.ndarray) -> dict:
    """Logical arrays of a host blob: q [N,K], z/s2 [N,G], s1 [N] (float16)."""
    n, k, g = blob_info(blob)
    groups = 1 if g == 0 else (0 if g == CODEBOOK_NF else k // g)
    q = np.empty((n, k), dtype=np.uint8)
    z = np.empty((n, groups), dtype=np.uint8)
    s2 = np.empty((n, groups), dtype=np.uint8)
    s1 = np.empty(n, dtype=np.uint16)
    _check(lib.w4a8_unpack(blob.ctypes.data, blob.nbytes, q.ctypes.data, z.ctypes.data,
                           s2.ctypes.data, s1.ctypes.data), "w4a8_unpack")
    out = {"q": q, "z": z, "s2": s2, "s1": s1.view(np.float16), "n": n, "k": k, "g": g}
    if g == CODEBOOK_NF:
        out["levels"] = blob[56:72].view(np.int8).astype(np.int32)
    return out


# ------------------------------------------------------------------ device side
def _torch():
    import torch
    return torch


def _stream_ptr(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def to_device(blob: np.ndarray, device="cuda"):
    """Copy a packed blob to device memory (a uint8 torch tensor)."""
    torch = _torch()
    return torch.from_numpy(blob).to(device)


def quant_act(a, a8=None, s_a=None, stream=None):
    """Per-token int8 quantization of an M x K float16 CUDA tensor."""
    torch = _torch()
    assert a.dtype == torch.float16 and a.is_cuda and a.dim() == 2 and a.stride(1) == 1
    m, k = a.shape
    if a8 is None:
        a8 = torch.empty((m, k), dtype=torch.int8, device=a.device)
    if s_a is None:
        s_a = torch.empty((m,), dtype=torch.float16, device=a.device)
    _check(lib.w4a8_quant_act(a.data_ptr(), m, k, a.stride(0), a8.data_ptr(), a8.stride(0),
                              s_a.data_ptr(), _stream_ptr(stream)), "w4a8_quant_act")
    return a8, s_a


def quant_act_static(a, scale, a8=None, s_a=None, stream=None):
    """Int8 quantization of an M x K float16 CUDA tensor with one static
    fp16 scale; s_a is filled with the scale for every row."""
    import numpy as np
    torch = _torch()
    assert a.dtype == torch.float16 and a.is_cuda and a.dim() == 2 and a.stride(1) == 1
    m, k = a.shape
    if a8 is None:
        a8 = torch.empty((m, k), dtype=torch.int8, device=a.device)
    if s_a is None:
        s_a = torch.empty((m,), dtype=torch.float16, device=a.device)
    bits = int(np.array([scale], dtype=np.float16).view(np.uint16)[0])
    _check(lib.w4a8_quant_act_static(a.data_ptr(), m, k, a.stride(0), bits, a8.data_ptr(),
                                     a8.stride(0), s_a.data_ptr(), _stream_ptr(stream)),
           "w4a8_quant_act_static")
    return a8, s_a


def gemm(a8, s_a, blob_dev, n: int, k: int, g: int, y=None, acc=None, want_acc=False,
         variant: int = 0, k_split: int = 0, n_tiles: int = 0, m_tiles: int = 0,
         stages: int = 0, row_groups: int = 0, slices: int = 0, workspace=None, stream=None):
    """Y = fp16(s_a * s1 * (A8 @ W8^.T)); returns y (and the int32 acc if asked)."""
    torch = _torch()
    m = a8.shape[0]
    assert a8.dtype == torch.int8 and a8.is_cuda and a8.stride(1) == 1
    if y is None:
        y = torch.empty((m, n), dtype=torch.float16, device=a8.device)
    if want_acc and acc is None:
        acc = torch.empty((m, n), dtype=torch.int32, device=a8.device)
    opts = None
    if variant or k_split or n_tiles or m_tiles or stages or row_groups or slices:
        opts = GemmOpts(variant, k_split, n_tiles, m_tiles, stages, row_groups, slices)
    ws_need = int(lib.w4a8_gemm_workspace_size(m, n, k, g,
                                               ctypes.byref(opts) if opts is not None else None))
    if ws_need and workspace is None:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=a8.device)
    st = lib.w4a8_gemm(a8.data_ptr(), a8.stride(0), s_a.data_ptr(), m, blob_dev.data_ptr(), n, k,
                       g, y.data_ptr(), y.stride(0),
                       acc.data_ptr() if acc is not None else None,
                       acc.stride(0) if acc is not None else 0,
                       workspace.data_ptr() if workspace is not None else None,
                       workspace.numel() if workspace is not None else 0,
                       ctypes.byref(opts) if opts is not None else None, _stream_ptr(stream))
    _check(st, "w4a8_gemm")
    return (y, acc) if acc is not None else y


def gemm_noalloc(a8, s_a, blob_dev, n: int, k: int, g: int, y, acc=None, slices: int = 0,
                 stream=None):
    """w4a8_gemm_noalloc: the GEMM with no workspace argument (a K split keeps
    its partial sums in the library's static device scratch).  y (and acc,
    if given) must be preallocated; nothing is allocated here."""
    torch = _torch()
    m = a8.shape[0]
    assert a8.dtype == torch.int8 and a8.is_cuda and a8.stride(1) == 1
    opts = GemmOpts(0, 0, 0, 0, 0, 0, slices) if slices else None
    st = lib.w4a8_gemm_noalloc(a8.data_ptr(), a8.stride(0), s_a.data_ptr(), m,
                               blob_dev.data_ptr(), n, k, g, y.data_ptr(), y.stride(0),
                               acc.data_ptr() if acc is not None else None,
                               acc.stride(0) if acc is not None else 0,
                               ctypes.byref(opts) if opts is not None else None,
                               _stream_ptr(stream))
    _check(st, "w4a8_gemm_noalloc")
    return (y, acc) if acc is not None else y


def linear(a, blob_dev, n: int, k: int, g: int, y=None, a8=None, s_a=None, acc=None,
           want_acc=False, variant: int = 0, k_split: int = 0, n_tiles: int = 0,
           m_tiles: int = 0, stages: int = 0, row_groups: int = 0, slices: int = 0,
           workgroups: int = 0, workspace=None, stream=None):
    """The whole layer from fp16 activations (fused for small M); returns
    (y, a8, s_a) or (y, a8, s_a, acc)."""
    torch = _torch()
    assert a.dtype == torch.float16 and a.is_cuda and a.dim() == 2 and a.stride(1) == 1
    m = a.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float16, device=a.device)
    if a8 is None:
        a8 = torch.empty((m, k), dtype=torch.int8, device=a.device)
    if s_a is None:
        s_a = torch.empty((m,), dtype=torch.float16, device=a.device)
    if want_acc and acc is None:
        acc = torch.empty((m, n), dtype=torch.int32, device=a.device)
    opts = None
    if variant or k_split or n_tiles or m_tiles or stages or row_groups or slices or workgroups:
        opts = GemmOpts(variant, k_split, n_tiles, m_tiles, stages, row_groups, slices, workgroups)
    ws_opts = opts if (opts is None or variant != 3) else None
    ws_need = 0 if variant == 3 else int(lib.w4a8_gemm_workspace_size(
        m, n, k, g, ctypes.byref(ws_opts) if ws_opts is not None else None))
    if ws_need and workspace is None:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=a.device)
    st = lib.w4a8_linear(a.data_ptr(), a.stride(0), m, k, blob_dev.data_ptr(), n, g,
                         y.data_ptr(), y.stride(0), a8.data_ptr(), a8.stride(0), s_a.data_ptr(),
                         acc.data_ptr() if acc is not None else None,
                         acc.stride(0) if acc is not None else 0,
                         workspace.data_ptr() if workspace is not None else None,
                         workspace.numel() if workspace is not None else 0,
                         ctypes.byref(opts) if opts is not None else None, _stream_ptr(stream))
    _check(st, "w4a8_linear")
    return (y, a8, s_a, acc) if acc is not None else (y, a8, s_a)


def w4a16(a, blob_dev, n: int, k: int, g: int, y=None, variant: int = 0, k_split: int = 0,
          n_tiles: int = 0, stream=None):
    """W4A16 comparison GEMM on the same blob: fp16 A times fp16-decoded weights."""
    torch = _torch()
    assert a.dtype == torch.float16 and a.is_cuda and a.dim() == 2 and a.stride(1) == 1
    m = a.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float16, device=a.device)
    opts = None
    if variant or k_split or n_tiles:
        opts = GemmOpts(variant, k_split, n_tiles)
    _check(lib.w4a16_gemm(a.data_ptr(), a.stride(0), m, k, blob_dev.data_ptr(), n, g,
                          y.data_ptr(), y.stride(0),
                          ctypes.byref(opts) if opts is not None else None, _stream_ptr(stream)),
           "w4a16_gemm")
    return y


def read_probe(buf, offset: int, nbytes: int, workgroups: int, sink, stream=None):
    """Measurement aid: a read-only stream over nbytes of the uint8 CUDA tensor
    `buf` from byte `offset` (w4a8_read_probe); sink is an int32 CUDA tensor of
    at least `workgroups` elements."""
    assert buf.is_cuda and 0 <= offset and offset + nbytes <= buf.numel() * buf.element_size()
    assert sink.numel() >= workgroups
    _check(lib.w4a8_read_probe(buf.data_ptr() + offset, nbytes, workgroups, sink.data_ptr(),
                               _stream_ptr(stream)), "w4a8_read_probe")
