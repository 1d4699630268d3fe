"""Driver run in a child process against the host-only sanitized build of the
C ABI (see test_host_sanitizers.py).  It imports no GPU runtime: it packs a
list of weight matrices, unpacks them into an .npz for the parent to check
against the oracle, and throws a few thousand random argument sets at every
entry point's validation and planning.  AddressSanitizer and
UndefinedBehaviorSanitizer abort the process on the first error.

    python san_driver.py LIB OUT.npz CASES.json
"""
import ctypes
import json
import sys

import numpy as np


def main():
    lib_path, out_path, cases_path = sys.argv[1:4]
    L = ctypes.CDLL(lib_path)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    sig = {
        "w4a8_packed_size": (Z, [I, I, I]),
        "w4a8_pack": (I, [P, I, I, I, I, P, Z, I]),
        "w4a8_blob_info": (I, [P, Z, P, P, P]),
        "w4a8_unpack": (I, [P, Z, P, P, P, P]),
        "w4a8_quant_act": (I, [P, I, I, I, P, I, P, P]),
        "w4a8_quant_act_static": (I, [P, I, I, I, ctypes.c_uint16, P, I, P, P]),
        "w4a8_gemm_workspace_size": (Z, [I, I, I, I, P]),
        "w4a8_gemm": (I, [P, I, P, I, P, I, I, I, P, I, P, I, P, Z, P, P]),
        "w4a8_gemm_noalloc": (I, [P, I, P, I, P, I, I, I, P, I, P, I, P, P]),
        "w4a8_linear": (I, [P, I, I, I, P, I, I, P, I, P, I, P, P, I, P, Z, P, P]),
        "w4a8_linear_launches": (I, [I, I, I, I, P]),
        "w4a16_gemm": (I, [P, I, I, I, P, I, I, P, I, P, P]),
        "w4a8_read_probe": (I, [P, Z, I, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args

    class Opts(ctypes.Structure):
        _fields_ = [(f, I) for f in ("variant", "k_split", "n_tiles", "m_tiles", "stages",
                                     "row_groups", "slices", "workgroups")]

    # ---- packing: every case packed, unpacked and handed back
    cases = json.load(open(cases_path))
    out = {}
    for ci, c in enumerate(cases):
        w = np.load(c["w_path"]).astype(np.float32)
        n, k = w.shape
        g = c["g"]
        size = L.w4a8_packed_size(n, k, g)
        blob = np.zeros(max(size, 1), dtype=np.uint8)
        st = L.w4a8_pack(w.ctypes.data, n, k, k, g, blob.ctypes.data, size, c.get("threads", 0))
        out[f"status_{ci}"] = np.array(st)
        if st != 0:
            continue
        groups = 1 if g in (0, k) else (0 if g == 1 else k // g)
        q = np.zeros((n, k), np.uint8)
        z = np.zeros((n, max(groups, 1)), np.uint8)
        s2 = np.zeros((n, max(groups, 1)), np.uint8)
        s1 = np.zeros(n, np.uint16)
        st = L.w4a8_unpack(blob.ctypes.data, size, q.ctypes.data, z.ctypes.data,
                           s2.ctypes.data, s1.ctypes.data)
        assert st == 0, st
        out[f"q_{ci}"], out[f"z_{ci}"], out[f"s2_{ci}"], out[f"s1_{ci}"] = q, z, s2, s1
        # a truncated or corrupted blob is refused, never read past its end
        for cut in (0, 16, 255, size - 1):
            if 0 <= cut < size:
                L.w4a8_blob_info(blob.ctypes.data, cut, None, None, None)
                L.w4a8_unpack(blob.ctypes.data, cut, None, None, None, None)
    np.savez(out_path, **out)

    # ---- validation and planning with extreme arguments (fake pointers are
    # never dereferenced: a call that passes validation reaches a stub launch)
    rng = np.random.default_rng(7)
    ints = [-(2 ** 31), -1, 0, 1, 2, 15, 16, 17, 31, 32, 63, 64, 65, 100, 127, 128, 129, 255, 256,
            1000, 1024, 4096, 4104, 14336, 24576, 49152, 131072, 131200, 1 << 20, 2 ** 30,
            2 ** 31 - 1]
    gs = [-1, 0, 1, 2, 16, 32, 64, 96, 128, 256, 4096]
    ptrs = [None, 4096, 4104, 1 << 40]
    statuses = set()
    for it in range(4000):
        pick = lambda xs: xs[int(rng.integers(len(xs)))]
        m, n, k, g = pick(ints), pick(ints), pick(ints), pick(gs)
        if rng.random() < 0.5:
            n = 16 * int(rng.integers(1, 4096))
            k = 128 * int(rng.integers(1, 1025))
            m = int(rng.integers(0, 5000))
        ld = pick(ints)
        o = Opts(*[int(pick([0, 0, 0, 1, 2, 3, 4, 8, 16, 17, -1, 2 ** 30])) for _ in range(8)])
        op = ctypes.byref(o) if rng.random() < 0.5 else None
        p1, p2, p3, p4 = pick(ptrs), pick(ptrs), pick(ptrs), pick(ptrs)
        ws = int(pick([0, 16, 1 << 20, 1 << 40]))
        statuses.add(L.w4a8_gemm_workspace_size(m, n, k, g, op) >= 0)
        statuses.add(L.w4a8_linear_launches(m, n, k, g, op))
        for st in (
            L.w4a8_gemm(p1, ld, p2, m, p3, n, k, g, p4, ld, None, 0, p1, ws, op, None),
            L.w4a8_gemm_noalloc(p1, ld, p2, m, p3, n, k, g, p4, ld, p2, ld, op, None),
            L.w4a8_linear(p1, ld, m, k, p2, n, g, p3, ld, p4, ld, p1, None, 0, p2, ws, op, None),
            L.w4a8_quant_act(p1, m, k, ld, p2, ld, p3, None),
            L.w4a8_quant_act_static(p1, m, k, ld, int(rng.integers(0, 65536)), p2, ld, p3, None),
            L.w4a16_gemm(p1, ld, m, k, p2, n, g, p3, ld, op, None),
            L.w4a8_read_probe(p1, ws, m, p2, None),
        ):
            assert 0 <= st <= 7, st
            statuses.add(("status", st))
    print(json.dumps({"ok": True, "statuses": sorted(str(s) for s in statuses)}))


if __name__ == "__main__":
    main()
