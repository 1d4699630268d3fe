"""Benchmark of the W4A8 linear layer on one MI355X.

One step = one pass of the whole hot path over a workload: for every run
(M, layer) of the workload, the per-token activation quantizer and the W4A8
GEMM through the C ABI library (one fused launch, w4a8_linear, where M is
small enough; else w4a8_quant_act then w4a8_gemm).  Inputs are resident in HBM
when the timed region starts.  Weight blobs rotate through a pool of copies
of at least 1 GiB so that every GEMM reads its weights from HBM rather than
from the 256 MB Infinity Cache or the L2.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

Prints one JSON line.  --gpus N > 1 is refused: the path runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, TOPS
# HBM counters are keyed to the sources of the kernel they were taken on
CSRC = os.path.join(ROOT, "w4a8_gemm_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_traffic.json")


CODEBOOK_NF = 1   # g value of the non-uniform codebook mode (no meta)

# sources of the kernels each counter entry covers (small M: fused and
# skinny; large M: tiled with its K-split reduction)
SKINNY_SOURCES = ["fused.hip", "skinny.hip", "gemm_common.h", "quant_common.h", "codebook.h"]
TILED_SOURCES = ["tiled.hip", "gemm_common.h", "quant_common.h", "codebook.h"]


def meta_bytes(n, k, g):
    if g == CODEBOOK_NF:
        return 0.0
    return 0.5 * n if g in (0, k) else 1.5 * n * k / g


def algo_bytes(m, n, k, g):
    """Bytes the method must move: codes, group meta, s1, A8, s_a, Y."""
    meta = meta_bytes(n, k, g)
    return n * k / 2 + meta + 2 * n + m * k + 2 * m + 2 * m * n


def w4a16_bytes(m, n, k, g):
    """The W4A16 comparison GEMM: the same weight bytes, fp16 A in, fp16 Y out."""
    meta = meta_bytes(n, k, g)
    return n * k / 2 + meta + 2 * n + 2 * m * k + 2 * m * n


def quant_bytes(m, k):
    return 3 * m * k + 2 * m


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash(files):
    h = hashlib.sha256()
    for name in files:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload):
    """Mean HBM bytes per GEMM launch on `workload` from committed rocprofv3
    counter runs, if they were taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            entries = json.load(f)["entries"]
    except (OSError, ValueError, KeyError):
        return None
    for t in entries:
        if t.get("workload") == workload and t.get("source_sha256_16") == source_hash(t["sources"]):
            return t.get("bytes_per_launch")
    return None


class HipEvent:
    """A HIP event created with hipEventDisableSystemFence, recorded on a given
    stream.  Timing-only events without the system-scope cache writeback and
    invalidate that a default event performs, so the interval between two of
    them is closer to the kernel in between.  Uses the HIP runtime torch has
    already loaded (same process-wide runtime as the library)."""
    _lib = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    @classmethod
    def lib(cls):
        if cls._lib is None:
            import ctypes
            import torch
            path = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
            h = ctypes.CDLL(path)
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                              ctypes.c_void_p]
            cls._lib = h
        return cls._lib

    def __init__(self):
        import ctypes
        self.h = ctypes.c_void_p()
        st = self.lib().hipEventCreateWithFlags(ctypes.byref(self.h), self.DISABLE_SYSTEM_FENCE)
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({st})")

    def record(self, stream_ptr):
        st = self.lib().hipEventRecord(self.h, stream_ptr)
        if st != 0:
            raise RuntimeError(f"hipEventRecord failed ({st})")

    def elapsed_time(self, end):
        import ctypes
        ms = ctypes.c_float()
        st = self.lib().hipEventElapsedTime(ctypes.byref(ms), self.h, end.h)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st})")
        return ms.value


def cpu_baseline(runs, weights, unit, budget_s=15.0):
    """The oracle, untuned, on a bounded sample of the same workload: every
    run, restricted to the first `cols` output columns of each layer.  The
    rate is in the metric's unit (GB/s of algorithmic bytes, or TOPS); the
    time of each oracle stage is reported beside it."""
    from oracle import ref
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    cols = 2048
    qws = {}
    for (layer, n, k, g), w in weights.items():
        qws[layer] = ref.quantize_weights(w[:cols], g)      # offline pack: not timed
    acts = {}
    for (m, layer, n, k, g, seed) in runs:
        acts[(m, layer)] = synth.activations(m, k, seed=seed)
    done_bytes = done_ops = 0.0
    stage = {"quant_act": 0.0, "decode_and_gemm": 0.0, "epilogue": 0.0}
    t0 = time.perf_counter()
    passes = 0
    while True:
        for (m, layer, n, k, g, seed) in runs:
            a = acts[(m, layer)]
            t1 = time.perf_counter()
            a8, s_a = ref.quant_act(a)
            t2 = time.perf_counter()
            w8hat = ref.decoded_weights(qws[layer])
            acc = ref.gemm_acc(a8, w8hat)
            t3 = time.perf_counter()
            ref.epilogue(acc, s_a, qws[layer]["s1"])
            t4 = time.perf_counter()
            stage["quant_act"] += t2 - t1
            stage["decode_and_gemm"] += t3 - t2
            stage["epilogue"] += t4 - t3
            ncols = min(cols, n)
            done_bytes += algo_bytes(m, ncols, k, g) + quant_bytes(m, k)
            done_ops += 2.0 * m * ncols * k
        passes += 1
        if time.perf_counter() - t0 >= budget_s or passes >= 200:
            break
    dt = time.perf_counter() - t0
    value = done_ops / dt / 1e12 if unit == "TOPS" else done_bytes / dt / 1e9
    return {"value": round(value, 4), "unit": unit, "cores": int(cores),
            "kind": "oracle",
            "sample": f"every run of the workload restricted to the first {cols} output "
                      f"columns of each layer, {passes} pass(es), {dt:.1f} s",
            "stage_seconds": {key: round(v, 3) for key, v in stage.items()}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama3_8b_decode",
                    choices=[k for k in synth.workloads() if k != "tiny"] + ["tiny"])
    ap.add_argument("--rotation-gib", type=float, default=1.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--runs-json", default="")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches instead of HIP-graph replays of the step")
    ap.add_argument("--static-scale", type=float, default=None,
                    help="quantize activations with this one static fp16 scale "
                         "(w4a8_quant_act_static) instead of per-token scales")
    ap.add_argument("--w4a16", action="store_true",
                    help="time the W4A16 comparison GEMM (same packed weights, fp16 "
                         "activations) in place of the W4A8 layer; M <= 64 workloads")
    ap.add_argument("--codebook", action="store_true",
                    help="pack every layer in the non-uniform codebook mode (register "
                         "table decode) instead of the workload's group size")
    ap.add_argument("--print-source-hash", action="store_true",
                    help="print the source hashes the HBM counter entries are keyed to")
    args = ap.parse_args()
    if args.print_source_hash:
        for files in (SKINNY_SOURCES, TILED_SOURCES):
            print(" + ".join(files), source_hash(files))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this W4A8 GEMM library has no multi-GPU path "
              "(the layer would shard by output columns or by K with an int32 all-reduce; "
              "neither is built).", file=sys.stderr)
        sys.exit(2)

    import torch
    import w4a8_gemm_amd as w4
    dev = torch.device("cuda:0")

    wl_names = list(synth.workloads().keys())
    items = synth.workloads()[args.workload]
    cfg_idx = wl_names.index(args.workload)
    if args.codebook:
        items = [(c, m, layer, n, k, CODEBOOK_NF, dist) for (c, m, layer, n, k, g, dist) in items]

    # weights: one per (layer, g); seeds as the parity tests use them
    layer_keys = []
    for (_, m, layer, n, k, g, dist) in items:
        key = (layer, n, k, g, dist)
        if key not in layer_keys:
            layer_keys.append(key)
    weights, blobs = {}, {}
    for shape_idx, (layer, n, k, g, dist) in enumerate(layer_keys):
        log(f"packing {layer} n={n} k={k} g={g}")
        w = synth.weights(n, k, seed=synth.weight_seed(cfg_idx, shape_idx, 0), dist=dist)
        blobs[(layer, g)] = w4.to_device(w4.pack(w, g), dev)
        if not args.no_cpu_baseline:
            weights[(layer, n, k, g)] = w[:2048].copy()
        del w
    per_copy = sum(b.numel() for b in blobs.values())
    ncopies = max(2, int(np.ceil(args.rotation_gib * 2 ** 30 / per_copy)))
    pool = [blobs] + [{key: b.clone() for key, b in blobs.items()} for _ in range(ncopies - 1)]
    log(f"rotation pool: {ncopies} copies x {per_copy / 2**20:.1f} MiB")

    runs = []   # (m, layer, n, k, g, seed)
    m_index = {}
    for (_, m, layer, n, k, g, dist) in items:
        shape_idx = layer_keys.index((layer, n, k, g, dist))
        mi = m_index.setdefault((layer, g), {}).setdefault(m, len(m_index[(layer, g)]))
        runs.append((m, layer, n, k, g, synth.act_seed(cfg_idx, shape_idx, mi)))

    bufs = []
    for (m, layer, n, k, g, seed) in runs:
        a = torch.from_numpy(synth.activations(m, k, seed=seed)).to(dev)
        a8 = torch.empty((m, k), dtype=torch.int8, device=dev)
        s_a = torch.empty((m,), dtype=torch.float16, device=dev)
        y = torch.empty((m, n), dtype=torch.float16, device=dev)
        ws_bytes = int(w4.lib.w4a8_gemm_workspace_size(m, n, k, g, None))
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
        bufs.append((a, a8, s_a, y, ws))

    nr = len(runs)

    stream_ptr = int(torch.cuda.current_stream().cuda_stream)

    # small M: quantization fused into the GEMM (one launch, w4a8_linear);
    # else the quantizer, then the GEMM; events bracket the GEMM launch
    fused = [int(w4.lib.w4a8_linear_launches(m, n, k, g, None)) == 1
             and args.static_scale is None and not args.w4a16 for (m, _, n, k, g, _) in runs]
    if args.w4a16 and max(r[0] for r in runs) > 64:
        print("--w4a16: the W4A16 comparison kernel covers M <= 64 only", file=sys.stderr)
        sys.exit(2)

    def launch_step(copy, record=None, gemm_only=False):
        for r, (m, layer, n, k, g, _) in enumerate(runs):
            a, a8, s_a, y, ws = bufs[r]
            if args.w4a16:
                if record is not None:
                    record[r][0].record(stream_ptr)
                w4.w4a16(a, copy[(layer, g)], n, k, g, y=y)
                if record is not None:
                    record[r][1].record(stream_ptr)
                continue
            if gemm_only:
                pass
            elif args.static_scale is not None:
                w4.quant_act_static(a, args.static_scale, a8=a8, s_a=s_a)
            elif not fused[r]:
                w4.quant_act(a, a8=a8, s_a=s_a)
            if record is not None:
                record[r][0].record(stream_ptr)
            if fused[r]:
                w4.linear(a, copy[(layer, g)], n, k, g, y=y, a8=a8, s_a=s_a, workspace=ws)
            else:
                w4.gemm(a8, s_a, copy[(layer, g)], n, k, g, y=y, workspace=ws)
            if record is not None:
                record[r][1].record(stream_ptr)

    def new_events():
        return [(HipEvent(), HipEvent()) for _ in range(nr)]

    # Pass 1 (per-launch durations for the roofline): `steps` eager steps
    # enqueued from the host behind a GPU spin kernel, so that the whole
    # region is queued when the GPU reaches it; events recorded on the launch
    # stream around each GEMM launch give its on-GPU duration.
    events = [new_events() for _ in range(args.steps)]
    for i in range(args.warmup):
        launch_step(pool[i % ncopies])
    torch.cuda.synchronize()
    t_start, t_end = HipEvent(), HipEvent()
    spin_s = max(0.02, 5e-5 * args.steps * nr)
    torch.cuda._sleep(int(2.4e9 * spin_s))          # GPU spin while the host enqueues
    t_start.record(stream_ptr)
    wall0 = time.perf_counter()
    for i in range(args.steps):
        launch_step(pool[i % ncopies], record=events[i])
    t_end.record(stream_ptr)
    enqueue_s = time.perf_counter() - wall0
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step_eager = total_ms / args.steps
    per_step_gemm = [[events[i][r][0].elapsed_time(events[i][r][1]) for r in range(nr)]
                     for i in range(args.steps)]
    log(f"eager pass: host enqueue {enqueue_s * 1e3:.1f} ms, GPU spin ~{spin_s * 1e3:.0f} ms, "
        f"timed GPU region {total_ms:.2f} ms")
    if enqueue_s * 1e3 > total_ms + 1e3 * spin_s:
        log("warning: the host enqueue outlasted the GPU spin; the GPU may have idled")

    # Pass 2 (the timed steps): each step captured once as a HIP graph (one
    # graph per weight copy of the rotation pool) and replayed, as a serving
    # loop runs its decode steps; `steps` replays are timed between two
    # synchronizations, enqueued behind a GPU spin.
    ms_per_step, timing = ms_per_step_eager, "eager launches"
    if not args.no_graph:
        try:
            graphs = []
            for i in range(ncopies):
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr):
                    launch_step(pool[i])
                graphs.append(gr)
            for i in range(args.warmup):
                graphs[i % ncopies].replay()
            torch.cuda.synchronize()
            g0 = torch.cuda.Event(enable_timing=True)
            g1 = torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(int(2.4e9 * spin_s))
            g0.record()
            for i in range(args.steps):
                graphs[i % ncopies].replay()
            g1.record()
            torch.cuda.synchronize()
            ms_per_step = g0.elapsed_time(g1) / args.steps
            timing = "HIP graph replay of each step"
        except Exception as e:
            log(f"graph replay unavailable ({e}); timing eager launches")
    log(f"ms per step: {ms_per_step:.4f} ({timing}); eager {ms_per_step_eager:.4f}")

    # Pass 3 (mean launch duration for the roofline): the step's GEMM (or
    # fused) launches alone, the quantizer launches left out (their outputs
    # are already in HBM), captured as one HIP graph per weight copy and
    # replayed `steps` times between two HIP events on the launch stream, so
    # the launches run back to back as in the timed steps and no event sits
    # between two of them.  Falls back to the eager pass's per-launch events.
    gemm_graph_us = None
    if timing.startswith("HIP graph"):
        try:
            ggraphs = []
            for i in range(ncopies):
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr):
                    launch_step(pool[i], gemm_only=True)
                ggraphs.append(gr)
            for i in range(args.warmup):
                ggraphs[i % ncopies].replay()
            torch.cuda.synchronize()
            h0, h1 = HipEvent(), HipEvent()
            torch.cuda._sleep(int(2.4e9 * spin_s))
            h0.record(stream_ptr)
            for i in range(args.steps):
                ggraphs[i % ncopies].replay()
            h1.record(stream_ptr)
            torch.cuda.synchronize()
            gemm_graph_us = h0.elapsed_time(h1) * 1e3 / (args.steps * nr)
            log(f"GEMM launches alone, graph replays: {gemm_graph_us:.3f} us per launch")
        except Exception as e:
            log(f"GEMM-only graph unavailable ({e}); launch durations from the eager pass")

    gemm_us = np.array(per_step_gemm) * 1e3
    med_us = np.median(gemm_us, axis=0)
    mean_us = gemm_us.mean(axis=0)
    p10_us, p90_us = np.percentile(gemm_us, 10, axis=0), np.percentile(gemm_us, 90, axis=0)
    step_bytes = sum(w4a16_bytes(m, n, k, g) if args.w4a16 else
                     algo_bytes(m, n, k, g) + quant_bytes(m, k) for (m, _, n, k, g, _) in runs)
    step_ops = sum(2.0 * m * n * k for (m, _, n, k, g, _) in runs)
    # bytes of the timed launch: a fused launch also reads A as fp16 and
    # writes A8 and s_a instead of reading A8 and s_a (2MK more)
    gemm_bytes = np.array([w4a16_bytes(m, n, k, g) if args.w4a16 else
                           algo_bytes(m, n, k, g) + (2 * m * k if fused[r] else 0)
                           for r, (m, _, n, k, g, _) in enumerate(runs)])
    gemm_ops = np.array([2.0 * m * n * k for (m, _, n, k, g, _) in runs])
    table = []
    for r, (m, layer, n, k, g, _) in enumerate(runs):
        t = med_us[r] * 1e-6
        table.append({"m": m, "layer": layer, "n": n, "k": k, "g": g, "fused": fused[r],
                      "gemm_us_median": round(float(med_us[r]), 3),
                      "gemm_us_mean": round(float(mean_us[r]), 3),
                      "gemm_us_p10": round(float(p10_us[r]), 3),
                      "gemm_us_p90": round(float(p90_us[r]), 3),
                      "GBps": round(gemm_bytes[r] / t / 1e9, 1),
                      "TOPS": round(gemm_ops[r] / t / 1e12, 2),
                      "frac_hbm": round(gemm_bytes[r] / t / 1e9 / HBM_PEAK_GBS, 3),
                      "frac_mfma": round(gemm_ops[r] / t / 1e12 / INT8_PEAK_TOPS, 4)})
        log(f"{layer:8s} m={m:5d} n={n:6d} k={k:6d} g={g:4d}  {'fused' if fused[r] else 'gemm '}"
            f" {med_us[r]:8.2f} us  "
            f"{table[-1]['GBps']:8.1f} GB/s ({table[-1]['frac_hbm']:.3f} HBM)  "
            f"{table[-1]['TOPS']:8.1f} TOPS ({table[-1]['frac_mfma']:.3f} MFMA)")
    if args.runs_json:
        with open(args.runs_json, "w") as f:
            json.dump(table, f, indent=1)

    # dominant kernel: the GEMM; average algorithmic bytes (or ops) per launch
    # over average launch duration
    avg_dur = (gemm_graph_us if gemm_graph_us is not None else float(mean_us.mean())) * 1e-6
    hbm_bound = args.workload in ("llama3_8b_decode", "tiny") or max(r[0] for r in runs) <= 64
    if hbm_bound:
        achieved = float(gemm_bytes.mean()) / avg_dur / 1e9
        peak, unit, bound = HBM_PEAK_GBS, "GB/s", "hbm"
    else:
        achieved = float(gemm_ops.mean()) / avg_dur / 1e12
        peak, unit, bound = INT8_PEAK_TOPS, "TFLOP/s", "mfma"
    traffic = (None if (args.w4a16 or args.codebook or args.static_scale is not None)
               else load_traffic(args.workload))
    value_gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    value_tops = step_ops / (ms_per_step * 1e-3) / 1e12
    if hbm_bound:
        metric_value, metric_unit = value_gbs, "GB/s"
    else:
        metric_value, metric_unit = value_tops, "TOPS"

    result = {
        "metric": "W4A8 GEMM TOPS + HBM GB/s vs roofline at M=1..4096 (Llama-3-8B layer shapes)",
        "value": round(metric_value, 2),
        "unit": metric_unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if args.w4a16 else "int8",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "runs": [f"M={m} {layer} N={n} K={k} g={g}" for (m, layer, n, k, g, _) in runs],
            "step": "every run: w4a8_linear fused (one launch) where it applies, "
                    "else w4a8_quant_act + w4a8_gemm",
            "fused_runs": int(sum(fused)),
            "weights": "codebook (NormalFloat-style levels)" if args.codebook else "uniform groups",
            "activation_scale": ("fp16 activations (W4A16 comparison)" if args.w4a16 else
                                 "static per-tensor %g" % args.static_scale
                                 if args.static_scale is not None else "per-token dynamic"),
            "weight_rotation_copies": ncopies,
            "timing": timing,
            "launch_durations": ("HIP graph of the step's GEMM launches alone, HIP events around its replays"
                                 if gemm_graph_us is not None else
                                 "separate eager pass, HIP events around every GEMM launch"),
            "parallelism": "single GPU",
        },
        "tops": round(value_tops, 3),
        "gbps": round(value_gbs, 2),
        "ms_per_step_eager": round(ms_per_step_eager, 4),
        "roofline": {"bound": bound, "achieved": round(achieved, 2), "peak": peak,
                     "unit": unit, "frac": round(achieved / peak, 4), "traffic": traffic},
    }
    if not args.no_cpu_baseline:
        sample_runs = [r for r in runs]
        log("timing the CPU oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline(sample_runs, weights, metric_unit)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
