"""Layers enqueued on two streams at once give the results they give alone.

Each call of the library keeps its state in the caller's buffers (the
quantized activations, the K-split workspace, the outputs), so calls on
different streams that share only read-only inputs may overlap.  Both
streams are created with torch's default priority."""
import numpy as np
import pytest

import synth
import w4a8_gemm_amd as w4
from gpu_util import log

pytestmark = pytest.mark.gpu

# (m, n, k, g): the fused kernel, the quantizer + skinny GEMM, the tiled GEMM
# with its K split through a workspace, and the 256 x 256 tiled kernel
LAYERS = [(1, 4096, 4096, 128), (16, 6144, 4096, 64), (256, 4096, 14336, 128),
          (1024, 4096, 4096, 128)]


def make_layer(idx, m, n, k, g, dev):
    import torch
    w = synth.weights(n, k, seed=40 + idx)
    wdev = w4.to_device(w4.pack(w, g), dev)
    a = torch.from_numpy(synth.activations(m, k, seed=60 + idx)).to(dev)
    ws_bytes = int(w4.lib.w4a8_gemm_workspace_size(m, n, k, g, None))
    bufs = {
        "a8": torch.empty((m, k), dtype=torch.int8, device=dev),
        "s_a": torch.empty((m,), dtype=torch.float16, device=dev),
        "y": torch.empty((m, n), dtype=torch.float16, device=dev),
        "acc": torch.empty((m, n), dtype=torch.int32, device=dev),
        "workspace": torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev),
    }
    return {"a": a, "w": wdev, "shape": (m, n, k, g), "bufs": bufs}


def run(layer, stream=None):
    m, n, k, g = layer["shape"]
    b = layer["bufs"]
    w4.linear(layer["a"], layer["w"], n, k, g, y=b["y"], a8=b["a8"], s_a=b["s_a"], acc=b["acc"],
              workspace=b["workspace"], stream=stream)


@pytest.mark.parametrize("pair", [(0, 2), (1, 3), (2, 3), (0, 1)])
def test_two_streams_match_one_stream(pair):
    import torch
    dev = torch.device("cuda:0")
    layers = [make_layer(i, *LAYERS[i], dev) for i in pair]
    expected = []
    for lay in layers:
        log(f"streams {pair}: alone {lay['shape']}")
        run(lay)
        torch.cuda.synchronize()
        expected.append({key: t.clone() for key, t in lay["bufs"].items() if key != "workspace"})
    streams = [torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)]
    for rep in range(3):
        for lay in layers:
            for key, t in lay["bufs"].items():
                t.fill_(0x11 if key == "workspace" else 0)
        torch.cuda.synchronize()
        log(f"streams {pair}: overlapped pass {rep}")
        # several calls per stream so the two queues interleave on the device
        for _ in range(4):
            for lay, s in zip(layers, streams):
                run(lay, stream=s)
        torch.cuda.synchronize()
        for lay, exp in zip(layers, expected):
            for key, want in exp.items():
                got = lay["bufs"][key]
                assert torch.equal(got, want), (pair, lay["shape"], key, rep)


def test_two_streams_same_weights_different_rows():
    """Two token batches of one layer on two streams, reading one weight copy."""
    import torch
    dev = torch.device("cuda:0")
    n, k, g = 6144, 4096, 128
    w = synth.weights(n, k, seed=71)
    wdev = w4.to_device(w4.pack(w, g), dev)
    batches = [torch.from_numpy(synth.activations(m, k, seed=72 + m)).to(dev) for m in (48, 512)]
    log("streams shared weights: alone")
    alone = [w4.linear(a, wdev, n, k, g)[0] for a in batches]
    torch.cuda.synchronize()
    alone = [y.clone() for y in alone]
    streams = [torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)]
    outs = [torch.empty_like(y) for y in alone]
    log("streams shared weights: overlapped")
    for _ in range(3):
        for a, y, s in zip(batches, outs, streams):
            with torch.cuda.stream(s):
                w4.linear(a, wdev, n, k, g, y=y, stream=s)
    torch.cuda.synchronize()
    for y, want in zip(outs, alone):
        assert torch.equal(y, want)
