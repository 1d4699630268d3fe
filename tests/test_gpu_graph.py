"""The layer captured in a HIP graph gives the eager result on every replay."""
import numpy as np
import pytest

import synth
import w4a8_gemm_amd as w4
from gpu_util import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("m,n,k,g", [(1, 4096, 4096, 128), (16, 6144, 4096, 64), (96, 512, 1024, 0)])
def test_graph_replays_match_eager(m, n, k, g):
    import torch
    dev = torch.device("cuda:0")
    w = synth.weights(n, k, seed=7)
    wdev = w4.to_device(w4.pack(w, g), dev)
    a = torch.from_numpy(synth.activations(m, k, seed=8)).to(dev)
    a8 = torch.empty((m, k), dtype=torch.int8, device=dev)
    s_a = torch.empty((m,), dtype=torch.float16, device=dev)
    y = torch.empty((m, n), dtype=torch.float16, device=dev)
    acc = torch.empty((m, n), dtype=torch.int32, device=dev)
    log(f"graph m={m} n={n} k={k} g={g}: eager")
    w4.quant_act(a, a8=a8, s_a=s_a)
    w4.gemm(a8, s_a, wdev, n, k, g, y=y, acc=acc)
    torch.cuda.synchronize()
    y_ref, acc_ref = y.clone(), acc.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        w4.quant_act(a, a8=a8, s_a=s_a)
        w4.gemm(a8, s_a, wdev, n, k, g, y=y, acc=acc)
    for rep in range(4):
        y.fill_(0)
        acc.fill_(0)
        a8.fill_(0)
        torch.cuda.synchronize()
        log(f"graph m={m} n={n} k={k} g={g}: replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(acc, acc_ref)
        assert torch.equal(y, y_ref)


@pytest.mark.parametrize("m,n,k,g", [(1, 4096, 4096, 128), (2, 6144, 4096, 32), (4, 4096, 14336, 128),
                                     (16, 6144, 4096, 128), (16, 16384, 4096, 128),
                                     (256, 4096, 14336, 128), (64, 512, 1024, 1), (100, 272, 768, 64)])
def test_graph_whole_layer_replays_match_eager(m, n, k, g):
    """w4a8_linear (fused up to 4 tokens here and at 16 tokens on 16384
    columns, quantizer + GEMM at 16 tokens on 6144 columns, K split
    through a workspace at M = 256, codebook weights) inside a captured graph:
    every replay, with eager work and synchronizations in between, equals
    the eager result."""
    import torch
    dev = torch.device("cuda:0")
    w = synth.weights(n, k, seed=17)
    wdev = w4.to_device(w4.pack(w, g), dev)
    a = torch.from_numpy(synth.activations(m, k, seed=18)).to(dev)
    a8 = torch.empty((m, k), dtype=torch.int8, device=dev)
    s_a = torch.empty((m,), dtype=torch.float16, device=dev)
    y = torch.empty((m, n), dtype=torch.float16, device=dev)
    acc = torch.empty((m, n), dtype=torch.int32, device=dev)
    ws_bytes = int(w4.lib.w4a8_gemm_workspace_size(m, n, k, g, None))
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    log(f"graph linear m={m} n={n} k={k} g={g}: eager (launches "
        f"{w4.lib.w4a8_linear_launches(m, n, k, g, None)})")
    w4.linear(a, wdev, n, k, g, y=y, a8=a8, s_a=s_a, acc=acc, workspace=ws)
    torch.cuda.synchronize()
    y_ref, acc_ref, a8_ref = y.clone(), acc.clone(), a8.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        w4.linear(a, wdev, n, k, g, y=y, a8=a8, s_a=s_a, acc=acc, workspace=ws)
    for rep in range(4):
        y.fill_(0)
        acc.fill_(0)
        a8.fill_(0)
        ws.fill_(0x5A)
        torch.cuda.synchronize()
        log(f"graph linear m={m} n={n} k={k} g={g}: replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(acc, acc_ref)
        assert torch.equal(y, y_ref)
        assert torch.equal(a8, a8_ref)
