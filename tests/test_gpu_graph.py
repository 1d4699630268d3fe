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
