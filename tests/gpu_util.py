"""Helpers shared by the GPU tests: run the library on numpy inputs."""
import sys

import numpy as np


def log(msg):
    """Name the case before each GPU step (so a fault still says where it was)."""
    print(msg, file=sys.stderr, flush=True)


def device():
    import torch
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def run_quant_act(a_np):
    import torch
    import w4a8_gemm_amd as w4
    dev = device()
    a = torch.from_numpy(a_np).to(dev)
    a8, s_a = w4.quant_act(a)
    torch.cuda.synchronize()
    return a8.cpu().numpy(), s_a.cpu().numpy()


def run_gemm(a8_np, s_a_np, blob_np, n, k, g, **kw):
    import torch
    import w4a8_gemm_amd as w4
    dev = device()
    a8 = torch.from_numpy(np.ascontiguousarray(a8_np)).to(dev)
    s_a = torch.from_numpy(np.ascontiguousarray(s_a_np)).to(dev)
    wdev = w4.to_device(blob_np, dev)
    y, acc = w4.gemm(a8, s_a, wdev, n, k, g, want_acc=True, **kw)
    torch.cuda.synchronize()
    return y.cpu().numpy(), acc.cpu().numpy()
