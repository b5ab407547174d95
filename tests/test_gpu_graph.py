"""HIP graph capture of the fused forward.

The library only launches kernels on the stream it is given and never
allocates, frees, synchronises or clears memory with a memset, so a decode
step can be captured once and replayed.  Each replay is checked against the
eager call on the same inputs, with eager work and synchronisation between
replays, and after new inputs are copied into the captured buffers.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _free_gpu():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _dsa():
    import long_context_sparse_14_amd as dsa
    dsa.library()
    return dsa


def _inputs(B, N, K, seed):
    wl = synth.WORKLOADS["dsa_decode_b32_128k"].replace(B=B, N=N, q_pos0=N - 1, K=K)
    return wl, {k: dev(v) for k, v in synth.make_inputs(wl, seed).items()}


@pytest.mark.parametrize("N,K", [(20000, 2048), (3000, 256)])   # long-row and one-workgroup top-k
def test_forward_graph_replays(N, K):
    dsa = _dsa()
    B = 3
    wl, d = _inputs(B, N, K, seed=1)
    _, d2 = _inputs(B, N, K, seed=2)
    ws = torch.empty(dsa.forward_workspace_size(B, 1, N, 128, 512, K, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty(B, 1, 128, 512, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, 1, 128, dtype=torch.float32, device="cuda")
    idx = torch.empty(B, 1, K, dtype=torch.int32, device="cuda")

    def call():
        dsa.forward(d["q_idx"], d["k_idx"], d["w"], d["q"], d["kv"], K, wl.scale, wl.q_pos0, out=out, lse=lse,
                    idx_out=idx, workspace=ws)

    def eager_result():
        call()
        torch.cuda.synchronize()
        return out.clone(), lse.clone(), idx.clone()

    ref1 = eager_result()
    saved = {k: v.clone() for k, v in d.items()}
    # new inputs -> the eager reference for the second set
    for k in d:
        d[k].copy_(d2[k])
    ref2 = eager_result()
    for k in d:
        d[k].copy_(saved[k])

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()

    for rep in range(3):
        ref = ref1 if rep != 1 else ref2
        src = saved if rep != 1 else d2
        for k in d:
            d[k].copy_(src[k])
        out.fill_(0)
        lse.fill_(0)
        idx.fill_(-7)
        x = torch.randn(512, 512, device="cuda")  # eager work between replays
        _ = x @ x
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[2]), f"replay {rep}: indices"
        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]), f"replay {rep}: attention"
