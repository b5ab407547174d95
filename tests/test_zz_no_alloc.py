"""dsa_forward_noalloc, the fused call that keeps its workspace in the
library's static per-GPU scratch, against dsa_forward with a caller
workspace: the two run the same kernels in the same launch shapes, so every
output must match bit for bit.  Calls follow each other on one GPU with
shrinking inputs (the scratch keeps the previous call's contents), and one
call goes through a stream other than the current one."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import dev

pytestmark = pytest.mark.gpu

WL = synth.WORKLOADS


def _dsa():
    import long_context_sparse_14_amd as dsa
    dsa.library()
    return dsa


def _run_both(dsa, wl, stream=None):
    print(f"noalloc case: {wl.name} B={wl.B} Tq={wl.Tq} N={wl.N} K={wl.K}", flush=True)
    x = synth.make_inputs(wl)
    d = {k: dev(v) for k, v in x.items()}
    a = (d["q_idx"], d["k_idx"], d["w"], d["q"], d["kv"], wl.K, wl.scale, wl.q_pos0, wl.DV)
    ref_out, ref_lse, ref_idx = dsa.forward(*a, return_idx=True)
    out = torch.full_like(ref_out, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    idx = torch.full_like(ref_idx, -7)
    if stream is None:
        dsa.forward_noalloc(*a, out=out, lse=lse, idx_out=idx)
    else:
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            dsa.forward_noalloc(*a, out=out, lse=lse, idx_out=idx, stream=stream)
        torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    assert torch.equal(idx, ref_idx), f"{wl.name}: indices differ"
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), f"{wl.name}: outputs differ"
    assert torch.equal(lse, ref_lse), f"{wl.name}: lse differs"


def test_noalloc_equals_forward_on_calls_of_shrinking_size():
    dsa = _dsa()
    dec = WL["dsa_decode_b32_128k"]
    _run_both(dsa, dec.replace(N=32768, q_pos0=32767))        # 32 queries: split partials, segmented top-k
    _run_both(dsa, dec.replace(B=3, N=5000, q_pos0=4999))     # smaller, on the scratch the first call left
    _run_both(dsa, WL["dsa_prefill_16k"].replace(Tq=300, N=300, K=64), stream=torch.cuda.Stream())


def test_noalloc_headline_decode_fits():
    """The 32-sequence decode at 131072-token context runs from the scratch."""
    dsa = _dsa()
    _run_both(dsa, WL["dsa_decode_b32_128k"])


def test_noalloc_refuses_a_problem_beyond_its_scratch():
    dsa = _dsa()
    wl = WL["dsa_prefill_16k"].replace(Tq=4096, N=4096)     # 64 MiB of scores alone
    qI = torch.zeros((1, 4096, 64, 128), dtype=torch.bfloat16, device="cuda")
    kI = torch.zeros((1, 4096, 128), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((1, 4096, 64), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((1, 4096, 128, 576), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, 4096, 576), dtype=torch.bfloat16, device="cuda")
    out = torch.full((1, 4096, 128, 512), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dsa.DSAError) as e:
        dsa.forward_noalloc(qI, kI, w, q, kv, wl.K, wl.scale, 0, 512, out=out)
    assert e.value.status == dsa.DSA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()), "a refused call must leave its outputs untouched"
