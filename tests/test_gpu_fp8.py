"""GPU parity for the FP8 indexer.

* Quantisation (Hadamard rotation, power-of-two row scale, E4M3 rounding):
  codes and scales bit-exact against the oracle, which takes every rounding
  decision on the same float32 values.
* Scores: against the oracle's float64 scores from the same codes, within the
  float32 rounding bound of the kernel's sums,
      |d| <= 200 * 2^-24 * sum_h |w_h| qs_h ks / 128 * sum_d |q8_d k8_d|
  (128 products and 64 heads summed in float32, two scalings; the products
  of E4M3 values are exact in the bf16 matrix cores).
* The fused forward: several selections are correct when scores tie within
  that bound, so each row is checked for what is unique -- every key whose
  oracle score beats the K-th largest by more than the bound is selected, no
  selected key falls below it by more than the bound, the row holds
  min(n, K) distinct visible keys in ascending order -- and the attention
  output is checked against the oracle on the indices the row selected.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, assert_lse_close, dev, host64

pytestmark = pytest.mark.gpu

FP8_WID = 41  # generator stream family of these tests
SCORE_ULPS = 200.0 * 2.0 ** -24


@pytest.fixture(autouse=True)
def _free_gpu():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _dsa():
    import long_context_sparse_14_amd as dsa
    dsa.library()
    return dsa


def gen(shape, tensor_id, dist, seed=0):
    n = int(np.prod(shape))
    return synth.fill(synth.stream_key(seed, FP8_WID, tensor_id), 0, n, dist, "bf16").reshape(shape)


def u8(t):
    return t.cpu().numpy().astype(np.uint8)


@pytest.mark.parametrize("rows,dist", [
    (1000, synth.INT4),       # the indexer inputs of the decode workloads
    (777, synth.NORMAL),
    (5, synth.Dist("int", 0, 0)),  # all-zero rows: scale 1, codes 0
])
def test_quantize_fp8_exact(rows, dist):
    dsa = _dsa()
    x = gen((rows, 128), 1, dist)
    codes, scales = dsa.indexer_quantize_fp8(dev(x))
    ref_codes, ref_scales = oracle.quantize_fp8_rows(x)
    assert np.array_equal(u8(codes), ref_codes), "codes differ"
    assert np.array_equal(scales.cpu().numpy(), ref_scales), "scales differ"


def _fp8_inputs(B, Tq, N, seed=0):
    q = gen((B, Tq, 64, 128), 2, synth.INT4, seed)
    k = gen((B, N, 128), 3, synth.INT4, seed)
    w = gen((B, Tq, 64), 4, synth.POW2_M4_0, seed)
    q8, qs = oracle.quantize_fp8_rows(q)
    k8, ks = oracle.quantize_fp8_rows(k)
    return q8, qs, k8, ks, w


def _score_bound(q8, qs, k8, ks, w, t, n):
    """float32 rounding bound of the kernel's score for keys 0..n-1 of query t."""
    qv = np.abs(oracle.e4m3_decode(q8[t]))                  # [64, 128]
    kv = np.abs(oracle.e4m3_decode(k8[:n]))                 # [n, 128]
    mag = (kv @ qv.T) * ks[:n, None].astype(np.float64) * qs[t][None, :].astype(np.float64) / 128.0
    return SCORE_ULPS * (mag @ np.abs(oracle.as_f64(w[t]))) + 1e-30


def _tdev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("B,Tq,N,q_pos0", [
    (2, 1, 5000, 4999),     # decode: every key visible, a ragged last tile
    (3, 4, 3000, 1000),     # causal rows of 1001..1004 keys, cache longer than the rows
    (1, 2, 40, 0),          # rows of one and two keys
    (1, 1, 131072, 131071), # one query over 128K keys: one round of 256-key workgroups
])
def test_index_scores_fp8(B, Tq, N, q_pos0):
    dsa = _dsa()
    q8, qs, k8, ks, w = _fp8_inputs(B, Tq, N)
    got = dsa.index_scores_fp8(_tdev(q8), _tdev(qs), _tdev(k8), _tdev(ks), dev(w), q_pos0).cpu().numpy()
    for b in range(B):
        ts = list(range(Tq))
        ref = oracle.index_scores_fp8_rows(q8[b], qs[b], k8[b], ks[b], w[b], ts, q_pos0)
        for t in ts:
            n = len(ref[t])
            tol = _score_bound(q8[b], qs[b], k8[b], ks[b], w[b], t, n)
            err = np.abs(got[b, t, :n].astype(np.float64) - ref[t])
            assert np.all(err <= tol), f"b={b} t={t}: worst excess {np.max(err - tol):.3e}"


def _check_selection(idx_row, ref_scores, tol, K):
    n = len(ref_scores)
    sel = idx_row[idx_row >= 0]
    assert len(sel) == min(n, K), f"{len(sel)} selected of {n} visible (K={K})"
    assert np.all(idx_row[len(sel):] == -1), "padding must follow the selection"
    assert np.all(np.diff(sel) > 0) and (len(sel) == 0 or sel[-1] < n), "selection must be ascending and visible"
    if n <= K:
        return
    order = np.lexsort((np.arange(n), -ref_scores))
    th = ref_scores[order[K - 1]]
    must = np.flatnonzero(ref_scores > th + tol)
    assert np.all(np.isin(must, sel)), "a clearly better key was not selected"
    assert np.all(ref_scores[sel] >= th - tol[sel]), "a clearly worse key was selected"


@pytest.mark.parametrize("B,N,K", [
    (2, 20000, 2048),   # segmented long-row top-k
    (3, 3000, 256),     # one-workgroup top-k
])
def test_forward_fp8_decode(B, N, K):
    dsa = _dsa()
    Tq, q_pos0 = 1, N - 1
    q8, qs, k8, ks, w = _fp8_inputs(B, Tq, N, seed=1)
    wl = synth.WORKLOADS["dsa_decode_b32_128k"].replace(B=B, N=N, q_pos0=q_pos0, K=K)
    x = synth.make_inputs(wl, 1)
    out, lse, idx = dsa.forward_fp8(_tdev(q8), _tdev(qs), _tdev(k8), _tdev(ks), dev(w), dev(x["q"]), dev(x["kv"]),
                                    K, wl.scale, q_pos0, return_idx=True)
    torch.cuda.synchronize()
    idx, out, lse = idx.cpu().numpy(), host64(out), host64(lse)
    for b in range(B):
        ref = oracle.index_scores_fp8_rows(q8[b], qs[b], k8[b], ks[b], w[b], [0], q_pos0)[0]
        tol = _score_bound(q8[b], qs[b], k8[b], ks[b], w[b], 0, len(ref))
        _check_selection(idx[b, 0], ref, tol, K)
        o, l = oracle.sparse_mla_rows(x["q"][b, 0], oracle.as_f64(x["kv"][b]), idx[b, 0], wl.scale, wl.DV)
        assert_close(out[b, 0], o, "bf16", f"attention b={b}")
        assert_lse_close(lse[b, 0], l, f"lse b={b}")


def test_index_scores_fp8_full_decode_sampled():
    """The 128K decode batch at full size (32 x 131072 keys): rows 0 and 31 against the oracle."""
    dsa = _dsa()
    B, N = 32, 131072
    q = gen((B, 1, 64, 128), 5, synth.INT4)
    w = gen((B, 1, 64), 6, synth.POW2_M4_0)
    k = torch.from_numpy(gen((B, N, 128), 7, synth.INT4).view(np.int16)).view(torch.bfloat16).cuda()
    k8, ks = dsa.indexer_quantize_fp8(k)
    q8, qs = dsa.indexer_quantize_fp8(dev(q))
    got = dsa.index_scores_fp8(q8, qs, k8, ks, dev(w), N - 1)
    torch.cuda.synchronize()
    for b in (0, B - 1):
        k8b, ksb = u8(k8[b]), ks[b].cpu().numpy()
        kb = k[b].view(torch.int16).cpu().numpy().view(np.uint16)
        rc, rs = oracle.quantize_fp8_rows(kb)
        assert np.array_equal(k8b, rc) and np.array_equal(ksb, rs), f"key cache quantisation b={b}"
        q8b, qsb = u8(q8[b]), qs[b].cpu().numpy()
        ref = oracle.index_scores_fp8_rows(q8b, qsb, k8b, ksb, w[b], [0], N - 1)[0]
        tol = _score_bound(q8b, qsb, k8b, ksb, w[b], 0, N)
        err = np.abs(got[b, 0].cpu().numpy().astype(np.float64) - ref)
        assert np.all(err <= tol), f"b={b}: worst excess {np.max(err - tol):.3e}"


@pytest.mark.parametrize("B,Tq,N,plant", [
    (8, 4, 40000, None),      # 32 rows of ~40000 keys: 16 segments of 2560 keys (the last one ragged), lists of 512
    (8, 4, 40000, "ties"),    # 3000 tied top keys: their segments cannot list them, the rows fall back
    (32, 1, 131072, None),    # the 128K decode batch: 16 segments of 8192 keys, lists of 512
])
def test_forward_fp8_presel(B, Tq, N, plant):
    """At these decode shapes the FP8 indexer also lists each segment's best keys and the top-k selects
    among the lists.  The fused forward must equal the staged plain FP8 indexer + top-k + sparse MLA on
    the GPU bit for bit, and sampled rows must select what the oracle's scores fix."""
    dsa = _dsa()
    K, q_pos0 = 2048, N - Tq
    print(f"fp8 presel case: B={B} Tq={Tq} N={N} plant={plant}", flush=True)
    q = gen((B, Tq, 64, 128), 12, synth.INT4, seed=2)
    w = gen((B, Tq, 64), 13, synth.POW2_M4_0, seed=2)
    k = gen((B, N, 128), 14, synth.INT4, seed=2)
    if plant == "ties":
        w[:, :, 0] = 0x3F80                                   # bf16 1.0 on head 0
        k[:, 1000:4000] = q[:, 0, 0][:, None, :]              # keys equal to query 0's head 0: a tied top block
    q8, qs = dsa.indexer_quantize_fp8(dev(q))
    k8, ks = dsa.indexer_quantize_fp8(torch.from_numpy(k.view(np.int16)).view(torch.bfloat16).cuda())
    wd = dev(w)
    g = torch.Generator(device="cuda")
    g.manual_seed(B * N + Tq)
    qm = (torch.randn((B, Tq, 128, 576), device="cuda", generator=g) * 0.5).to(torch.bfloat16)
    kv = (torch.randn((B, N, 576), device="cuda", generator=g) * 0.5).to(torch.bfloat16)
    scale = 192 ** -0.5
    out, lse, idx = dsa.forward_fp8(q8, qs, k8, ks, wd, qm, kv, K, scale, q_pos0, return_idx=True)
    # entries past a row's visible keys are never written: start both score buffers equal
    fill = lambda: torch.full((B, Tq, N), -3.5, dtype=torch.float32, device="cuda")
    scores = dsa.index_scores_fp8(q8, qs, k8, ks, wd, q_pos0, scores=fill())
    plain_idx = dsa.topk(scores, K, q_pos0)
    plain_out, plain_lse = dsa.sparse_mla(qm, kv, plain_idx, scale)
    pre_scores, ws = dsa.index_scores_fp8_presel(q8, qs, k8, ks, wd, K, q_pos0, scores=fill())
    pre_idx = dsa.topk_presel_fp8(pre_scores, K, ws, q_pos0)
    torch.cuda.synchronize()
    assert torch.equal(pre_scores, scores), "the pre-selecting FP8 indexer must write the same scores"
    assert torch.equal(pre_idx, plain_idx), "the staged pre-selection pair differs from the plain top-k"
    assert torch.equal(idx, plain_idx), "pre-selected FP8 top-k differs from the plain top-k"
    assert torch.equal(out, plain_out) and torch.equal(lse, plain_lse), "attention differs from the staged path"
    for b in sorted({0, B - 1}):
        k8b, ksb, q8b, qsb = u8(k8[b]), ks[b].cpu().numpy(), u8(q8[b]), qs[b].cpu().numpy()
        ts = list(range(Tq))
        ref = oracle.index_scores_fp8_rows(q8b, qsb, k8b, ksb, w[b], ts, q_pos0)
        for t in ts:
            tol = _score_bound(q8b, qsb, k8b, ksb, w[b], t, len(ref[t]))
            _check_selection(idx[b, t].cpu().numpy(), ref[t], tol, K)
