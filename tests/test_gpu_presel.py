"""GPU parity for the decode top-k from the indexer's pre-selection.

At long-context decode shapes the bf16 indexer also lists, per segment of a
row, every key at or above a threshold it picks from its own scores; the
top-k then selects among those lists and falls back to the row's full scores
when a truncated list does not reach the row's K-th key.  Every case checks
the indices bit for bit against the C++ oracle's top-k of the oracle's
scores, and against the plain indexer + top-k on the GPU.  The adversarial
cases place far more of a row's best keys in one segment than its list
holds (a block of tied keys; a block of distinct high keys), which the check
must catch so that the row is selected from its full scores.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, assert_lse_close, dev, host64

pytestmark = pytest.mark.gpu

WL = synth.WORKLOADS


@pytest.fixture(autouse=True)
def _free_gpu():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _dsa():
    import long_context_sparse_14_amd as dsa
    dsa.library()
    return dsa


def _case(B, Tq, N, q_pos0, K=2048, seed=0):
    wl = WL["dsa_decode_b32_128k"].replace(B=B, Tq=Tq, N=N, q_pos0=q_pos0, K=K)
    print(f"presel case: B={B} Tq={Tq} N={N} q_pos0={q_pos0} K={K}", flush=True)
    return wl, synth.make_inputs(wl, seed)


def _oracle_idx(x, K, rows, q_pos0, N):
    """The oracle's scores and top-k for the listed (b, t) rows."""
    sc = oracle.index_scores_batch(x["q_idx"], x["k_idx"], x["w"], rows, q_pos0)
    pos0 = np.broadcast_to(np.asarray(q_pos0, dtype=np.int64), (x["q_idx"].shape[0],))
    nv = [oracle.n_valid_keys(t, int(pos0[b]), N) for b, t in rows]
    return oracle.topk_rows(np.nan_to_num(sc, nan=0.0).astype(np.float32), nv, K)


def _check_staged(dsa, wl, x):
    """The staged pre-selection pair equals the plain indexer + top-k and the oracle."""
    d = {k: dev(x[k]) for k in ("q_idx", "k_idx", "w")}
    # entries past a row's visible keys are never written: start both score buffers equal
    fill = lambda: torch.full((wl.B, wl.Tq, wl.N), -3.5, dtype=torch.float32, device="cuda")
    scores, ws = dsa.index_scores_presel(d["q_idx"], d["k_idx"], d["w"], wl.K, wl.q_pos0, scores=fill())
    idx = dsa.topk_presel(scores, wl.K, ws, torch.bfloat16, wl.q_pos0)
    plain_scores = dsa.index_scores(d["q_idx"], d["k_idx"], d["w"], wl.q_pos0, scores=fill())
    plain_idx = dsa.topk(plain_scores, wl.K, wl.q_pos0)
    torch.cuda.synchronize()
    assert torch.equal(scores, plain_scores), "the pre-selecting indexer must write the same scores"
    assert torch.equal(idx, plain_idx), "pre-selected top-k differs from the plain top-k"
    rows = [(b, t) for b in range(wl.B) for t in range(wl.Tq)]
    ref = _oracle_idx(x, wl.K, rows, wl.q_pos0, wl.N)
    got = idx.cpu().numpy().reshape(len(rows), wl.K)
    bad = ~(got == ref).all(1)
    assert not bad.any(), f"rows {np.flatnonzero(bad)[:8]} differ from the oracle"


def test_presel_decode_batch():
    """8 sequences of 65536 keys: 32 segments of 2048 keys per row, lists of 256."""
    dsa = _dsa()
    wl, x = _case(8, 1, 65536, 65535)
    _check_staged(dsa, wl, x)


def test_presel_three_queries_per_sequence():
    dsa = _dsa()
    wl, x = _case(4, 3, 50000, 49997, seed=3)
    _check_staged(dsa, wl, x)


def test_presel_fallback_on_a_block_of_ties():
    """3000 keys equal to a copy of head 0's query (weight 1): they tie at the top of the row, so every
    segment they cover holds far more of the row's best keys than its list: the row must fall back."""
    dsa = _dsa()
    wl, x = _case(2, 1, 40000, 39999, seed=5)
    for b in range(2):
        x["w"][b, 0, 0] = 0x3F80                            # bf16 1.0
        x["k_idx"][b, 1000:4000] = x["q_idx"][b, 0, 0]
    _check_staged(dsa, wl, x)


def test_presel_fallback_on_a_block_of_high_keys():
    """600 distinct high-scoring keys inside one 2048-key segment whose list holds 256."""
    dsa = _dsa()
    wl, x = _case(8, 1, 65536, 65535, seed=6)
    rng = np.random.default_rng(6)
    for b in range(8):
        x["w"][b, 0, 0] = 0x3F80
        blk = np.repeat(x["q_idx"][b, 0, 0][None], 600, axis=0).copy()
        # perturb one channel per key so that the scores differ
        col = rng.integers(0, 128, size=600)
        val = ((x["q_idx"][b, 0, 0][col].astype(np.uint32) << 16).view(np.float32) - 1).astype(np.float32)
        val = np.clip(val, -4, 4)
        blk[np.arange(600), col] = (val.view(np.uint32) >> 16).astype(np.uint16)
        x["k_idx"][b, 4096 + 100:4096 + 700] = blk
    _check_staged(dsa, wl, x)


def test_presel_fused_forward_varlen():
    """Per-sequence lengths (one row at most 16384 keys, one shorter than the segments of the longest):
    the fused varlen forward, whose indexer pre-selects, against the oracle on each sequence."""
    dsa = _dsa()
    lens = [70000, 20000, 16000, 100000]
    wl, x = _case(4, 1, 100000, 0, seed=7)
    d = {k: dev(v) for k, v in x.items()}
    out, lse, idx = dsa.forward_varlen(d["q_idx"], d["k_idx"], d["w"], d["q"], d["kv"], wl.K, wl.scale,
                                       torch.tensor(lens, dtype=torch.int64, device="cuda"), return_idx=True)
    torch.cuda.synchronize()
    ix, o, ls = idx.cpu().numpy(), host64(out), host64(lse)
    for b, n in enumerate(lens):
        ref = oracle.forward_rows(x["q_idx"][b], x["k_idx"][b], x["w"][b], x["q"][b], x["kv"][b], [0], n - 1, wl.K,
                                  wl.scale, wl.DV)[0]
        assert np.array_equal(ix[b, 0], ref["idx"]), f"idx b={b}"
        assert_close(o[b, 0], ref["o"], "bf16", f"out b={b}")
        assert_lse_close(ls[b, 0], ref["lse"], f"lse b={b}")


def test_presel_fused_forward_paged():
    """The paged forward (pre-selecting indexer over block tables) equals the static varlen forward."""
    dsa = _dsa()
    lens, bs = [40000, 30000], 128
    B = len(lens)
    max_blocks = -(-max(lens) // bs) + 1
    N = max_blocks * bs
    wl, x = _case(B, 1, N, 0, seed=8)
    rng = np.random.default_rng(9)
    need = [-(-n // bs) for n in lens]
    nblocks = sum(need) + 3
    perm = rng.permutation(nblocks)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    k = 0
    for b, nb in enumerate(need):
        table[b, :nb] = perm[k:k + nb]
        k += nb
    pools = {}
    for name in ("k_idx", "kv"):
        pool = np.zeros((nblocks * bs, x[name].shape[-1]), dtype=x[name].dtype)
        for b, n in enumerate(lens):
            r = np.arange(n)
            pool[table[b, r // bs] * bs + r % bs] = x[name][b, :n]
        pools[name] = pool
    tl = torch.tensor(lens, dtype=torch.int64, device="cuda")
    d = {k_: dev(v) for k_, v in x.items()}
    out_p, lse_p, idx_p = dsa.forward_paged(d["q_idx"], dev(pools["k_idx"]), d["w"], d["q"], dev(pools["kv"]), wl.K,
                                            wl.scale, tl, torch.from_numpy(table).cuda(), bs, return_idx=True)
    out_s, lse_s, idx_s = dsa.forward_varlen(d["q_idx"], d["k_idx"], d["w"], d["q"], d["kv"], wl.K, wl.scale, tl,
                                             return_idx=True)
    torch.cuda.synchronize()
    assert torch.equal(idx_p, idx_s) and torch.equal(out_p, out_s) and torch.equal(lse_p, lse_s)
    ref = _oracle_idx(x, wl.K, [(b, 0) for b in range(B)], np.array(lens) - 1, N)
    assert np.array_equal(idx_p[:, 0].cpu().numpy(), ref)


def test_presel_entry_points_without_a_preselection():
    """fp32 and prefill shapes: the pair is the plain indexer and top-k."""
    dsa = _dsa()
    wl = WL["tiny_prefill_f32"]
    x = synth.make_inputs(wl)
    d = {k: dev(v) for k, v in x.items()}
    scores, ws = dsa.index_scores_presel(d["q_idx"], d["k_idx"], d["w"], wl.K, 0)
    idx = dsa.topk_presel(scores, wl.K, ws, torch.float32, 0)
    plain = dsa.topk(dsa.index_scores(d["q_idx"], d["k_idx"], d["w"], 0), wl.K, 0)
    torch.cuda.synchronize()
    assert torch.equal(idx, plain)
