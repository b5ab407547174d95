"""The C++ CPU oracle pinned to facts outside itself (runs without a GPU).

Each pin in tests/pins.py must hold for the oracle.  That the pins have teeth
is shown in test_oracle_mutants.py: mistakes planted in the oracle's source
are each rejected by at least one of them.
"""
import numpy as np
import pytest

import oracle
import pins


def test_indexer_golden():
    assert pins.pin_indexer_golden(oracle.index_scores_rows)


def test_indexer_hadamard_invariance():
    assert pins.pin_indexer_hadamard(oracle.index_scores_rows, oracle.sylvester_hadamard)


def test_indexer_unit_queries():
    assert pins.pin_indexer_unit_queries(oracle.index_scores_rows)


def test_indexer_causal():
    assert pins.pin_indexer_causal(oracle.index_scores_rows)


def test_indexer_heads():
    assert pins.pin_indexer_heads(oracle.index_scores_rows)


def test_topk_golden():
    assert pins.pin_topk_golden(oracle.topk_row)


def test_topk_bruteforce():
    assert pins.pin_topk_bruteforce(oracle.topk_row)


def test_topk_short_rows():
    assert pins.pin_topk_short_rows(oracle.topk_row)


def test_mla_golden():
    assert pins.pin_mla_golden(oracle.sparse_mla_rows)


def test_mla_single_key():
    assert pins.pin_mla_single_key(oracle.sparse_mla_rows)


def test_mla_uniform():
    assert pins.pin_mla_uniform(oracle.sparse_mla_rows)


def test_mla_permutation_and_mask():
    assert pins.pin_mla_permutation_and_mask(oracle.sparse_mla_rows)


def test_mla_sdpa_special_case():
    assert pins.pin_mla_sdpa(oracle.sparse_mla, oracle.dense_masked_mla)


def test_mla_sparse_equals_dense():
    assert pins.pin_mla_sparse_equals_dense(oracle.sparse_mla, oracle.dense_masked_mla)


def test_forward_rows_composes_the_steps():
    """forward_rows is indexer -> top-k -> sparse MLA; with K >= L it is causal attention."""
    r = np.random.default_rng(5)
    T, HI, DI, H, D, DV = 12, 2, 4, 2, 6, 4
    qI = r.integers(-3, 4, size=(T, HI, DI)).astype(np.float32)
    kI = r.integers(-3, 4, size=(T, DI)).astype(np.float32)
    w = np.ones((T, HI), dtype=np.float32)
    q = r.standard_normal((T, H, D))
    kv = r.standard_normal((T, D))
    res = oracle.forward_rows(qI, kI, w, q, kv, range(T), 0, 3, 0.5, DV)
    for x in res:
        exp_idx = oracle.topk_row(x["scores"].astype(np.float32), 3)
        assert np.array_equal(x["idx"], exp_idx)
        o, lse = oracle.sparse_mla_rows(q[x["t"]], kv, exp_idx, 0.5, DV)
        assert np.array_equal(o, x["o"]) and np.array_equal(lse, x["lse"])
    full = oracle.forward_rows(qI, kI, w, q, kv, range(T), 0, T, 0.5, DV)
    od, _ = oracle.dense_masked_mla(q[None], kv[None], np.stack([x["idx"] for x in full])[None], 0.5, DV, 0)
    for x in full:
        assert np.allclose(x["o"], od[0, x["t"]], atol=1e-13)


def test_compressed_visibility():
    assert pins.pin_compressed_visibility(oracle.n_valid_keys)


def test_compressed_pipeline():
    assert pins.pin_compressed_pipeline(oracle.index_scores, oracle.topk)


def test_mla_naive_sdpa():
    assert pins.pin_mla_naive_sdpa(oracle.mla_naive_rows)


def test_mla_absorbed_equals_naive():
    assert pins.pin_mla_absorbed_equals_naive(oracle.mla_absorb_query, oracle.sparse_mla_rows,
                                              oracle.mla_output_projection, oracle.mla_naive_rows)


def test_linear():
    assert pins.pin_linear(oracle.linear)


def test_e4m3():
    assert pins.pin_e4m3(oracle.e4m3_decode, oracle.e4m3_encode_rne)


def test_fwht():
    assert pins.pin_fwht(oracle.fwht_f32, oracle.sylvester_hadamard)


def test_pow2_scale():
    assert pins.pin_pow2_scale(oracle.pow2_scale_exp)


def test_quantize_fp8():
    assert pins.pin_quantize_fp8(oracle.quantize_fp8_rows, oracle.fwht_f32, oracle.e4m3_decode)


def test_fp8_scores_near_bf16():
    assert pins.pin_fp8_scores_near_bf16(oracle.quantize_fp8_rows, oracle.index_scores_fp8_rows,
                                         oracle.index_scores_rows, oracle.fwht_f32, oracle.e4m3_decode)


def test_paged_gather():
    assert pins.pin_paged_gather(oracle.paged_gather)


def test_forward_pin():
    assert pins.pin_forward(oracle.forward_rows)


def test_topk_long_ties():
    assert pins.pin_topk_long_ties(oracle.topk_row)


def test_thread_count_changes_no_bit(monkeypatch):
    """Rows are dealt to threads whole, so one thread and many give the same bits."""
    r = np.random.default_rng(8)
    T, HI, DI, H, D, DV = 40, 3, 8, 4, 12, 8
    qI = r.integers(-3, 4, size=(1, T, HI, DI)).astype(np.float32)
    kI = r.integers(-3, 4, size=(1, T, DI)).astype(np.float32)
    w = r.choice([0.5, 1.0, 2.0], size=(1, T, HI)).astype(np.float32)
    q = r.standard_normal((1, T, H, D))
    kv = r.standard_normal((1, T, D))
    rows = [(0, t) for t in range(T)]
    outs = []
    for n in ("1", "7"):
        monkeypatch.setenv("DSA_ORACLE_THREADS", n)
        outs.append(oracle.forward_batch(qI, kI, w, q, kv, rows, 0, 5, 0.3, DV))
    for k in ("scores", "idx", "o", "lse"):
        assert np.array_equal(outs[0][k], outs[1][k], equal_nan=True), k


def test_rejects_bad_arguments():
    """Invalid shapes and rows are refused before anything is computed."""
    q = np.zeros((1, 2, 1, 4), np.float32)
    k = np.zeros((1, 3, 4), np.float32)
    w = np.ones((1, 2, 1), np.float32)
    with pytest.raises(ValueError):
        oracle.index_scores_batch(q, k, w, [(0, 2)], 0)          # query 2 of a 2-query sequence
    with pytest.raises(ValueError):
        oracle.index_scores_batch(q, k, w, [(1, 0)], 0)          # sequence 1 of a 1-sequence batch
    with pytest.raises(ValueError):
        oracle.e4m3_encode_rne(np.array([449.0], np.float32))
    with pytest.raises(ValueError):
        oracle.topk_rows(np.zeros((1, 4), np.float32), [5], 2)   # more visible keys than the row holds
