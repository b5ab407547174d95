"""The CPU oracle pinned to facts outside itself (runs without a GPU).

Each pin in tests/pins.py must hold for the oracle, and for each planted
mistake (a broken copy of an oracle function, made here on the CPU) at least
one pin must fail.
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


# ----------------------------------------------------------- planted mistakes

def _mut_no_relu(q_b, k_b, w_b, ts, p0):
    kI = oracle.as_f64(k_b)
    return [(kI[:oracle.n_valid_keys(t, p0, kI.shape[0])] @ oracle.as_f64(q_b[t]).T) @ oracle.as_f64(w_b[t])
            for t in ts]


def _mut_exclusive_diag(q_b, k_b, w_b, ts, p0):
    return [r[:-1] for r in oracle.index_scores_rows(q_b, k_b, w_b, ts, p0)]


def _mut_weight_order(q_b, k_b, w_b, ts, p0):
    return oracle.index_scores_rows(q_b, k_b, np.asarray(w_b)[:, ::-1], ts, p0)


def _mut_relu_after_sum(q_b, k_b, w_b, ts, p0):
    kI = oracle.as_f64(k_b)
    return [np.maximum((kI[:oracle.n_valid_keys(t, p0, kI.shape[0])] @ oracle.as_f64(q_b[t]).T)
                       @ oracle.as_f64(w_b[t]), 0) for t in ts]


def _mut_key_dim_reversed(q_b, k_b, w_b, ts, p0):
    return oracle.index_scores_rows(q_b, np.asarray(k_b)[:, ::-1], w_b, ts, p0)


@pytest.mark.parametrize("mutant", [_mut_no_relu, _mut_exclusive_diag, _mut_weight_order,
                                    _mut_relu_after_sum, _mut_key_dim_reversed])
def test_indexer_pins_catch_planted_mistakes(mutant):
    checks = [pins.pin_indexer_golden(mutant), pins.pin_indexer_hadamard(mutant, oracle.sylvester_hadamard),
              pins.pin_indexer_unit_queries(mutant), pins.pin_indexer_causal(mutant),
              pins.pin_indexer_heads(mutant)]
    assert not all(checks)


def _mut_ties_high(v, K):
    v = np.asarray(v, dtype=np.float32)
    n = len(v)
    out = np.full(K, -1, dtype=np.int32)
    if n <= K:
        out[:n] = np.arange(n)
        return out
    order = np.lexsort((-np.arange(n), -v.astype(np.float64)))
    out[:] = np.sort(order[:K])
    return out


def _mut_rank_order(v, K):
    v = np.asarray(v, dtype=np.float32)
    n = len(v)
    out = np.full(K, -1, dtype=np.int32)
    if n <= K:
        out[:n] = np.arange(n)
        return out
    out[:] = np.lexsort((np.arange(n), -v.astype(np.float64)))[:K]
    return out


def _mut_smallest(v, K):
    return oracle.topk_row(-np.asarray(v, dtype=np.float32), K)


def _mut_pad_zero(v, K):
    out = oracle.topk_row(v, K)
    out[out < 0] = 0
    return out


@pytest.mark.parametrize("mutant", [_mut_ties_high, _mut_rank_order, _mut_smallest, _mut_pad_zero])
def test_topk_pins_catch_planted_mistakes(mutant):
    checks = [pins.pin_topk_golden(mutant), pins.pin_topk_bruteforce(mutant), pins.pin_topk_short_rows(mutant)]
    assert not all(checks)


def _mut_value_from_rope(q, kv, idx, scale, DV):
    """value read from the last DV entries of the row instead of the first DV"""
    kv = np.asarray(kv, dtype=np.float64)
    swapped = np.concatenate([kv[:, -DV:], kv[:, :-DV]], axis=1)
    o, _ = oracle.sparse_mla_rows(q, swapped, idx, scale, DV)
    _, lse = oracle.sparse_mla_rows(q, kv, idx, scale, DV)
    return o, lse


def _mut_no_scale(q, kv, idx, scale, DV):
    return oracle.sparse_mla_rows(q, kv, idx, 1.0, DV)


def _mut_mask_ignored(q, kv, idx, scale, DV):
    idx = np.where(np.asarray(idx) < 0, 0, idx)
    return oracle.sparse_mla_rows(q, kv, idx, scale, DV)


def _mut_lse_log2(q, kv, idx, scale, DV):
    o, lse = oracle.sparse_mla_rows(q, kv, idx, scale, DV)
    return o, lse / np.log(2.0)


def _mut_no_max_shift_wrong_norm(q, kv, idx, scale, DV):
    o, lse = oracle.sparse_mla_rows(q, kv, idx, scale, DV)
    sel = [int(i) for i in np.asarray(idx) if int(i) >= 0]
    return o * len(sel) / max(1, len(sel) + 1), lse


@pytest.mark.parametrize("mutant", [_mut_value_from_rope, _mut_no_scale, _mut_mask_ignored, _mut_lse_log2,
                                    _mut_no_max_shift_wrong_norm])
def test_mla_pins_catch_planted_mistakes(mutant):
    checks = [pins.pin_mla_golden(mutant), pins.pin_mla_single_key(mutant), pins.pin_mla_uniform(mutant),
              pins.pin_mla_permutation_and_mask(mutant)]
    assert not all(checks)


def test_compressed_visibility():
    assert pins.pin_compressed_visibility(oracle.n_valid_keys)


def test_compressed_pipeline():
    assert pins.pin_compressed_pipeline(oracle.index_scores, oracle.topk)


def _mut_vis_open_window(t, q_pos0, N, m=1):
    """an entry counted as soon as its window opens"""
    p = q_pos0 + t
    return 0 if p < 0 else min(N, p // m + 1)


def _mut_vis_off_by_one(t, q_pos0, N, m=1):
    """own position left out of the closing test"""
    p = q_pos0 + t
    return 0 if p <= 0 else min(N, p // m)


def _mut_vis_rate_ignored(t, q_pos0, N, m=1):
    return oracle.n_valid_keys(t, q_pos0, N, 1)


def _mut_vis_no_cap(t, q_pos0, N, m=1):
    p1 = q_pos0 + t + 1
    return 0 if p1 <= 0 else p1 // m


@pytest.mark.parametrize("mutant", [_mut_vis_open_window, _mut_vis_off_by_one, _mut_vis_rate_ignored,
                                    _mut_vis_no_cap])
def test_compressed_pins_catch_planted_mistakes(mutant):
    assert not pins.pin_compressed_visibility(mutant)


def test_mla_naive_sdpa():
    assert pins.pin_mla_naive_sdpa(oracle.mla_naive_rows)


def test_mla_absorbed_equals_naive():
    assert pins.pin_mla_absorbed_equals_naive(oracle.mla_absorb_query, oracle.sparse_mla_rows,
                                              oracle.mla_output_projection, oracle.mla_naive_rows)


def _mut_absorb_no_rope(q, W_UK):
    out = oracle.mla_absorb_query(q, W_UK)
    out[..., W_UK.shape[2]:] = 0.0
    return out


def _mut_absorb_transposed(q, W_UK):
    """W_UK used as if stored [d_c, d_nope] (only runs where the shapes allow)"""
    d_nope = W_UK.shape[1]
    q = np.asarray(q, dtype=np.float64)
    return np.concatenate([np.einsum("hn,hcn->hc", q[:, :d_nope], W_UK.transpose(0, 2, 1).reshape(
        W_UK.shape[0], W_UK.shape[2], d_nope)[:, :, ::-1]), q[:, d_nope:]], axis=-1)


def _mut_out_proj_transposed(o_lat, W_UV):
    return np.einsum("hc,hvc->hv", np.asarray(o_lat)[:, ::-1], W_UV)


def _mut_naive_value_from_key(q, c, kr, idx, W_UK, W_UV, scale):
    """values read through the key projection padded to d_v columns"""
    H, d_nope, d_c = W_UK.shape
    W = np.zeros_like(W_UV)
    n = min(d_nope, W_UV.shape[1])
    W[:, :n] = W_UK[:, :n]
    return oracle.mla_naive_rows(q, c, kr, idx, W_UK, W, scale)


def _mut_naive_no_rope(q, c, kr, idx, W_UK, W_UV, scale):
    return oracle.mla_naive_rows(q, c, np.zeros_like(kr), idx, W_UK, W_UV, scale)


@pytest.mark.parametrize("mutant", [_mut_absorb_no_rope, _mut_absorb_transposed])
def test_absorb_pin_catches_planted_mistakes(mutant):
    assert not pins.pin_mla_absorbed_equals_naive(mutant, oracle.sparse_mla_rows, oracle.mla_output_projection,
                                                  oracle.mla_naive_rows)


def test_out_proj_pin_catches_planted_mistake():
    assert not pins.pin_mla_absorbed_equals_naive(oracle.mla_absorb_query, oracle.sparse_mla_rows,
                                                  _mut_out_proj_transposed, oracle.mla_naive_rows)


@pytest.mark.parametrize("mutant", [_mut_naive_value_from_key, _mut_naive_no_rope])
def test_naive_pin_catches_planted_mistakes(mutant):
    assert not pins.pin_mla_naive_sdpa(mutant)


def test_absorbed_pin_catches_value_from_rope():
    """the value read from the wrong end of the latent row breaks absorbed == naive"""
    def mla_rows_mut(q, kv, idx, scale, DV):
        kv = np.asarray(kv, dtype=np.float64)
        return oracle.sparse_mla_rows(q, kv[:, ::-1], idx, scale, DV)
    assert not pins.pin_mla_absorbed_equals_naive(oracle.mla_absorb_query, mla_rows_mut,
                                                  oracle.mla_output_projection, oracle.mla_naive_rows)


def test_linear():
    assert pins.pin_linear(oracle.linear)


@pytest.mark.parametrize("mutant", [lambda x, W: np.asarray(x) @ np.asarray(W),
                                    lambda x, W: np.asarray(x)[:, ::-1] @ np.asarray(W).T])
def test_linear_pin_catches_planted_mistakes(mutant):
    assert not pins.pin_linear(mutant)


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


def _mut_e4m3_fnuz(codes):
    """bias 8 instead of 7"""
    return oracle.e4m3_decode(codes) / 2.0


def _mut_e4m3_truncate(v):
    v = np.asarray(v, dtype=np.float32)
    d = oracle.e4m3_decode(oracle.e4m3_encode_rne(v))
    over = np.abs(d) > np.abs(v.astype(np.float64))
    out = oracle.e4m3_encode_rne(v).astype(np.int64)
    return np.where(over, out - 1, out).astype(np.uint8)


def test_e4m3_pin_catches_planted_mistakes():
    assert not pins.pin_e4m3(_mut_e4m3_fnuz, oracle.e4m3_encode_rne)
    assert not pins.pin_e4m3(oracle.e4m3_decode, _mut_e4m3_truncate)


def test_fwht_pin_catches_planted_mistake():
    assert not pins.pin_fwht(lambda x: oracle.fwht_f32(x)[..., ::-1], oracle.sylvester_hadamard)


def test_pow2_pin_catches_planted_mistake():
    assert not pins.pin_pow2_scale(lambda a: oracle.pow2_scale_exp(a) + 1)


def test_fp8_score_pin_catches_planted_mistakes():
    def no_div(q8, qs, k8, ks, w, ts, p0):
        return [r * 128.0 for r in oracle.index_scores_fp8_rows(q8, qs, k8, ks, w, ts, p0)]

    def no_key_scale(q8, qs, k8, ks, w, ts, p0):
        return oracle.index_scores_fp8_rows(q8, qs, k8, np.ones_like(ks), w, ts, p0)

    for mut in (no_div, no_key_scale):
        assert not pins.pin_fp8_scores_near_bf16(oracle.quantize_fp8_rows, mut, oracle.index_scores_rows,
                                                 oracle.fwht_f32, oracle.e4m3_decode)


def test_paged_gather():
    assert pins.pin_paged_gather(oracle.paged_gather)


def test_paged_gather_pin_catches_planted_mistake():
    def swapped(pool, table_row, bs, n):
        t = np.asarray(table_row)
        r = np.arange(n)
        return np.asarray(pool)[t[r % len(t)] * bs + r // len(t)]
    assert not pins.pin_paged_gather(swapped)
