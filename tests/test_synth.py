"""The seeded input generator: deterministic, sliceable, and within the recipe."""
import numpy as np

import oracle
import synth


def test_slices_match_whole_tensor():
    wl = synth.WORKLOADS["tiny_prefill_f32"]
    kv = synth.tensor(wl, "kv")
    assert kv.shape == (1, 256, 80)
    part = synth.rows(wl, "kv", 0, [3, 200, 7])
    assert np.array_equal(part, kv[0, [3, 200, 7]])
    blk = synth.row_block(wl, "kv", 0, 10, 20)
    assert np.array_equal(blk, kv[0, 10:20])


def test_deterministic_and_seeded():
    wl = synth.WORKLOADS["tiny_prefill_f32"]
    a = synth.tensor(wl, "q")
    b = synth.tensor(wl, "q")
    c = synth.tensor(wl, "q", seed=1)
    assert np.array_equal(a, b) and not np.array_equal(a, c)


def test_distributions_follow_the_recipe():
    wl = synth.WORKLOADS["indexer_topk_prefill_8k"].replace(Tq=64, N=64)
    qi = oracle.as_f64(synth.tensor(wl, "q_idx"))
    assert set(np.unique(qi)) == set(range(-4, 5))
    w = oracle.as_f64(synth.tensor(wl, "w"))
    assert set(np.unique(w)) <= {2.0 ** e for e in range(-4, 1)}
    wl1 = synth.WORKLOADS["tiny_prefill_f32"]
    assert set(np.unique(synth.tensor(wl1, "w"))) == {0.25, 0.5, 1.0, 2.0}
    assert set(np.unique(synth.tensor(wl1, "k_idx"))) == set(range(-3, 4))
    x = synth.fill(99, 0, 200000, synth.NORMAL, "f32")
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01


def test_floyd_rows_are_distinct_and_in_range():
    idx = synth.floyd(1234, 50, 300, 100)
    for row in idx:
        assert len(set(row.tolist())) == 100 and row.min() >= 0 and row.max() < 300


def test_bf16_rounding_is_nearest_even():
    # normals drawn in fp32 then rounded: the bf16 value is the nearest bf16 of the fp32 value
    f = synth.fill(7, 0, 4096, synth.NORMAL, "f32")
    h = synth.fill(7, 0, 4096, synth.NORMAL, "bf16")
    hv = oracle.as_f64(h)
    ulp = np.exp2(np.floor(np.log2(np.abs(f.astype(np.float64)))) - 7)
    assert np.all(np.abs(hv - f) <= ulp / 2)


def test_config_value_bounds_keep_scores_exact_in_fp32():
    """The integer-valued indexer inputs make every partial sum an exact fp32 value:
    |q.k| <= D_I*max|q|*max|k| and |score| <= H_I*max|w|*that, all on a 2^-4 grid
    below 2^24 steps."""
    for name in ["tiny_prefill_f32", "indexer_topk_prefill_8k", "dsa_prefill_16k", "dsa_decode_b32_128k"]:
        wl = synth.WORKLOADS[name]
        qmax = max(abs(wl.dists["q_idx"].lo), abs(wl.dists["q_idx"].hi))
        kmax = max(abs(wl.dists["k_idx"].lo), abs(wl.dists["k_idx"].hi))
        wd = wl.dists["w"]
        wmax = max(wd.values) if wd.kind == "choice" else 2.0 ** wd.hi
        wmin = min(wd.values) if wd.kind == "choice" else 2.0 ** wd.lo
        bound = wl.H_I * wmax * wl.D_I * qmax * kmax
        assert bound / wmin < 2 ** 24, name
