"""Planted mistakes in the C++ oracle: every one must be caught by the pins.

Each mutant is the oracle's own source (oracle/dsa_oracle.cpp) with one
plausible mistake written into it: a dropped term, a wrong sign, index or
constant, a reversed operand, a missed mask.  The mutant is compiled on the
CPU into a library of its own and run through the pins of the step it
breaks; at least one pin must fail.  Every replacement must match the source
exactly as often as stated, so a change to the oracle that moves the code
under a mutant fails here instead of silently testing nothing.  Mutants only
change values, never the extent of an access, so none of them reads or writes
outside its buffers.
"""
import concurrent.futures
import os
import subprocess

import pytest

import oracle
import pins

# (name, pin group, old text, new text, occurrences of the old text to replace)
MUTANTS = [
    # O1 indexer
    ("no_relu", "indexer", "I += w_t[h] * relu(dot);", "I += w_t[h] * dot;", 1),
    ("relu_after_head_sum", "indexer", "I += w_t[h] * relu(dot);\n  }\n  return I;",
     "I += w_t[h] * dot;\n  }\n  return relu(I);", 1),
    ("head_weights_reversed", "indexer", "I += w_t[h] * relu(dot);", "I += w_t[H_I - 1 - h] * relu(dot);", 1),
    ("key_channels_reversed", "indexer", "dot += q_t[h * D_I + d] * k_s[d];",
     "dot += q_t[h * D_I + d] * k_s[D_I - 1 - d];", 1),
    ("query_head_and_channel_swapped", "indexer", "dot += q_t[h * D_I + d] * k_s[d];",
     "dot += q_t[d * H_I + h] * k_s[d];", 1),
    ("next_key_row", "indexer", "widen_into(k_idx, k_dt, (b * N + s) * D_I, D_I, k_s.data());",
     "widen_into(k_idx, k_dt, (b * N + (s + 1) % N) * D_I, D_I, k_s.data());", 1),
    ("own_key_excluded", "indexer", "const int64_t p1 = q_pos0 + t + 1;", "const int64_t p1 = q_pos0 + t;", 1),
    # O2 top-k
    ("ties_to_higher_index", "topk", "[v](int64_t a, int64_t b) { return v[a] > v[b]; }",
     "[v](int64_t a, int64_t b) { return v[a] > v[b] || (v[a] == v[b] && a > b); }", 1),
    ("smallest_kept", "topk", "return v[a] > v[b]; }", "return v[a] < v[b]; }", 1),
    ("rank_order_not_ascending", "topk", "std::sort(cand.begin(), cand.begin() + K);", "", 1),
    ("unstable_sort", "topk", "std::stable_sort(cand.begin()", "std::sort(cand.begin()", 1),
    ("padding_zero", "topk", "static_cast<int32_t>(i) : -1;", "static_cast<int32_t>(i) : 0;", 1),
    # O3 sparse MLA
    ("value_from_rope_end", "mla", "values[j] = &rows[j * D];", "values[j] = &rows[j * D + (D - DV)];", 1),
    ("no_scale", "mla", "      logits[j] = scale * dot;\n    }\n    softmax_attend(logits, values,",
     "      logits[j] = dot;\n    }\n    softmax_attend(logits, values,", 1),
    ("mask_ignored", "mla", "const int64_t i = idx_row[j];\n    if (i < 0 || i >= N) continue;",
     "const int64_t i = idx_row[j] < 0 ? 0 : idx_row[j];\n    if (i >= N) continue;", 1),
    ("lse_log2", "mla", "*lse_h = m + std::log(l);", "*lse_h = m + std::log2(l);", 1),
    ("lse_without_max", "mla", "*lse_h = m + std::log(l);", "*lse_h = std::log(l);", 1),
    ("exp_without_max", "mla", "p[j] = std::exp(logits[j] - m);", "p[j] = std::exp(logits[j]);", 1),
    ("normaliser_off", "mla", "o_h[c] = acc[c] / l;\n  *lse_h", "o_h[c] = acc[c] / (l + 1.0);\n  *lse_h", 1),
    ("gather_ignores_sequence", "mla", "widen_into(kv, kv_dt, (b * N + sel[j]) * D, D, &rows[j * D]);",
     "widen_into(kv, kv_dt, sel[j] * D, D, &rows[j * D]);", 1),
    ("query_head_zero", "mla",
     "widen_into(q, q_dt, ((b * Tq + t) * H + h) * D, D, q_h.data());\n    for (size_t j",
     "widen_into(q, q_dt, ((b * Tq + t) * H + 0) * D, D, q_h.data());\n    for (size_t j", 1),
    # O3' dense masked form
    ("dense_mask_ignored", "mla", "std::vector<double> mask(n_visible, kNegInf);",
     "std::vector<double> mask(n_visible, 0.0);", 1),
    ("dense_own_key_excluded", "mla",
     "const int64_t n = n_valid_keys(t, q_pos0[b], N, 1);\n      dense_masked_mla_row",
     "const int64_t n = n_valid_keys(t, q_pos0[b], N, 1) - 1;\n      dense_masked_mla_row", 1),
    # O4 composition
    ("forward_attends_query_zero", "forward", "scale, b, t, o + r * H * DV,\n                     lse + r * H);\n    });\n  });\n}\n\nint dsao_sylvester",
     "scale, b, 0, o + r * H * DV,\n                     lse + r * H);\n    });\n  });\n}\n\nint dsao_sylvester", 1),
    ("forward_scores_of_query_zero", "forward",
     "index_scores_row(q_idx, qi_dt, k_idx, ki_dt, w, w_dt, Tq, N, H_I, D_I, b, t, n, s.data());",
     "index_scores_row(q_idx, qi_dt, k_idx, ki_dt, w, w_dt, Tq, N, H_I, D_I, b, 0, n, s.data());", 1),
    # compressed key axis
    ("window_counted_when_open", "compressed", "return std::min(N, p1 / m);", "return std::min(N, (p1 - 1) / m + 1);",
     1),
    ("rate_ignored", "compressed", "return std::min(N, p1 / m);", "return std::min(N, p1);", 1),
    ("cap_one_short_of_cache_length", "compressed", "return std::min(N, p1 / m);", "return std::min(N - 1, p1 / m);",
     1),
    # projections and the naive form
    ("absorb_drops_rope", "proj", "out[ob + d_c + r] = qh[d_nope + r];", "out[ob + d_c + r] = 0.0;", 1),
    ("absorb_latent_reversed", "proj", "* d_c + c] * qh[n];", "* d_c + (d_c - 1 - c)] * qh[n];", 1),
    ("out_proj_latent_reversed", "proj", "* d_c + c] * oh[c];", "* d_c + c] * oh[d_c - 1 - c];", 1),
    ("linear_input_reversed", "proj", "acc += xm[k] * w[n * K_in + k];", "acc += xm[K_in - 1 - k] * w[n * K_in + k];",
     1),
    ("naive_drops_rope", "proj", "keys[j * kw + d_nope + r] = kr[j * d_rope + r];", "keys[j * kw + d_nope + r] = 0.0;",
     1),
    ("naive_value_through_key_projection", "proj", "acc += w_uv[static_cast<int64_t>(v) * d_c + x] * c[j * d_c + x];",
     "acc += w_uk[static_cast<int64_t>(v % d_nope) * d_c + x] * c[j * d_c + x];", 1),
    # FP8 indexer
    ("e4m3_bias_8", "fp8", "std::ldexp(1.0, E - 7);", "std::ldexp(1.0, E - 8);", 1),
    ("e4m3_subnormal_step", "fp8", "M * std::ldexp(1.0, -9);", "M * std::ldexp(1.0, -10);", 1),
    ("e4m3_truncating_encode", "fp8", "std::nearbyint((a / std::ldexp(1.0, e) - 1.0) * 8.0)",
     "std::floor((a / std::ldexp(1.0, e) - 1.0) * 8.0)", 1),
    ("e4m3_truncating_subnormal", "fp8", "std::nearbyint(a * 512.0)", "std::floor(a * 512.0)", 1),
    ("fwht_sign", "fp8", "y[base + dist + i] = a - b;", "y[base + dist + i] = b - a;", 1),
    ("pow2_scale_one_too_big", "fp8", "--e;\n  return e;", "--e;\n  return e + 1;", 1),
    ("fp8_score_rotation_factor_kept", "fp8", "relu(qs_t[h] * ks_s / D * dot)", "relu(qs_t[h] * ks_s * dot)", 1),
    ("fp8_score_no_key_scale", "fp8", "relu(qs_t[h] * ks_s / D * dot)", "relu(qs_t[h] / D * dot)", 1),
    ("quantize_scale_inverted", "fp8", "*scale = std::ldexp(1.0f, e);", "*scale = std::ldexp(1.0f, -e);", 1),
    # test helper, paged gather
    ("hadamard_sign", "fp8", "out[(i + k) * n + (j + k)] = -h;", "out[(i + k) * n + (j + k)] = h;", 1),
    ("paged_rows_reversed_in_block", "paged", "* block_size + r % block_size;",
     "* block_size + (block_size - 1 - r % block_size);", 2),
]


def _holds(pin, *args):
    """A pin's verdict; a pin that cannot even run (the mutant's library rejects the call) fails."""
    try:
        return bool(pin(*args))
    except ValueError:
        return False


def _group_checks(o, group):
    return [_holds(pin, *args) for pin, *args in _group_pins(o, group)]


def _group_pins(o, group):
    if group == "indexer":
        f = o.index_scores_rows
        return [(pins.pin_indexer_golden, f), (pins.pin_indexer_hadamard, f, o.sylvester_hadamard),
                (pins.pin_indexer_unit_queries, f), (pins.pin_indexer_causal, f), (pins.pin_indexer_heads, f)]
    if group == "topk":
        f = o.topk_row
        return [(pins.pin_topk_golden, f), (pins.pin_topk_bruteforce, f), (pins.pin_topk_short_rows, f),
                (pins.pin_topk_long_ties, f)]
    if group == "mla":
        f = o.sparse_mla_rows
        return [(pins.pin_mla_golden, f), (pins.pin_mla_single_key, f), (pins.pin_mla_uniform, f),
                (pins.pin_mla_permutation_and_mask, f), (pins.pin_mla_sdpa, o.sparse_mla, o.dense_masked_mla),
                (pins.pin_mla_sparse_equals_dense, o.sparse_mla, o.dense_masked_mla)]
    if group == "forward":
        return [(pins.pin_forward, o.forward_rows)]
    if group == "compressed":
        return [(pins.pin_compressed_visibility, o.n_valid_keys), (pins.pin_compressed_pipeline, o.index_scores, o.topk)]
    if group == "proj":
        return [(pins.pin_mla_naive_sdpa, o.mla_naive_rows), (pins.pin_linear, o.linear),
                (pins.pin_mla_absorbed_equals_naive, o.mla_absorb_query, o.sparse_mla_rows, o.mla_output_projection,
                                                   o.mla_naive_rows)]
    if group == "fp8":
        return [(pins.pin_e4m3, o.e4m3_decode, o.e4m3_encode_rne), (pins.pin_fwht, o.fwht_f32, o.sylvester_hadamard),
                (pins.pin_pow2_scale, o.pow2_scale_exp),
                (pins.pin_quantize_fp8, o.quantize_fp8_rows, o.fwht_f32, o.e4m3_decode),
                (pins.pin_fp8_scores_near_bf16, o.quantize_fp8_rows, o.index_scores_fp8_rows, o.index_scores_rows,
                                              o.fwht_f32, o.e4m3_decode)]
    if group == "paged":
        return [(pins.pin_paged_gather, o.paged_gather)]
    raise KeyError(group)


def _mutant_source(old, new, count):
    with open(oracle.SOURCE) as f:
        src = f.read()
    assert src.count(old) == count, f"mutation pattern found {src.count(old)} times, expected {count}: {old!r}"
    return src.replace(old, new)


@pytest.fixture(scope="module")
def mutant_libs(tmp_path_factory):
    """Every mutant compiled (in parallel) into its own shared library."""
    d = tmp_path_factory.mktemp("oracle_mutants")

    def build(m):
        name, _, old, new, count = m
        src = d / f"{name}.cpp"
        src.write_text(_mutant_source(old, new, count))
        lib = d / f"lib_{name}.so"
        subprocess.run(["g++", "-O1", "-std=c++17", "-fPIC", "-shared", "-pthread", "-I",
                        os.path.dirname(oracle.SOURCE), str(src), "-o", str(lib)], check=True, capture_output=True)
        return name, str(lib)

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        return dict(ex.map(build, MUTANTS))


def test_every_group_passes_on_the_oracle():
    for group in ("indexer", "topk", "mla", "forward", "compressed", "proj", "fp8", "paged"):
        assert all(_group_checks(oracle.default(), group)), group


@pytest.mark.parametrize("name,group", [(m[0], m[1]) for m in MUTANTS])
def test_pins_catch_planted_mistake(mutant_libs, name, group):
    checks = _group_checks(oracle.Oracle(mutant_libs[name]), group)
    assert not all(checks), f"planted mistake {name!r} passes every {group} pin"
