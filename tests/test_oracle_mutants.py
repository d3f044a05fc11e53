"""Planted mistakes in the oracle must be caught by its pins (no GPU).

Each case copies ``oracle/attn_oracle.c``, plants one plausible mistake in the
copy (a dropped term, a wrong sign, a wrong or transposed index), compiles it
with gcc into a temporary library, points the oracle wrapper at it, and checks
that at least one pin from ``test_oracle.py`` fails.  The real oracle source is
never modified.
"""
import os
import subprocess

import pytest

import oracle
import oracle.oracle as oracle_mod
import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle_mod.__file__), "attn_oracle.c")

# (name, text in attn_oracle.c, replacement)
MUTANTS = [
    ("scale_dropped", "s[j] = scale * dot;", "s[j] = dot;"),
    ("exp_sign_flipped", "double e = exp(s[j] - m);", "double e = exp(m - s[j]);"),
    ("max_not_subtracted", "double e = exp(s[j] - m);", "double e = exp(s[j]);"),
    ("normalisation_dropped", "out[d] /= z;", "out[d] /= 1.0;"),
    ("lse_max_dropped", "*lse = m + log(z);", "*lse = log(z);"),
    ("head_dim_reversed_in_rows",
     "dst[(r - a) * D + d] = elem(x, (r * H + h) * (int64_t)D + d, dtype);",
     "dst[(r - a) * D + d] = elem(x, (r * H + h) * (int64_t)D + (D - 1 - d), dtype);"),
    ("key_range_from_query_bounds",
     "int64_t qa = cu_q[i], qb = cu_q[i + 1], ka = cu_k[i], kb = cu_k[i + 1];",
     "int64_t qa = cu_q[i], qb = cu_q[i + 1], ka = cu_q[i], kb = cu_q[i + 1];"),
    ("last_key_dropped", "attend_row(qrow, K, V, nk, D, scale, s,\n",
     "attend_row(qrow, K, V, nk - (nk > 1), D, scale, s,\n"),
    ("decode_last_key_dropped", "attend_row(qrow, K, V, L, D, scale, sc,",
     "attend_row(qrow, K, V, L - (L > 1), D, scale, sc,"),
    ("slot_offset_wrong", "int o = t % block_size;", "int o = (t + 1) % block_size;"),
    ("k_layout_transposed",
     "(head_size / x) + d / x) * block_size + o) * x + d % x;",
     "block_size + o) * (head_size / x) + d / x) * x + d % x;"),
    ("v_layout_transposed",
     "int64_t vi = ((b * num_kv_heads + hk) * (int64_t)head_size + d) * block_size + o;",
     "int64_t vi = ((b * num_kv_heads + hk) * (int64_t)block_size + o) * head_size + d;"),
    ("gqa_mapping_modulo", "int hk = hq / G;", "int hk = hq % num_kv_heads;"),
    ("query_head_from_kv_head",
     "qrow[d] = elem(query, ((int64_t)s * num_query_heads + hq) * D + d, dtype);",
     "qrow[d] = elem(query, ((int64_t)s * num_query_heads + hk) * D + d, dtype);"),
    ("bf16_shift_wrong", "uint32_t u = (uint32_t)bits << 16;", "uint32_t u = (uint32_t)bits << 15;"),
    ("fp16_bias_wrong", "expo - 25", "expo - 24"),
    ("fp16_subnormal_wrong", "ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
]

# The pins run against each mutant (the test functions of test_oracle.py).
PINS = [
    pins.test_bf16_decoding_every_pattern,
    pins.test_fp16_decoding_every_pattern,
    lambda: pins.test_prefill_matches_library_sdpa("bf16", [4, 0, 6], [3, 5, 9], 2, 16),
    lambda: pins.test_decode_matches_library_sdpa("bf16", 4, 33, 8, 2, 8, [33, 1, 16, 17]),
    pins.test_single_key_returns_value_row_exactly,
    pins.test_two_keys_logistic_blend,
    lambda: pins.test_uniform_weights_average_values("zero_query"),
    pins.test_identical_value_rows_return_that_row,
    pins.test_softmax_weights_sum_to_one,
    pins.test_lse_matches_log_sum_exp_of_scores,
    pins.test_large_scores_stay_finite,
    lambda: pins.test_gather_matches_numpy_layout_bitwise("bf16"),
    pins.test_grouped_query_heads_equal_repeated_kv_heads,
]


def _caught(lib):
    saved = oracle_mod._lib
    oracle_mod._lib = lib
    try:
        for pin in PINS:
            try:
                pin()
            except (AssertionError, ValueError):
                return True
        return False
    finally:
        oracle_mod._lib = saved


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new)
    c = tmp_path / "mutant.c"
    so = tmp_path / "libmutant.so"
    c.write_text(mutated)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(c), "-lm"],
                   check=True)
    assert _caught(oracle_mod.load(str(so))), f"no pin catches the planted mistake {name}"


def test_unmutated_copy_passes_every_pin(tmp_path):
    c = tmp_path / "same.c"
    so = tmp_path / "libsame.so"
    c.write_text(open(SRC).read())
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(c), "-lm"],
                   check=True)
    assert not _caught(oracle_mod.load(str(so)))
