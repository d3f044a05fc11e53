"""Planted mistakes in the chunked delta-rule output oracle must be caught by
its pins (no GPU).

Each case copies ``oracle/chunk_oracle.c``, plants one plausible mistake (a
flipped condition or sign, a dropped factor or rounding, a wrong index),
compiles the copy with gcc, points the wrapper at it and checks that at least
one pin of ``test_chunk_oracle.py`` fails.  The real source is never modified.
"""
import os
import subprocess

import pytest

import oracle.chunk as chunk_mod
import test_chunk_oracle as pins

SRC = os.path.join(os.path.dirname(chunk_mod.__file__), "chunk_oracle.c")

MUTANTS = [
    ("mask_direction_flipped", "if (j <= i && G[i] <= G[j]) {", "if (j <= i && G[i] >= G[j]) {"),
    ("causal_mask_dropped", "if (j <= i && G[i] <= G[j]) {", "if (G[i] <= G[j]) {"),
    ("gate_sign_flipped", "a = oracle_round_to_dtype(dot * exp(G[i] - G[j]), dtype);",
     "a = oracle_round_to_dtype(dot * exp(G[j] - G[i]), dtype);"),
    ("score_rounding_dropped", "a = oracle_round_to_dtype(dot * exp(G[i] - G[j]), dtype);",
     "a = dot * exp(G[i] - G[j]);"),
    ("state_gate_dropped", "const double gate = exp(G[i]);", "const double gate = 1.0;"),
    ("scale_on_one_term", "orow[e] = scale * (gate * inter + intra);",
     "orow[e] = scale * gate * inter + intra;"),
    ("intra_term_dropped", "orow[e] = scale * (gate * inter + intra);",
     "orow[e] = scale * (gate * inter);"),
    ("query_head_modulo", "int hq = hd / per_q;\n                if", "int hq = hd % Hq;\n                if"),
    ("state_from_next_chunk", "const int64_t hbase = (((int64_t)b * num_chunks + c) * H + hd)",
     "const int64_t hbase = (((int64_t)b * num_chunks + (c + 1) % num_chunks) * H + hd)"),
    ("state_transposed", "const double qv = Q[(size_t)i * K + d], hv = Hc[(size_t)d * V + e];",
     "const double qv = Q[(size_t)i * K + d], hv = Hc[(size_t)e * K + d];"),
    ("gate_from_query_head", "G[i] = (double)g[t * H + hd];", "G[i] = (double)g[t * H + hq];"),
    ("value_from_query_head", "Vc[(size_t)i * V + e] = value(v, (t * H + hd) * (int64_t)V + e, dtype);",
     "Vc[(size_t)i * V + e] = value(v, (t * H + hq) * (int64_t)V + e, dtype);"),
    ("key_row_is_query_row", "dot += Q[(size_t)i * K + d] * Kc[(size_t)j * K + d];",
     "dot += Q[(size_t)i * K + d] * Kc[(size_t)i * K + d];"),
    ("ties_away_from_zero", "return ldexp(nearbyint(ldexp(x, -qe)), qe);",
     "return ldexp(round(ldexp(x, -qe)), qe);"),
    ("bf16_subnormal_quantum_wrong", "dtype == ORACLE_BF16 ? -133 : -24", "dtype == ORACLE_BF16 ? -132 : -24"),
    ("fp16_precision_wrong", "dtype == ORACLE_BF16 ? 8 : 11", "dtype == ORACLE_BF16 ? 8 : 10"),
    ("chunk_start_wrong", "const int t0 = c * chunk;\n", "const int t0 = c * chunk + (c > 0);\n"),
]

PINS = [
    pins.test_rounding_ties_to_even,
    lambda: pins.test_rounding_matches_torch_from_float32(pins.torch.float16, 1),
    lambda: pins.test_constant_gate_reduces_to_masked_matmul(21, 8),
    lambda: pins.test_constant_gate_reduces_to_masked_matmul(70, 64),
    pins.test_token_gate_decides_mask_and_weights,
    pins.test_decreasing_gate_matches_recurrence,
    pins.test_padding_rows_are_inert,
    pins.test_grouped_heads_match_repeated_query_heads,
    pins.test_each_chunk_uses_its_own_state,
    pins.test_linear_in_value_state_and_scale,
    pins.test_rows_entry_matches_whole_output,
]


def _caught(lib):
    saved = chunk_mod._lib
    chunk_mod._lib = lib
    try:
        for pin in PINS:
            try:
                pin()
            except (AssertionError, ValueError):
                return True
        return False
    finally:
        chunk_mod._lib = saved


def _compile(tmp_path, text, stem):
    c = tmp_path / f"{stem}.c"
    so = tmp_path / f"lib{stem}.so"
    c.write_text(text)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(c), "-lm"],
                   check=True)
    return chunk_mod.load(str(so))


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    assert _caught(_compile(tmp_path, src.replace(old, new, 1), "mutant")), \
        f"no pin catches the planted mistake {name}"


def test_unmutated_copy_passes_every_pin(tmp_path):
    assert not _caught(_compile(tmp_path, open(SRC).read(), "same"))
