"""The named workloads and input generators match the pages' tables (no GPU).

Sizes are checked against the Shapes tables of atrex-bench
"attention_forward" (#001) and "paged_attention_decode" (#024), stored under
tests/golden/; layouts against those pages' Input Generation sections.
"""
import os
import sys

import torch

sys.path.insert(0, os.path.join(os.path.dirname(__file__), "golden"))
import shapes  # noqa: E402

from softmax_attention_flashattention_amd import inputs as gen  # noqa: E402


def test_prefill_workloads_are_table_rows():
    rows = {r["row"]: r for r in shapes.prefill_rows()}
    assert len(rows) == 21
    for name, row in [("prefill_s276_h4_d72", 11), ("prefill_s8136_h16_d72", 4),
                      ("prefill_s16742_h32_d128", 9), ("prefill_s65556_h16_d72", 8)]:
        w = gen.WORKLOADS[name]
        assert w["seq_lens"] == [rows[row]["seq_len"]]
        assert w["num_heads"] == rows[row]["num_heads"]
        assert w["head_dim"] == rows[row]["head_dim"]


def test_decode_workload_is_table_row_0():
    r = shapes.decode_rows()[0]
    w = gen.WORKLOADS["decode_b256_ctx64_h16_kv16_d128"]
    for key in ("num_seqs", "ctx_len", "num_query_heads", "num_kv_heads", "head_size",
                "block_size", "dtype"):
        assert w[key] == r[key], key


def test_decode_inputs_layout():
    d = gen.decode_inputs(256, 64, 16, 16, 128, seed=1)
    assert d["query"].shape == (256, 16, 128)
    assert d["k_cache"].shape == (1040, 16, 16, 16, 8)        # 4 * 256 + 16 spare blocks
    assert d["v_cache"].shape == (1040, 16, 128, 16)
    assert d["block_tables"].dtype == torch.int32
    assert d["block_tables"][3].tolist() == [12, 13, 14, 15]
    assert d["seq_lens"].tolist() == [64] * 256


def test_prefill_inputs_layout_and_determinism():
    a = gen.prefill_inputs([5, 7], 3, 72, seed=4)
    b = gen.prefill_inputs([5, 7], 3, 72, seed=4)
    assert a["q"].shape == (12, 3, 72) and a["q"].dtype == torch.bfloat16
    assert a["cu_seqlens_q"].tolist() == [0, 5, 12] == a["cu_seqlens_k"].tolist()
    assert all(torch.equal(a[k], b[k]) for k in ("q", "k", "v"))
    # standard normal, drawn in float32 and rounded to bf16
    big = gen.prefill_inputs([4096], 4, 64, seed=9)["q"].float()
    assert abs(big.mean().item()) < 0.01 and abs(big.std().item() - 1.0) < 0.01


def test_permute_blocks_moves_data_consistently():
    d = gen.decode_inputs(4, 40, 2, 2, 16, seed=3)
    p = gen.permute_blocks(d, seed=5)
    for s in range(4):
        for j in range(d["block_tables"].shape[1]):
            a, b = d["block_tables"][s, j], p["block_tables"][s, j]
            assert torch.equal(d["k_cache"][a], p["k_cache"][b])
            assert torch.equal(d["v_cache"][a], p["v_cache"][b])
