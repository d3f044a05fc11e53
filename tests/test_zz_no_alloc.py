"""attn_paged_decode_noalloc through the C ABI against attn_paged_decode.

The no-allocation entry point keeps a split context's partial results in the
library's static per-GPU buffer instead of a caller workspace.  Its output
must equal, bit for bit, that of attn_paged_decode with a workspace (the same
kernels), and meet the parity bars against the oracle
("paged_attention_decode" #024, Reference Implementation), on two calls in a
row, the second smaller (the buffer then still holds the first call's
partials), and with no split at all.
"""
import ctypes

import pytest
import torch

import oracle
from parity import check, f64, to_gpu
from softmax_attention_flashattention_amd import attn_paged_decode, binding, inputs as gen

pytestmark = pytest.mark.gpu


def noalloc_via_abi(inp, partition_size, out):
    lib = binding._load()
    q, kc, vc = inp["query"], inp["k_cache"], inp["v_cache"]
    bt, sl = inp["block_tables"], inp["seq_lens"]
    S, Hq, D = q.shape
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = lib.attn_paged_decode_noalloc(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), bt.data_ptr(),
                                       sl.data_ptr(), S, Hq, vc.shape[1], D, vc.shape[3],
                                       bt.shape[1], vc.shape[0], D ** -0.5,
                                       0 if q.dtype == torch.bfloat16 else 1, partition_size,
                                       out.data_ptr(), stream)
    torch.cuda.synchronize()
    return rc


def compare(inp, partition_size, what):
    print(f"[noalloc] {what}", flush=True)
    d = to_gpu(inp)
    out = torch.full_like(d["query"], float("nan"))
    assert noalloc_via_abi(d, partition_size, out) == 0
    ref_call = attn_paged_decode(d["query"], d["k_cache"], d["v_cache"], d["block_tables"],
                                 d["seq_lens"], partition_size=partition_size)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_call), f"{what}: differs from attn_paged_decode"
    args = (inp["query"], inp["k_cache"], inp["v_cache"], inp["block_tables"], inp["seq_lens"])
    ref = oracle.paged_decode(*args)
    ref_abs = oracle.paged_decode(inp["query"], inp["k_cache"], inp["v_cache"].abs(),
                                  inp["block_tables"], inp["seq_lens"])
    check(f64(out), ref, what, ref_abs=ref_abs)


def test_two_calls_in_a_row_the_second_smaller():
    big = gen.decode_inputs(64, 1000, 16, 4, 128, seed=201,
                            seq_lens=[1000, 17, 0, 640, 999, 1, 512, 513] * 8)
    assert binding.attn_paged_decode_num_partitions(64, 4, 63, 16, 64) == 16
    compare(big, 64, "64 seqs x ctx <= 1000, 16 partitions of 64 tokens")
    small = gen.decode_inputs(8, 300, 8, 8, 256, seed=202, dtype="fp16",
                              seq_lens=[300, 33, 1, 0, 288, 100, 17, 256])
    compare(small, 32, "8 seqs x ctx <= 300, head_size 256, fp16, partitions of 32 tokens")


def test_one_partition_uses_no_buffer():
    inp = gen.workload_inputs("decode_b256_ctx64_h16_kv16_d128")
    compare(inp, 0, "256 seqs x ctx 64, one partition")


def test_automatic_partitions_use_the_buffer():
    # partition_size 0 on few long contexts: the library splits them into
    # 128-token partitions (24 here), whose partials go to the static buffer
    inp = gen.decode_inputs(2, 3000, 8, 1, 128, seed=203, seq_lens=[3000, 77])
    assert binding.attn_paged_decode_num_partitions(2, 1, inp["block_tables"].shape[1], 16) == 24
    compare(inp, 0, "2 seqs x 1 KV head x ctx <= 3000, automatic partitions")


def test_grouped_heads_on_matrix_cores_use_the_buffer():
    # 8 and 16 query heads per KV head on device-filling grids run on the
    # MFMA decode kernel; their split contexts' partials go to the static
    # buffer too (two calls, the second smaller)
    big = gen.decode_inputs(64, 1000, 32, 4, 128, seed=204,
                            seq_lens=[1000, 17, 0, 640, 999, 1, 512, 513] * 8)
    compare(big, 256, "64 seqs x 32/4 heads x ctx <= 1000, partitions of 256 tokens, MFMA kernel")
    small = gen.decode_inputs(32, 600, 64, 4, 256, seed=205, dtype="fp16",
                              seq_lens=[600, 33, 1, 0, 288, 100, 17, 256] * 4)
    compare(small, 128, "32 seqs x 64/4 heads x ctx <= 600, head_size 256, fp16, MFMA kernel")
