"""GPU parity of attn_paged_decode against the CPU oracle.

Operator: atrex-bench "paged_attention_decode" (#024), Reference
Implementation and Input Generation.  Every case feeds the HIP library and
the oracle the same seeded inputs and applies the bar of tests/parity.py.
Index work is checked bit for bit: a cache whose blocks are moved and whose
table is rewritten to match must give identical output bits, and a
one-token context must return the gathered value row exactly.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import check, f64, to_gpu
from softmax_attention_flashattention_amd import attn_paged_decode, inputs as gen

pytestmark = pytest.mark.gpu


def run(inp, partition_size=0):
    d = to_gpu(inp)
    o = attn_paged_decode(d["query"], d["k_cache"], d["v_cache"], d["block_tables"],
                          d["seq_lens"], partition_size=partition_size)
    torch.cuda.synchronize()
    return o


def ref_of(inp, v_abs=False):
    v = inp["v_cache"].abs() if v_abs else inp["v_cache"]
    return oracle.paged_decode(inp["query"], inp["k_cache"], v, inp["block_tables"],
                               inp["seq_lens"])


def full_check(inp, what, partition_size=0, bar1=True):
    print(f"[decode] {what}", flush=True)
    out = run(inp, partition_size)
    return check(f64(out), ref_of(inp), what, ref_abs=ref_of(inp, True), bar1=bar1), out


def test_workload_b256_ctx64_h16_kv16_d128():
    full_check(gen.workload_inputs("decode_b256_ctx64_h16_kv16_d128"),
               "decode_b256_ctx64_h16_kv16_d128")


def test_permuted_block_table_is_bitwise_identical():
    inp = gen.decode_inputs(64, 100, 8, 4, 128, seed=3,
                            seq_lens=[100, 1, 16, 17, 0, 64, 33, 99] * 8)
    per = gen.permute_blocks(inp, seed=11)
    a = run(inp).cpu()
    b = run(per).cpu()
    assert torch.equal(a, b)
    check(f64(a), ref_of(inp), "identity table", ref_abs=ref_of(inp, True))


def test_ragged_and_empty_contexts():
    lens = [1, 2, 15, 16, 17, 31, 33, 47, 48, 49, 63, 64, 0, -3, 5, 60]
    inp = gen.decode_inputs(16, 64, 4, 4, 128, seed=5, seq_lens=lens)
    _, out = full_check(inp, "ragged contexts")
    o = out.cpu()
    assert torch.count_nonzero(o[12]).item() == 0 and torch.count_nonzero(o[13]).item() == 0


def test_sharp_attention_over_a_long_context():
    # query x 32 (exact in bf16): scores spread over hundreds of log2 units
    # and the split-K partitions see very different maxima
    inp = gen.decode_inputs(8, 1000, 8, 2, 128, seed=57)
    inp["query"] = (inp["query"].float() * 32).to(torch.bfloat16)
    full_check(inp, "sharp, one partition")
    full_check(inp, "sharp, 64-token partitions", partition_size=64)


@pytest.mark.parametrize("dtype,head_size,partition_size",
                         [("bf16", 128, 0), ("fp16", 128, 0), ("bf16", 128, 64), ("bf16", 256, 32)])
def test_identical_value_rows_return_that_row(dtype, head_size, partition_size):
    # Every token of a KV head carries the same value row u, so out =
    # (sum_j w_j) u / sum_j w_j for any weights.  The weights that multiply V
    # are rounded to 16 bits; when the row sum adds up those same rounded
    # weights, the quotient is u up to fp32 rounding and rounds back to u bit
    # for bit (a sum of the unrounded weights misses by up to one unit in the
    # last place).  Contexts from 1 token to several partitions.
    lens = [1, 15, 16, 17, 100, 333, 700, 0]
    inp = gen.decode_inputs(8, 700, 8, 2, head_size, seed=61, dtype=dtype, seq_lens=lens)
    inp["query"] = (inp["query"].float() * 4).to(inp["query"].dtype)   # weights spread over 2^10 and more
    u = inp["v_cache"][0, :, :, 0].clone()                              # [Hkv, D]
    inp["v_cache"] = u[None, :, :, None].expand_as(inp["v_cache"]).contiguous()
    print(f"[decode] identical V rows {dtype} D={head_size} partition {partition_size}", flush=True)
    out = run(inp, partition_size).cpu()
    for s, n in enumerate(lens):
        for hq in range(8):
            want = u[hq // 4] if n > 0 else torch.zeros_like(u[0])
            assert torch.equal(out[s, hq], want), (s, n, hq)


def test_automatic_partitions_for_few_long_contexts():
    # Few workgroups (sequence x KV head) and long contexts: the library's
    # own choice (partition_size 0) splits the context into 128-token
    # partitions, which must match the explicit 128-token split bit for bit
    # and the oracle to the parity bar.
    from softmax_attention_flashattention_amd import attn_paged_decode_num_partitions
    cases = [(1, 16, 2, 128, "bf16", [1000]), (2, 8, 1, 128, "bf16", [3000, 77]),
             (3, 16, 2, 256, "fp16", [700, 1, 513])]
    for i, (n, hq, hkv, D, dtype, lens) in enumerate(cases):
        inp = gen.decode_inputs(n, max(lens), hq, hkv, D, seed=71 + i, dtype=dtype, seq_lens=lens)
        maxb = inp["block_tables"].shape[1]
        parts = attn_paged_decode_num_partitions(n, hkv, maxb, 16)
        assert parts == (maxb * 16 + 127) // 128, (parts, maxb)
        what = f"{n} seqs x {hkv} KV heads, contexts {lens}, D {D} {dtype}: {parts} automatic partitions"
        _, auto = full_check(inp, what)
        explicit = run(inp, 128)
        assert torch.equal(auto, explicit), what


def test_one_token_context_returns_value_row_exactly():
    inp = gen.decode_inputs(8, 1, 4, 2, 128, seed=7)
    per = gen.permute_blocks(inp, seed=8)
    out = run(per).cpu()
    for s in range(8):
        b = int(per["block_tables"][s, 0])
        for hq in range(4):
            v = per["v_cache"][b, hq // 2, :, 0]      # token 0 of the block: [D]
            assert torch.equal(out[s, hq], v), (s, hq)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("Hq,Hkv", [(16, 16), (16, 8), (32, 8), (40, 8), (12, 4), (64, 8),
                                    (32, 2), (16, 1)])
def test_grouped_query_heads(dtype, Hq, Hkv):
    inp = gen.decode_inputs(6, 128, Hq, Hkv, 128, seed=Hq * 100 + Hkv, dtype=dtype,
                            seq_lens=[128, 77, 1, 16, 100, 0])
    full_check(inp, f"GQA {dtype} Hq={Hq} Hkv={Hkv}")


@pytest.mark.parametrize("partition_size", [16, 48, 112, 256])
@pytest.mark.parametrize("G", [1, 4])
def test_split_context_merge(partition_size, G):
    lens = [1000, 333, 17, 0, 512, 1]
    inp = gen.decode_inputs(6, 1000, 4 * G, 4, 128, seed=51 + G, seq_lens=lens)
    (_, _), split = full_check(inp, f"split P={partition_size} G={G}", partition_size)
    whole = run(inp, partition_size=16 * 64)            # one partition
    assert torch.count_nonzero(split[3]).item() == 0
    check(f64(split), f64(whole).astype(np.float64), "split vs whole")


@pytest.mark.parametrize("ctx,num_seqs", [(4096, 4), (32768, 2)])
def test_long_contexts(ctx, num_seqs):
    inp = gen.decode_inputs(num_seqs, ctx, 8, 2, 128, seed=ctx)
    full_check(inp, f"long ctx {ctx}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_page_table_rows(dtype):
    # the remaining rows of the decode Shapes table that fit head_size 128
    for (S, L, Hq, Hkv) in [(128, 64, 3, 3), (4, 128, 32, 4), (4, 128, 32, 8), (1, 128, 4, 1),
                            (4, 128, 40, 8), (4, 128, 64, 8)]:
        full_check(gen.decode_inputs(S, L, Hq, Hkv, 128, seed=S + L + Hq, dtype=dtype),
                   f"table row {S}x{L} Hq={Hq} Hkv={Hkv} {dtype}")


def test_scaled_values_tighten_the_floor():
    inp = gen.decode_inputs(32, 300, 8, 2, 128, seed=61)
    inp["v_cache"] = (inp["v_cache"].float() * 64.0).to(torch.bfloat16)
    full_check(inp, "V*64", bar1=False)


def test_runs_are_bitwise_deterministic():
    inp = gen.decode_inputs(16, 700, 8, 2, 128, seed=71)
    assert torch.equal(run(inp, 64).cpu(), run(inp, 64).cpu())


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("S,L,Hq,Hkv,lens", [
    (1, 128, 16, 2, None),                        # decode Shapes table row 1
    (5, 300, 8, 8, [300, 1, 0, 17, 256]),
    (3, 700, 32, 4, [700, 64, 1]),
])
def test_head_size_256(dtype, S, L, Hq, Hkv, lens):
    inp = gen.decode_inputs(S, L, Hq, Hkv, 256, seed=S * L + Hq, dtype=dtype, seq_lens=lens)
    full_check(inp, f"D=256 {dtype} {S}x{L} Hq={Hq} Hkv={Hkv}")
    if L > 256:
        full_check(inp, f"D=256 split {dtype}", partition_size=128)


def test_binding_rejects_mismatched_tensors():
    # the binding refuses, naming the argument, what the library could not
    # read correctly: host memory, another dtype, a strided view, a bad out
    inp = gen.decode_inputs(2, 40, 4, 2, 128, seed=61)
    d = to_gpu(inp)
    args = [d["query"], d["k_cache"], d["v_cache"], d["block_tables"], d["seq_lens"]]
    bad = list(args)
    bad[2] = inp["v_cache"]
    with pytest.raises(ValueError, match="v_cache must be a GPU tensor"):
        attn_paged_decode(*bad)
    bad = list(args)
    bad[1] = d["k_cache"].half()
    with pytest.raises(TypeError, match="k_cache has dtype"):
        attn_paged_decode(*bad)
    bad = list(args)
    bad[3] = d["block_tables"].t().contiguous().t()
    with pytest.raises(ValueError, match="block_tables must be contiguous"):
        attn_paged_decode(*bad)
    with pytest.raises(TypeError, match="out has dtype"):
        attn_paged_decode(*args, out=d["query"].float())
    with pytest.raises(ValueError, match="out must have query's shape"):
        attn_paged_decode(*args, out=d["query"][:1])


@pytest.mark.parametrize("S,L,Hq,Hkv,D,dtype", [
    (85, 100, 5, 1, 128, "bf16"),     # 85 units: G = 5 dealt as 2 + 2 + 1 heads
    (1, 128, 16, 2, 256, "bf16"),     # 2 units: one query head per workgroup
    (3, 700, 16, 1, 128, "fp16"),     # split context (18 units) and heads dealt out: 8 x 2
    (128, 64, 8, 4, 128, "bf16"),     # 512 units fill the device: all 2 heads in one workgroup
])
def test_query_heads_dealt_to_workgroups(S, L, Hq, Hkv, D, dtype):
    # grids with fewer (sequence, KV head, partition) units than compute
    # units spread each KV head's query heads over several workgroups; every
    # output row must still come out once, right
    lens = [L - (7 * i) % max(L // 3, 1) for i in range(S)]
    inp = gen.decode_inputs(S, L, Hq, Hkv, D, seed=S + L + Hq + D, dtype=dtype, seq_lens=lens)
    d = to_gpu(inp)
    out = torch.full_like(d["query"], float("nan"))
    attn_paged_decode(d["query"], d["k_cache"], d["v_cache"], d["block_tables"], d["seq_lens"],
                      out=out)
    torch.cuda.synchronize()
    what = f"decode {S} x {L} Hq {Hq} Hkv {Hkv} D {D} {dtype}, heads dealt to workgroups"
    print(f"[decode] {what}", flush=True)
    check(f64(out), ref_of(inp), what, ref_abs=ref_of(inp, True))


@pytest.mark.parametrize("S,L,Hq,Hkv,D,dtype,ps", [
    (64, 300, 32, 8, 128, "bf16", 0),       # G 4, 19 blocks a workgroup
    (40, 700, 40, 8, 128, "fp16", 0),       # G 5: heads padded to 16 columns
    (128, 300, 16, 8, 128, "fp16", 0),      # G 2 with 19 blocks
    (70, 1000, 64, 4, 128, "bf16", 256),    # G 16, split context, merge kernel
    (64, 400, 64, 8, 128, "bf16", 32),      # G 8, 2-block partitions: a block per wave
    (48, 600, 64, 8, 256, "bf16", 0),       # G 8, head_size 256, 32 blocks a workgroup
    (32, 900, 128, 8, 256, "fp16", 128),    # G 16, head_size 256, split context
    (300, 17, 32, 4, 128, "bf16", 0),       # G 8, contexts of one or two blocks
    (128, 130, 64, 8, 256, "fp16", 0),      # G 8, head_size 256, 9 blocks a workgroup
    (64, 600, 32, 8, 256, "bf16", 0),       # G 4, head_size 256, 38 blocks a workgroup
    (512, 40, 16, 8, 128, "bf16", 0),       # G 2, three blocks a workgroup
    (256, 50, 24, 8, 128, "fp16", 0),       # G 3 over four blocks
    (256, 70, 16, 8, 256, "bf16", 0),       # G 2, head_size 256
    (256, 130, 16, 16, 128, "bf16", 0),     # one query head per KV head, 9 blocks a workgroup
    (128, 300, 8, 8, 256, "fp16", 0),       # one query head per KV head, head_size 256
    (64, 1000, 8, 8, 128, "bf16", 128),     # one query head per KV head, 8-block partitions, merge
])
def test_grouped_heads_on_matrix_cores(S, L, Hq, Hkv, D, dtype, ps):
    # device-filling grids (sequence x KV head x partition units at least the
    # compute units) with grouped query heads run the score and value
    # products on MFMAs (decode_mfma_kernel, from 2 query heads per KV head
    # when no heads are dealt out, with one where a workgroup walks 8 blocks
    # or more); ragged contexts, an empty one, scattered blocks
    lens = [L - (13 * i) % max(L // 2, 1) for i in range(S)]
    lens[1] = 0
    inp = gen.decode_inputs(S, L, Hq, Hkv, D, seed=S + Hq + D + ps, dtype=dtype, seq_lens=lens)
    inp = gen.permute_blocks(inp, seed=S * 7 + Hq)
    d = to_gpu(inp)
    out = torch.full_like(d["query"], float("nan"))
    attn_paged_decode(d["query"], d["k_cache"], d["v_cache"], d["block_tables"], d["seq_lens"], out=out,
                      partition_size=ps)
    torch.cuda.synchronize()
    what = f"decode {S} x {L} Hq {Hq} Hkv {Hkv} D {D} {dtype} partition {ps or 'auto'}, grouped heads on MFMAs"
    print(f"[decode] {what}", flush=True)
    check(f64(out), ref_of(inp), what, ref_abs=ref_of(inp, True))
    assert torch.count_nonzero(out[1]).item() == 0, what


@pytest.mark.parametrize("S,L,Hq,Hkv,D,dtype,ps", [
    (64, 300, 64, 8, 128, "bf16", 0),       # G 8, whole contexts
    (64, 200, 128, 8, 256, "fp16", 0),      # G 16, head_size 256
    (64, 700, 32, 8, 128, "bf16", 128),     # G 4, 8-block partitions, merge kernel
])
def test_identical_value_rows_on_matrix_cores(S, L, Hq, Hkv, D, dtype, ps):
    # The invariant of test_identical_value_rows_return_that_row on grids
    # that run the MFMA decode kernel: its row sum adds the same 16-bit
    # weights that form the B operand of the value product, so every output
    # row is the KV head's value row bit for bit, through the split-context
    # merge too.
    lens = [(1, 15, 16, 17, 100, L, L - 3, 33)[i % 8] for i in range(S)]
    lens[5] = 0
    inp = gen.decode_inputs(S, L, Hq, Hkv, D, seed=90 + S + Hq + D, dtype=dtype, seq_lens=lens)
    inp["query"] = (inp["query"].float() * 4).to(inp["query"].dtype)
    u = inp["v_cache"][0, :, :, 0].clone()                              # [Hkv, D]
    inp["v_cache"] = u[None, :, :, None].expand_as(inp["v_cache"]).contiguous()
    inp = gen.permute_blocks(inp, seed=S + D)
    print(f"[decode] identical V rows on MFMAs {S} x {L} Hq {Hq} Hkv {Hkv} D {D} {dtype} partition {ps}",
          flush=True)
    out = run(inp, ps).cpu()
    G = Hq // Hkv
    for s, n in enumerate(lens):
        for hq in range(Hq):
            want = u[hq // G] if n > 0 else torch.zeros_like(u[0])
            assert torch.equal(out[s, hq], want), (s, n, hq)
