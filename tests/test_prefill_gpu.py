"""GPU parity of attn_varlen_fwd against the CPU oracle.

Operator: atrex-bench "attention_forward" (#001), Reference Implementation.
Every case feeds the HIP library and the oracle the same seeded inputs and
applies the bar of tests/parity.py elementwise.  The full-size workloads run
with their output filled with NaN first, so an unwritten row cannot pass:
the 276-, 8136- and 16742-token ones are compared on every element, the
65556-token one on one row from every work item after checking that every
element was written.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import check, f64, to_gpu
from softmax_attention_flashattention_amd import attn_varlen_fwd, inputs as gen

pytestmark = pytest.mark.gpu

SENTINEL = -12352.0      # exactly representable in bf16 and fp16


def run(inp, out=None):
    d = to_gpu(inp)
    o = attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"],
                        max_seqlen_q=inp["max_seqlen_q"], out=out)
    torch.cuda.synchronize()
    return o


def refs(inp):
    """Oracle output and the same weights applied to |v| (the scale of bar 2)."""
    return oracle.varlen_fwd(inp["q"], inp["k"], inp["v"], inp["cu_seqlens_q"],
                             inp["cu_seqlens_k"], return_abs=True)


def full_check(inp, what, bar1=True):
    print(f"[prefill] {what}", flush=True)
    out = run(inp)
    ref, ref_abs = refs(inp)
    m = ~np.isnan(ref)
    return check(f64(out)[m], ref[m], what, ref_abs=ref_abs[m], bar1=bar1)


@pytest.mark.parametrize("D", [72, 128])
@pytest.mark.parametrize("S", [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 276])
def test_single_sequence_lengths(D, S):
    full_check(gen.prefill_inputs([S], 2, D, seed=100 + S), f"S={S} D={D}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("D", [72, 128])
def test_varlen_batch_with_empty_and_unequal_segments(dtype, D):
    # an empty query segment, S_q != S_k, a sequence with no keys, ragged tiles
    inp = gen.prefill_inputs([5, 0, 300, 64, 129, 1], 3, D, seed=7, dtype=dtype,
                             seq_lens_k=[7, 3, 250, 0, 129, 200])
    full_check(inp, f"varlen {dtype} D={D}")


@pytest.mark.parametrize("D", [72, 128])
def test_rows_outside_segments_are_untouched(D):
    inp = gen.prefill_inputs([40, 70], 2, D, seed=9)
    # 30 extra rows after the last segment belong to no sequence
    pad = torch.zeros(30, 2, D, dtype=torch.bfloat16)
    inp["q"] = torch.cat([inp["q"], pad])
    d = to_gpu(inp)
    out = torch.full_like(d["q"], SENTINEL)
    attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"],
                    max_seqlen_q=70, out=out)
    torch.cuda.synchronize()
    o = f64(out)
    assert np.all(o[110:] == SENTINEL)
    ref, ref_abs = refs(inp)
    check(o[:110], ref[:110], f"sentinel D={D}", ref_abs=ref_abs[:110])


@pytest.mark.parametrize("D", [72, 128])
def test_segment_longer_than_max_seqlen_q_writes_nothing_wrong(D):
    # a caller error: max_seqlen_q = 100 below a 300-row segment.  Rows under
    # the bound are computed; every other row is either left as it was or
    # holds its correct value (whole query tiles are computed) -- nothing else.
    inp = gen.prefill_inputs([300, 40], 2, D, seed=11)
    d = to_gpu(inp)
    out = torch.full_like(d["q"], SENTINEL)
    attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"],
                    max_seqlen_q=100, out=out)
    torch.cuda.synchronize()
    o = f64(out)
    ref, ref_abs = refs(inp)
    under = np.r_[0:100, 300:340]
    check(o[under], ref[under], f"rows under the bound D={D}", ref_abs=ref_abs[under])
    rest = o[100:300]
    untouched = np.all(rest == SENTINEL, axis=(1, 2))
    assert untouched.any(), "rows far past the bound were written"
    written = ~untouched
    check(rest[written], ref[100:300][written], f"rows past the bound D={D}",
          ref_abs=ref_abs[100:300][written])


def scaled_check(inp, scale, what):
    d = to_gpu(inp)
    out = attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"],
                          max_seqlen_q=inp["max_seqlen_q"], scale=scale)
    torch.cuda.synchronize()
    args = (inp["cu_seqlens_q"], inp["cu_seqlens_k"])
    ref = oracle.varlen_fwd(inp["q"], inp["k"], inp["v"], *args, scale=scale)
    ref_abs = oracle.varlen_fwd(inp["q"], inp["k"], inp["v"].abs(), *args, scale=scale)
    m = ~np.isnan(ref)
    check(f64(out)[m], ref[m], what, ref_abs=ref_abs[m])


@pytest.mark.parametrize("D", [72, 128])
def test_sharp_attention_with_growing_maxima(D):
    # q x 32 (exact): scores spread over hundreds of log2 units, so the
    # running max grows past the lazy-rescale threshold on many tiles and
    # most weights underflow; keys are ordered so maxima keep rising
    inp = gen.prefill_inputs([700, 90], 2, D, seed=55)
    inp["q"] = (inp["q"].float() * 32).to(torch.bfloat16)
    k = inp["k"].clone()
    norms = k[:700].float().norm(dim=2).sum(dim=1)
    k[:700] = k[:700][torch.argsort(norms)]          # growing key norms in sequence 0
    inp["k"] = k
    full_check(inp, f"sharp D={D}")


@pytest.mark.parametrize("scale", [0.0, -0.3])
@pytest.mark.parametrize("D", [72, 128])
def test_zero_and_negative_scale(D, scale):
    # the definition holds for any finite scale: 0 gives the mean of the
    # segment's values, a negative one favours the least similar keys.  Key
    # lengths leave a partial last key tile, where the kernel masks keys.
    inp = gen.prefill_inputs([100, 37, 200], 2, D, seed=51, seq_lens_k=[70, 129, 5])
    scaled_check(inp, scale, f"scale {scale} D={D}")


@pytest.mark.parametrize("scale", [0.0, -0.3])
def test_zero_and_negative_scale_on_split_items(scale):
    # 2024 tokens x 4 heads: every work item is split into key ranges and merged
    inp = gen.prefill_inputs([2024], 4, 128, seed=53, seq_lens_k=[2000])
    scaled_check(inp, scale, f"scale {scale} split items")


@pytest.mark.parametrize("D", [72, 128])
def test_scaled_values_tighten_the_floor(D):
    # out is linear in V and a power-of-two scale is exact in bf16; with V
    # scaled up the output errors are judged by the scale-free bar 2 only.
    inp = gen.prefill_inputs([1000], 2, D, seed=21, v_scale=64.0)
    full_check(inp, f"V*64 D={D}", bar1=False)


@pytest.mark.parametrize("D", [72, 128])
def test_single_key_returns_value_rows_exactly(D):
    # one key per sequence: softmax weight 1, so out == v bit for bit
    inp = gen.prefill_inputs([50, 3], 4, D, seed=31, seq_lens_k=[1, 1])
    out = run(inp)
    v = inp["v"]
    assert torch.equal(out[:50].cpu(), v[0:1].expand(50, 4, D))
    assert torch.equal(out[50:].cpu(), v[1:2].expand(3, 4, D))


@pytest.mark.parametrize("D,dtype,S", [(72, "bf16", 300), (128, "bf16", 300), (72, "fp16", 300),
                                         (128, "fp16", 300), (72, "bf16", 2100), (128, "bf16", 2100)])
def test_identical_value_rows_return_that_row(D, dtype, S):
    # All keys carry the same value row u, so out = (sum_j p_j) u / sum_j p_j.
    # The row sum adds up the same 16-bit weights that multiply V, so the
    # quotient is u up to fp32 rounding and rounds back to u bit for bit.
    # 2100 tokens x 2 heads is a small grid: every item runs as key ranges
    # merged by log-sum-exp (at head_dim 128 by a second kernel, at 72
    # inside the key-splitting workgroups).
    inp = gen.prefill_inputs([S], 2, D, seed=33, dtype=dtype)
    inp["q"] = (inp["q"].float() * 4).to(inp["q"].dtype)   # weights spread over 2^10 and more
    inp["v"] = inp["v"][7:8].expand(S, 2, D).contiguous()
    print(f"[prefill] identical V rows D={D} {dtype} S={S}", flush=True)
    out = run(inp).cpu()
    assert torch.equal(out, inp["v"])


@pytest.mark.parametrize("D", [72, 128])
def test_no_keys_gives_zero_rows(D):
    inp = gen.prefill_inputs([17], 2, D, seed=35, seq_lens_k=[0])
    out = run(inp)
    assert torch.count_nonzero(out).item() == 0


def test_binding_rejects_host_buffers():
    # every tensor handed to the library must be GPU memory of q's device
    inp = gen.prefill_inputs([20], 2, 128, seed=43)
    d = to_gpu(inp)
    args = (d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"])
    with pytest.raises(ValueError):
        attn_varlen_fwd(*args, max_seqlen_q=20, workspace=torch.empty(16, dtype=torch.uint8))
    with pytest.raises(ValueError):
        attn_varlen_fwd(*args, max_seqlen_q=20, out=torch.empty_like(inp["q"]))
    with pytest.raises(ValueError):
        attn_varlen_fwd(d["q"], inp["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"],
                        max_seqlen_q=20)
    # and of the right type, layout and shape
    with pytest.raises(TypeError, match="v has dtype"):
        attn_varlen_fwd(d["q"], d["k"], d["v"].half(), d["cu_seqlens_q"], d["cu_seqlens_k"],
                        max_seqlen_q=20)
    with pytest.raises(ValueError, match="k must be contiguous"):
        kt = d["k"].transpose(0, 1).contiguous().transpose(0, 1)
        attn_varlen_fwd(d["q"], kt, d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"], max_seqlen_q=20)
    with pytest.raises(TypeError, match="cu_seqlens_k has dtype"):
        attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"].long(),
                        max_seqlen_q=20)
    with pytest.raises(TypeError, match="out has dtype"):
        attn_varlen_fwd(*args, max_seqlen_q=20, out=d["q"].float())
    with pytest.raises(ValueError, match="out must have q's shape"):
        attn_varlen_fwd(*args, max_seqlen_q=20, out=d["q"][:10])
    with pytest.raises(ValueError, match="k and v must be"):
        attn_varlen_fwd(d["q"], d["k"][:, :1].contiguous(), d["v"][:, :1].contiguous(),
                        d["cu_seqlens_q"], d["cu_seqlens_k"], max_seqlen_q=20)


def test_runs_are_bitwise_deterministic():
    inp = gen.prefill_inputs([777], 4, 128, seed=41)
    a = run(inp).cpu()
    b = run(inp).cpu()
    assert torch.equal(a, b)


def run_nan_filled(inp):
    """The call with `out` filled with NaN first, so a row no work item
    writes stays NaN and fails the finiteness checks."""
    d = to_gpu(inp)
    out = torch.full_like(d["q"], float("nan"))
    attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"],
                    max_seqlen_q=inp["max_seqlen_q"], out=out)
    torch.cuda.synchronize()
    return out


def oracle_at(inp, rows, heads):
    """Oracle output and |v|-weighted magnitude at (row, head) pairs of a
    single-sequence input, evaluated head by head: each head's chosen query
    rows form one query segment against all of the sequence's keys, which is
    the definition for those rows (query and key lengths may differ)."""
    assert inp["cu_seqlens_q"].numel() == 2, "single-sequence inputs only"
    rows, heads = np.asarray(rows, dtype=np.int64), np.asarray(heads, dtype=np.int64)
    D = inp["q"].shape[2]
    ref = np.empty((rows.size, D))
    ref_abs = np.empty((rows.size, D))
    for h in np.unique(heads):
        sel = np.nonzero(heads == h)[0]
        r = torch.from_numpy(rows[sel])
        q = inp["q"][r, h:h + 1].contiguous()
        k = inp["k"][:, h:h + 1].contiguous()
        v = inp["v"][:, h:h + 1].contiguous()
        cu_q = torch.tensor([0, sel.size], dtype=torch.int32)
        o, a = oracle.varlen_fwd(q, k, v, cu_q, inp["cu_seqlens_k"], return_abs=True)
        ref[sel], ref_abs[sel] = o[:, 0], a[:, 0]
    return ref, ref_abs


def rows_of_every_tile(S, H, tile, seed, extra_last=True):
    """One seeded random query row from every (head, tile of `tile` rows),
    plus the first and last rows of the last, partial tile of every head."""
    rng = np.random.default_rng(seed)
    nt = (S + tile - 1) // tile
    rows, heads = [], []
    for h in range(H):
        for t in range(nt):
            rows.append(int(rng.integers(t * tile, min(S, (t + 1) * tile))))
            heads.append(h)
        if extra_last:
            rows += [(nt - 1) * tile, S - 1]
            heads += [h, h]
    return np.array(rows), np.array(heads)


def every_item_check(name, tile, seed, inp=None):
    inp = gen.workload_inputs(name) if inp is None else inp
    S, H, _ = inp["q"].shape
    print(f"[prefill] workload {name}: every work item", flush=True)
    out = run_nan_filled(inp)
    # every element lies inside the one segment: all must have been written
    assert bool(torch.isfinite(out).all()), f"{name}: rows left unwritten or non-finite"
    rows, heads = rows_of_every_tile(S, H, tile, seed)
    ref, ref_abs = oracle_at(inp, rows, heads)
    got = f64(out[torch.from_numpy(rows).cuda(), torch.from_numpy(heads).cuda()])
    check(got, ref, f"{name}: one row per {tile}-row tile", ref_abs=ref_abs)
    return inp, out


def test_workload_s276_h4_d72_full():
    full_check(gen.workload_inputs("prefill_s276_h4_d72"), "prefill_s276_h4_d72")


def test_workload_s8136_h16_d72_every_element():
    # 16 heads x 8136 rows at head_dim 72 (one wave of 512 items of 256 rows,
    # 64 query rows per wave), every output element against the oracle
    name = "prefill_s8136_h16_d72"
    inp = gen.workload_inputs(name)
    print(f"[prefill] workload {name}: every element", flush=True)
    out = run_nan_filled(inp)
    ref, ref_abs = oracle.varlen_fwd(inp["q"], inp["k"], inp["v"], inp["cu_seqlens_q"],
                                     inp["cu_seqlens_k"], return_abs=True)
    check(f64(out), ref, name, ref_abs=ref_abs)


def test_workload_s16742_h32_d128_every_element():
    # 66 query tiles x 32 heads = 2112 work items of 256 rows on 512 resident
    # workgroups: 4 full waves, and the last 64 items (head 31, query tiles
    # 2..65) run as key ranges merged by log-sum-exp.  Every output element
    # against the oracle (about 40 s of the oracle on 16 cores).
    name = "prefill_s16742_h32_d128"
    inp = gen.workload_inputs(name)
    print(f"[prefill] workload {name}: every element", flush=True)
    out = run_nan_filled(inp)
    ref, ref_abs = oracle.varlen_fwd(inp["q"], inp["k"], inp["v"], inp["cu_seqlens_q"],
                                     inp["cu_seqlens_k"], return_abs=True)
    check(f64(out), ref, name, ref_abs=ref_abs)


def test_workload_s65556_h16_d72_every_work_item():
    # 257 tiles of 256 rows x 16 heads = 4112 items of 64-row waves (512
    # resident workgroups): 8 full waves, and the last 16 items (head 15)
    # split into key ranges.  One row from every 128-row half of every item.
    every_item_check("prefill_s65556_h16_d72", 128, seed=13)


def test_largest_shapes_row_s30793_h32_d128_every_work_item():
    # the largest head_dim-128 row of the page's Shapes table (row 10):
    # 121 query tiles of 256 rows x 32 heads = 3872 work items: 7 full waves
    # of 512 and a last wave of 288 (split into key ranges where that
    # finishes it sooner); every element written and finite, one row of
    # every 256-row tile of every head against the oracle
    inp = gen.prefill_inputs([30793], 32, 128, seed=2010)
    every_item_check("prefill_s30793_h32_d128", 256, seed=14, inp=inp)


@pytest.mark.parametrize("D", [72, 128])
@pytest.mark.parametrize("Sk", [1, 17, 38, 300])
def test_keys_past_the_last_segment_are_never_read(D, Sk):
    # k and v are the leading rows of buffers whose further rows hold NaN: a
    # tile load that reached past the last key would pull NaN into the
    # product (0 weight times NaN is NaN).  Key lengths leave a partial last
    # key tile and a partial 4-row DMA group; a second sequence ends there.
    H = 3
    for lens_q, lens_k in (([50], [Sk]), ([20, 33], [64, Sk])):
        inp = gen.prefill_inputs(lens_q, H, D, seed=90 + Sk, seq_lens_k=lens_k)
        tk = inp["k"].shape[0]
        d = to_gpu(inp)
        kb = torch.full((tk + 80, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        vb = torch.full((tk + 80, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        kb[:tk] = d["k"]
        vb[:tk] = d["v"]
        out = torch.full_like(d["q"], float("nan"))
        attn_varlen_fwd(d["q"], kb[:tk], vb[:tk], d["cu_seqlens_q"], d["cu_seqlens_k"],
                        max_seqlen_q=inp["max_seqlen_q"], out=out)
        torch.cuda.synchronize()
        ref, ref_abs = refs(inp)
        check(f64(out), ref, f"NaN past the keys D={D} Sk={Sk} {lens_k}", ref_abs=ref_abs)


def test_many_sequences_of_random_lengths():
    # 40 sequences, query lengths 0..700 and key lengths 0..900: most query
    # tiles of the grid (sized by the longest sequence) exit at once
    rng = np.random.default_rng(5)
    lq = [int(x) for x in rng.integers(0, 701, 40)]
    lk = [int(x) for x in rng.integers(0, 901, 40)]
    lq[3], lk[3] = 700, 900
    inp = gen.prefill_inputs(lq, 2, 128, seed=61, seq_lens_k=lk)
    full_check(inp, "40 sequences")


def test_varlen_batch_with_split_tail():
    # 3 sequences x 4 heads, up to 16 query tiles of 256 rows: 192 items,
    # under half of the 512 resident workgroups, so every item is split into
    # key ranges, each over its own sequence's keys
    from softmax_attention_flashattention_amd import attn_varlen_fwd_workspace_size
    lens = [3000, 1500, 4096]
    inp = gen.prefill_inputs(lens, 4, 128, seed=62, seq_lens_k=[2500, 4100, 4096])
    assert attn_varlen_fwd_workspace_size(3, 4096, 4, 128) > 0
    d = to_gpu(inp)
    print("[prefill] varlen batch, split tail", flush=True)
    split = attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"],
                            max_seqlen_q=4096)
    whole = attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"],
                            max_seqlen_q=4096,
                            workspace=torch.empty(0, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    starts = np.cumsum([0] + lens)
    rows = np.concatenate([starts[i] + np.concatenate([[0, lens[i] - 1], rng.integers(0, lens[i], 20)])
                           for i in range(3)])
    heads = rng.integers(0, 4, rows.size)
    args = (inp["cu_seqlens_q"], inp["cu_seqlens_k"], rows, heads)
    ref = oracle.varlen_fwd_rows(inp["q"], inp["k"], inp["v"], *args)
    ref_abs = oracle.varlen_fwd_rows(inp["q"], inp["k"], inp["v"].abs(), *args)
    idx = (torch.from_numpy(rows).cuda(), torch.from_numpy(heads).cuda())
    check(f64(split[idx]), ref, "varlen split", ref_abs=ref_abs)
    check(f64(split), f64(whole), "varlen split vs whole")


@pytest.mark.parametrize("D", [72, 128])
def test_split_last_wave_matches_whole_items(D):
    # 516 heads x 300 rows: two query tiles of 256 rows, so two full waves of
    # 512 workgroups plus 8 items, which the library splits into key ranges
    # (10 key tiles of 32 rows over up to 8 ranges) and merges
    from softmax_attention_flashattention_amd import attn_varlen_fwd_workspace_size
    inp = gen.prefill_inputs([300], 516, D, seed=77)
    assert attn_varlen_fwd_workspace_size(1, 300, 516, D) > 0
    d = to_gpu(inp)
    split = attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"],
                            max_seqlen_q=300)
    whole = attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"],
                            max_seqlen_q=300,
                            workspace=torch.empty(0, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    rows = rng.integers(0, 300, 64)
    heads = np.concatenate([rng.integers(0, 516, 32), rng.integers(508, 516, 32)])
    args = (inp["cu_seqlens_q"], inp["cu_seqlens_k"], rows, heads)
    ref = oracle.varlen_fwd_rows(inp["q"], inp["k"], inp["v"], *args)
    ref_abs = oracle.varlen_fwd_rows(inp["q"], inp["k"], inp["v"].abs(), *args)
    idx = (torch.from_numpy(rows).cuda(), torch.from_numpy(heads).cuda())
    check(f64(split[idx]), ref, f"split D={D}", ref_abs=ref_abs)
    check(f64(whole[idx]), ref, f"whole D={D}", ref_abs=ref_abs)
    check(f64(split), f64(whole), f"split vs whole D={D}")


@pytest.mark.parametrize("S,H", [(5888, 12), (33024, 2)])
def test_head_dim_72_items_with_a_split_last_wave(S, H):
    # 5888 tokens x 12 heads: 276 work items of 256 query rows, enough to fill
    # the 256 resident 8-wave workgroups of 32-row waves (too few for the
    # 64-row waves' 512, and the sequences are short), so one full wave plus
    # 20 items, which are split into key ranges and merged.  33024 tokens x 2
    # heads: 258 items of 64-row waves (long sequences take them on any grid),
    # a more-than-half-full single wave whose items are split into ranges.
    from softmax_attention_flashattention_amd import attn_varlen_fwd_workspace_size
    D = 72
    inp = gen.prefill_inputs([S], H, D, seed=79)
    assert attn_varlen_fwd_workspace_size(1, S, H, D) > 0
    d = to_gpu(inp)
    split = attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"],
                            max_seqlen_q=S)
    whole = attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"],
                            max_seqlen_q=S,
                            workspace=torch.empty(0, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = np.concatenate([[0, 255, 256, S - 257, S - 256, S - 1], rng.integers(0, S, 40),
                           rng.integers(S - 512, S, 16)])
    heads = rng.integers(0, H, rows.size)
    args = (inp["cu_seqlens_q"], inp["cu_seqlens_k"], rows, heads)
    ref = oracle.varlen_fwd_rows(inp["q"], inp["k"], inp["v"], *args)
    ref_abs = oracle.varlen_fwd_rows(inp["q"], inp["k"], inp["v"].abs(), *args)
    idx = (torch.from_numpy(rows).cuda(), torch.from_numpy(heads).cuda())
    check(f64(split[idx]), ref, f"{S}x{H} split", ref_abs=ref_abs)
    check(f64(whole[idx]), ref, f"{S}x{H} whole", ref_abs=ref_abs)
    check(f64(split), f64(whole), f"{S}x{H} split vs whole")


@pytest.mark.parametrize("D", [72, 128])
def test_fp16_on_a_device_filling_grid(D):
    # 8136 tokens x 16 heads in fp16: exactly one wave of 512 items of 256
    # rows, with 64 query rows per wave at either head_dim
    S, H = 8136, 16
    inp = gen.prefill_inputs([S], H, D, seed=81, dtype="fp16")
    out = run(inp)
    rng = np.random.default_rng(9)
    rows = np.concatenate([[0, S - 1, (S // 256) * 256, (S // 128) * 128], rng.integers(0, S, 60)])
    heads = rng.integers(0, H, rows.size)
    args = (inp["cu_seqlens_q"], inp["cu_seqlens_k"], rows, heads)
    ref = oracle.varlen_fwd_rows(inp["q"], inp["k"], inp["v"], *args)
    ref_abs = oracle.varlen_fwd_rows(inp["q"], inp["k"], inp["v"].abs(), *args)
    got = f64(out[torch.from_numpy(rows).cuda(), torch.from_numpy(heads).cuda()])
    check(got, ref, f"fp16 {S}x{H} D={D}", ref_abs=ref_abs)


@pytest.mark.parametrize("D", [72, 128])
def test_small_grid_splits_every_item(D):
    # far fewer work items than the device holds, so every item is split into
    # key ranges and merged: head_dim 128, 8 query tiles of 256 rows x 4
    # heads; head_dim 72, 16 tiles of 128 rows x 10 heads (with 4 heads the
    # 32-row items of the key-splitting workgroups would all fit at once,
    # and those need no merge)
    from softmax_attention_flashattention_amd import attn_varlen_fwd_workspace_size
    H = 10 if D == 72 else 4
    inp = gen.prefill_inputs([2024], H, D, seed=78)
    assert attn_varlen_fwd_workspace_size(1, 2024, H, D) > 0
    d = to_gpu(inp)
    print(f"[prefill] small grid split D={D}", flush=True)
    split = attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"],
                            max_seqlen_q=2024)
    whole = attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"],
                            max_seqlen_q=2024,
                            workspace=torch.empty(0, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    ref = oracle.varlen_fwd(inp["q"], inp["k"], inp["v"], inp["cu_seqlens_q"], inp["cu_seqlens_k"])
    ref_abs = oracle.varlen_fwd(inp["q"], inp["k"], inp["v"].abs(), inp["cu_seqlens_q"],
                                inp["cu_seqlens_k"])
    check(f64(split), ref, f"small grid split D={D}", ref_abs=ref_abs)
    check(f64(split), f64(whole), f"small grid split vs whole D={D}")


@pytest.mark.parametrize("H", [52, 20])
def test_more_than_half_full_wave_is_split(H):
    # 16 query tiles of 256 rows (head_dim 128) x H heads at 64 key tiles of
    # 64 rows: with 512 resident workgroups, 52 heads leave 320 items for a
    # second wave and 20 heads make one wave of 320; either tail is split
    # into the number of key ranges that finishes it soonest (3 here) and
    # merged
    from softmax_attention_flashattention_amd import attn_varlen_fwd_workspace_size
    S = 4096
    inp = gen.prefill_inputs([S], H, 128, seed=80 + H)
    assert attn_varlen_fwd_workspace_size(1, S, H, 128) > 0
    d = to_gpu(inp)
    print(f"[prefill] tail split, {H} heads", flush=True)
    split = attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"],
                            max_seqlen_q=S)
    whole = attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"],
                            max_seqlen_q=S,
                            workspace=torch.empty(0, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    rng = np.random.default_rng(H)
    rows = np.concatenate([[0, S - 1], rng.integers(0, S, 62)])
    heads = np.concatenate([[H - 1, H - 1], rng.integers(0, H, 62)])
    args = (inp["cu_seqlens_q"], inp["cu_seqlens_k"], rows, heads)
    ref = oracle.varlen_fwd_rows(inp["q"], inp["k"], inp["v"], *args)
    ref_abs = oracle.varlen_fwd_rows(inp["q"], inp["k"], inp["v"].abs(), *args)
    idx = (torch.from_numpy(rows).cuda(), torch.from_numpy(heads).cuda())
    check(f64(split[idx]), ref, f"tail split H={H}", ref_abs=ref_abs)
    check(f64(split), f64(whole), f"tail split vs whole H={H}")


def test_small_grid_split_with_uneven_key_lengths():
    # the split count is estimated from the query lengths; a sequence with
    # many more keys, and one with fewer key tiles than ranges, stay exact
    from softmax_attention_flashattention_amd import attn_varlen_fwd_workspace_size
    inp = gen.prefill_inputs([600, 1100], 2, 128, seed=79, seq_lens_k=[4000, 7])
    assert attn_varlen_fwd_workspace_size(2, 1100, 2, 128) > 0
    d = to_gpu(inp)
    print("[prefill] small grid split, uneven keys", flush=True)
    out = attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"],
                          max_seqlen_q=1100)
    torch.cuda.synchronize()
    ref = oracle.varlen_fwd(inp["q"], inp["k"], inp["v"], inp["cu_seqlens_q"], inp["cu_seqlens_k"])
    ref_abs = oracle.varlen_fwd(inp["q"], inp["k"], inp["v"].abs(), inp["cu_seqlens_q"],
                                inp["cu_seqlens_k"])
    check(f64(out), ref, "uneven keys", ref_abs=ref_abs)


# ---- head_dim 72 with 64 query rows per wave (prefill_fwd_d72_kernel): the
# library takes it when the 256-row work items fill the device's 512
# resident workgroups at least once, so these cases use enough heads for that.

def wide_heads(max_len):
    """Heads that make at least 512 work items of 256 query rows."""
    return -(-512 // -(-max_len // 256))


@pytest.mark.parametrize("S", [1, 17, 31, 32, 33, 255, 256, 257, 300])
def test_d72_64_row_waves_single_sequence_lengths(S):
    H = wide_heads(S)
    full_check(gen.prefill_inputs([S], H, 72, seed=600 + S), f"64-row waves S={S} H={H}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_d72_64_row_waves_varlen_batch(dtype):
    # an empty query segment, S_q != S_k, a sequence with no keys, ragged tiles
    inp = gen.prefill_inputs([5, 0, 300, 64, 129, 1], 48, 72, seed=607, dtype=dtype,
                             seq_lens_k=[7, 3, 250, 0, 129, 200])
    full_check(inp, f"64-row waves varlen {dtype}")


@pytest.mark.parametrize("scale", [0.0, -0.3])
def test_d72_64_row_waves_zero_and_negative_scale(scale):
    inp = gen.prefill_inputs([100, 37, 200], 176, 72, seed=651, seq_lens_k=[70, 129, 5])
    scaled_check(inp, scale, f"64-row waves scale {scale}")


def test_d72_64_row_waves_sharp_attention():
    # rising maxima: the rescale branch on many tiles
    inp = gen.prefill_inputs([700, 90], 96, 72, seed=655)
    inp["q"] = (inp["q"].float() * 32).to(torch.bfloat16)
    k = inp["k"].clone()
    norms = k[:700].float().norm(dim=2).sum(dim=1)
    k[:700] = k[:700][torch.argsort(norms)]
    inp["k"] = k
    full_check(inp, "64-row waves sharp")


@pytest.mark.parametrize("Sk", [1, 17, 38, 300])
def test_d72_64_row_waves_never_read_past_the_keys(Sk):
    H = 256
    inp = gen.prefill_inputs([20, 300], H, 72, seed=690 + Sk, seq_lens_k=[64, Sk])
    tk = inp["k"].shape[0]
    d = to_gpu(inp)
    kb = torch.full((tk + 80, H, 72), float("nan"), dtype=torch.bfloat16, device="cuda")
    vb = torch.full((tk + 80, H, 72), float("nan"), dtype=torch.bfloat16, device="cuda")
    kb[:tk] = d["k"]
    vb[:tk] = d["v"]
    out = torch.full_like(d["q"], float("nan"))
    attn_varlen_fwd(d["q"], kb[:tk], vb[:tk], d["cu_seqlens_q"], d["cu_seqlens_k"],
                    max_seqlen_q=inp["max_seqlen_q"], out=out)
    torch.cuda.synchronize()
    ref, ref_abs = refs(inp)
    check(f64(out), ref, f"64-row waves, NaN past the keys Sk={Sk}", ref_abs=ref_abs)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_d72_64_row_waves_identical_value_rows(dtype):
    S, H = 300, 256
    inp = gen.prefill_inputs([S], H, 72, seed=633, dtype=dtype)
    inp["q"] = (inp["q"].float() * 4).to(inp["q"].dtype)
    inp["v"] = inp["v"][7:8].expand(S, H, 72).contiguous()
    out = run(inp).cpu()
    assert torch.equal(out, inp["v"])


def test_d72_64_row_waves_rows_outside_segments_untouched():
    inp = gen.prefill_inputs([40, 300], 256, 72, seed=609)
    pad = torch.zeros(30, 256, 72, dtype=torch.bfloat16)
    inp["q"] = torch.cat([inp["q"], pad])
    d = to_gpu(inp)
    out = torch.full_like(d["q"], SENTINEL)
    attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"],
                    max_seqlen_q=300, out=out)
    torch.cuda.synchronize()
    o = f64(out)
    assert np.all(o[340:] == SENTINEL)
    ref, ref_abs = refs(inp)
    check(o[:340], ref[:340], "64-row waves sentinel", ref_abs=ref_abs[:340])


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_d72_64_row_waves_random_batches(seed):
    # random varlen batches (empty segments, S_q != S_k, ragged tiles), bf16
    # or fp16, a scale of either sign, with enough heads for the 64-row waves;
    # every element against the oracle
    rng = np.random.default_rng(700 + seed)
    n = int(rng.integers(1, 7))
    lq = [int(x) for x in rng.integers(0, 701, n)]
    lk = [int(x) for x in rng.integers(0, 901, n)]
    lq[0] = max(lq[0], 1)
    H = wide_heads(max(lq)) // n + 1
    dtype = "fp16" if seed % 2 else "bf16"
    scale = float(rng.choice([-1.0, 1.0]) * rng.uniform(0.05, 0.2))
    inp = gen.prefill_inputs(lq, H, 72, seed=710 + seed, dtype=dtype, seq_lens_k=lk)
    scaled_check(inp, scale, f"64-row waves random batch {seed}: {n} seqs, {H} heads, {dtype}, scale {scale:.3f}")


# ---- head_dim 72 on small grids (prefill_fwd_split_kernel): the library
# takes it when the items of 32 query rows all fit the device at once (512
# resident workgroups) and max_seqlen_q <= 8192.  Each of a workgroup's 4
# waves walks a quarter of the key tiles; the quarters are merged in LDS.
# The short cases earlier in this file (2-3 heads) run here too: they cover
# wave ranges left empty (fewer than 4 key tiles), sequences without keys,
# both dtypes, scale 0 and negative scales.

def test_split_kernel_long_single_sequence():
    # 8192 tokens x 1 head: 256 items whose waves walk 64 key tiles each (the
    # steady-state loop); every element written, one row of every 32-row
    # item and the first and last rows against the oracle
    S = 8192
    inp = gen.prefill_inputs([S], 1, 72, seed=820)
    print("[prefill] key-splitting workgroups, 8192 x 1", flush=True)
    out = run_nan_filled(inp)
    assert bool(torch.isfinite(out).all())
    rows, heads = rows_of_every_tile(S, 1, 32, seed=821)
    ref, ref_abs = oracle_at(inp, rows, heads)
    got = f64(out[torch.from_numpy(rows).cuda(), torch.from_numpy(heads).cuda()])
    check(got, ref, "8192 x 1: one row per 32-row item", ref_abs=ref_abs)


@pytest.mark.parametrize("S", [1024, 1025])
def test_split_kernel_slot_boundary(S):
    # 1024 tokens x 16 heads make exactly 512 items of 32 rows (the
    # key-splitting workgroups); 1025 make 528, which run on the 32-row waves
    # with key ranges merged by a second kernel.  Both against the oracle on
    # one row of every 32-row tile of every head.
    H = 16
    inp = gen.prefill_inputs([S], H, 72, seed=830 + S)
    print(f"[prefill] slot boundary {S} x {H}", flush=True)
    out = run_nan_filled(inp)
    assert bool(torch.isfinite(out).all())
    rows, heads = rows_of_every_tile(S, H, 32, seed=S)
    ref, ref_abs = oracle_at(inp, rows, heads)
    got = f64(out[torch.from_numpy(rows).cuda(), torch.from_numpy(heads).cuda()])
    check(got, ref, f"{S} x {H}", ref_abs=ref_abs)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_split_kernel_varlen_batch_uneven_ranges(dtype):
    # sequences whose key counts leave 0-3 of a workgroup's 4 wave ranges
    # empty, one with no keys, one with no queries, one with far more keys
    # than queries (long ranges), a negative scale; every element
    lq = [33, 1, 0, 90, 200, 31]
    lk = [40, 0, 7, 95, 2100, 3]
    inp = gen.prefill_inputs(lq, 3, 72, seed=840, dtype=dtype, seq_lens_k=lk)
    scaled_check(inp, -0.15, f"key-splitting workgroups, uneven ranges, {dtype}")


# ---- head_dim 72 on the 32-row waves (prefill_fwd_kernel<72, T, 4>): grids
# with more than 512 items of 32 rows but fewer than 256 of 256 rows.  These
# cases use enough heads for that and otherwise mirror the edge cases above.

@pytest.mark.parametrize("S", [257, 300, 511])
def test_d72_32_row_waves_single_sequence_lengths(S):
    full_check(gen.prefill_inputs([S], 64, 72, seed=860 + S), f"32-row waves S={S} H=64")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_d72_32_row_waves_varlen_batch(dtype):
    inp = gen.prefill_inputs([5, 0, 300, 64, 129, 1], 12, 72, seed=867, dtype=dtype,
                             seq_lens_k=[9, 4, 300, 1, 200, 64])
    full_check(inp, f"32-row waves varlen {dtype}")


@pytest.mark.parametrize("Sk", [1, 17, 38, 300])
def test_d72_32_row_waves_keys_past_the_segment_are_never_read(Sk):
    H = 64
    inp = gen.prefill_inputs([300], H, 72, seed=870 + Sk, seq_lens_k=[Sk])
    tk = inp["k"].shape[0]
    d = to_gpu(inp)
    kb = torch.full((tk + 80, H, 72), float("nan"), dtype=torch.bfloat16, device="cuda")
    vb = torch.full((tk + 80, H, 72), float("nan"), dtype=torch.bfloat16, device="cuda")
    kb[:tk] = d["k"]
    vb[:tk] = d["v"]
    out = torch.full_like(d["q"], float("nan"))
    attn_varlen_fwd(d["q"], kb[:tk], vb[:tk], d["cu_seqlens_q"], d["cu_seqlens_k"],
                    max_seqlen_q=300, out=out)
    torch.cuda.synchronize()
    ref, ref_abs = refs(inp)
    check(f64(out), ref, f"32-row waves, NaN past the keys Sk={Sk}", ref_abs=ref_abs)


def test_d72_32_row_waves_identical_value_rows():
    S, H = 300, 64
    inp = gen.prefill_inputs([S], H, 72, seed=875)
    inp["q"] = (inp["q"].float() * 4).to(inp["q"].dtype)
    inp["v"] = inp["v"][7:8].expand(S, H, 72).contiguous()
    out = run(inp).cpu()
    assert torch.equal(out, inp["v"])


def test_d72_32_row_waves_rows_outside_segments_untouched():
    inp = gen.prefill_inputs([40, 300], 32, 72, seed=877)
    pad = torch.zeros(30, 32, 72, dtype=torch.bfloat16)
    inp["q"] = torch.cat([inp["q"], pad])
    d = to_gpu(inp)
    out = torch.full_like(d["q"], SENTINEL)
    attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"],
                    max_seqlen_q=300, out=out)
    torch.cuda.synchronize()
    o = f64(out)
    assert np.all(o[340:] == SENTINEL)
    ref, ref_abs = refs(inp)
    check(o[:340], ref[:340], "32-row waves sentinel", ref_abs=ref_abs[:340])
