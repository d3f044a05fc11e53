"""Seeded random paged-decode batches through attn_paged_decode, every element
against the oracle ("paged_attention_decode" #024, Reference Implementation).

Each case draws from its seed the batch (1-200 sequences with ragged and
empty contexts of up to 3000 tokens), the KV and query head counts (query
heads per KV head 1-16), the head size, the 16-bit type, the scale, the
partition size (the library's own choice or 16-512 tokens) and a random
placement of the cache blocks, so the cases land on every combination of
context split, query-head dealing (fewer sequence x KV head x partition
units than compute units) and the device-filling grids that keep each KV
head's query heads together.  The output is filled with NaN first, so a
row no workgroup writes fails the finiteness check.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import check, f64, to_gpu
from softmax_attention_flashattention_amd import attn_paged_decode, inputs as gen

pytestmark = pytest.mark.gpu


def draw(seed):
    rng = np.random.default_rng(5000 + seed)
    big = seed % 4 == 3                          # a quarter of the cases fill the device
    S = int(rng.integers(64, 201)) if big else int(rng.integers(1, 9))
    Hkv = int(rng.choice([1, 2, 4, 8, 16] if big else [1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
    D = int(rng.choice([128, 256]))
    ctx = int(rng.choice([16, 100, 700]) if big else rng.choice([1, 64, 128, 700, 3000]))
    lens = [int(x) for x in rng.integers(0, ctx + 1, S)]
    lens[0] = ctx
    if S > 2:
        lens[1] = 0                              # an empty context: zero rows
    dtype = "fp16" if rng.random() < 0.3 else "bf16"
    scale = [D ** -0.5, float(rng.uniform(0.02, 0.2)), -float(rng.uniform(0.02, 0.1))][int(rng.integers(0, 3))]
    ps = int(rng.choice([0, 0, 16, 32, 64, 128, 256, 512]))
    return S, Hkv, G, D, lens, dtype, scale, ps


@pytest.mark.parametrize("seed", range(24))
def test_random_decode_batches(seed):
    S, Hkv, G, D, lens, dtype, scale, ps = draw(seed)
    what = (f"random decode {seed}: {S} seqs, contexts up to {max(lens)}, {G * Hkv}/{Hkv} heads, "
            f"D {D}, {dtype}, scale {scale:.3f}, partition {ps or 'auto'}")
    inp = gen.decode_inputs(S, max(lens), G * Hkv, Hkv, D, seed=6000 + seed, dtype=dtype, seq_lens=lens)
    inp = gen.permute_blocks(inp, seed=7000 + seed)
    print(f"[decode] {what}", flush=True)
    d = to_gpu(inp)
    out = torch.full_like(d["query"], float("nan"))
    attn_paged_decode(d["query"], d["k_cache"], d["v_cache"], d["block_tables"], d["seq_lens"],
                      scale=scale, out=out, partition_size=ps)
    torch.cuda.synchronize()
    args = (inp["query"], inp["k_cache"], inp["v_cache"], inp["block_tables"], inp["seq_lens"])
    ref = oracle.paged_decode(*args, scale=scale)
    ref_abs = oracle.paged_decode(inp["query"], inp["k_cache"], inp["v_cache"].abs(), inp["block_tables"],
                                  inp["seq_lens"], scale=scale)
    check(f64(out), ref, what, ref_abs=ref_abs)
    empty = np.array(lens) <= 0
    if empty.any():
        assert torch.count_nonzero(out[torch.from_numpy(empty).to(out.device)]).item() == 0, what
