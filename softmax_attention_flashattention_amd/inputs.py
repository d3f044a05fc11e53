"""Seeded synthetic inputs shaped like the operator pages' workloads.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic, so the GPU path and the CPU oracle can both be fed from
it without sharing any of the method.

Distributions and layouts follow the pages' input generators (atrex-bench
"attention_forward" #001 and "paged_attention_decode" #024, Input Generation):
i.i.d. standard-normal q, k, v in bfloat16 packed ``[tokens, heads, dim]`` with
equal query and key boundaries; for decode a standard-normal query, K cache
``[num_blocks, kv_heads, head_size/x, block_size, x]`` (x = 16 bytes per
element size), V cache ``[num_blocks, kv_heads, head_size, block_size]``,
``num_blocks = max_blocks_per_seq * num_seqs + 16`` spare blocks, an
identity-ordered block table ``bt[i][j] = i * max_blocks_per_seq + j`` and
every ``seq_lens`` entry equal to ``ctx_len``.

For the chunked delta-rule output ("chunk_delta_rule_output" #004, Input
Generation): q ~ 0.02 N(0, 1) ``[batch, tokens, q_heads, key_dim]``, k ~ N(0, 1)
of q's shape (the page draws it with randn_like, unscaled), v ~ 0.02 N(0, 1)
``[batch, tokens, heads, value_dim]``, h ~ 0.02 N(0, 1) ``[batch, chunks,
heads, key_dim, value_dim]`` and float32 g = -U[0, 1) ``[batch, tokens,
heads]``.

The pages draw without a seed on the device; here every tensor is drawn on the
CPU from ``torch.Generator().manual_seed(seed)`` in float32, in the pages'
order (q, k, v; query, k_cache, v_cache; q, k, v, h, g) and rounded to the
16-bit type with round-to-nearest-even (a scaled draw is rounded, scaled in
float32 and rounded again, as the page's 16-bit multiply does), so the oracle
and the GPU see the same bits.
"""
import torch

_DT = {"bf16": torch.bfloat16, "fp16": torch.float16}

# The five workloads the benchmark and the parity tests are built around,
# named by what they are.  Sizes come from the pages' Shapes tables:
# "attention_forward" rows 11, 4, 9 and 8 and "paged_attention_decode" row 0.
WORKLOADS = {
    "prefill_s276_h4_d72": dict(kind="prefill", seq_lens=[276], num_heads=4, head_dim=72,
                                seed=1001),
    "prefill_s8136_h16_d72": dict(kind="prefill", seq_lens=[8136], num_heads=16, head_dim=72,
                                  seed=1002),
    "prefill_s16742_h32_d128": dict(kind="prefill", seq_lens=[16742], num_heads=32,
                                    head_dim=128, seed=1003),
    "decode_b256_ctx64_h16_kv16_d128": dict(kind="decode", num_seqs=256, ctx_len=64,
                                            num_query_heads=16, num_kv_heads=16,
                                            head_size=128, block_size=16, dtype="bf16",
                                            seed=1004),
    "prefill_s65556_h16_d72": dict(kind="prefill", seq_lens=[65556], num_heads=16, head_dim=72,
                                   seed=1005),
}

# Chunked delta-rule output workloads: rows 15, 13, 8 and 0 of the
# "chunk_delta_rule_output" Shapes table (chunk 64, key_dim = value_dim = 128).
CHUNK_WORKLOADS = {
    "chunk_t14807_h32_hq16": dict(batch=1, tokens=14807, num_q_heads=16, num_heads=32, seed=1006),
    "chunk_t4195_h32_hq16": dict(batch=1, tokens=4195, num_q_heads=16, num_heads=32, seed=1007),
    "chunk_t704_h16_hq8": dict(batch=1, tokens=704, num_q_heads=8, num_heads=16, seed=1008),
    "chunk_t64_h32_hq16": dict(batch=1, tokens=64, num_q_heads=16, num_heads=32, seed=1009),
}


def _randn(gen, shape, dtype):
    return torch.randn(*shape, generator=gen, dtype=torch.float32).to(_DT[dtype])


def _cumsum_i32(lens):
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + int(n))
    return torch.tensor(cu, dtype=torch.int32)


def prefill_inputs(seq_lens, num_heads, head_dim, seed, dtype="bf16", seq_lens_k=None,
                   v_scale=1.0):
    """q, k, v [total, H, D] and cu_seqlens_q/k [num_seqs + 1] (int32), on the CPU.

    ``seq_lens_k`` (default: ``seq_lens``) gives key lengths that differ from
    the query lengths; ``v_scale`` multiplies v by a power of two (exact).
    """
    seq_lens_k = list(seq_lens) if seq_lens_k is None else list(seq_lens_k)
    if len(seq_lens_k) != len(seq_lens):
        raise ValueError("seq_lens and seq_lens_k must have one entry per sequence")
    gen = torch.Generator().manual_seed(int(seed))
    tq, tk = sum(seq_lens), sum(seq_lens_k)
    q = _randn(gen, (tq, num_heads, head_dim), dtype)
    k = _randn(gen, (tk, num_heads, head_dim), dtype)
    v = _randn(gen, (tk, num_heads, head_dim), dtype)
    if v_scale != 1.0:
        v = (v.float() * v_scale).to(_DT[dtype])
    return {"q": q, "k": k, "v": v,
            "cu_seqlens_q": _cumsum_i32(seq_lens), "cu_seqlens_k": _cumsum_i32(seq_lens_k),
            "max_seqlen_q": max(list(seq_lens) + [0])}


def decode_inputs(num_seqs, ctx_len, num_query_heads, num_kv_heads, head_size, seed,
                  block_size=16, dtype="bf16", seq_lens=None, spare_blocks=16):
    """query, k_cache, v_cache, block_tables, seq_lens on the CPU.

    ``seq_lens`` (a list) overrides the uniform ``ctx_len``; the table is
    then sized for the longest entry.
    """
    lens = [ctx_len] * num_seqs if seq_lens is None else [int(x) for x in seq_lens]
    if len(lens) != num_seqs:
        raise ValueError("seq_lens must have num_seqs entries")
    longest = max(lens + [0])
    maxb = (longest + block_size - 1) // block_size
    num_blocks = maxb * num_seqs + spare_blocks
    x = 16 // 2
    gen = torch.Generator().manual_seed(int(seed))
    query = _randn(gen, (num_seqs, num_query_heads, head_size), dtype)
    k_cache = _randn(gen, (num_blocks, num_kv_heads, head_size // x, block_size, x), dtype)
    v_cache = _randn(gen, (num_blocks, num_kv_heads, head_size, block_size), dtype)
    block_tables = (torch.arange(num_seqs, dtype=torch.int32)[:, None] * maxb
                    + torch.arange(maxb, dtype=torch.int32)[None, :]).contiguous()
    return {"query": query, "k_cache": k_cache, "v_cache": v_cache,
            "block_tables": block_tables, "seq_lens": torch.tensor(lens, dtype=torch.int32)}


def permute_blocks(inputs, seed):
    """Moves every physical block to a random new position and rewrites the
    block table to match: the same logical keys, stored elsewhere."""
    gen = torch.Generator().manual_seed(int(seed))
    nb = inputs["k_cache"].shape[0]
    perm = torch.randperm(nb, generator=gen)          # block b moves to perm[b]
    k_new = torch.empty_like(inputs["k_cache"])
    v_new = torch.empty_like(inputs["v_cache"])
    k_new[perm] = inputs["k_cache"]
    v_new[perm] = inputs["v_cache"]
    bt = perm.to(torch.int32)[inputs["block_tables"].long()].contiguous()
    out = dict(inputs)
    out.update(k_cache=k_new, v_cache=v_new, block_tables=bt)
    return out


def chunk_inputs(batch, tokens, num_q_heads, num_heads, seed, key_dim=128, value_dim=128,
                 chunk_size=64, dtype="bf16"):
    """q, k, v, h (16-bit) and g (float32) of the chunked delta-rule output, on the CPU."""
    gen = torch.Generator().manual_seed(int(seed))
    dt = _DT[dtype]
    nc = (tokens + chunk_size - 1) // chunk_size

    def scaled(shape):
        return (_randn(gen, shape, dtype).float() * 0.02).to(dt)

    q = scaled((batch, tokens, num_q_heads, key_dim))
    k = _randn(gen, (batch, tokens, num_q_heads, key_dim), dtype)
    v = scaled((batch, tokens, num_heads, value_dim))
    h = scaled((batch, nc, num_heads, key_dim, value_dim))
    g = -torch.rand(batch, tokens, num_heads, generator=gen, dtype=torch.float32)
    return {"q": q, "k": k, "v": v, "h": h, "g": g, "chunk_size": chunk_size}


def workload_inputs(name):
    """Inputs of one named workload from ``WORKLOADS`` or ``CHUNK_WORKLOADS``."""
    if name in CHUNK_WORKLOADS:
        return chunk_inputs(**CHUNK_WORKLOADS[name])
    w = dict(WORKLOADS[name])
    kind = w.pop("kind")
    if kind == "prefill":
        return prefill_inputs(**w)
    return decode_inputs(**w)
