"""Offsets past 2^31 elements (4 GiB of 16-bit data) in prefill, decode and
the chunked output, against the oracle ("attention_forward" #001,
"paged_attention_decode" #024 and "chunk_delta_rule_output" #004, Reference
Implementation).

The tensors repeat a seeded pattern (1000 token rows, 1000 cache blocks or
250 chunks) copied on the GPU, so that the inputs are cheap to build and the
oracle only needs the pattern.  The period does not divide 2^31 elements, so a device
offset that wrapped at 32 bits would read rows holding other values and fail
the comparison.  The checked rows are those whose byte offsets lie past 2^32
(and a few below, for contrast).
"""
import numpy as np
import pytest
import torch

import oracle
from parity import check, f64
from softmax_attention_flashattention_amd import attn_paged_decode, attn_varlen_fwd, inputs as gen

pytestmark = pytest.mark.gpu

PERIOD = 1000


def tiled(x, n):
    """x [PERIOD, ...] (CPU) repeated along dim 0 to n rows, on the GPU."""
    reps = (n + x.shape[0] - 1) // x.shape[0]
    return x.cuda().repeat(reps, *([1] * (x.dim() - 1)))[:n].contiguous()


def test_prefill_offsets_past_4_gib():
    # 17 x 2^20 tokens x 1 head x 128 dims: q, k, v and out are 4.56 GB each
    # (element offsets up to 2.28e9); 17408 sequences of 1024 tokens
    H, D, L = 1, 128, 1024
    N = 17 << 20
    nseq = N // L
    pat = gen.prefill_inputs([PERIOD], H, D, seed=81)
    print(f"[prefill] {N} tokens x {H} x {D}: offsets past 2^31 elements", flush=True)
    q, k, v = tiled(pat["q"], N), tiled(pat["k"], N), tiled(pat["v"], N)
    cu = torch.arange(0, N + 1, L, dtype=torch.int32, device="cuda")
    out = torch.full_like(q, float("nan"))
    attn_varlen_fwd(q, k, v, cu, cu, max_seqlen_q=L, out=out)
    torch.cuda.synchronize()
    first_high = (1 << 31) // (H * D) // L            # the first sequence past 2^31 elements
    for s in [0, 5, first_high - 1, first_high, first_high + 1, nseq - 2, nseq - 1]:
        rows = np.arange(s * L, (s + 1) * L) % PERIOD
        idx = torch.from_numpy(rows)
        qs, ks, vs = pat["q"][idx].contiguous(), pat["k"][idx].contiguous(), pat["v"][idx].contiguous()
        cu1 = torch.tensor([0, L], dtype=torch.int32)
        ref, ref_abs = oracle.varlen_fwd(qs, ks, vs, cu1, cu1, return_abs=True)
        got = f64(out[s * L:(s + 1) * L])
        check(got, ref, f"sequence {s} (element offsets from {s * L * H * D})", ref_abs=ref_abs)
    del q, k, v, out, cu
    torch.cuda.empty_cache()


def test_decode_offsets_past_4_gib():
    # 2^20 + 2^17 cache blocks of one KV head at head_size 128 (2048 elements
    # a block): K and V caches are 4.8 GB each; the tables point at blocks on
    # both sides of 2^20 (element offset 2^31)
    Hq, Hkv, D, bs = 8, 1, 128, 16
    nb = (1 << 20) + (1 << 17)
    S, ctx = 8, 300
    pat = gen.decode_inputs(1, PERIOD * bs, Hq, Hkv, D, seed=83, spare_blocks=0)
    kp, vp = pat["k_cache"][:PERIOD], pat["v_cache"][:PERIOD]     # PERIOD distinct blocks
    print(f"[decode] {nb} cache blocks: offsets past 2^31 elements", flush=True)
    kc, vc = tiled(kp, nb), tiled(vp, nb)
    rng = np.random.default_rng(85)
    maxb = (ctx + bs - 1) // bs
    bt = np.empty((S, maxb), dtype=np.int32)
    for s in range(S):
        lo = 0 if s < 2 else (1 << 20) - 8
        bt[s] = rng.integers(lo, nb, maxb) if s >= 2 else rng.integers(0, 1 << 17, maxb)
    bt[3] = np.arange(nb - maxb, nb)                    # the very last blocks
    lens = np.array([ctx - 7 * s for s in range(S)], dtype=np.int32)
    query = gen.decode_inputs(S, 1, Hq, Hkv, D, seed=87)["query"]
    out = torch.full((S, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    attn_paged_decode(query.cuda(), kc, vc, torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda(),
                      out=out)
    torch.cuda.synchronize()
    # the oracle on a small cache of the pattern blocks the tables name
    small_bt = torch.from_numpy((bt % PERIOD).astype(np.int32))
    ref = oracle.paged_decode(query, kp, vp, small_bt, torch.from_numpy(lens))
    ref_abs = oracle.paged_decode(query, kp, vp.abs(), small_bt, torch.from_numpy(lens))
    check(f64(out), ref, "decode, blocks past element offset 2^31", ref_abs=ref_abs)
    del kc, vc, out
    torch.cuda.empty_cache()


def test_chunk_output_offsets_past_4_gib():
    # 9600 chunks of 64 tokens, 32 value / 16 query heads, key and value dim
    # 128: h is 10 GB (element offsets up to 5.0e9), v and out 5 GB each.
    # Each chunk's output depends on that chunk's q, k, v, g and state only,
    # so the oracle checks a chunk on its pattern chunk alone.
    import oracle.chunk as ch
    from softmax_attention_flashattention_amd import attn_chunk_delta_out
    from test_chunk_gpu import bar
    Hq, H, cs, P = 16, 32, 64, 250                     # P pattern chunks
    nc = 9600
    T = nc * cs
    pat = gen.chunk_inputs(1, P * cs, Hq, H, seed=89)
    print(f"[chunk] {T} tokens x {H} heads: offsets past 2^31 elements", flush=True)

    def tile_tokens(x):                                # [1, P*cs, ...] -> [1, T, ...]
        return tiled(x[0], T).unsqueeze(0)
    q, k, v, g = (tile_tokens(pat[n]) for n in ("q", "k", "v", "g"))
    h = tiled(pat["h"][0], nc).unsqueeze(0)
    out = torch.full_like(v, float("nan"))
    attn_chunk_delta_out(q, k, v, h, g, chunk_size=cs, out=out)
    torch.cuda.synchronize()
    # h passes element offset 2^31 at chunk 4096, v and out at chunk 8192
    for c in [0, 7, 4095, 4096, 4097, 8191, 8192, nc - 1]:
        pc = c % P
        t0 = pc * cs
        one = {n: pat[n][:, t0:t0 + cs].contiguous() for n in ("q", "k", "v", "g")}
        hc = pat["h"][:, pc:pc + 1].contiguous()
        ref = ch.chunk_delta_out(one["q"], one["k"], one["v"], hc, one["g"])
        A = ch.chunk_delta_out(one["q"], one["k"], one["v"], hc, one["g"], absolute=True)
        bar(f64(out[:, c * cs:(c + 1) * cs]), ref, A, f"chunk {c}")
    del q, k, v, g, h, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("lens,H,D,path", [
    ([300, 17, 290], 4, 72, "key-splitting workgroups"),
    ([9000], 1, 72, "64-row waves, items split into key ranges"),
    ([2116, 1500], 16, 72, "32-row waves"),
    ([1000, 600], 2, 128, "head_dim 128, items split into key ranges"),
])
def test_prefill_segments_past_4_gib(lens, H, D, path):
    # few work items whose segments start past element offset 2^31 of
    # buffers of 4.3-4.6 GB: query and key segments begin at different rows,
    # so every kernel path the grid selects addresses q, k, v and out far out
    rs = H * D
    a_q = (1 << 31) // rs + 123                  # first query row of the segments
    a_k = (1 << 31) // rs + 777                  # first key row
    tot = sum(lens)
    nq, nk = a_q + tot, a_k + tot
    pat = gen.prefill_inputs([PERIOD], H, D, seed=91 + D + H)
    print(f"[prefill] {path}: segments {lens} x {H} heads at rows {a_q} (q), {a_k} (k, v)", flush=True)
    q, k, v = tiled(pat["q"], nq), tiled(pat["k"], nk), tiled(pat["v"], nk)
    cu_q = torch.tensor(np.concatenate([[0], np.cumsum(lens)]) + a_q, dtype=torch.int32, device="cuda")
    cu_k = torch.tensor(np.concatenate([[0], np.cumsum(lens)]) + a_k, dtype=torch.int32, device="cuda")
    out = torch.full_like(q, float("nan"))
    attn_varlen_fwd(q, k, v, cu_q, cu_k, max_seqlen_q=max(lens), out=out)
    torch.cuda.synchronize()
    qi = torch.from_numpy((np.arange(a_q, nq) % PERIOD))
    ki = torch.from_numpy((np.arange(a_k, nk) % PERIOD))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    ref, ref_abs = oracle.varlen_fwd(pat["q"][qi].contiguous(), pat["k"][ki].contiguous(),
                                     pat["v"][ki].contiguous(), cu, cu, return_abs=True)
    check(f64(out[a_q:nq]), ref, f"{path}: segments past 2^31 elements", ref_abs=ref_abs)
    # the rows before the segments are outside every segment: untouched
    assert bool(torch.isnan(out[a_q - 64:a_q]).all()), f"{path}: rows before the segments written"
    del q, k, v, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("D", [72, 128])
def test_prefill_largest_head_count(D):
    # the most heads the library accepts, num_heads * head_dim < 2^25: one
    # token row is then almost 64 MiB, so a 64-key tile spans almost 2^32
    # bytes, the most its 32-bit byte offsets reach.  64 tokens, heads
    # repeating a pattern of 1000 heads; the output is NaN-filled first and
    # every element must be written; all heads of the first and last 3000
    # and every 97th head are compared with the oracle
    H = ((1 << 32) - 1) // (2 * 64 * D)          # largest H with H * D * 2 * 64 < 2^32
    assert H * D * 2 * 64 < (1 << 32) <= (H + 1) * D * 2 * 64
    S, HP = 64, 1000
    pat = gen.prefill_inputs([S], HP, D, seed=93 + D)
    print(f"[prefill] {S} tokens x {H} heads x {D}: key tiles spanning almost 2^32 bytes", flush=True)

    def tile_heads(x):                             # [S, HP, D] -> [S, H, D] on the GPU
        return x.cuda().repeat(1, (H + HP - 1) // HP, 1)[:, :H].contiguous()
    q, k, v = tile_heads(pat["q"]), tile_heads(pat["k"]), tile_heads(pat["v"])
    cu = torch.tensor([0, S], dtype=torch.int32, device="cuda")
    out = torch.full_like(q, float("nan"))
    attn_varlen_fwd(q, k, v, cu, cu, max_seqlen_q=S, out=out)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()), f"D={D}: rows left unwritten or non-finite"
    ref, ref_abs = oracle.varlen_fwd(pat["q"], pat["k"], pat["v"], pat["cu_seqlens_q"],
                                     pat["cu_seqlens_k"], return_abs=True)
    heads = np.unique(np.concatenate([np.arange(3000), np.arange(H - 3000, H), np.arange(0, H, 97)]))
    for i in range(0, heads.size, 4096):
        hs = heads[i:i + 4096]
        got = f64(out[:, torch.from_numpy(hs).cuda()])
        check(got, ref[:, hs % HP], f"D={D}, heads {hs[0]}..{hs[-1]}", ref_abs=ref_abs[:, hs % HP])
    del q, k, v, out
    torch.cuda.empty_cache()
