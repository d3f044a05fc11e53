"""Pins of the chunked delta-rule output oracle against facts that do not come
from the oracle itself (no GPU).

Source: atrex-bench "chunk_delta_rule_output" (#004), Reference
Implementation.  The page prints no output values, so the pins are special
cases with a closed form or a library reduction, an independent (recurrent)
formulation, exact invariants, and the rounding rule checked against torch's
own conversion.
"""
import math

import numpy as np
import pytest
import torch

import oracle.chunk as ch

BF16, FP16 = 0, 1


def _ints(gen, shape, lo, hi, dtype=torch.bfloat16):
    return torch.randint(lo, hi + 1, shape, generator=gen).to(dtype)


def _rand(gen, shape, scale=1.0, dtype=torch.bfloat16):
    return (torch.randn(*shape, generator=gen) * scale).to(dtype)


def _f64(x):
    return x.to(torch.float64).numpy()


# ---- the rounding of the intra-chunk scores to the value dtype -------------

def test_rounding_ties_to_even():
    r = ch.round_to_dtype
    assert r(1 + 2 ** -8, BF16) == 1.0                     # halfway, even neighbour below
    assert r(1 + 3 * 2 ** -8, BF16) == 1 + 2 ** -6         # halfway, even neighbour above
    assert r(-(1 + 3 * 2 ** -8), BF16) == -(1 + 2 ** -6)
    assert r(1 + 2 ** -8 + 2 ** -30, BF16) == 1 + 2 ** -7  # just past halfway
    assert r(1 + 2 ** -11, FP16) == 1.0
    assert r(1 + 3 * 2 ** -11, FP16) == 1 + 2 ** -9
    assert r(2 ** -134, BF16) == 0.0                       # half the bf16 subnormal quantum
    assert r(3 * 2 ** -134, BF16) == 2 ** -132
    assert r(2 ** -133, BF16) == 2 ** -133                  # the smallest bf16 subnormal
    assert r(5 * 2 ** -134, BF16) == 2 ** -132              # 2.5 quanta: even neighbour
    assert r(2 ** -25, FP16) == 0.0                        # half the fp16 subnormal quantum
    assert r(3 * 2 ** -25, FP16) == 2 ** -23
    assert r(2 ** -24, FP16) == 2 ** -24                    # the smallest fp16 subnormal
    assert r(0.0, BF16) == 0.0


@pytest.mark.parametrize("dtype,code", [(torch.bfloat16, BF16), (torch.float16, FP16)])
def test_rounding_matches_torch_from_float32(dtype, code):
    # values exactly representable in float32: one rounding, as torch's own
    gen = torch.Generator().manual_seed(3)
    x = torch.cat([torch.randn(3000, generator=gen) * 10.0 ** e for e in (-6, -3, 0, 2)])
    ref = x.to(dtype).to(torch.float64).numpy()
    got = np.array([ch.round_to_dtype(float(v), code) for v in x.tolist()])
    assert np.array_equal(got, ref)


# ---- special cases with a library reduction ---------------------------------

def _chunks(T, C):
    return [(c0, min(c0 + C, T)) for c0 in range(0, T, C)]


@pytest.mark.parametrize("T,C", [(1, 8), (8, 8), (21, 8), (64, 64), (70, 64)])
def test_constant_gate_reduces_to_masked_matmul(T, C):
    # g equal for every token: the condition g_i <= g_j always holds and the
    # gate is 1, so the intra-chunk scores are tril(Q K^T); small integer q, k
    # make them exact in bf16.  out = scale (e^g Q H + tril(Q K^T) V).
    gen = torch.Generator().manual_seed(T)
    B, Hq, H, K, V = 1, 2, 2, 16, 16
    q = _ints(gen, (B, T, Hq, K), -2, 2)
    k = _ints(gen, (B, T, Hq, K), -2, 2)
    v = _rand(gen, (B, T, H, V))
    nc = -(-T // C)
    h = _rand(gen, (B, nc, H, K, V))
    g = torch.full((B, T, H), -0.3, dtype=torch.float32)
    got = ch.chunk_delta_out(q, k, v, h, g, chunk_size=C)
    scale = K ** -0.5
    for hd in range(H):
        Q, Kk, Vv = _f64(q[0, :, hd]), _f64(k[0, :, hd]), _f64(v[0, :, hd])
        for c, (a, b) in enumerate(_chunks(T, C)):
            S = np.tril(Q[a:b] @ Kk[a:b].T)
            exp_g = float(np.exp(np.float64(np.float32(-0.3))))
            ref = scale * (exp_g * Q[a:b] @ _f64(h[0, c, hd]) + S @ Vv[a:b])
            np.testing.assert_allclose(got[0, a:b, hd], ref, rtol=1e-12, atol=1e-14)


def test_token_gate_decides_mask_and_weights():
    # g alternates 0 (even tokens) and -1 (odd tokens).  An even row i sees
    # the even tokens j <= i with weight 1 (odd ones have g_j < g_i); an odd
    # row sees every token j <= i, even ones with weight e^-1, odd ones with 1.
    gen = torch.Generator().manual_seed(11)
    B, T, Hq, H, K, V, C = 1, 16, 1, 1, 16, 8, 16
    q = _ints(gen, (B, T, Hq, K), -2, 2)
    k = _ints(gen, (B, T, Hq, K), -2, 2)
    v = _rand(gen, (B, T, H, V))
    h = _rand(gen, (B, 1, H, K, V))
    g = torch.tensor([0.0 if t % 2 == 0 else -1.0 for t in range(T)]).reshape(1, T, 1)
    got = ch.chunk_delta_out(q, k, v, h, g, chunk_size=C)[0, :, 0]
    Q, Kk, Vv, Hh = _f64(q[0, :, 0]), _f64(k[0, :, 0]), _f64(v[0, :, 0]), _f64(h[0, 0, 0])
    e1 = math.exp(-1.0)
    for i in range(T):
        acc = np.zeros(V)
        for j in range(i + 1):
            s = float(Q[i] @ Kk[j])
            if i % 2 == 0:
                if j % 2 == 1:
                    continue
                a = s                                   # exact integer
            else:
                a = s if j % 2 == 1 else ch.round_to_dtype(s * e1, BF16)
            acc += a * Vv[j]
        inter = (1.0 if i % 2 == 0 else e1) * (Q[i] @ Hh)
        np.testing.assert_allclose(got[i], K ** -0.5 * (inter + acc), rtol=1e-12, atol=1e-14)


# ---- an independent formulation: the recurrent form of the chunk ----------

def test_decreasing_gate_matches_recurrence():
    # For a decreasing gate (a cumulative log-decay) the condition g_i <= g_j
    # holds for every j <= i, and the intra-chunk term equals q_i . S_i with
    # the state recurrence S_i = e^(g_i - g_(i-1)) S_(i-1) + k_i v_i^T.  The
    # oracle rounds each score to bf16 (relative error <= 2^-9 each), the
    # recurrence does not.
    gen = torch.Generator().manual_seed(5)
    B, T, Hq, H, K, V, C = 1, 40, 2, 2, 16, 16, 16
    q = _rand(gen, (B, T, Hq, K), 0.3)
    k = _rand(gen, (B, T, Hq, K))
    v = _rand(gen, (B, T, H, V))
    nc = -(-T // C)
    h = _rand(gen, (B, nc, H, K, V), 0.5)
    steps = torch.rand(B, T, H, generator=gen) * 0.2
    g = -torch.cumsum(steps, dim=1)
    got = ch.chunk_delta_out(q, k, v, h, g, chunk_size=C)
    scale = K ** -0.5
    for hd in range(H):
        Q, Kk, Vv = _f64(q[0, :, hd]), _f64(k[0, :, hd]), _f64(v[0, :, hd])
        G = g[0, :, hd].to(torch.float64).numpy()
        for c, (a, b) in enumerate(_chunks(T, C)):
            S = np.zeros((K, V))
            Hc = _f64(h[0, c, hd])
            for i in range(a, b):
                if i > a:
                    S = math.exp(G[i] - G[i - 1]) * S
                S = S + np.outer(Kk[i], Vv[i])
                ref = scale * (math.exp(G[i]) * Q[i] @ Hc + Q[i] @ S)
                bound = 2 ** -8 * scale * (np.abs(Q[i] @ Kk[a:i + 1].T) @ np.abs(Vv[a:i + 1]))
                assert np.all(np.abs(got[0, i, hd] - ref) <= bound + 1e-12), (hd, i)


# ---- exact invariants --------------------------------------------------------

def _case(seed, B=1, T=50, Hq=2, H=4, K=16, V=16, C=16):
    gen = torch.Generator().manual_seed(seed)
    nc = -(-T // C)
    return dict(q=_rand(gen, (B, T, Hq, K), 0.3), k=_rand(gen, (B, T, Hq, K)),
                v=_rand(gen, (B, T, H, V)), h=_rand(gen, (B, nc, H, K, V), 0.5),
                g=-torch.rand(B, T, H, generator=gen))


def test_padding_rows_are_inert():
    # the page pads the last chunk with zero q, k, v, g rows: extending the
    # inputs with such rows must leave the real rows unchanged
    x = _case(7, T=37, C=16)
    base = ch.chunk_delta_out(**x, chunk_size=16)
    pad = 48 - 37
    y = dict(q=torch.cat([x["q"], torch.zeros(1, pad, 2, 16, dtype=torch.bfloat16)], 1),
             k=torch.cat([x["k"], torch.zeros(1, pad, 2, 16, dtype=torch.bfloat16)], 1),
             v=torch.cat([x["v"], torch.zeros(1, pad, 4, 16, dtype=torch.bfloat16)], 1),
             h=x["h"], g=torch.cat([x["g"], torch.zeros(1, pad, 4)], 1))
    ext = ch.chunk_delta_out(**y, chunk_size=16)
    assert np.array_equal(ext[:, :37], base)


def test_grouped_heads_match_repeated_query_heads():
    # value head hd reads query head hd // (H / Hq): the same as H query heads
    # made by repeating each of the Hq query heads H / Hq times
    x = _case(8, Hq=2, H=4)
    grouped = ch.chunk_delta_out(**x, chunk_size=16)
    y = dict(x, q=x["q"].repeat_interleave(2, dim=2), k=x["k"].repeat_interleave(2, dim=2))
    assert np.array_equal(ch.chunk_delta_out(**y, chunk_size=16), grouped)


def test_more_query_heads_than_value_heads_use_the_first_ones():
    # H < Hq: one query head per value head, head hd reads query head hd
    x = _case(9, Hq=4, H=2)
    got = ch.chunk_delta_out(**x, chunk_size=16)
    y = dict(x, q=x["q"][:, :, :2].contiguous(), k=x["k"][:, :, :2].contiguous())
    assert np.array_equal(ch.chunk_delta_out(**y, chunk_size=16), got)


def test_each_chunk_uses_its_own_state():
    # swapping chunks 0 and 1 (their tokens and their states) swaps the output
    x = _case(10, T=32, C=16)
    base = ch.chunk_delta_out(**x, chunk_size=16)
    sw = lambda t: torch.cat([t[:, 16:32], t[:, 0:16]], 1)
    y = dict(q=sw(x["q"]), k=sw(x["k"]), v=sw(x["v"]), g=sw(x["g"]),
             h=x["h"][:, [1, 0]].contiguous())
    got = ch.chunk_delta_out(**y, chunk_size=16)
    assert np.array_equal(got[:, 0:16], base[:, 16:32])
    assert np.array_equal(got[:, 16:32], base[:, 0:16])


def test_batches_are_independent():
    x = _case(12, B=2, T=20)
    both = ch.chunk_delta_out(**x, chunk_size=16)
    for b in range(2):
        one = ch.chunk_delta_out(**{n: t[b:b + 1] for n, t in x.items()}, chunk_size=16)
        assert np.array_equal(both[b:b + 1], one)


def test_linear_in_value_state_and_scale():
    # the scores do not depend on v or h, so scaling both by 4 (exact in
    # bf16) scales the output by 4; the scale multiplies the whole output
    x = _case(13)
    base = ch.chunk_delta_out(**x, chunk_size=16)
    y = dict(x, v=(x["v"].float() * 4).to(torch.bfloat16), h=(x["h"].float() * 4).to(torch.bfloat16))
    assert np.array_equal(ch.chunk_delta_out(**y, chunk_size=16), 4 * base)
    assert np.allclose(ch.chunk_delta_out(**x, chunk_size=16, scale=2 * 16 ** -0.5), 2 * base,
                       rtol=1e-15, atol=0)


def test_zero_query_gives_zero():
    x = _case(14)
    x["q"] = torch.zeros_like(x["q"])
    assert not np.any(ch.chunk_delta_out(**x, chunk_size=16))


def test_rows_entry_matches_whole_output():
    x = _case(15, B=2, T=45)
    full = ch.chunk_delta_out(**x, chunk_size=16)
    gen = np.random.default_rng(0)
    rows = gen.integers(0, 2 * 45, 40)
    heads = gen.integers(0, 4, 40)
    part = ch.chunk_delta_out_rows(**x, rows=rows, heads=heads, chunk_size=16)
    ref = full.reshape(2 * 45, 4, 16)[rows, heads]
    np.testing.assert_allclose(part, ref, rtol=1e-13, atol=1e-16)
    partA = ch.chunk_delta_out_rows(**x, rows=rows, heads=heads, chunk_size=16, absolute=True)
    fullA = ch.chunk_delta_out(**x, chunk_size=16, absolute=True).reshape(2 * 45, 4, 16)
    np.testing.assert_allclose(partA, fullA[rows, heads], rtol=1e-13, atol=1e-16)


def test_absolute_mode_bounds_the_output():
    x = _case(16)
    out = ch.chunk_delta_out(**x, chunk_size=16)
    A = ch.chunk_delta_out(**x, chunk_size=16, absolute=True)
    assert np.all(np.abs(out) <= A * (1 + 1e-12))
    assert np.all(A >= 0)
