"""GPU parity of attn_chunk_delta_out against the CPU oracle.

Operator: atrex-bench "chunk_delta_rule_output" (#004), Reference
Implementation and Input Generation.  Every case feeds the HIP library and
the oracle (oracle/chunk_oracle.c) the same seeded inputs.

Bar (derived from the arithmetic; the outputs of this operator are of order
1e-3, so the absolute 1e-2 floor of the softmax bar would test nothing):
the kernel accumulates in fp32 (error ~2^-17 of the magnitude A below), may
round an intra-chunk score to the neighbouring 16-bit value when its fp32
value sits within ~2^-17 of a rounding tie (one unit, 2^-8 of that score's
term), and rounds the output once (2^-9 |ref|).  With A the oracle's
absolute-value magnitude (every product taken in absolute value),
    |gpu - ref| <= 2^-8 |ref| + 2^-8 A,
and the relative RMS error must stay below 4e-3.
"""
import numpy as np
import pytest
import torch

import oracle.chunk as ch
from parity import f64, to_gpu
from softmax_attention_flashattention_amd import attn_chunk_delta_out, inputs as gen

pytestmark = pytest.mark.gpu


def bar(gpu, ref, A, what):
    gpu = np.asarray(gpu, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    err = np.abs(gpu - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -8 * A
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {err.size} outside 2^-8 |ref| + 2^-8 A; "
                           f"worst ratio {(err / np.maximum(bound, 1e-300)).max():.3f}")
    rms = float(np.sqrt((err ** 2).sum() / max((ref ** 2).sum(), 1e-300)))
    assert rms <= 4e-3, f"{what}: relative RMS error {rms:.3e}"
    return float(err.max()), rms


def run(x, scale=None):
    # the output starts as NaN, so an element no workgroup writes fails the
    # finiteness check
    d = to_gpu(x)
    o = torch.full_like(d["v"], float("nan"))
    attn_chunk_delta_out(d["q"], d["k"], d["v"], d["h"], d["g"], chunk_size=x.get("chunk_size", 64),
                         scale=scale, out=o)
    torch.cuda.synchronize()
    return o


def full_check(x, what, scale=None):
    print(f"[chunk] {what}", flush=True)
    out = run(x, scale)
    ref = ch.chunk_delta_out(x["q"], x["k"], x["v"], x["h"], x["g"], scale=scale)
    A = ch.chunk_delta_out(x["q"], x["k"], x["v"], x["h"], x["g"], scale=scale, absolute=True)
    return bar(f64(out), ref, A, what), out


@pytest.mark.parametrize("T", [1, 2, 31, 32, 33, 63, 64, 65, 100, 128, 129, 200])
def test_token_counts(T):
    x = gen.chunk_inputs(1, T, 2, 4, seed=300 + T)
    full_check(x, f"T={T} Hq=2 H=4")


@pytest.mark.parametrize("B,T,Hq,H", [(2, 150, 2, 4), (1, 130, 4, 4), (1, 90, 4, 2), (3, 64, 1, 3)])
def test_batches_and_head_groups(B, T, Hq, H):
    x = gen.chunk_inputs(B, T, Hq, H, seed=400 + B * T + H)
    full_check(x, f"B={B} T={T} Hq={Hq} H={H}")


def test_fp16():
    x = gen.chunk_inputs(1, 160, 2, 4, seed=501, dtype="fp16")
    full_check(x, "fp16 T=160")


def test_explicit_scale():
    x = gen.chunk_inputs(1, 96, 2, 4, seed=502)
    full_check(x, "scale 0.3", scale=0.3)


def test_token_gate_masks_keys():
    # gates alternating 0 and -1: half of the earlier keys are masked for the
    # even rows (g_i > g_j), every earlier key is kept for the odd rows
    x = gen.chunk_inputs(1, 128, 2, 2, seed=503)
    g = torch.zeros_like(x["g"])
    g[:, 1::2] = -1.0
    x["g"] = g
    full_check(x, "alternating gate")


def test_decreasing_gate():
    # a cumulative log-decay (every earlier key kept, weights decaying)
    x = gen.chunk_inputs(1, 192, 2, 4, seed=504)
    x["g"] = -torch.cumsum(-x["g"] * 0.1, dim=1)
    full_check(x, "decreasing gate")


def test_zero_query_gives_exact_zero():
    x = gen.chunk_inputs(1, 100, 2, 4, seed=505)
    x["q"] = torch.zeros_like(x["q"])
    out = run(x)
    assert not torch.any(out != 0)


def test_state_only_when_keys_are_zero():
    x = gen.chunk_inputs(1, 100, 2, 4, seed=506)
    x["k"] = torch.zeros_like(x["k"])
    full_check(x, "k = 0 (state term only)")


def test_scores_only_when_state_is_zero():
    x = gen.chunk_inputs(1, 100, 2, 4, seed=507)
    x["h"] = torch.zeros_like(x["h"])
    full_check(x, "h = 0 (intra-chunk term only)")


def test_deterministic():
    x = gen.chunk_inputs(1, 300, 2, 4, seed=508)
    a, b = run(x), run(x)
    assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["chunk_t64_h32_hq16", "chunk_t704_h16_hq8", "chunk_t4195_h32_hq16",
                                  "chunk_t14807_h32_hq16"])
def test_workloads_in_full(name):
    # every element, the largest (14807 tokens x 32 heads, the benchmark's
    # chunk workload) included
    full_check(gen.workload_inputs(name), name)


def test_binding_rejects_mismatched_tensors():
    # the binding refuses, naming the argument, what the kernel could not read
    # correctly: host memory, another dtype, a strided view, a bad out
    x = gen.chunk_inputs(1, 128, 2, 2, seed=97)
    d = to_gpu(x)
    args = [d["q"], d["k"], d["v"], d["h"], d["g"]]
    bad = list(args)
    bad[4] = x["g"]
    with pytest.raises(ValueError, match="g must be a GPU tensor"):
        attn_chunk_delta_out(*bad)
    bad = list(args)
    bad[4] = d["g"].double()
    with pytest.raises(TypeError, match="g has dtype"):
        attn_chunk_delta_out(*bad)
    bad = list(args)
    bad[3] = d["h"].transpose(3, 4).contiguous().transpose(3, 4)
    with pytest.raises(ValueError, match="h must be contiguous"):
        attn_chunk_delta_out(*bad)
    with pytest.raises(TypeError, match="out has dtype"):
        attn_chunk_delta_out(*args, out=d["v"].float())
    with pytest.raises(ValueError, match="out must have v's shape"):
        attn_chunk_delta_out(*args, out=d["v"][:, :64].contiguous())
