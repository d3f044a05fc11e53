"""Seeded random varlen prefill batches through attn_varlen_fwd, every
element against the oracle ("attention_forward" #001, Reference
Implementation).

Each case draws a batch (1-6 sequences, query lengths up to 1500, key
lengths up to 1.3 times that, empty segments included), a head count, the
head_dim, the 16-bit type and the scale from its seed, so the cases land on
every small- and mid-grid path the library chooses between: the
key-splitting workgroups and the 32-row waves at head_dim 72, the
head_dim-128 kernel whole and (for the long-key cases) with its items split
into key ranges merged by a second kernel.
"""
import numpy as np
import pytest

from test_prefill_gpu import scaled_check
from softmax_attention_flashattention_amd import inputs as gen

pytestmark = pytest.mark.gpu


def draw(seed):
    rng = np.random.default_rng(3000 + seed)
    if seed % 6 == 5:
        # few items of head_dim 128 with long keys: split into key ranges
        n, H, D = int(rng.integers(1, 3)), int(rng.choice([1, 2, 4])), 128
        lq = [int(x) for x in rng.integers(1, 1500, n)]
        lq[0] = max(lq[0], 1100)
        lk = [int(x) for x in rng.integers(500, 4000, n)]
    else:
        n = int(rng.integers(1, 7))
        H = int(rng.choice([1, 2, 3, 4, 8, 12, 16, 32, 64]))
        D = int(rng.choice([72, 128]))
        maxlen = int(rng.choice([64, 300, 800, 1500]))
        lq = [int(x) for x in rng.integers(0, maxlen + 1, n)]
        lk = [int(x) for x in rng.integers(0, int(maxlen * 1.3) + 1, n)]
        lq[0] = max(lq[0], 1)
        while sum(a * b for a, b in zip(lq, lk)) * H * D * 4 > 4e9:   # keep the oracle in seconds
            H = max(1, H // 2)
            if H == 1:
                break
    dtype = "fp16" if rng.random() < 0.3 else "bf16"
    scale = [D ** -0.5, float(rng.uniform(0.02, 0.2)), -float(rng.uniform(0.02, 0.2)), 0.0][int(rng.integers(0, 4))]
    return lq, lk, H, D, dtype, scale


@pytest.mark.parametrize("seed", range(24))
def test_random_batches(seed):
    lq, lk, H, D, dtype, scale = draw(seed)
    inp = gen.prefill_inputs(lq, H, D, seed=4000 + seed, dtype=dtype, seq_lens_k=lk)
    print(f"[prefill] random batch {seed}: q {lq} k {lk} H {H} D {D} {dtype} scale {scale:.3f}", flush=True)
    scaled_check(inp, scale, f"random batch {seed}: q {lq} k {lk} H {H} D {D} {dtype} scale {scale:.3f}")
