"""Helpers shared by the GPU parity tests: device transfer and the comparison
bars.

Bar 1 (the target's own): elementwise |gpu - ref| <= 1e-2 + 1e-2 |ref| on the
16-bit output against the unrounded float64 oracle.

Bar 2 (derived from the kernels' arithmetic, scale-free): the prefill kernel
rounds each softmax weight p_j to the 16-bit type before the P V product
(relative error <= 2^-9 per weight) and the output is rounded once more
(<= 2^-9 relative).  With w_j the exact normalised weights and
A = sum_j w_j |v_j| (the oracle run on |v|), the error is at most about
2^-9 A + 2^-8 |ref|; the bar allows twice that:
    |gpu - ref| <= 2^-8 A + 2^-7 |ref|.
Unlike bar 1 it does not loosen as outputs shrink at long sequence lengths,
and it holds for value tensors of any scale.

Both bars also require the relative RMS error to stay below 1e-2.
"""
import numpy as np
import torch

ATOL = 1e-2
RTOL = 1e-2


def to_gpu(inputs):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inputs.items()}


def f64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def check(gpu, ref, what="", ref_abs=None, bar1=True):
    """Asserts the bars; returns (max abs error, relative RMS error)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU output"
    err = np.abs(gpu - ref)
    if bar1:
        bad = err > ATOL + RTOL * np.abs(ref)
        assert not bad.any(), (f"{what}: {int(bad.sum())} of {err.size} elements outside "
                               f"1e-2 + 1e-2|ref|; worst {err.max():.3e}")
    if ref_abs is not None:
        ref_abs = np.asarray(ref_abs, dtype=np.float64)
        bound = 2.0 ** -8 * ref_abs + 2.0 ** -7 * np.abs(ref)
        bad = err > bound
        assert not bad.any(), (f"{what}: {int(bad.sum())} of {err.size} elements outside "
                               f"2^-8 A + 2^-7 |ref|; worst ratio {(err / np.maximum(bound, 1e-300)).max():.3f}")
    rms = float(np.sqrt((err ** 2).sum() / max((ref ** 2).sum(), 1e-300)))
    assert rms <= 1e-2, f"{what}: relative RMS error {rms:.3e}"
    return float(err.max()), rms
