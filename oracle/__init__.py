"""CPU oracles -- test infrastructure only: exact softmax attention forward
(``oracle.py``) and the output step of chunked gated delta-rule linear
attention (``chunk.py``).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package; the GPU library and its Python binding never do.
"""
from .oracle import (build, load, decode_bits, varlen_fwd, varlen_fwd_rows, paged_decode,
                     paged_gather, num_threads)

from . import chunk

__all__ = ["chunk", "build", "load", "decode_bits", "varlen_fwd", "varlen_fwd_rows", "paged_decode",
           "paged_gather", "num_threads"]
