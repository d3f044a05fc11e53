"""CPU oracle for exact softmax attention forward -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package; the GPU library and its Python binding never do.
"""
from .oracle import (build, load, decode_bits, varlen_fwd, varlen_fwd_rows, paged_decode,
                     paged_gather, num_threads)

__all__ = ["build", "load", "decode_bits", "varlen_fwd", "varlen_fwd_rows", "paged_decode",
           "paged_gather", "num_threads"]
