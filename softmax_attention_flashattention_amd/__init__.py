"""libattn: exact softmax attention forward on MI355X (gfx950), and the
output step of chunked gated delta-rule linear attention.

The Python names mirror the C entry points declared in ``include/attn.h``;
they only marshal arguments (shapes, pointers, the current HIP stream) and
call the HIP library.  Nothing is computed here.
"""
from .binding import (attn_varlen_fwd, attn_varlen_fwd_workspace_size, attn_paged_decode,
                      attn_paged_decode_noalloc, attn_paged_decode_workspace_size,
                      attn_paged_decode_num_partitions, attn_chunk_delta_out, attn_status_string,
                      AttnError, library_path)

__all__ = ["attn_varlen_fwd", "attn_varlen_fwd_workspace_size", "attn_paged_decode",
           "attn_paged_decode_noalloc", "attn_paged_decode_workspace_size", "attn_paged_decode_num_partitions",
           "attn_chunk_delta_out", "attn_status_string", "AttnError", "library_path"]
