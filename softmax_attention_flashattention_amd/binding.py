"""ctypes binding of libattn (``include/attn.h``): argument marshalling only.

Each function here has the name of the C entry point it calls.  It takes the
scalar sizes from the tensor shapes under the shape conventions of the
operator pages (atrex-bench "attention_forward" #001 and
"paged_attention_decode" #024, Reference Implementation): the three
dimensions of the decode query are the sequence count, the query-head count
and the head size, and the value cache's second and fourth dimensions are the
KV-head count and the block size.  It allocates outputs and the decode
workspace with torch, passes raw device pointers and torch's current HIP
stream, and raises on a non-OK status.  Every step of the computation runs in the HIP library; if the
library is missing the call fails loudly -- there is no fallback.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libattn.so"
_lib = None

_DTYPE = {torch.bfloat16: 0, torch.float16: 1}
_STATUS = {0: "ATTN_OK", 1: "ATTN_ERR_INVALID_ARG", 2: "ATTN_ERR_UNSUPPORTED",
           3: "ATTN_ERR_WORKSPACE", 4: "ATTN_ERR_HIP"}


class AttnError(RuntimeError):
    """A libattn call returned a status other than ATTN_OK."""

    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {_STATUS.get(status, status)}")


def library_path():
    """Where the built HIP library is expected (inside this package)."""
    return os.path.join(_PKG, _LIB_NAME)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"libattn is not built ({path} is missing); run "
                           "`python -c 'import __graft_entry__ as g; g.build()'` first")
    lib = ctypes.CDLL(path)
    P, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                            ctypes.c_size_t)
    lib.attn_varlen_fwd.argtypes = [P, P, P, P, P, i32, i32, i64, i64, i32, i32, f32, i32, P, sz, P, P]
    lib.attn_varlen_fwd.restype = ctypes.c_int
    lib.attn_varlen_fwd_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.attn_varlen_fwd_workspace_size.restype = sz
    lib.attn_paged_decode.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32, i64, f32, i32,
                                      i32, P, sz, P, P]
    lib.attn_paged_decode.restype = ctypes.c_int
    lib.attn_paged_decode_noalloc.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32, i64, f32,
                                              i32, i32, P, P]
    lib.attn_paged_decode_noalloc.restype = ctypes.c_int
    lib.attn_paged_decode_num_partitions.argtypes = [i32, i32, i32, i32, i32]
    lib.attn_paged_decode_num_partitions.restype = i32
    lib.attn_paged_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.attn_paged_decode_workspace_size.restype = sz
    lib.attn_chunk_delta_out.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32, f32, i32,
                                         P, P]
    lib.attn_chunk_delta_out.restype = ctypes.c_int
    lib.attn_status_string.argtypes = [i32]
    lib.attn_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _ptr(t):
    """A tensor's device address as a plain int (ctypes passes it as void *)."""
    return t.data_ptr() if t is not None else None


# torch's current stream on a device as a raw handle; the private accessor
# skips building a Stream object (about 2 us of host time per call)
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(dev):
    """torch's current stream on GPU index `dev`, as an int handle."""
    if _raw_stream is not None:
        return _raw_stream(dev)
    return torch.cuda.current_stream(dev).cuda_stream


def _ok(t, dtype, ndim, dev):
    """The common case of the checks `_need` spells out, in a few cheap
    attribute reads: a contiguous tensor of `dtype` with `ndim` dimensions on
    GPU index `dev`."""
    return (isinstance(t, torch.Tensor) and t.dtype is dtype and t.dim() == ndim
            and t.get_device() == dev and t.is_contiguous())


def _gpu_index(t):
    """The GPU index of a 16-bit floating-point tensor, -1 for anything else."""
    if isinstance(t, torch.Tensor) and t.dtype in _DTYPE:
        return t.get_device()
    return -1


# workspace sizes the library reported, by the sizes of the call and the GPU
# index (5-tuples: prefill, 8-tuples: decode)
_ws_sizes = {}


def _need(t, name, dtype=None, ndim=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the call runs on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, has {t.dim()}")


def attn_status_string(status):
    """The library's name for a status code."""
    return _load().attn_status_string(int(status)).decode()


def attn_varlen_fwd_workspace_size(num_seqs, max_seqlen_q, num_heads, head_dim):
    """Workspace bytes a varlen prefill call can use on the current device."""
    return _load().attn_varlen_fwd_workspace_size(int(num_seqs), int(max_seqlen_q),
                                                  int(num_heads), int(head_dim))


def _varlen_ws_bytes(num_seqs, max_seqlen_q, H, D, dev):
    key = (num_seqs, max_seqlen_q, H, D, dev)
    n = _ws_sizes.get(key)
    if n is None:
        if len(_ws_sizes) > 4096:
            _ws_sizes.clear()
        n = _ws_sizes[key] = attn_varlen_fwd_workspace_size(num_seqs, max_seqlen_q, H, D)
    return n


def attn_varlen_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q=None, scale=None,
                    out=None, workspace=None):
    """Non-causal varlen prefill attention (calls ``attn_varlen_fwd``).

    q [total_q, H, D], k/v [total_k, H, D] in bf16 or fp16; cu_seqlens_* int32
    [num_seqs + 1] on the GPU.  ``max_seqlen_q`` defaults to the longest
    query segment (read back from the GPU: a synchronisation).  ``scale``
    defaults to D**-0.5.  Rows outside every query segment of a
    caller-provided ``out`` are left untouched.  ``workspace`` (a GPU
    tensor) defaults to one allocated here of the size the library asks for;
    an empty tensor runs every work item whole.
    """
    dev = _gpu_index(q)
    dt = q.dtype if dev >= 0 else None
    if not (dev >= 0 and q.dim() == 3 and q.is_contiguous() and _ok(k, dt, 3, dev)
            and _ok(v, dt, 3, dev) and _ok(cu_seqlens_q, torch.int32, 1, dev)
            and _ok(cu_seqlens_k, torch.int32, 1, dev)):
        fp16 = (torch.bfloat16, torch.float16)   # name the first failing check
        _need(q, "q", fp16, 3)
        _need(k, "k", q.dtype, 3, device=q.device)
        _need(v, "v", q.dtype, 3, device=q.device)
        _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1, device=q.device)
        _need(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1, device=q.device)
    total_q, H, D = q.shape
    ks = k.shape
    if ks[1] != H or ks[2] != D or v.shape != ks:
        raise ValueError("k and v must be [total_k, H, D] with q's H and D")
    n1 = cu_seqlens_q.numel()
    if cu_seqlens_k.numel() != n1 or n1 < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have num_seqs + 1 entries each")
    num_seqs = n1 - 1
    if max_seqlen_q is None:
        max_seqlen_q = int((cu_seqlens_q[1:] - cu_seqlens_q[:-1]).max().item()) if num_seqs else 0
    else:
        max_seqlen_q = int(max_seqlen_q)
    scale = float(D) ** -0.5 if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    elif not _ok(out, dt, 3, dev) or out.shape != q.shape:
        _need(out, "out", q.dtype, 3, device=q.device)
        raise ValueError("out must have q's shape")
    if workspace is None:
        ws_len = _varlen_ws_bytes(num_seqs, max_seqlen_q, H, D, dev)
        # held until the call has enqueued its kernels
        workspace = torch.empty(ws_len, dtype=torch.uint8, device=q.device) if ws_len else None
        ws_ptr = workspace.data_ptr() if ws_len else None
    else:
        _need(workspace, "workspace", device=q.device)
        ws_len = workspace.numel() * workspace.element_size()
        ws_ptr = workspace.data_ptr() if ws_len else None
    rc = _load().attn_varlen_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens_q.data_ptr(),
                                 cu_seqlens_k.data_ptr(), num_seqs, max_seqlen_q, total_q, ks[0], H,
                                 D, scale, _DTYPE[dt], ws_ptr, ws_len, out.data_ptr(), _stream(dev))
    if rc != 0:
        raise AttnError("attn_varlen_fwd", rc)
    return out


def attn_paged_decode_num_partitions(num_seqs, num_kv_heads, max_blocks_per_seq, block_size,
                                     partition_size=0):
    """Context partitions the decode call will use on the current device
    (calls the C function)."""
    n = _load().attn_paged_decode_num_partitions(int(num_seqs), int(num_kv_heads),
                                                 int(max_blocks_per_seq), int(block_size),
                                                 int(partition_size))
    if n < 0:
        raise AttnError("attn_paged_decode_num_partitions", -n)
    return n


def attn_paged_decode_workspace_size(num_seqs, num_query_heads, num_kv_heads, head_size,
                                     max_blocks_per_seq, block_size, partition_size=0):
    """Workspace bytes for a decode call on the current device (calls the C
    function)."""
    return _load().attn_paged_decode_workspace_size(int(num_seqs), int(num_query_heads),
                                                    int(num_kv_heads), int(head_size),
                                                    int(max_blocks_per_seq), int(block_size),
                                                    int(partition_size))


def _decode_sizes(query, k_cache, v_cache, block_tables, seq_lens, scale, out):
    """Checks the decode tensors, derives the sizes from their shapes and
    returns (sizes, scale, out, GPU index)."""
    dev = _gpu_index(query)
    dt = query.dtype if dev >= 0 else None
    if not (dev >= 0 and query.dim() == 3 and query.is_contiguous() and _ok(k_cache, dt, 5, dev)
            and _ok(v_cache, dt, 4, dev) and _ok(block_tables, torch.int32, 2, dev)
            and _ok(seq_lens, torch.int32, 1, dev)):
        fp16 = (torch.bfloat16, torch.float16)   # name the first failing check
        _need(query, "query", fp16, 3)
        _need(k_cache, "k_cache", query.dtype, 5, device=query.device)
        _need(v_cache, "v_cache", query.dtype, 4, device=query.device)
        _need(block_tables, "block_tables", torch.int32, 2, device=query.device)
        _need(seq_lens, "seq_lens", torch.int32, 1, device=query.device)
    num_seqs, num_query_heads, head_size = query.shape
    num_blocks, num_kv_heads, v_dim, block_size = v_cache.shape
    if k_cache.shape != (num_blocks, num_kv_heads, head_size // 8, block_size, 8):
        raise ValueError("k_cache must be [num_blocks, num_kv_heads, head_size/8, block_size, 8]")
    if v_dim != head_size:
        raise ValueError("v_cache must be [num_blocks, num_kv_heads, head_size, block_size]")
    if block_tables.shape[0] != num_seqs or seq_lens.numel() != num_seqs:
        raise ValueError("block_tables and seq_lens need one row/entry per sequence")
    maxb = block_tables.shape[1]
    scale = float(head_size) ** -0.5 if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(query)
    elif not _ok(out, dt, 3, dev) or out.shape != query.shape:
        _need(out, "out", query.dtype, 3, device=query.device)
        raise ValueError("out must have query's shape")
    sizes = (num_seqs, num_query_heads, num_kv_heads, head_size, block_size, maxb, num_blocks)
    return sizes, scale, out, dev


def attn_paged_decode(query, k_cache, v_cache, block_tables, seq_lens, scale=None, out=None,
                      partition_size=0, workspace=None):
    """Paged single-query decode with grouped-query heads (calls ``attn_paged_decode``).

    query [num_seqs, Hq, D]; k_cache [num_blocks, Hkv, D/8, block_size, 8];
    v_cache [num_blocks, Hkv, D, block_size]; block_tables int32
    [num_seqs, max_blocks_per_seq]; seq_lens int32 [num_seqs].  ``scale``
    defaults to D**-0.5.  ``partition_size`` (tokens; 0 lets the library
    choose) sets the split-K granularity; the workspace it needs is
    allocated here unless one is passed.
    """
    sizes, scale, out, dev = _decode_sizes(query, k_cache, v_cache, block_tables, seq_lens, scale,
                                           out)
    num_seqs, num_query_heads, num_kv_heads, head_size, block_size, maxb, num_blocks = sizes
    key = (num_seqs, num_query_heads, num_kv_heads, head_size, maxb, block_size, partition_size, dev)
    ws_bytes = _ws_sizes.get(key)
    if ws_bytes is None:
        if len(_ws_sizes) > 4096:
            _ws_sizes.clear()
        ws_bytes = _ws_sizes[key] = attn_paged_decode_workspace_size(
            num_seqs, num_query_heads, num_kv_heads, head_size, maxb, block_size, partition_size)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=query.device)
    elif workspace is not None:
        _need(workspace, "workspace", device=query.device)
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = _load().attn_paged_decode(_ptr(query), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                   _ptr(seq_lens), num_seqs, num_query_heads, num_kv_heads,
                                   head_size, block_size, maxb, num_blocks, scale,
                                   _DTYPE[query.dtype], int(partition_size), _ptr(workspace),
                                   ws_len, _ptr(out), _stream(dev))
    if rc != 0:
        raise AttnError("attn_paged_decode", rc)
    return out


def attn_paged_decode_noalloc(query, k_cache, v_cache, block_tables, seq_lens, scale=None,
                              out=None, partition_size=0):
    """``attn_paged_decode`` without a workspace (calls ``attn_paged_decode_noalloc``).

    The library keeps a split context's partial results in its own static
    per-GPU buffer, so the call allocates nothing when ``out`` is passed;
    calls that may overlap on one GPU race for that buffer.  Raises
    AttnError(ATTN_ERR_WORKSPACE) when the split needs more than the buffer
    holds.
    """
    sizes, scale, out, dev = _decode_sizes(query, k_cache, v_cache, block_tables, seq_lens, scale,
                                           out)
    num_seqs, num_query_heads, num_kv_heads, head_size, block_size, maxb, num_blocks = sizes
    rc = _load().attn_paged_decode_noalloc(_ptr(query), _ptr(k_cache), _ptr(v_cache),
                                           _ptr(block_tables), _ptr(seq_lens), num_seqs,
                                           num_query_heads, num_kv_heads, head_size, block_size,
                                           maxb, num_blocks, scale, _DTYPE[query.dtype],
                                           int(partition_size), _ptr(out), _stream(dev))
    if rc != 0:
        raise AttnError("attn_paged_decode_noalloc", rc)
    return out


def attn_chunk_delta_out(q, k, v, h, g, chunk_size=64, scale=None, out=None):
    """Output step of chunked gated delta-rule linear attention (calls
    ``attn_chunk_delta_out``).

    q, k [B, T, Hq, K] and v [B, T, H, V] in bf16 or fp16; h [B, ceil(T /
    chunk_size), H, K, V] in the same dtype; g [B, T, H] float32.  Shapes are
    derived as the operator page does (``batch, tokens, num_q_heads, key_dim
    = q.shape``, ``num_heads, value_dim = v.shape[2], v.shape[3]``).
    ``scale`` defaults to K**-0.5.  Returns out [B, T, H, V] in v's dtype.
    """
    dev = _gpu_index(q)
    dt = q.dtype if dev >= 0 else None
    if not (dev >= 0 and q.dim() == 4 and q.is_contiguous() and _ok(k, dt, 4, dev)
            and _ok(v, dt, 4, dev) and _ok(h, dt, 5, dev) and _ok(g, torch.float32, 3, dev)):
        fp16 = (torch.bfloat16, torch.float16)   # name the first failing check
        _need(q, "q", fp16, 4)
        _need(k, "k", q.dtype, 4, device=q.device)
        _need(v, "v", q.dtype, 4, device=q.device)
        _need(h, "h", q.dtype, 5, device=q.device)
        _need(g, "g", torch.float32, 3, device=q.device)
    B, T, Hq, K = q.shape
    H, V = v.shape[2], v.shape[3]
    nc = (T + chunk_size - 1) // chunk_size
    if tuple(k.shape) != (B, T, Hq, K) or tuple(v.shape[:2]) != (B, T):
        raise ValueError("q, k must be [B, T, Hq, K] and v [B, T, H, V]")
    if tuple(h.shape) != (B, nc, H, K, V) or tuple(g.shape) != (B, T, H):
        raise ValueError("h must be [B, ceil(T / chunk_size), H, K, V] and g [B, T, H]")
    scale = float(K) ** -0.5 if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(v)
    elif not _ok(out, dt, 4, dev) or out.shape != v.shape:
        _need(out, "out", v.dtype, 4, device=q.device)
        raise ValueError("out must have v's shape")
    rc = _load().attn_chunk_delta_out(_ptr(q), _ptr(k), _ptr(v), _ptr(h), _ptr(g), B, T, Hq, H, K,
                                      V, int(chunk_size), scale, _DTYPE[dt], _ptr(out),
                                      _stream(dev))
    if rc != 0:
        raise AttnError("attn_chunk_delta_out", rc)
    return out
