"""CPU oracle for exact softmax attention forward -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  It wraps ``attn_oracle.c`` (plain C, double precision, OpenMP)
through ctypes and shares nothing with the GPU library: not its kernels, not
its header, not its Python binding.

Sizes come from the tensor shapes under the shape conventions of the
operator pages (atrex-bench "attention_forward" #001 and
"paged_attention_decode" #024, Reference Implementation):

* prefill: ``q``, ``k``, ``v`` are packed ``[tokens, num_heads, head_dim]``;
* decode: the query is ``[num_seqs, num_query_heads, head_size]``, and the
  value cache's second and fourth dimensions are the KV-head count and the
  block size.

The default scale is ``head_dim ** -0.5``, the default of the
scaled-dot-product routine both pages call.  Inputs are CPU tensors in
bfloat16 or float16 (or numpy float16 arrays); results are float64 numpy
arrays.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

BF16, FP16 = 0, 1


def build(force=True):
    """Compiles attn_oracle.c to liboracle.so with gcc (no fast-math)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp"
    subprocess.run(
        ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
         "-fno-fast-math", "-o", tmp, _SRC, "-lm"],
        check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def load(path=None):
    """Loads the oracle library (building it first if it is missing)."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _lib is None:
        override = os.environ.get("ATTN_ORACLE_LIB")   # another build of the same source
        if override:
            _lib = _declare(ctypes.CDLL(override))
            return _lib
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = _declare(ctypes.CDLL(_LIB_PATH))
    return _lib


def _declare(lib):
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.oracle_decode_bits_f64.argtypes = [P, i64, i32, P]
    lib.oracle_varlen_fwd_f64.argtypes = [P, P, P, i32, P, P, i32, i64, i64, i32, i32, f64, P, P, P,
                                          P]
    lib.oracle_varlen_fwd_rows_f64.argtypes = [P, P, P, i32, P, P, i32, i64, i64, i32, i32, f64,
                                               P, P, i64, P, P, P]
    lib.oracle_paged_gather_f64.argtypes = [P, P, i32, P, i32, i32, i32, i32, i32, i32, i32, i32,
                                            P, P, P]
    lib.oracle_paged_decode_f64.argtypes = [P, P, P, i32, P, P, i32, i32, i32, i32, i32, i32, i32,
                                            f64, P, P]
    lib.oracle_num_threads.argtypes = []
    for name in ("oracle_decode_bits_f64", "oracle_varlen_fwd_f64", "oracle_varlen_fwd_rows_f64",
                 "oracle_paged_gather_f64", "oracle_paged_decode_f64", "oracle_num_threads"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


def _bits(x):
    """Returns (contiguous uint16 bit patterns, dtype code) of a 16-bit float tensor."""
    if isinstance(x, np.ndarray):
        if x.dtype == np.float16:
            return np.ascontiguousarray(x).view(np.uint16), FP16
        raise TypeError(f"numpy input must be float16, got {x.dtype}")
    import torch
    if x.dtype == torch.bfloat16:
        code = BF16
    elif x.dtype == torch.float16:
        code = FP16
    else:
        raise TypeError(f"expected bfloat16 or float16, got {x.dtype}")
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16), code


def _i32(x):
    if not isinstance(x, np.ndarray):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(x, dtype=np.int32)


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"{what}: oracle rejected its arguments (code {rc})")


def decode_bits(x):
    """Decodes a bf16/fp16 tensor to float64 with the oracle's own decoder."""
    bits, code = _bits(x)
    out = np.empty(bits.shape, dtype=np.float64)
    _check(load().oracle_decode_bits_f64(_p(bits), bits.size, code, _p(out)), "decode_bits")
    return out


def varlen_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, scale=None, return_lse=False,
               return_wsum=False, return_abs=False):
    """Whole varlen prefill; rows outside every query segment come back NaN.

    ``return_abs`` also returns the same softmax weights applied to |v|
    (what ``varlen_fwd`` gives for ``v.abs()``, computed in the same pass):
    the magnitude the parity bar scales rounding errors with.  Extra results
    follow ``out`` in the order lse, wsum, abs.
    """
    qb, code = _bits(q)
    kb, kcode = _bits(k)
    vb, vcode = _bits(v)
    if not (code == kcode == vcode):
        raise TypeError("q, k and v must share one dtype")
    total_q, H, D = qb.shape
    total_k = kb.shape[0]
    if kb.shape[1:] != (H, D) or vb.shape != kb.shape:
        raise ValueError("k and v must be [total_k, H, D] with q's H and D")
    cq, ck = _i32(cu_seqlens_q), _i32(cu_seqlens_k)
    if cq.shape != ck.shape or cq.ndim != 1 or cq.size < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must be 1-D of equal length")
    scale = D ** -0.5 if scale is None else float(scale)
    out = np.empty((total_q, H, D), dtype=np.float64)
    lse = np.empty((total_q, H), dtype=np.float64) if return_lse else None
    wsum = np.empty((total_q, H), dtype=np.float64) if return_wsum else None
    oabs = np.empty((total_q, H, D), dtype=np.float64) if return_abs else None
    rc = load().oracle_varlen_fwd_f64(_p(qb), _p(kb), _p(vb), code, _p(cq), _p(ck), cq.size - 1,
                                      total_q, total_k, H, D, scale, _p(out), _p(lse), _p(wsum),
                                      _p(oabs))
    _check(rc, "varlen_fwd")
    res = ([out] + ([lse] if return_lse else []) + ([wsum] if return_wsum else [])
           + ([oabs] if return_abs else []))
    return res[0] if len(res) == 1 else tuple(res)


def varlen_fwd_rows(q, k, v, cu_seqlens_q, cu_seqlens_k, rows, heads, scale=None,
                    return_lse=False, return_abs=False):
    """The prefill definition at chosen (row, head) pairs only: out [n, D].

    ``return_abs`` as in ``varlen_fwd``; extra results follow ``out`` in the
    order lse, abs."""
    qb, code = _bits(q)
    kb, _ = _bits(k)
    vb, _ = _bits(v)
    total_q, H, D = qb.shape
    cq, ck = _i32(cu_seqlens_q), _i32(cu_seqlens_k)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    heads = np.ascontiguousarray(heads, dtype=np.int32)
    if rows.shape != heads.shape or rows.ndim != 1:
        raise ValueError("rows and heads must be 1-D of equal length")
    scale = D ** -0.5 if scale is None else float(scale)
    out = np.empty((rows.size, D), dtype=np.float64)
    lse = np.empty(rows.size, dtype=np.float64) if return_lse else None
    oabs = np.empty((rows.size, D), dtype=np.float64) if return_abs else None
    rc = load().oracle_varlen_fwd_rows_f64(_p(qb), _p(kb), _p(vb), code, _p(cq), _p(ck),
                                           cq.size - 1, total_q, kb.shape[0], H, D, scale,
                                           _p(rows), _p(heads), rows.size, _p(out), _p(lse),
                                           _p(oabs))
    _check(rc, "varlen_fwd_rows")
    res = [out] + ([lse] if return_lse else []) + ([oabs] if return_abs else [])
    return res[0] if len(res) == 1 else tuple(res)


def _decode_dims(query, k_cache, v_cache, block_tables):
    num_seqs, num_query_heads, head_size = query.shape
    num_kv_heads = v_cache.shape[1]
    block_size = v_cache.shape[3]
    num_blocks = v_cache.shape[0]
    x = 16 // 2
    if tuple(k_cache.shape) != (num_blocks, num_kv_heads, head_size // x, block_size, x):
        raise ValueError(f"k_cache shape {tuple(k_cache.shape)} does not match the layout "
                         "[blocks, kv_heads, head_size/x, block_size, x]")
    if tuple(v_cache.shape) != (num_blocks, num_kv_heads, head_size, block_size):
        raise ValueError("v_cache must be [blocks, kv_heads, head_size, block_size]")
    if block_tables.ndim != 2 or block_tables.shape[0] != num_seqs:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
    return num_seqs, num_query_heads, num_kv_heads, head_size, block_size, num_blocks


def paged_decode(query, k_cache, v_cache, block_tables, seq_lens, scale=None, return_lse=False):
    """Whole paged decode: out [num_seqs, num_query_heads, head_size] float64."""
    qb, code = _bits(query)
    kb, _ = _bits(k_cache)
    vb, _ = _bits(v_cache)
    bt, sl = _i32(block_tables), _i32(seq_lens)
    S, Hq, Hkv, D, bs, nb = _decode_dims(qb, kb, vb, bt)
    scale = D ** -0.5 if scale is None else float(scale)
    out = np.empty((S, Hq, D), dtype=np.float64)
    lse = np.empty((S, Hq), dtype=np.float64) if return_lse else None
    rc = load().oracle_paged_decode_f64(_p(qb), _p(kb), _p(vb), code, _p(bt), _p(sl), S, Hq, Hkv,
                                        D, bs, bt.shape[1], nb, scale, _p(out), _p(lse))
    _check(rc, "paged_decode")
    return (out, lse) if return_lse else out


def paged_gather(k_cache, v_cache, block_tables, seq, ctx_len, kv_head):
    """The oracle's gather of one sequence: (K [L, D], V [L, D], slots [L])."""
    kb, code = _bits(k_cache)
    vb, _ = _bits(v_cache)
    bt = _i32(block_tables)
    nb, Hkv, D, bs = vb.shape
    L = int(ctx_len)
    K = np.empty((max(L, 0), D), dtype=np.float64)
    V = np.empty((max(L, 0), D), dtype=np.float64)
    slots = np.empty(max(L, 0), dtype=np.int64)
    rc = load().oracle_paged_gather_f64(_p(kb), _p(vb), code, _p(bt), int(seq), L, nb, Hkv, D, bs,
                                        bt.shape[1], int(kv_head), _p(K), _p(V), _p(slots))
    _check(rc, "paged_gather")
    return K, V, slots


def num_threads():
    """Threads the oracle's OpenMP regions use."""
    return load().oracle_num_threads()
