"""CPU oracle for the output step of chunked gated delta-rule linear attention
-- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  It wraps ``chunk_oracle.c`` (plain C, double precision, OpenMP)
through ctypes and shares nothing with the GPU library.

Shapes follow the operator page (atrex-bench "chunk_delta_rule_output" #004,
Reference Implementation): ``q`` and ``k`` are ``[batch, tokens, num_q_heads,
key_dim]``, ``v`` is ``[batch, tokens, num_heads, value_dim]`` (its last two
dimensions give the value-head count and the value width), ``h`` is
``[batch, num_chunks, num_heads, key_dim, value_dim]`` and ``g`` is float32
``[batch, tokens, num_heads]``.  The default scale is ``key_dim ** -0.5``.
Inputs are CPU tensors (q, k, v, h in bfloat16 or float16, g in float32);
results are float64 numpy arrays of v's shape.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "chunk_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libchunk_oracle.so")
_lib = None

BF16, FP16 = 0, 1


def build(force=True):
    """Compiles chunk_oracle.c to libchunk_oracle.so with gcc (no fast-math)."""
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
    """Loads the library (building it first if it is missing)."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _lib is None:
        override = os.environ.get("ATTN_CHUNK_ORACLE_LIB")   # another build of the same source
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
    lib.oracle_chunk_delta_out_f64.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32,
                                               f64, i32, i32, P]
    lib.oracle_chunk_delta_out_f64.restype = ctypes.c_int
    lib.oracle_chunk_delta_out_rows_f64.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32,
                                                    i32, f64, i32, i32, P, P, i64, P]
    lib.oracle_chunk_delta_out_rows_f64.restype = ctypes.c_int
    lib.oracle_round_to_dtype.argtypes = [f64, i32]
    lib.oracle_round_to_dtype.restype = ctypes.c_double
    return lib


def _bits(x):
    import torch
    if x.dtype == torch.bfloat16:
        code = BF16
    elif x.dtype == torch.float16:
        code = FP16
    else:
        raise TypeError(f"expected bfloat16 or float16, got {x.dtype}")
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16), code


def _f32(x):
    if not isinstance(x, np.ndarray):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(x, dtype=np.float32)


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dims(q, k, v, h, g, chunk_size):
    B, T, Hq, K = q.shape
    H, V = v.shape[2], v.shape[3]
    nc = (T + chunk_size - 1) // chunk_size
    if tuple(k.shape) != (B, T, Hq, K) or tuple(v.shape[:2]) != (B, T):
        raise ValueError("q, k must be [B, T, Hq, K] and v [B, T, H, V]")
    if tuple(h.shape) != (B, nc, H, K, V) or tuple(g.shape) != (B, T, H):
        raise ValueError("h must be [B, num_chunks, H, K, V] and g [B, T, H]")
    return B, T, Hq, H, K, V


def round_to_dtype(x, dtype_code):
    """The oracle's rounding of a double to bf16 (0) or fp16 (1) values."""
    return load().oracle_round_to_dtype(float(x), int(dtype_code))


def chunk_delta_out(q, k, v, h, g, chunk_size=64, scale=None, absolute=False):
    """Whole output, float64 [B, T, H, V].  With ``absolute`` the bound
    magnitude (every product taken in absolute value) instead."""
    B, T, Hq, H, K, V = _dims(q, k, v, h, g, chunk_size)
    qb, code = _bits(q)
    kb, c2 = _bits(k)
    vb, c3 = _bits(v)
    hb, c4 = _bits(h)
    if len({code, c2, c3, c4}) != 1:
        raise TypeError("q, k, v, h must share one dtype")
    gf = _f32(g)
    scale = K ** -0.5 if scale is None else float(scale)
    out = np.zeros((B, T, H, V), dtype=np.float64)
    rc = load().oracle_chunk_delta_out_f64(_p(qb), _p(kb), _p(vb), _p(hb), _p(gf), B, T, Hq, H, K,
                                           V, int(chunk_size), scale, code, int(bool(absolute)),
                                           _p(out))
    if rc != 0:
        raise ValueError(f"chunk_delta_out: oracle rejected its arguments (code {rc})")
    return out


def chunk_delta_out_rows(q, k, v, h, g, rows, heads, chunk_size=64, scale=None, absolute=False):
    """Selected output rows: ``rows`` are flat token indices b * T + t,
    ``heads`` value heads; float64 [len(rows), V]."""
    B, T, Hq, H, K, V = _dims(q, k, v, h, g, chunk_size)
    qb, code = _bits(q)
    kb, _ = _bits(k)
    vb, _ = _bits(v)
    hb, _ = _bits(h)
    gf = _f32(g)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    heads = np.ascontiguousarray(heads, dtype=np.int32)
    if rows.shape != heads.shape:
        raise ValueError("rows and heads must have the same length")
    scale = K ** -0.5 if scale is None else float(scale)
    out = np.zeros((rows.size, V), dtype=np.float64)
    rc = load().oracle_chunk_delta_out_rows_f64(_p(qb), _p(kb), _p(vb), _p(hb), _p(gf), B, T, Hq,
                                                H, K, V, int(chunk_size), scale, code,
                                                int(bool(absolute)), _p(rows), _p(heads),
                                                rows.size, _p(out))
    if rc != 0:
        raise ValueError(f"chunk_delta_out_rows: oracle rejected its arguments (code {rc})")
    return out
