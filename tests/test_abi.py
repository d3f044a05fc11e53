"""The C ABI of libattn without a GPU: the library loads, exports every
function include/attn.h declares, and rejects bad arguments on the host
before anything is enqueued (no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")
LIB = os.path.join(ROOT, "softmax_attention_flashattention_amd", "libattn.so")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = 4096          # an aligned, never-dereferenced stand-in for a device pointer


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libattn.so is not built")
    from softmax_attention_flashattention_amd import binding
    return binding._load()


def test_every_declared_function_is_exported(lib):
    names = declared_functions()
    assert set(names) >= {"attn_varlen_fwd", "attn_varlen_fwd_workspace_size",
                          "attn_paged_decode", "attn_status_string",
                          "attn_paged_decode_workspace_size", "attn_paged_decode_num_partitions",
                          "attn_chunk_delta_out", "attn_paged_decode_noalloc"}
    for n in names:
        assert hasattr(lib, n), f"{n} declared in attn.h but not exported"


def test_status_strings(lib):
    assert lib.attn_status_string(0) == b"ATTN_OK"
    assert lib.attn_status_string(1) == b"ATTN_ERR_INVALID_ARG"
    assert lib.attn_status_string(2) == b"ATTN_ERR_UNSUPPORTED"
    assert lib.attn_status_string(3) == b"ATTN_ERR_WORKSPACE"
    assert lib.attn_status_string(4) == b"ATTN_ERR_HIP"
    assert lib.attn_status_string(99) == b"ATTN_ERR_UNKNOWN"


def varlen(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, cu_q=FAKE, cu_k=FAKE, num_seqs=1, max_seqlen_q=16,
             total_q=16, total_k=16, num_heads=2, head_dim=128, scale=0.1, dtype=0, ws=None,
             ws_bytes=0, out=FAKE)
    a.update(kw)
    return lib.attn_varlen_fwd(a["q"], a["k"], a["v"], a["cu_q"], a["cu_k"], a["num_seqs"],
                               a["max_seqlen_q"], a["total_q"], a["total_k"], a["num_heads"],
                               a["head_dim"], a["scale"], a["dtype"], a["ws"], a["ws_bytes"],
                               a["out"], None)


def test_varlen_argument_errors(lib):
    assert varlen(lib, head_dim=64) == UNSUPPORTED
    assert varlen(lib, head_dim=0) == INVALID
    assert varlen(lib, num_heads=0) == INVALID
    assert varlen(lib, num_seqs=-1) == INVALID
    assert varlen(lib, max_seqlen_q=-5) == INVALID
    assert varlen(lib, total_k=-1) == INVALID
    assert varlen(lib, dtype=7) == INVALID
    assert varlen(lib, scale=float("nan")) == INVALID
    assert varlen(lib, scale=float("inf")) == INVALID
    assert varlen(lib, q=None) == INVALID
    assert varlen(lib, out=None) == INVALID
    assert varlen(lib, cu_k=None) == INVALID
    assert varlen(lib, k=None) == INVALID              # keys exist (total_k = 16)
    assert varlen(lib, k=FAKE + 8) == INVALID          # not 16-byte aligned
    assert varlen(lib, cu_q=FAKE + 2) == INVALID       # not 4-byte aligned
    assert varlen(lib, ws=FAKE + 16, ws_bytes=1 << 20) == INVALID   # not 256-byte aligned
    # a 64-row key tile must be addressable with 32-bit byte offsets
    assert varlen(lib, num_heads=(1 << 25) // 128) == INVALID
    assert varlen(lib, num_heads=(1 << 25) // 72 + 1, head_dim=72) == INVALID


def test_varlen_empty_work_is_ok_without_launch(lib):
    assert varlen(lib, num_seqs=0, q=None, out=None) == OK
    assert varlen(lib, max_seqlen_q=0, q=None) == OK
    assert varlen(lib, total_q=0, q=None) == OK


def decode(lib, **kw):
    a = dict(query=FAKE, k=FAKE, v=FAKE, bt=FAKE, sl=FAKE, num_seqs=4, hq=16, hkv=16, d=128,
             bs=16, maxb=4, nb=32, scale=0.1, dtype=0, part=0, ws=None, ws_bytes=0, out=FAKE)
    a.update(kw)
    return lib.attn_paged_decode(a["query"], a["k"], a["v"], a["bt"], a["sl"], a["num_seqs"],
                                 a["hq"], a["hkv"], a["d"], a["bs"], a["maxb"], a["nb"], a["scale"],
                                 a["dtype"], a["part"], a["ws"], a["ws_bytes"], a["out"], None)


def test_decode_argument_errors(lib):
    assert decode(lib, hkv=3) == INVALID               # 16 % 3 != 0
    assert decode(lib, d=64) == UNSUPPORTED
    assert decode(lib, d=192) == UNSUPPORTED
    assert decode(lib, d=12) == INVALID                # not a multiple of x = 8
    assert decode(lib, bs=32) == UNSUPPORTED
    assert decode(lib, hq=34, hkv=2) == UNSUPPORTED    # group of 17
    assert decode(lib, part=24) == INVALID             # not a multiple of block_size
    assert decode(lib, part=-16) == INVALID
    assert decode(lib, num_seqs=-1) == INVALID
    assert decode(lib, nb=-1) == INVALID
    assert decode(lib, dtype=2) == INVALID
    assert decode(lib, scale=float("nan")) == INVALID
    assert decode(lib, query=None) == INVALID
    assert decode(lib, bt=None) == INVALID
    assert decode(lib, v=FAKE + 4) == INVALID
    assert decode(lib, sl=FAKE + 1) == INVALID


def test_decode_workspace_rules(lib):
    # (num_seqs, num_kv_heads, max_blocks_per_seq, block_size, partition_size)
    # 64 x 16 workgroups fill the device at the default 512-token partition:
    # 64 blocks per sequence give 2 partitions
    assert lib.attn_paged_decode_num_partitions(64, 16, 64, 16, 0) == 2
    assert lib.attn_paged_decode_num_partitions(64, 16, 4, 16, 0) == 1
    # 1 sequence x 2 KV heads: 512 tokens halved down to 128, so 1024 tokens
    # give 8 partitions; 128 tokens stay one
    assert lib.attn_paged_decode_num_partitions(1, 2, 64, 16, 0) == 8
    assert lib.attn_paged_decode_num_partitions(1, 2, 8, 16, 0) == 1
    assert lib.attn_paged_decode_num_partitions(4, 16, 4, 16, 16) == 4
    assert lib.attn_paged_decode_num_partitions(4, 16, 4, 16, 24) == -INVALID
    assert lib.attn_paged_decode_num_partitions(4, 0, 4, 16, 0) == -INVALID
    # (num_seqs, num_query_heads, num_kv_heads, head_size, max_blocks_per_seq, ...)
    need64 = lib.attn_paged_decode_workspace_size(64, 16, 16, 128, 64, 16, 0)
    rows = 64 * 16 * 2
    assert need64 == (rows * 8 + 255) // 256 * 256 + rows * 128 * 4
    assert lib.attn_paged_decode_workspace_size(64, 16, 16, 128, 4, 16, 0) == 0
    need = lib.attn_paged_decode_workspace_size(4, 16, 16, 128, 64, 16, 0)
    assert need > 0
    assert decode(lib, maxb=64, ws=None, ws_bytes=0) == WORKSPACE
    assert decode(lib, maxb=64, ws=FAKE, ws_bytes=need - 1) == WORKSPACE
    assert decode(lib, maxb=64, ws=FAKE + 16, ws_bytes=need) == WORKSPACE   # not 256-aligned


def decode_noalloc(lib, **kw):
    a = dict(query=FAKE, k=FAKE, v=FAKE, bt=FAKE, sl=FAKE, num_seqs=4, hq=16, hkv=16, d=128,
             bs=16, maxb=4, nb=32, scale=0.1, dtype=0, part=0, out=FAKE)
    a.update(kw)
    return lib.attn_paged_decode_noalloc(a["query"], a["k"], a["v"], a["bt"], a["sl"],
                                         a["num_seqs"], a["hq"], a["hkv"], a["d"], a["bs"],
                                         a["maxb"], a["nb"], a["scale"], a["dtype"], a["part"],
                                         a["out"], None)


def test_decode_noalloc_rejects_what_its_buffer_cannot_hold(lib):
    # the same argument checks as attn_paged_decode, then the split's partial
    # results must fit the static 64 MiB buffer: refused before any device call
    assert decode_noalloc(lib, hkv=3) == INVALID
    assert decode_noalloc(lib, d=64) == UNSUPPORTED
    assert decode_noalloc(lib, part=24) == INVALID
    assert decode_noalloc(lib, query=None) == INVALID
    limit = 64 << 20
    big = dict(num_seqs=256, hq=64, hkv=8, maxb=64, part=16)      # 64 partitions each
    need = lib.attn_paged_decode_workspace_size(256, 64, 8, 128, 64, 16, 16)
    assert need > limit
    assert decode_noalloc(lib, **big) == WORKSPACE
    fits = lib.attn_paged_decode_workspace_size(256, 64, 8, 128, 64, 16, 256)   # 4 partitions
    assert 0 < fits <= limit


def test_decode_empty_batch_is_ok_without_launch(lib):
    assert decode(lib, num_seqs=0, query=None) == OK


def chunk(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, h=FAKE, g=FAKE, batch=1, tokens=100, hq=16, hv=32, kd=128,
             vd=128, cs=64, scale=0.1, dtype=0, out=FAKE)
    a.update(kw)
    return lib.attn_chunk_delta_out(a["q"], a["k"], a["v"], a["h"], a["g"], a["batch"], a["tokens"],
                                    a["hq"], a["hv"], a["kd"], a["vd"], a["cs"], a["scale"],
                                    a["dtype"], a["out"], None)


def test_chunk_argument_errors(lib):
    assert chunk(lib, kd=64) == UNSUPPORTED
    assert chunk(lib, vd=256) == UNSUPPORTED
    assert chunk(lib, cs=32) == UNSUPPORTED
    assert chunk(lib, batch=-1) == INVALID
    assert chunk(lib, tokens=-5) == INVALID
    assert chunk(lib, hq=0) == INVALID
    assert chunk(lib, hv=0) == INVALID
    assert chunk(lib, cs=0) == INVALID
    assert chunk(lib, dtype=3) == INVALID
    assert chunk(lib, scale=float("inf")) == INVALID
    assert chunk(lib, h=None) == INVALID
    assert chunk(lib, g=None) == INVALID
    assert chunk(lib, out=FAKE + 8) == INVALID         # not 16-byte aligned
    assert chunk(lib, g=FAKE + 2) == INVALID           # not 4-byte aligned
    # one chunk of q/k or v rows must be addressable with 32-bit offsets
    assert chunk(lib, hv=131072) == INVALID
    assert chunk(lib, hq=131072) == INVALID


def test_chunk_empty_input_is_ok_without_launch(lib):
    assert chunk(lib, tokens=0, q=None, k=None, v=None, h=None, g=None, out=None) == OK
    assert chunk(lib, batch=0, q=None) == OK


def test_binding_names_match_the_header():
    import softmax_attention_flashattention_amd as pkg
    for n in declared_functions():
        assert hasattr(pkg, n), f"binding lacks {n}"


def test_binding_checks_tensors_before_any_call():
    # host tensors and non-tensors are refused by the binding with the name
    # of the offending argument; nothing reaches the library (these run
    # without a GPU)
    import torch
    import softmax_attention_flashattention_amd as pkg
    q = torch.zeros(8, 2, 128, dtype=torch.bfloat16)
    cu = torch.tensor([0, 8], dtype=torch.int32)
    with pytest.raises(ValueError, match="q must be a GPU tensor"):
        pkg.attn_varlen_fwd(q, q, q, cu, cu, max_seqlen_q=8)
    with pytest.raises(TypeError, match="q must be a torch.Tensor"):
        pkg.attn_varlen_fwd(None, q, q, cu, cu, max_seqlen_q=8)
    query = torch.zeros(2, 4, 128, dtype=torch.float16)
    kc = torch.zeros(3, 4, 16, 16, 8, dtype=torch.float16)
    vc = torch.zeros(3, 4, 128, 16, dtype=torch.float16)
    bt = torch.zeros(2, 1, dtype=torch.int32)
    sl = torch.ones(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="query must be a GPU tensor"):
        pkg.attn_paged_decode(query, kc, vc, bt, sl)
    with pytest.raises(ValueError, match="query must be a GPU tensor"):
        pkg.attn_paged_decode_noalloc(query, kc, vc, bt, sl)
    x = torch.zeros(1, 64, 2, 128, dtype=torch.bfloat16)
    h = torch.zeros(1, 1, 2, 128, 128, dtype=torch.bfloat16)
    g = torch.zeros(1, 64, 2)
    with pytest.raises(ValueError, match="q must be a GPU tensor"):
        pkg.attn_chunk_delta_out(x, x, x, h, g)
