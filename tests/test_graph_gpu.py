"""The entry points captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: every replay must reproduce the eager call's output bit for bit.

Launch-bound callers (small shapes, serving loops) replay captured calls
instead of paying the per-call host path each time.  A call enqueues its
kernels on the caller's stream and does no host synchronisation, device
allocation or memset, so it can be captured as it is (prefill needs
`max_seqlen_q` passed in: deriving it reads the sequence bounds back to the
host).  Each case uses the work split that adds a second kernel (prefill key
ranges and their merge, decode context partitions and their merge), and
each replay is checked with eager calls and synchronisations in between.
"""
import pytest
import torch

from parity import to_gpu
from softmax_attention_flashattention_amd import (attn_chunk_delta_out, attn_paged_decode,
                                                  attn_varlen_fwd, inputs as gen)

pytestmark = pytest.mark.gpu


def replay_matches_eager(call, what, reps=4):
    print(f"[graph] {what}", flush=True)
    eager = call().clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = call()
    torch.cuda.synchronize()
    for i in range(reps):
        out.fill_(7.0)           # the replay must rewrite every element
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"{what}: replay {i} differs from the eager call"
        again = call()           # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(again, eager), f"{what}: eager call after replay {i} differs"


@pytest.mark.parametrize("D", [72, 128])
def test_prefill_split_and_merge_replays(D):
    # few work items (2024 tokens x 4 heads at head_dim 128, x 10 heads at
    # 72): every item is split into key ranges, so the graph holds the
    # prefill kernel and the merge kernel
    H = 10 if D == 72 else 4
    inp = gen.prefill_inputs([2024], H, D, seed=90 + D)
    d = to_gpu(inp)
    replay_matches_eager(
        lambda: attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"],
                                max_seqlen_q=2024),
        f"prefill 2024 x {H} heads, D={D}")


@pytest.mark.parametrize("S,H", [(276, 4), (2024, 4)])
def test_prefill_key_splitting_workgroups_replay(S, H):
    # head_dim 72 on a small grid: one kernel whose workgroups merge their
    # waves' key ranges in LDS
    inp = gen.prefill_inputs([S], H, 72, seed=97 + S)
    d = to_gpu(inp)
    replay_matches_eager(
        lambda: attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"],
                                max_seqlen_q=S),
        f"prefill {S} x {H} heads, D=72, key-splitting workgroups")


@pytest.mark.parametrize("S,H", [(5888, 12), (33024, 2)])
def test_prefill_head_dim_72_split_replays(S, H):
    # head_dim 72 with a split last wave, merged: 5888 x 12 heads on 8-wave
    # workgroups of 32-row waves, 33024 x 2 heads on 64-row waves
    inp = gen.prefill_inputs([S], H, 72, seed=95)
    d = to_gpu(inp)
    replay_matches_eager(
        lambda: attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"],
                                max_seqlen_q=S),
        f"prefill {S} x {H} heads, D=72")


def test_prefill_varlen_batch_replays():
    inp = gen.prefill_inputs([300, 1, 777], 2, 128, seed=93)
    d = to_gpu(inp)
    replay_matches_eager(
        lambda: attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"],
                                max_seqlen_q=777),
        "prefill varlen batch")


def test_decode_partitions_and_merge_replay():
    lens = [1000, 333, 17, 0, 512, 1]
    inp = gen.decode_inputs(6, 1000, 8, 4, 128, seed=94, seq_lens=lens)
    d = to_gpu(inp)
    replay_matches_eager(
        lambda: attn_paged_decode(d["query"], d["k_cache"], d["v_cache"], d["block_tables"],
                                  d["seq_lens"], partition_size=112),
        "decode, 112-token partitions")


def test_decode_workload_replays():
    d = to_gpu(gen.workload_inputs("decode_b256_ctx64_h16_kv16_d128"))
    replay_matches_eager(
        lambda: attn_paged_decode(d["query"], d["k_cache"], d["v_cache"], d["block_tables"],
                                  d["seq_lens"]),
        "decode 256 x 64")


def test_chunk_output_replays():
    x = gen.chunk_inputs(2, 300, 2, 4, seed=95)
    d = to_gpu(x)
    replay_matches_eager(
        lambda: attn_chunk_delta_out(d["q"], d["k"], d["v"], d["h"], d["g"]),
        "chunk output 2 x 300 tokens")


def test_calls_take_torch_current_stream():
    # the binding hands the library torch's current stream of the tensors'
    # device: inside a stream context that stream's handle, outside it the
    # default one
    from softmax_attention_flashattention_amd import binding
    dev = torch.cuda.current_device()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        assert binding._stream(dev) == s.cuda_stream
    assert binding._stream(dev) == torch.cuda.current_stream(dev).cuda_stream
    # and a call issued inside the context runs on that stream, ordered after
    # the work already queued there
    inp = gen.prefill_inputs([300], 2, 72, seed=99)
    d = to_gpu(inp)
    eager = attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"], max_seqlen_q=300)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        q2 = d["q"].clone()          # queued on s before the call
        out = attn_varlen_fwd(q2, d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"], max_seqlen_q=300)
    s.synchronize()
    assert torch.equal(out, eager)
