/*
 * attn.h -- libattn: exact softmax attention forward on AMD Instinct MI355X
 * (gfx950, CDNA4), and the output step of chunked linear attention.
 *
 * Two operators share one definition: for every sequence and head,
 *
 *     out = softmax(scale * Q K^T) V,
 *
 * accumulated in fp32 and written in the input's 16-bit type (bf16 or fp16).
 * The definition and both data layouts are those of the atrex-bench operator
 * pages "attention_forward" (#001) and "paged_attention_decode" (#024),
 * sections "Reference Implementation" and "Input Generation".  A third entry
 * point, attn_chunk_delta_out, computes the page "chunk_delta_rule_output"
 * (#004): a gated, causal, unnormalised variant over chunks of 64 tokens.
 *
 * Conventions shared by every entry point
 *  - Every tensor pointer is device memory owned by the caller.  The library
 *    never allocates, frees or synchronises; it writes only `out` and the
 *    caller's `workspace` (prefill's key-range split, decode's context
 *    partitions), or for attn_paged_decode_noalloc its static buffer.
 *  - Calls enqueue their kernels on `stream` (a hipStream_t; NULL is the null
 *    stream) and return at once.  They never read device memory on the host
 *    and issue no memset, so a call can be captured into a HIP graph and
 *    replayed (the captured pointers and sizes are reused as they are).
 *  - 16-bit tensors are contiguous, row-major, and 16-byte aligned; int32
 *    index arrays are contiguous and 4-byte aligned.
 *  - Calls return an attn_status and never print, throw or abort.  Argument
 *    errors are detected on the host before anything is enqueued; a launch
 *    failure reported by the HIP runtime maps to ATTN_ERR_HIP.
 *  - Device-side contents that contradict the sizes passed (cu_seqlens that
 *    decrease or point past total_q / total_k, block-table entries outside
 *    [0, num_blocks), seq_lens above max_blocks_per_seq * block_size) are a
 *    caller error with unspecified output values; the kernels clamp such
 *    indices so that they never read or write outside the buffers described
 *    by the size arguments.
 *  - The only mutable global state is attn_paged_decode_noalloc's device
 *    buffer (one per GPU) and its looked-up address, and facts about each
 *    device the launch plans use (compute units, resident workgroups per
 *    kernel), queried once on a device's first call and kept; other calls on
 *    different streams may run concurrently as long as their
 *    `out`/`workspace` buffers differ.
 */
#ifndef LIBATTN_ATTN_H
#define LIBATTN_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_INVALID_ARG = 1, /* null/misaligned pointer, negative size, Hq % Hkv != 0, bad scale */
    ATTN_ERR_UNSUPPORTED = 2, /* well-formed request outside the built kernels (head_dim, block_size) */
    ATTN_ERR_WORKSPACE = 3,   /* decode workspace missing or too small */
    ATTN_ERR_HIP = 4          /* the HIP runtime reported an error at launch */
} attn_status;

typedef enum attn_dtype {
    ATTN_DTYPE_BF16 = 0,
    ATTN_DTYPE_FP16 = 1
} attn_dtype;

/*
 * attn_varlen_fwd -- non-causal variable-length prefill attention.
 *
 * Defined by "attention_forward" (#001), Reference Implementation: for each
 * sequence i, query rows [cu_seqlens_q[i], cu_seqlens_q[i+1]) attend to key
 * rows [cu_seqlens_k[i], cu_seqlens_k[i+1]) of the same head, with no mask.
 *
 *  q              [total_q, num_heads, head_dim], dtype
 *  k, v           [total_k, num_heads, head_dim], dtype; may be NULL when
 *                 total_k == 0
 *  cu_seqlens_q   [num_seqs + 1] int32, non-decreasing, cu_seqlens_q[0] >= 0,
 *                 cu_seqlens_q[num_seqs] <= total_q
 *  cu_seqlens_k   [num_seqs + 1] int32, the same rules against total_k
 *  max_seqlen_q   an upper bound on cu_seqlens_q[i+1] - cu_seqlens_q[i]; it
 *                 sizes the grid (whole tiles of query rows), so a segment
 *                 longer than it is a caller error: its rows past the last
 *                 tile the bound covers are left unwritten
 *  head_dim       72 or 128 (others return ATTN_ERR_UNSUPPORTED)
 *  num_heads      num_heads * head_dim < 2^25 (a key tile of 64 rows is
 *                 addressed with 32-bit byte offsets); larger returns
 *                 ATTN_ERR_INVALID_ARG
 *  scale          finite, of either sign or 0; the pages use head_dim^-1/2
 *  workspace      optional device memory, 256-byte aligned, of
 *                 attn_varlen_fwd_workspace_size(...) bytes.  When the work
 *                 items would leave the device's last wave of workgroups
 *                 partly empty, the items of that wave may be split into key
 *                 ranges (when there are fewer items than half the device
 *                 holds at once, every item is) whose partial results go
 *                 here and a second kernel merges them.  NULL (or too small)
 *                 runs every item whole: the same result up to rounding,
 *                 only slower in those cases.  head_dim-72 grids whose
 *                 32-row items all fit the device at once (and
 *                 max_seqlen_q <= 8192) split the keys inside each
 *                 workgroup instead and use no workspace (size 0).
 *  out            [total_q, num_heads, head_dim], dtype.  Only rows inside a
 *                 query segment are written; a sequence with query rows but
 *                 no key rows gets all-zero rows.  Other rows are untouched.
 *
 * num_seqs == 0, max_seqlen_q == 0 or total_q == 0 is a valid no-op.
 */
attn_status attn_varlen_fwd(const void *q, const void *k, const void *v,
                    const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                    int32_t num_seqs, int32_t max_seqlen_q,
                    int64_t total_q, int64_t total_k,
                    int32_t num_heads, int32_t head_dim, float scale,
                    int32_t dtype, void *workspace, size_t workspace_bytes,
                    void *out, void *stream);

/*
 * Workspace bytes attn_varlen_fwd can use for these sizes on the current
 * device (0 when no split applies, on invalid sizes, or when the device
 * cannot be queried).
 */
size_t attn_varlen_fwd_workspace_size(int32_t num_seqs, int32_t max_seqlen_q,
                                      int32_t num_heads, int32_t head_dim);

/*
 * attn_paged_decode -- single-query attention over a paged KV cache with
 * grouped-query heads.
 *
 * Defined by "paged_attention_decode" (#024), Reference Implementation and
 * Input Generation.  Token t of sequence s lives in physical block
 * block_tables[s][t / block_size] at slot t % block_size; query head hq
 * reads KV head hq / (num_query_heads / num_kv_heads).
 *
 *  query          [num_seqs, num_query_heads, head_size], dtype
 *  k_cache        [num_blocks, num_kv_heads, head_size / 8, block_size, 8]
 *                 (x = 16 bytes / element size = 8)
 *  v_cache        [num_blocks, num_kv_heads, head_size, block_size]
 *  block_tables   [num_seqs, max_blocks_per_seq] int32; only the first
 *                 ceil(seq_lens[s] / block_size) entries of a row are read
 *  seq_lens       [num_seqs] int32; seq_lens[s] <= 0 gives an all-zero row
 *  head_size      128 or 256 (others return ATTN_ERR_UNSUPPORTED)
 *  block_size     16 (others return ATTN_ERR_UNSUPPORTED)
 *  num_query_heads % num_kv_heads must be 0; the group size
 *                 num_query_heads / num_kv_heads must be at most 16
 *  partition_size tokens per split of the context (split-K); a positive
 *                 value must be a multiple of block_size.  0 lets the
 *                 library choose: 512 tokens, halved down to 128 while
 *                 num_seqs x num_kv_heads x partitions (one workgroup each)
 *                 is below the current device's compute-unit count.  With
 *                 more than one partition the kernel writes per-partition
 *                 (max, sum, partial output) into `workspace` and a second
 *                 kernel merges them by log-sum-exp.
 *  workspace      device memory of attn_paged_decode_workspace_size(...)
 *                 bytes, 256-byte aligned; may be NULL when that size is 0
 *  out            [num_seqs, num_query_heads, head_size], dtype; every row is
 *                 written
 *
 * num_seqs == 0 is a valid no-op.
 */
attn_status attn_paged_decode(const void *query, const void *k_cache, const void *v_cache,
                      const int32_t *block_tables, const int32_t *seq_lens,
                      int32_t num_seqs, int32_t num_query_heads, int32_t num_kv_heads,
                      int32_t head_size, int32_t block_size, int32_t max_blocks_per_seq,
                      int64_t num_blocks, float scale, int32_t dtype,
                      int32_t partition_size, void *workspace, size_t workspace_bytes,
                      void *out, void *stream);

/*
 * attn_paged_decode_noalloc -- attn_paged_decode without a caller workspace,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  It
 * allocates nothing.  Arguments, layouts, results and errors are those of
 * attn_paged_decode; a split context keeps its per-partition partial results
 * in a static device buffer of ATTN_NOALLOC_SCRATCH_BYTES instead (one per
 * GPU, held until the process ends).
 *
 *  - Returns ATTN_ERR_WORKSPACE, before touching the device, when
 *    attn_paged_decode_workspace_size(...) for the call exceeds
 *    ATTN_NOALLOC_SCRATCH_BYTES (pick a larger partition_size, or use
 *    attn_paged_decode with a workspace).
 *  - The first call on a device looks the buffer's address up (a runtime
 *    symbol query, no allocation); make it outside graph capture if the
 *    capture mode forbids runtime queries.  `stream` must belong to the
 *    current device.
 *  - Every call on one GPU shares that GPU's buffer: calls that may overlap
 *    on one GPU (different streams, different host threads) race and give
 *    unspecified output.  Calls in one stream are ordered and safe.  Nothing
 *    in the buffer needs to start zeroed: each partition a merge reads is
 *    written by the same call.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
attn_status attn_paged_decode_noalloc(const void *query, const void *k_cache, const void *v_cache,
                              const int32_t *block_tables, const int32_t *seq_lens,
                              int32_t num_seqs, int32_t num_query_heads, int32_t num_kv_heads,
                              int32_t head_size, int32_t block_size, int32_t max_blocks_per_seq,
                              int64_t num_blocks, float scale, int32_t dtype,
                              int32_t partition_size, void *out, void *stream);

/*
 * Number of context partitions attn_paged_decode will use for these sizes on
 * the current device (1 means no split and no workspace).  Returns a
 * negative attn_status value on invalid sizes.
 */
int32_t attn_paged_decode_num_partitions(int32_t num_seqs, int32_t num_kv_heads,
                                         int32_t max_blocks_per_seq, int32_t block_size,
                                         int32_t partition_size);

/*
 * Workspace bytes attn_paged_decode needs for these sizes on the current
 * device (0 when one partition suffices).  Returns 0 on invalid sizes as
 * well; the decode call itself reports those.
 */
size_t attn_paged_decode_workspace_size(int32_t num_seqs, int32_t num_query_heads,
                                        int32_t num_kv_heads, int32_t head_size,
                                        int32_t max_blocks_per_seq, int32_t block_size,
                                        int32_t partition_size);

/*
 * attn_chunk_delta_out -- output step of chunked gated delta-rule linear
 * attention.
 *
 * Defined by "chunk_delta_rule_output" (#004), Reference Implementation and
 * Input Generation.  For every batch b, value head hd and chunk c of
 * chunk_size consecutive tokens (the last chunk may be short), with query
 * head hq = min(hd / max(num_heads / num_q_heads, 1), num_q_heads - 1) and
 * token rows i, j of the chunk:
 *   a[i][j] = <q_i, k_j> exp(g_i - g_j) if j <= i and g_i <= g_j, else 0,
 *             rounded to the 16-bit type (to nearest, ties to even)
 *   out_i   = scale (exp(g_i) q_i h_c + sum_j a[i][j] v_j)
 * accumulated in fp32.  Unlike the softmax entries there is no normalisation.
 *
 *  q, k      [batch, tokens, num_q_heads, key_dim], dtype
 *  v         [batch, tokens, num_heads, value_dim], dtype
 *  h         [batch, ceil(tokens / chunk_size), num_heads, key_dim, value_dim],
 *            dtype: the state each chunk starts from
 *  g         [batch, tokens, num_heads] float32 (log gates), 4-byte aligned
 *  key_dim, value_dim  128; chunk_size 64 (others: ATTN_ERR_UNSUPPORTED)
 *  num_q_heads, num_heads  below 131072 each (one chunk of rows is
 *            addressed with 32-bit offsets); larger: ATTN_ERR_INVALID_ARG
 *  scale     finite; the page uses key_dim^-1/2
 *  out       [batch, tokens, num_heads, value_dim], dtype; every row written
 *
 * batch == 0 or tokens == 0 is a valid no-op (pointers may then be NULL).
 */
attn_status attn_chunk_delta_out(const void *q, const void *k, const void *v, const void *h,
                         const float *g, int32_t batch, int32_t tokens, int32_t num_q_heads,
                         int32_t num_heads, int32_t key_dim, int32_t value_dim,
                         int32_t chunk_size, float scale, int32_t dtype, void *out,
                         void *stream);

/* A static, human-readable name for a status code. */
const char *attn_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* LIBATTN_ATTN_H */
