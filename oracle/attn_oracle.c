/*
 * attn_oracle.c -- plain, slow CPU oracle for exact softmax attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * links it, includes it or calls it, and this file shares no code, header,
 * table or helper with the GPU path.
 *
 * What it computes is the plain definition, written out in double precision:
 *
 *   out[r, h, :] = sum_j softmax_j(scale * <q[r,h,:], k[j,h,:]>) * v[j,h,:]
 *
 * over the keys j of the sequence that row r belongs to.  The tiled
 * online-softmax method of the GPU kernels reaches the same value up to
 * floating-point rounding, so the oracle does not follow that method: it
 * forms every score of a row, takes their maximum, exponentiates, sums and
 * divides, in that order, with no blocking or fusion.
 *
 * Sources (atrex-bench operator catalogue):
 *  - "attention_forward" (#001), Reference Implementation: per sequence,
 *    query rows [cu_q[i], cu_q[i+1]) attend non-causally to key rows
 *    [cu_k[i], cu_k[i+1]) of the same head; a sequence with no query rows is
 *    skipped, and rows outside every query segment are left unspecified
 *    (the reference allocates its output with empty_like).
 *  - "paged_attention_decode" (#024), Reference Implementation and Input
 *    Generation: one query row per sequence; key/value token t of sequence s
 *    sits in physical block block_tables[s][t / block_size] at slot
 *    t % block_size; the K cache is [blocks, kv_heads, head_size/x,
 *    block_size, x] with x = 16 bytes / element size, the V cache is
 *    [blocks, kv_heads, head_size, block_size]; query head hq reads KV head
 *    hq / (num_query_heads / num_kv_heads) (repeat_interleave); a sequence
 *    with seq_lens <= 0 keeps an all-zero output (zeros_like).
 *  - Both pages call scaled_dot_product_attention with no scale argument, so
 *    the scale is 1/sqrt(head_dim); here it is an explicit argument.
 *
 * Readings of points the pages leave open (each listed in the design notes):
 *  - a sequence with query rows but no key rows yields all-zero rows;
 *  - rows outside every query segment are written as NaN here, so a test
 *    can exclude them from comparison;
 *  - inputs are 16-bit bit patterns (bf16 or fp16) decoded exactly to double.
 *
 * Every function returns 0 on success and a negative number on an invalid
 * argument.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_BF16 0
#define ORACLE_FP16 1

/* ---- exact decoding of 16-bit floating-point bit patterns -------------- */

/* bfloat16 is the upper half of an IEEE binary32. */
static double bf16_bits_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double fp16_bits_to_double(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int expo = (bits >> 10) & 0x1f;
    int frac = bits & 0x3ff;
    double mag;
    if (expo == 0)
        mag = ldexp((double)frac, -24);               /* subnormal or zero */
    else if (expo == 31)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexp((double)(1024 + frac), expo - 25); /* (1 + f/1024) 2^(e-15) */
    return sign ? -mag : mag;
}

static double elem(const uint16_t *base, int64_t index, int dtype)
{
    return dtype == ORACLE_BF16 ? bf16_bits_to_double(base[index])
                                : fp16_bits_to_double(base[index]);
}

/* Decodes n bit patterns to double (exposed so the decoding can be checked). */
int oracle_decode_bits_f64(const uint16_t *bits, int64_t n, int dtype, double *out)
{
    if (n < 0 || (dtype != ORACLE_BF16 && dtype != ORACLE_FP16)) return -1;
    for (int64_t i = 0; i < n; ++i)
        out[i] = elem(bits, i, dtype);
    return 0;
}

/* ---- one query row against n key/value rows ---------------------------- */

/*
 * qrow[D], K[n][D], V[n][D] in double.  Writes out[D]; if lse is non-NULL it
 * receives log(sum_j exp(s_j)), and if wsum is non-NULL the sum of the
 * normalised softmax weights.  If out_abs is non-NULL it receives the same
 * weights applied to |V| (sum_j w_j |v_j|, term for term what out would be
 * for |V|): the magnitude that rounding errors of a weighted sum scale with.
 * s is caller scratch of n doubles.  n == 0 gives an all-zero row (and
 * out_abs), lse = -inf and wsum = 0.
 */
static void attend_row(const double *qrow, const double *K, const double *V,
                       int64_t n, int D, double scale, double *s, double *out,
                       double *lse, double *wsum, double *out_abs)
{
    for (int d = 0; d < D; ++d)
        out[d] = 0.0;
    if (out_abs)
        for (int d = 0; d < D; ++d)
            out_abs[d] = 0.0;
    if (n == 0) {
        if (lse) *lse = -INFINITY;
        if (wsum) *wsum = 0.0;
        return;
    }
    /* scores and their maximum */
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += qrow[d] * K[j * D + d];
        s[j] = scale * dot;
        if (s[j] > m) m = s[j];
    }
    /* unnormalised weights, their sum, and the weighted sum of values */
    double z = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        double e = exp(s[j] - m);
        s[j] = e;
        z += e;
        for (int d = 0; d < D; ++d)
            out[d] += e * V[j * D + d];
        if (out_abs)
            for (int d = 0; d < D; ++d)
                out_abs[d] += e * fabs(V[j * D + d]);
    }
    for (int d = 0; d < D; ++d)
        out[d] /= z;
    if (out_abs)
        for (int d = 0; d < D; ++d)
            out_abs[d] /= z;
    if (lse) *lse = m + log(z);
    if (wsum) {
        double w = 0.0;
        for (int64_t j = 0; j < n; ++j)
            w += s[j] / z;
        *wsum = w;
    }
}

/* ---- varlen prefill ------------------------------------------------------ */

static int check_cu(const int32_t *cu, int num_seqs)
{
    if (cu[0] < 0) return -1;
    for (int i = 0; i < num_seqs; ++i)
        if (cu[i + 1] < cu[i]) return -1;
    return 0;
}

/* Copies head h of rows [a, b) of a packed [tokens, H, D] tensor to dst[b-a][D]. */
static void gather_rows(const uint16_t *x, int dtype, int64_t a, int64_t b,
                        int H, int D, int h, double *dst)
{
    for (int64_t r = a; r < b; ++r)
        for (int d = 0; d < D; ++d)
            dst[(r - a) * D + d] = elem(x, (r * H + h) * (int64_t)D + d, dtype);
}

/*
 * Full varlen prefill.  q [total_q, H, D], k and v [total_k, H, D] (16-bit
 * bit patterns), cu_q and cu_k [num_seqs + 1].  out [total_q, H, D] double;
 * rows outside every query segment are set to NaN.  lse (optional,
 * [total_q, H]), wsum (optional, [total_q, H]) and out_abs (optional,
 * [total_q, H, D]) as in attend_row.
 */
int oracle_varlen_fwd_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                          int dtype, const int32_t *cu_q, const int32_t *cu_k,
                          int num_seqs, int64_t total_q, int64_t total_k,
                          int H, int D, double scale,
                          double *out, double *lse, double *wsum, double *out_abs)
{
    if (num_seqs < 0 || H <= 0 || D <= 0 || (dtype != ORACLE_BF16 && dtype != ORACLE_FP16))
        return -1;
    if (check_cu(cu_q, num_seqs) || check_cu(cu_k, num_seqs)) return -2;
    if (cu_q[num_seqs] > total_q || cu_k[num_seqs] > total_k) return -3;

    for (int64_t i = 0; i < total_q * H * (int64_t)D; ++i) out[i] = NAN;
    if (out_abs) for (int64_t i = 0; i < total_q * H * (int64_t)D; ++i) out_abs[i] = NAN;
    if (lse) for (int64_t i = 0; i < total_q * H; ++i) lse[i] = NAN;
    if (wsum) for (int64_t i = 0; i < total_q * H; ++i) wsum[i] = NAN;

    int failed = 0;
    for (int i = 0; i < num_seqs; ++i) {
        int64_t qa = cu_q[i], qb = cu_q[i + 1], ka = cu_k[i], kb = cu_k[i + 1];
        if (qb <= qa) continue;                  /* no query rows: skipped */
        int64_t nk = kb - ka;
        for (int h = 0; h < H; ++h) {
            double *K = malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1) * D);
            double *V = malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1) * D);
            if (!K || !V) { free(K); free(V); return -4; }
            gather_rows(k, dtype, ka, kb, H, D, h, K);
            gather_rows(v, dtype, ka, kb, H, D, h, V);
            #pragma omp parallel for schedule(dynamic, 16)
            for (int64_t r = qa; r < qb; ++r) {
                double *qrow = malloc(sizeof(double) * D);
                double *s = malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
                if (!qrow || !s) {
                    #pragma omp atomic write
                    failed = 1;
                } else {
                    for (int d = 0; d < D; ++d)
                        qrow[d] = elem(q, (r * H + h) * (int64_t)D + d, dtype);
                    attend_row(qrow, K, V, nk, D, scale, s,
                               out + (r * H + h) * (int64_t)D,
                               lse ? lse + r * H + h : NULL,
                               wsum ? wsum + r * H + h : NULL,
                               out_abs ? out_abs + (r * H + h) * (int64_t)D : NULL);
                }
                free(qrow);
                free(s);
            }
            free(K);
            free(V);
        }
    }
    return failed ? -4 : 0;
}

/*
 * The same definition evaluated only at n chosen (row, head) pairs, for
 * inputs too large to evaluate whole.  rows[i] must lie inside some query
 * segment.  out [n, D] double; lse optional [n]; out_abs optional [n, D].
 */
int oracle_varlen_fwd_rows_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               int dtype, const int32_t *cu_q, const int32_t *cu_k,
                               int num_seqs, int64_t total_q, int64_t total_k,
                               int H, int D, double scale,
                               const int64_t *rows, const int32_t *heads, int64_t n,
                               double *out, double *lse, double *out_abs)
{
    if (num_seqs <= 0 || H <= 0 || D <= 0 || n < 0 || (dtype != ORACLE_BF16 && dtype != ORACLE_FP16))
        return -1;
    if (check_cu(cu_q, num_seqs) || check_cu(cu_k, num_seqs)) return -2;
    if (cu_q[num_seqs] > total_q || cu_k[num_seqs] > total_k) return -3;
    for (int64_t i = 0; i < n; ++i) {
        int seq = -1;
        for (int s = 0; s < num_seqs; ++s)
            if (rows[i] >= cu_q[s] && rows[i] < cu_q[s + 1]) { seq = s; break; }
        if (seq < 0 || heads[i] < 0 || heads[i] >= H) return -5;
    }

    int failed = 0;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n; ++i) {
        int64_t r = rows[i];
        int h = heads[i], seq = 0;
        for (int s = 0; s < num_seqs; ++s)
            if (r >= cu_q[s] && r < cu_q[s + 1]) { seq = s; break; }
        int64_t ka = cu_k[seq], kb = cu_k[seq + 1], nk = kb - ka;
        double *K = malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1) * D);
        double *V = malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1) * D);
        double *qrow = malloc(sizeof(double) * D);
        double *s = malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
        if (!K || !V || !qrow || !s) {
            #pragma omp atomic write
            failed = 1;
        } else {
            gather_rows(k, dtype, ka, kb, H, D, h, K);
            gather_rows(v, dtype, ka, kb, H, D, h, V);
            for (int d = 0; d < D; ++d)
                qrow[d] = elem(q, (r * H + h) * (int64_t)D + d, dtype);
            attend_row(qrow, K, V, nk, D, scale, s, out + i * D,
                       lse ? lse + i : NULL, NULL, out_abs ? out_abs + i * D : NULL);
        }
        free(K); free(V); free(qrow); free(s);
    }
    return failed ? -4 : 0;
}

/* ---- paged decode -------------------------------------------------------- */

/* Element count per 16 bytes: the innermost K-cache dimension x. */
static int x_of(int dtype) { (void)dtype; return 16 / 2; }

/*
 * Gathers the first L tokens of sequence s, KV head hk, from the paged
 * caches into Kout[L][D] and Vout[L][D] (double), and writes the physical
 * slot index block * block_size + offset of each token to slots[L] (if
 * non-NULL).  Returns a negative number if a table entry is out of range.
 */
int oracle_paged_gather_f64(const uint16_t *k_cache, const uint16_t *v_cache, int dtype,
                            const int32_t *block_tables, int s, int L,
                            int num_blocks, int num_kv_heads, int head_size,
                            int block_size, int max_blocks_per_seq, int hk,
                            double *Kout, double *Vout, int64_t *slots)
{
    const int x = x_of(dtype);
    if (L < 0 || L > max_blocks_per_seq * block_size) return -1;
    if (head_size % x) return -1;
    for (int t = 0; t < L; ++t) {
        int64_t b = block_tables[(int64_t)s * max_blocks_per_seq + t / block_size];
        int o = t % block_size;
        if (b < 0 || b >= num_blocks) return -6;
        if (slots) slots[t] = b * block_size + o;
        for (int d = 0; d < head_size; ++d) {
            /* k_cache[b][hk][d / x][o][d % x] */
            int64_t ki = (((b * num_kv_heads + hk) * (head_size / x) + d / x) * block_size + o) * x + d % x;
            /* v_cache[b][hk][d][o] */
            int64_t vi = ((b * num_kv_heads + hk) * (int64_t)head_size + d) * block_size + o;
            if (Kout) Kout[(int64_t)t * head_size + d] = elem(k_cache, ki, dtype);
            if (Vout) Vout[(int64_t)t * head_size + d] = elem(v_cache, vi, dtype);
        }
    }
    return 0;
}

/*
 * Full paged decode.  query [num_seqs, Hq, D]; caches as in the header
 * comment; block_tables [num_seqs, max_blocks_per_seq]; seq_lens
 * [num_seqs].  out [num_seqs, Hq, D] double; lse optional [num_seqs, Hq].
 */
int oracle_paged_decode_f64(const uint16_t *query, const uint16_t *k_cache,
                            const uint16_t *v_cache, int dtype,
                            const int32_t *block_tables, const int32_t *seq_lens,
                            int num_seqs, int num_query_heads, int num_kv_heads,
                            int head_size, int block_size, int max_blocks_per_seq,
                            int num_blocks, double scale, double *out, double *lse)
{
    if (num_seqs < 0 || num_query_heads <= 0 || num_kv_heads <= 0 || head_size <= 0 ||
        block_size <= 0 || max_blocks_per_seq < 0 || (dtype != ORACLE_BF16 && dtype != ORACLE_FP16))
        return -1;
    if (num_query_heads % num_kv_heads) return -1;
    if (head_size % x_of(dtype)) return -1;
    const int G = num_query_heads / num_kv_heads;  /* queries per KV head */
    const int D = head_size;

    for (int64_t i = 0; i < (int64_t)num_seqs * num_query_heads * D; ++i) out[i] = 0.0;
    if (lse) for (int64_t i = 0; i < (int64_t)num_seqs * num_query_heads; ++i) lse[i] = -INFINITY;

    int failed = 0;
    #pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int s = 0; s < num_seqs; ++s) {
        for (int hq = 0; hq < num_query_heads; ++hq) {
            int L = seq_lens[s];
            if (L <= 0) continue;                 /* zero context: row stays 0 */
            int hk = hq / G;
            double *K = malloc(sizeof(double) * (size_t)L * D);
            double *V = malloc(sizeof(double) * (size_t)L * D);
            double *qrow = malloc(sizeof(double) * D);
            double *sc = malloc(sizeof(double) * (size_t)L);
            int rc = (K && V && qrow && sc) ? 0 : -4;
            if (!rc)
                rc = oracle_paged_gather_f64(k_cache, v_cache, dtype, block_tables, s, L,
                                             num_blocks, num_kv_heads, head_size, block_size,
                                             max_blocks_per_seq, hk, K, V, NULL);
            if (!rc) {
                for (int d = 0; d < D; ++d)
                    qrow[d] = elem(query, ((int64_t)s * num_query_heads + hq) * D + d, dtype);
                attend_row(qrow, K, V, L, D, scale, sc,
                           out + ((int64_t)s * num_query_heads + hq) * D,
                           lse ? lse + (int64_t)s * num_query_heads + hq : NULL, NULL, NULL);
            } else {
                #pragma omp atomic write
                failed = rc;
            }
            free(K); free(V); free(qrow); free(sc);
        }
    }
    return failed;
}

/* Number of threads the OpenMP runtime will use for a parallel region. */
int oracle_num_threads(void)
{
    int n = 1;
    #pragma omp parallel
    {
        #pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
