/*
 * chunk_oracle.c -- plain, slow CPU oracle for the output step of chunked
 * gated delta-rule linear attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * links it, includes it or calls it, and this file shares no code, header,
 * table or helper with the GPU path.
 *
 * Source: atrex-bench operator catalogue, "chunk_delta_rule_output" (#004),
 * Reference Implementation and Input Generation.  Shapes: q and k are
 * [batch, tokens, num_q_heads, key_dim], v is [batch, tokens, num_heads,
 * value_dim], h is [batch, num_chunks, num_heads, key_dim, value_dim] (one
 * key_dim x value_dim state per chunk and value head), g is float32
 * [batch, tokens, num_heads]; the output has v's shape and dtype.
 *
 * What it computes, written out in double precision for every batch b,
 * value head hd and chunk c of `chunk` consecutive tokens (the last chunk
 * may be short; the page pads it with zero rows, which contribute nothing):
 *
 *   hq          = min(hd / max(num_heads / num_q_heads, 1), num_q_heads - 1)
 *   o[i, :]     = exp(g[i]) * sum_k q[i, k] h_c[k, :]
 *   a[i, j]     = <q[i, :], k[j, :]> * exp(g[i] - g[j])
 *                   for token rows j <= i of the chunk with g[i] <= g[j],
 *                 0 otherwise
 *   a16[i, j]   = a[i, j] rounded to the value dtype, to nearest, ties even
 *   out[i, :]   = scale * (o[i, :] + sum_j a16[i, j] v[j, :])
 *
 * with q, k taken from query head hq, v, g and h from value head hd, and
 * scale = key_dim^-0.5 unless given.  The gate g is used as given per token
 * (the page's inputs draw it independently per token, so the condition
 * g[i] <= g[j] is not implied by j <= i).  Rounding a[i, j] to 16 bits
 * before the product with v is part of the page's definition; here it is one
 * rounding from the double-precision value.
 *
 * With `absolute` set the same loops accumulate absolute values instead,
 *   A[i, :] = scale * (exp(g[i]) * sum_k |q[i, k]| |h_c[k, :]|
 *                      + sum_j |a16[i, j]| |v[j, :]|),
 * the magnitude that rounding errors of a floating-point evaluation scale
 * with.
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

static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;   /* bfloat16 is the top half of binary32 */
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double fp16_value(uint16_t bits)
{
    int sign = (bits >> 15) & 1, expo = (bits >> 10) & 0x1f, frac = bits & 0x3ff;
    double mag;
    if (expo == 0)
        mag = ldexp((double)frac, -24);
    else if (expo == 31)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexp((double)(1024 + frac), expo - 25);
    return sign ? -mag : mag;
}

static double value(const uint16_t *x, int64_t i, int dtype)
{
    return dtype == ORACLE_BF16 ? bf16_value(x[i]) : fp16_value(x[i]);
}

/* x rounded to the nearest value of the 16-bit type, ties to even:
 * bfloat16 keeps 8 significant bits down to 2^-126 and then a fixed quantum
 * of 2^-133; binary16 keeps 11 down to 2^-14 and then 2^-24.  Overflow is
 * not handled (the operator's values stay far below either range's top). */
double oracle_round_to_dtype(double x, int dtype)
{
    if (x == 0.0 || !isfinite(x))
        return x;
    int e;
    frexp(x, &e);                       /* |x| = m 2^e, 0.5 <= m < 1 */
    const int bits = dtype == ORACLE_BF16 ? 8 : 11;
    const int min_quantum = dtype == ORACLE_BF16 ? -133 : -24;
    int qe = e - bits;
    if (qe < min_quantum)
        qe = min_quantum;
    return ldexp(nearbyint(ldexp(x, -qe)), qe);   /* default mode: to nearest, ties even */
}

int oracle_chunk_delta_out_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               const uint16_t *h, const float *g, int batch, int tokens,
                               int num_q_heads, int num_heads, int key_dim, int value_dim,
                               int chunk, double scale, int dtype, int absolute, double *out)
{
    if (batch < 0 || tokens < 0 || num_q_heads <= 0 || num_heads <= 0 || key_dim <= 0 ||
        value_dim <= 0 || chunk <= 0 || (dtype != ORACLE_BF16 && dtype != ORACLE_FP16))
        return -1;
    if (batch == 0 || tokens == 0)
        return 0;
    if (!q || !k || !v || !h || !g || !out)
        return -1;
    const int K = key_dim, V = value_dim, H = num_heads, Hq = num_q_heads;
    const int num_chunks = (tokens + chunk - 1) / chunk;
    const int per_q = H / Hq > 1 ? H / Hq : 1;
    int failed = 0;

#pragma omp parallel for collapse(3) schedule(dynamic)
    for (int b = 0; b < batch; ++b)
        for (int hd = 0; hd < H; ++hd)
            for (int c = 0; c < num_chunks; ++c) {
                int hq = hd / per_q;
                if (hq > Hq - 1)
                    hq = Hq - 1;
                const int t0 = c * chunk;
                const int n = tokens - t0 < chunk ? tokens - t0 : chunk;
                double *Q = malloc(sizeof(double) * (size_t)n * K);
                double *Kc = malloc(sizeof(double) * (size_t)n * K);
                double *Vc = malloc(sizeof(double) * (size_t)n * V);
                double *Hc = malloc(sizeof(double) * (size_t)K * V);
                double *G = malloc(sizeof(double) * (size_t)n);
                double *A = malloc(sizeof(double) * (size_t)n);
                if (!Q || !Kc || !Vc || !Hc || !G || !A) {
#pragma omp atomic write
                    failed = 1;
                    free(Q); free(Kc); free(Vc); free(Hc); free(G); free(A);
                    continue;
                }
                for (int i = 0; i < n; ++i) {
                    const int64_t t = (int64_t)b * tokens + t0 + i;
                    for (int d = 0; d < K; ++d) {
                        Q[(size_t)i * K + d] = value(q, (t * Hq + hq) * K + d, dtype);
                        Kc[(size_t)i * K + d] = value(k, (t * Hq + hq) * K + d, dtype);
                    }
                    for (int e = 0; e < V; ++e)
                        Vc[(size_t)i * V + e] = value(v, (t * H + hd) * (int64_t)V + e, dtype);
                    G[i] = (double)g[t * H + hd];
                }
                const int64_t hbase = (((int64_t)b * num_chunks + c) * H + hd) * (int64_t)K * V;
                for (int64_t x = 0; x < (int64_t)K * V; ++x)
                    Hc[x] = value(h, hbase + x, dtype);

                for (int i = 0; i < n; ++i) {
                    /* row i of the gated, masked, rounded intra-chunk scores */
                    for (int j = 0; j < n; ++j) {
                        double a = 0.0;
                        if (j <= i && G[i] <= G[j]) {
                            double dot = 0.0;
                            for (int d = 0; d < K; ++d)
                                dot += Q[(size_t)i * K + d] * Kc[(size_t)j * K + d];
                            a = oracle_round_to_dtype(dot * exp(G[i] - G[j]), dtype);
                        }
                        A[j] = absolute ? fabs(a) : a;
                    }
                    const double gate = exp(G[i]);
                    double *orow = out + (((int64_t)b * tokens + t0 + i) * H + hd) * (int64_t)V;
                    for (int e = 0; e < V; ++e) {
                        double inter = 0.0, intra = 0.0;
                        for (int d = 0; d < K; ++d) {
                            const double qv = Q[(size_t)i * K + d], hv = Hc[(size_t)d * V + e];
                            inter += absolute ? fabs(qv) * fabs(hv) : qv * hv;
                        }
                        for (int j = 0; j < n; ++j) {
                            const double vv = Vc[(size_t)j * V + e];
                            intra += A[j] * (absolute ? fabs(vv) : vv);
                        }
                        orow[e] = scale * (gate * inter + intra);
                    }
                }
                free(Q); free(Kc); free(Vc); free(Hc); free(G); free(A);
            }
    return failed ? -2 : 0;
}

/* Only the listed (token, head) rows of the output: rows[i] is a flat token
 * index b * tokens + t, heads[i] a value head; out is [count, value_dim].
 * Same arithmetic as oracle_chunk_delta_out_f64, for sampled checks of large
 * workloads. */
int oracle_chunk_delta_out_rows_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                    const uint16_t *h, const float *g, int batch, int tokens,
                                    int num_q_heads, int num_heads, int key_dim, int value_dim,
                                    int chunk, double scale, int dtype, int absolute,
                                    const int64_t *rows, const int32_t *heads, int64_t count,
                                    double *out)
{
    if (batch <= 0 || tokens <= 0 || num_q_heads <= 0 || num_heads <= 0 || key_dim <= 0 ||
        value_dim <= 0 || chunk <= 0 || count < 0 || (dtype != ORACLE_BF16 && dtype != ORACLE_FP16))
        return -1;
    if (!q || !k || !v || !h || !g || !rows || !heads || (count && !out))
        return -1;
    for (int64_t r = 0; r < count; ++r)
        if (rows[r] < 0 || rows[r] >= (int64_t)batch * tokens || heads[r] < 0 || heads[r] >= num_heads)
            return -1;
    const int K = key_dim, V = value_dim, H = num_heads, Hq = num_q_heads;
    const int num_chunks = (tokens + chunk - 1) / chunk;
    const int per_q = H / Hq > 1 ? H / Hq : 1;

#pragma omp parallel for schedule(dynamic)
    for (int64_t r = 0; r < count; ++r) {
        const int b = (int)(rows[r] / tokens), ti = (int)(rows[r] % tokens), hd = heads[r];
        int hq = hd / per_q;
        if (hq > Hq - 1)
            hq = Hq - 1;
        const int c = ti / chunk, t0 = c * chunk;
        const int64_t ti_flat = (int64_t)b * tokens + ti;
        const double gi = (double)g[ti_flat * H + hd];
        double *orow = out + r * (int64_t)V;
        for (int e = 0; e < V; ++e)
            orow[e] = 0.0;
        /* inter-chunk term */
        const int64_t hbase = (((int64_t)b * num_chunks + c) * H + hd) * (int64_t)K * V;
        for (int e = 0; e < V; ++e) {
            double inter = 0.0;
            for (int d = 0; d < K; ++d) {
                const double qv = value(q, (ti_flat * Hq + hq) * K + d, dtype);
                const double hv = value(h, hbase + (int64_t)d * V + e, dtype);
                inter += absolute ? fabs(qv) * fabs(hv) : qv * hv;
            }
            orow[e] = exp(gi) * inter;
        }
        /* intra-chunk term */
        for (int tj = t0; tj <= ti; ++tj) {
            const int64_t tj_flat = (int64_t)b * tokens + tj;
            const double gj = (double)g[tj_flat * H + hd];
            if (!(gi <= gj))
                continue;
            double dot = 0.0;
            for (int d = 0; d < K; ++d)
                dot += value(q, (ti_flat * Hq + hq) * K + d, dtype) * value(k, (tj_flat * Hq + hq) * K + d, dtype);
            double a = oracle_round_to_dtype(dot * exp(gi - gj), dtype);
            if (absolute)
                a = fabs(a);
            for (int e = 0; e < V; ++e) {
                const double vv = value(v, (tj_flat * H + hd) * (int64_t)V + e, dtype);
                orow[e] += a * (absolute ? fabs(vv) : vv);
            }
        }
        for (int e = 0; e < V; ++e)
            orow[e] *= scale;
    }
    return 0;
}
