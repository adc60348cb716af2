/*
 * attn_oracle.c -- plain, slow, fp64 CPU oracle for exact scaled-dot-product
 * attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code with the HIP library.
 *
 * What it computes is the plain definition of attention, written out with no
 * tiling, no online softmax and no reordering:
 *
 *   for every batch b, query head h and query row i:
 *     hk   = floor(h / (Hq / Hkv))               (contiguous GQA/MQA groups)
 *     s_j  = scale * sum_c q[b,h,i,c] * k[b,hk,j,c]   for every visible j
 *     m    = max_j s_j
 *     e_j  = exp(s_j - m)
 *     l    = sum_j e_j
 *     o[b,h,i,c] = sum_j e_j * v[b,hk,j,c] / l
 *     lse[b,h,i] = m + ln(l)
 *
 * Sources (the pages these follow):
 *  - "Lab 02 - Forward de flash attention en Triton", section "Bloque C":
 *    the naive reference: S = Q K^T * sm_scale, masked with -inf, row softmax,
 *    then P V.  Section "La estructura del kernel" and "Bloque B" define the
 *    log-sum-exp output as m + log(l) per row, with m the max of the scaled
 *    scores.
 *  - "Optimizaciones de Atencion" (cruxr.ai), section "FlashAttention: Nunca
 *    materializar la matriz de atencion": the standard branch of the demo
 *    (row max, exponentials, their sum, normalised weights, weighted V sum).
 *  - Causal visibility j <= i: "Lab 02", "Bloque B" (mask keeps offs_m >=
 *    offs_n) and "Errores tipicos" (a position attends to itself).
 *  - Sliding window: "00 - Por que la atencion domina la inferencia", section
 *    "Otras tres variantes": each token sees only its last W tokens.  Reading
 *    taken: key j is visible from row i iff 0 <= i - j < W (W keys including
 *    the token itself); W = 0 means no window.
 *  - GQA/MQA: same page, same section, and "Optimizaciones de Atencion",
 *    section "Multi-Head Latent Attention": K/V are shared by groups of query
 *    heads.  Reading taken: contiguous groups, kv head = floor(h / G).
 *  - A row with no visible key (unreachable through the library's argument
 *    rules) yields o = 0 and lse = -inf, the limit of the all-masked-row guard
 *    in "Lab 02", "Errores tipicos".
 *  - Paged K/V ("00 - Por que la atencion domina la inferencia", section
 *    "PagedAttention es un problema distinto": the cache lives in fixed-size
 *    blocks with a table of blocks per request, and the kernel follows the
 *    table).  Reading taken for the layout: pools (num_pages, Hkv, page_size,
 *    d); key j of request b is slot j % page_size of page
 *    block_table[b][j / page_size]; request b has seq_lens[b] keys.  The
 *    oracle walks the table to gather each request's keys in order and then
 *    applies the definition above.
 *  - Fewer queries than keys (Nq < Nk, the decoding case of "Optimizaciones de
 *    Atencion", section "FlashDecoding": a few new query tokens against a
 *    cached sequence): the pages do not say how the causal mask aligns.
 *    Reading taken: the Nq queries are the last Nq positions of the sequence,
 *    so query row i sits at position Nk - Nq + i and the masks above apply to
 *    that position (bottom-right alignment).  With Nq = Nk this is the plain
 *    case.
 *
 * Inputs are the raw bit patterns the GPU receives (fp16 or bf16), decoded
 * exactly to double by the decoders below; a float64 input mode exists for
 * tests that need inputs no 16-bit format can hold.  The scale is the fp32
 * value passed to the library, widened exactly.  Scores are formed one row at
 * a time, so memory is O(N) per thread, never O(N^2).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F16 = 0, ORACLE_BF16 = 1, ORACLE_F64 = 2 };

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double decode_f16(uint16_t h)
{
    int sign = h >> 15;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double mag;
    if (expo == 0)
        mag = ldexp((double)frac, -24);                 /* subnormal: frac * 2^-24 */
    else if (expo == 31)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexp((double)(frac | 0x400), expo - 25); /* 1.frac * 2^(expo-15) */
    return sign ? -mag : mag;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
static double decode_bf16(uint16_t b)
{
    int sign = b >> 15;
    int expo = (b >> 7) & 0xff;
    int frac = b & 0x7f;
    double mag;
    if (expo == 0)
        mag = ldexp((double)frac, -133);                /* subnormal: frac * 2^-133 */
    else if (expo == 255)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexp((double)(frac | 0x80), expo - 134); /* 1.frac * 2^(expo-127) */
    return sign ? -mag : mag;
}

static double load_elem(const void *base, int dtype, int64_t idx)
{
    if (dtype == ORACLE_F16)
        return decode_f16(((const uint16_t *)base)[idx]);
    if (dtype == ORACLE_BF16)
        return decode_bf16(((const uint16_t *)base)[idx]);
    return ((const double *)base)[idx];
}

/* Exposed so the tests can pin the decoders against library conversions. */
double attn_oracle_decode(uint16_t bits, int dtype)
{
    return dtype == ORACLE_F16 ? decode_f16(bits) : decode_bf16(bits);
}

int attn_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Visible key range [lo, hi] of query row i of Nq against Nk keys (empty
 * when lo > hi); the row sits at sequence position Nk - Nq + i. */
static void visible_range(int64_t i, int64_t Nq, int64_t Nk, int causal, int64_t window,
                          int64_t *lo, int64_t *hi)
{
    int64_t pos = Nk - Nq + i;
    *hi = causal ? (pos < Nk - 1 ? pos : Nk - 1) : Nk - 1;
    *lo = 0;
    if (window > 0 && pos - window + 1 > 0)
        *lo = pos - window + 1;
}

/*
 * One output row: o_row[0..d) and *lse_out for (b, h, i).
 * s is scratch for at least Nk doubles, qrow scratch for d doubles.
 */
static void oracle_row(const void *q, const void *k, const void *v,
                       int64_t b, int64_t h, int64_t i,
                       int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                       int causal, int64_t window, double scale, int dtype,
                       double *o_row, double *lse_out, double *s, double *qrow)
{
    int64_t group = Hq / Hkv;
    int64_t hk = h / group;
    int64_t qbase = ((b * Hq + h) * Nq + i) * d;
    int64_t kvhead = (b * Hkv + hk) * Nk * d;
    int64_t lo, hi;
    visible_range(i, Nq, Nk, causal, window, &lo, &hi);

    for (int64_t c = 0; c < d; ++c) {
        o_row[c] = 0.0;
        qrow[c] = load_elem(q, dtype, qbase + c);
    }
    if (lo > hi) {
        *lse_out = -INFINITY;
        return;
    }

    /* scores s_j = scale * <q_i, k_j> */
    double m = -INFINITY;
    for (int64_t j = lo; j <= hi; ++j) {
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c)
            dot += qrow[c] * load_elem(k, dtype, kvhead + j * d + c);
        s[j - lo] = scale * dot;
        if (s[j - lo] > m)
            m = s[j - lo];
    }

    /* softmax weights and the weighted sum of V rows */
    double l = 0.0;
    for (int64_t j = lo; j <= hi; ++j) {
        double e = exp(s[j - lo] - m);
        l += e;
        for (int64_t c = 0; c < d; ++c)
            o_row[c] += e * load_elem(v, dtype, kvhead + j * d + c);
    }
    for (int64_t c = 0; c < d; ++c)
        o_row[c] /= l;
    *lse_out = m + log(l);
}

/*
 * Full forward, Nq queries against Nk keys.  q, o: (B, Hq, Nq, d); k, v:
 * (B, Hkv, Nk, d); lse: (B, Hq, Nq); all row-major.  o and lse are float64.
 * Returns 0, or -1 on bad arguments, -2 when scratch cannot be allocated.
 */
int attn_oracle_fwd_qk(const void *q, const void *k, const void *v,
                       double *o, double *lse,
                       int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                       int causal, int64_t window, float scale, int dtype)
{
    if (B < 0 || Hq < 1 || Hkv < 1 || Nq < 0 || Nk < 0 || d < 1 || Hq % Hkv != 0 ||
        window < 0 || dtype < ORACLE_F16 || dtype > ORACLE_F64)
        return -1;
    int64_t N = Nq;
    int64_t rows = B * Hq * Nq;
    int failed = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
        double *qrow = (double *)malloc(sizeof(double) * (size_t)d);
        if (!s || !qrow) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < rows; ++r) {
                int64_t i = r % N;
                int64_t h = (r / N) % Hq;
                int64_t b = r / (N * Hq);
                oracle_row(q, k, v, b, h, i, Hq, Hkv, Nq, Nk, d, causal, window,
                           (double)scale, dtype, o + r * d, lse + r, s, qrow);
            }
        }
        free(s);
        free(qrow);
    }
    return failed ? -2 : 0;
}

/* Full forward with Nq = Nk = N. */
int attn_oracle_fwd(const void *q, const void *k, const void *v,
                    double *o, double *lse,
                    int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                    int causal, int64_t window, float scale, int dtype)
{
    return attn_oracle_fwd_qk(q, k, v, o, lse, B, Hq, Hkv, N, N, d, causal, window, scale, dtype);
}

/*
 * Selected rows only, for full-size checks where the whole output would take
 * too long on the CPU.  row_ids[r] is the flat row index (b * Hq + h) * Nq + i.
 * o: (nrows, d) float64; lse: (nrows,) float64.
 */
int attn_oracle_rows_qk(const void *q, const void *k, const void *v,
                        const int64_t *row_ids, int64_t nrows,
                        double *o, double *lse,
                        int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                        int causal, int64_t window, float scale, int dtype)
{
    if (B < 0 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || d < 1 || Hq % Hkv != 0 ||
        window < 0 || dtype < ORACLE_F16 || dtype > ORACLE_F64 || nrows < 0)
        return -1;
    int64_t N = Nq;
    for (int64_t r = 0; r < nrows; ++r)
        if (row_ids[r] < 0 || row_ids[r] >= B * Hq * N)
            return -1;
    int failed = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)Nk);
        double *qrow = (double *)malloc(sizeof(double) * (size_t)d);
        if (!s || !qrow) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < nrows; ++r) {
                int64_t id = row_ids[r];
                int64_t i = id % N;
                int64_t h = (id / N) % Hq;
                int64_t b = id / (N * Hq);
                oracle_row(q, k, v, b, h, i, Hq, Hkv, Nq, Nk, d, causal, window,
                           (double)scale, dtype, o + r * d, lse + r, s, qrow);
            }
        }
        free(s);
        free(qrow);
    }
    return failed ? -2 : 0;
}

/* Selected rows with Nq = Nk = N. */
int attn_oracle_rows(const void *q, const void *k, const void *v,
                     const int64_t *row_ids, int64_t nrows,
                     double *o, double *lse,
                     int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                     int causal, int64_t window, float scale, int dtype)
{
    return attn_oracle_rows_qk(q, k, v, row_ids, nrows, o, lse, B, Hq, Hkv, N, N, d,
                               causal, window, scale, dtype);
}

/*
 * Paged K/V forward.  q, o: (B, Hq, Nq, d); k_pool, v_pool: (num_pages, Hkv,
 * page_size, d); block_table: (B, max_pages) int32; seq_lens: (B,) int32;
 * lse: (B, Hq, Nq).  For each request b the keys 0 .. seq_lens[b]-1 are
 * gathered by walking its page table (key j: page block_table[b][j /
 * page_size], slot j % page_size) into contiguous (1, Hkv, seq_lens[b], d)
 * arrays, and the Nq-against-Nk forward above runs on them.  Returns 0, -1 on
 * bad arguments or a table entry outside [0, num_pages), -2 when memory cannot
 * be allocated.
 */
int attn_oracle_fwd_paged(const void *q, const void *k_pool, const void *v_pool,
                          const int32_t *block_table, const int32_t *seq_lens,
                          double *o, double *lse,
                          int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t d,
                          int64_t page_size, int64_t num_pages, int64_t max_pages,
                          int causal, int64_t window, float scale, int dtype)
{
    if (B < 0 || Hq < 1 || Hkv < 1 || Nq < 0 || d < 1 || Hq % Hkv != 0 || page_size < 1 ||
        num_pages < 1 || max_pages < 1 || window < 0 || dtype < ORACLE_F16 || dtype > ORACLE_F64)
        return -1;
    size_t esize = dtype == ORACLE_F64 ? sizeof(double) : sizeof(uint16_t);
    for (int64_t b = 0; b < B; ++b)
        if (seq_lens[b] < 0 || seq_lens[b] > max_pages * page_size)
            return -1;
    for (int64_t b = 0; b < B; ++b) {
        int64_t nk = seq_lens[b];
        size_t rows = (size_t)(Hkv * (nk > 0 ? nk : 1));
        char *kg = (char *)malloc(rows * (size_t)d * esize);
        char *vg = (char *)malloc(rows * (size_t)d * esize);
        if (!kg || !vg) {
            free(kg);
            free(vg);
            return -2;
        }
        int bad = 0;
        for (int64_t hk = 0; hk < Hkv && !bad; ++hk)
            for (int64_t j = 0; j < nk; ++j) {
                int64_t page = block_table[b * max_pages + j / page_size];
                if (page < 0 || page >= num_pages) {
                    bad = 1;
                    break;
                }
                int64_t src = ((page * Hkv + hk) * page_size + j % page_size) * d;
                int64_t dst = (hk * nk + j) * d;
                memcpy(kg + (size_t)dst * esize, (const char *)k_pool + (size_t)src * esize, (size_t)d * esize);
                memcpy(vg + (size_t)dst * esize, (const char *)v_pool + (size_t)src * esize, (size_t)d * esize);
            }
        const char *qb = (const char *)q + (size_t)(b * Hq * Nq * d) * esize;
        int rc = bad ? -1 : 0;
        if (!bad && nk > 0) {
            rc = attn_oracle_fwd_qk(qb, kg, vg, o + b * Hq * Nq * d, lse + b * Hq * Nq,
                                    1, Hq, Hkv, Nq, nk, d, causal, window, scale, dtype);
        } else if (!bad) {
            for (int64_t r = 0; r < Hq * Nq; ++r) {
                for (int64_t c = 0; c < d; ++c)
                    o[(b * Hq * Nq + r) * d + c] = 0.0;
                lse[b * Hq * Nq + r] = -INFINITY;
            }
        }
        free(kg);
        free(vg);
        if (rc != 0)
            return rc;
    }
    return 0;
}

/*
 * Backward pass: the gradients of the scalar sum_{b,h,i,c} dO[b,h,i,c] *
 * O[b,h,i,c] with respect to q, k and v, where O is the forward above (Nq = Nk
 * = N).  The pages leave the backward out of their scope; they say only that
 * it recomputes the scores from Q and K instead of storing them, and that the
 * per-row log-sum-exp is kept for it ("Optimizaciones de Atencion", section
 * "FlashAttention: Nunca materializar la matriz de atencion"; "Fase 27", the
 * out-of-scope list).  What it computes is plain calculus on the definition,
 * written out per query row i of head (b, h) with kv head hk = floor(h / G):
 *
 *   P_j   = exp(s_j - m) / l              (the forward's softmax weights)
 *   dP_j  = sum_c dO[i,c] * v[hk,j,c]     (gradient of the weights)
 *   D     = sum_j P_j * dP_j              (softmax Jacobian term)
 *   dS_j  = P_j * (dP_j - D)              (gradient of the scaled scores)
 *   dq[i,c]    = scale * sum_j dS_j * k[hk,j,c]
 *   dk[hk,j,c] += scale * dS_j * q[i,c]   (summed over i and the G heads)
 *   dv[hk,j,c] += P_j * dO[i,c]           (summed over i and the G heads)
 *
 * Masked keys have P_j = 0 and so contribute nothing; a row with no visible
 * key contributes nothing at all.
 */
static void bwd_row(const void *q, const void *k, const void *v, const void *dout,
                    int64_t b, int64_t h, int64_t i, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                    int causal, int64_t window, double scale, int dtype,
                    double *dq_row, double *dk_head, double *dv_head,
                    double *s, double *qrow, double *dorow)
{
    int64_t hk = h / (Hq / Hkv);
    int64_t qbase = ((b * Hq + h) * N + i) * d;
    int64_t kvhead = (b * Hkv + hk) * N * d;
    int64_t lo, hi;
    visible_range(i, N, N, causal, window, &lo, &hi);
    for (int64_t c = 0; c < d; ++c) {
        dq_row[c] = 0.0;
        qrow[c] = load_elem(q, dtype, qbase + c);
        dorow[c] = load_elem(dout, dtype, qbase + c);
    }
    if (lo > hi)
        return;
    double m = -INFINITY;
    for (int64_t j = lo; j <= hi; ++j) {
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c)
            dot += load_elem(k, dtype, kvhead + j * d + c) * qrow[c];
        s[j - lo] = dot * scale;
        m = s[j - lo] > m ? s[j - lo] : m;
    }
    double l = 0.0;
    for (int64_t j = lo; j <= hi; ++j)
        l += exp(s[j - lo] - m);
    /* s[] now becomes P_j, and dP_j goes into the second half of the buffer */
    double *dp = s + (hi - lo + 1);
    double dsum = 0.0;
    for (int64_t j = lo; j <= hi; ++j) {
        double p = exp(s[j - lo] - m) / l;
        double g = 0.0;
        for (int64_t c = 0; c < d; ++c)
            g += dorow[c] * load_elem(v, dtype, kvhead + j * d + c);
        s[j - lo] = p;
        dp[j - lo] = g;
        dsum += p * g;
    }
    for (int64_t j = lo; j <= hi; ++j) {
        double p = s[j - lo];
        double ds = p * (dp[j - lo] - dsum);
        for (int64_t c = 0; c < d; ++c)
            dq_row[c] += scale * ds * load_elem(k, dtype, kvhead + j * d + c);
        if (dk_head)
            for (int64_t c = 0; c < d; ++c) {
                dk_head[j * d + c] += scale * ds * qrow[c];
                dv_head[j * d + c] += p * dorow[c];
            }
    }
}

/*
 * Whole backward.  q, dout, dq: (B, Hq, N, d); k, v, dk, dv: (B, Hkv, N, d);
 * dq, dk, dv are float64.  One OpenMP task per (batch, kv head), which owns
 * that head's dk and dv, so nothing is summed across threads.  Returns 0, -1
 * on bad arguments, -2 when scratch cannot be allocated.
 */
int attn_oracle_bwd(const void *q, const void *k, const void *v, const void *dout,
                    double *dq, double *dk, double *dv,
                    int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                    int causal, int64_t window, float scale, int dtype)
{
    if (B < 0 || Hq < 1 || Hkv < 1 || N < 0 || d < 1 || Hq % Hkv != 0 || window < 0 ||
        dtype < ORACLE_F16 || dtype > ORACLE_F64)
        return -1;
    int64_t group = Hq / Hkv;
    int failed = 0;
    memset(dk, 0, sizeof(double) * (size_t)(B * Hkv * N * d));
    memset(dv, 0, sizeof(double) * (size_t)(B * Hkv * N * d));
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(2 * (N > 0 ? N : 1)));
        double *qrow = (double *)malloc(sizeof(double) * (size_t)d);
        double *dorow = (double *)malloc(sizeof(double) * (size_t)d);
        if (!s || !qrow || !dorow) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t g = 0; g < B * Hkv; ++g) {
                int64_t b = g / Hkv, hk = g % Hkv;
                double *dkh = dk + g * N * d, *dvh = dv + g * N * d;
                for (int64_t h = hk * group; h < (hk + 1) * group; ++h)
                    for (int64_t i = 0; i < N; ++i)
                        bwd_row(q, k, v, dout, b, h, i, Hq, Hkv, N, d, causal, window, (double)scale,
                                dtype, dq + ((b * Hq + h) * N + i) * d, dkh, dvh, s, qrow, dorow);
            }
        }
        free(s);
        free(qrow);
        free(dorow);
    }
    return failed ? -2 : 0;
}

/*
 * dq for selected rows only (row_ids[r] = (b * Hq + h) * N + i); each row's
 * dq needs nothing but that row, so this is the per-row part of the backward
 * above.  dq: (nrows, d) float64.
 */
int attn_oracle_bwd_rows(const void *q, const void *k, const void *v, const void *dout,
                         const int64_t *row_ids, int64_t nrows, double *dq,
                         int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                         int causal, int64_t window, float scale, int dtype)
{
    if (B < 0 || Hq < 1 || Hkv < 1 || N < 1 || d < 1 || Hq % Hkv != 0 || window < 0 ||
        dtype < ORACLE_F16 || dtype > ORACLE_F64 || nrows < 0)
        return -1;
    for (int64_t r = 0; r < nrows; ++r)
        if (row_ids[r] < 0 || row_ids[r] >= B * Hq * N)
            return -1;
    int failed = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(2 * N));
        double *qrow = (double *)malloc(sizeof(double) * (size_t)d);
        double *dorow = (double *)malloc(sizeof(double) * (size_t)d);
        if (!s || !qrow || !dorow) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < nrows; ++r) {
                int64_t id = row_ids[r];
                int64_t i = id % N, h = (id / N) % Hq, b = id / (N * Hq);
                bwd_row(q, k, v, dout, b, h, i, Hq, Hkv, N, d, causal, window, (double)scale, dtype,
                        dq + r * d, NULL, NULL, s, qrow, dorow);
            }
        }
        free(s);
        free(qrow);
        free(dorow);
    }
    return failed ? -2 : 0;
}

/*
 * dk and dv for selected keys only (key_ids[r] = (b * Hkv + hk) * N + j), for
 * full-size checks.  A key's gradients need the softmax normaliser and the
 * Jacobian term D of every row that sees it, so the caller passes them per
 * query row, as computed by this oracle: lse (B, Hq, N) = m + ln l from the
 * forward, and drow (B, Hq, N) = sum_j P_j dP_j, which equals sum_c dO[c] *
 * O[c] for the forward's O.  Then for every head h of the group and every
 * row i that sees key j:  P = exp(s_ij - lse_i), dP = dO_i . v_j, and
 *   dk[j] += scale * P * (dP - drow_i) * q_i,   dv[j] += P * dO_i.
 * dk, dv: (nkeys, d) float64.
 */
int attn_oracle_bwd_keys(const void *q, const void *k, const void *v, const void *dout,
                         const double *lse, const double *drow,
                         const int64_t *key_ids, int64_t nkeys, double *dk, double *dv,
                         int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                         int causal, int64_t window, float scale, int dtype)
{
    if (B < 0 || Hq < 1 || Hkv < 1 || N < 1 || d < 1 || Hq % Hkv != 0 || window < 0 ||
        dtype < ORACLE_F16 || dtype > ORACLE_F64 || nkeys < 0)
        return -1;
    for (int64_t r = 0; r < nkeys; ++r)
        if (key_ids[r] < 0 || key_ids[r] >= B * Hkv * N)
            return -1;
    int64_t group = Hq / Hkv;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nkeys; ++r) {
        int64_t id = key_ids[r];
        int64_t j = id % N, hk = (id / N) % Hkv, b = id / (N * Hkv);
        int64_t kvhead = (b * Hkv + hk) * N * d;
        double *dkr = dk + r * d, *dvr = dv + r * d;
        for (int64_t c = 0; c < d; ++c)
            dkr[c] = dvr[c] = 0.0;
        for (int64_t h = hk * group; h < (hk + 1) * group; ++h)
            for (int64_t i = 0; i < N; ++i) {
                int64_t lo, hi;
                visible_range(i, N, N, causal, window, &lo, &hi);
                if (j < lo || j > hi)
                    continue;
                int64_t row = (b * Hq + h) * N + i;
                double dot = 0.0, g = 0.0;
                for (int64_t c = 0; c < d; ++c) {
                    double kc = load_elem(k, dtype, kvhead + j * d + c);
                    dot += load_elem(q, dtype, row * d + c) * kc;
                    g += load_elem(dout, dtype, row * d + c) * load_elem(v, dtype, kvhead + j * d + c);
                }
                double p = exp((double)scale * dot - lse[row]);
                double ds = p * (g - drow[row]);
                for (int64_t c = 0; c < d; ++c) {
                    dkr[c] += (double)scale * ds * load_elem(q, dtype, row * d + c);
                    dvr[c] += p * load_elem(dout, dtype, row * d + c);
                }
            }
    }
    return 0;
}
