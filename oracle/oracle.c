/*
 * Plain CPU fp64 oracle for fused scaled-dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header or constant with
 * the HIP library.
 *
 * What it computes is the plain definition, written out with no blocking,
 * no fusion and no reordering beyond the definition itself:
 *
 *   Attention(Q, K, V) = softmax(Q K^T / sqrt(d_k)) V
 *     -- "FlashInfer kernel library ..." (zyxy.net/archives/24491),
 *        section 1 "Background and challenges": similarity of Q and K, a
 *        softmax that turns the weights into a probability distribution, then
 *        the weighted sum with V.
 *
 * The softmax is the numerically stable form (subtract the row maximum
 * before exponentiating, then divide by the sum), as the same page's
 * section 3 example and the TensorRT-LLM FMHA page (zyxy.net/?p=24414,
 * section 2, "numerical stability") ask for.  The full score matrix of each
 * (batch, head) is materialised in fp64.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - the scale is an explicit argument (1/sqrt(d) in every workload);
 *   - lse_i = ln sum_j exp(s_ij), natural log of the scaled scores, so
 *     lse_i = m_i + ln l_i with m_i the row max and l_i the sum of
 *     exp(s_ij - m_i);
 *   - causal: key j is masked for query i when j > i + (Tk - Tq)
 *     (bottom-right alignment; identical to top-left when Tq == Tk);
 *   - a row with every key masked gives O = 0 and lse = -inf;
 *   - grouped heads: query head h reads key/value head h / (Hq / Hkv);
 *   - paged cache: token t of sequence b lives in physical page
 *     block_table[b][t / page_size], slot t % page_size, and a page holds
 *     [Hkv][page_size][D] elements (the paged-attention description on the
 *     xhh.club page, "how does paged attention manage the KV cache": fixed
 *     size blocks mapped logical-to-physical through a block table);
 *   - merging two partial states (o_a, lse_a), (o_b, lse_b) of disjoint key
 *     sets gives the state of their union:
 *       M = max(lse_a, lse_b); w_x = exp(lse_x - M);
 *       lse = M + ln(w_a + w_b); o = (w_a o_a + w_b o_b) / (w_a + w_b),
 *     with (anything, -inf) as the identity.  (The FlashDecoding++ summary,
 *     wenjunhu.com/d/2311396.html, section 1, says split partial softmax
 *     results are combined at the end; the formula is not printed there.)
 *
 * Element types: inputs may be fp64, fp32 or bf16 (given as raw 16-bit
 * patterns); every element is widened to fp64 exactly before use.  A paged
 * cache may also hold 8-bit floats (OCP FP8 E4M3, one byte per element) with
 * one scale per tensor: the element's value is scale * e4m3(byte), and
 * attention is the plain definition on those values (quantised caches are
 * named as an inference optimisation on the TensorRT-LLM FMHA page,
 * sections 3, 4 and 7; the format is the OCP 8-bit floating point one).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F64 = 0, ORC_F32 = 1, ORC_BF16 = 2 };

/* Exact widening of one stored element to fp64. */
static double load_elem(const void *base, int dtype, size_t idx)
{
    if (dtype == ORC_F64)
        return ((const double *)base)[idx];
    if (dtype == ORC_F32)
        return (double)((const float *)base)[idx];
    /* bf16: the 16 stored bits are the top half of an fp32 pattern */
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/*
 * OCP FP8 E4M3 byte -> fp64, from the format's definition: 1 sign bit, 4
 * exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
 * subnormals m/8 * 2^-6; the pattern S.1111.111 is NaN (there is no
 * infinity), so the largest finite magnitude is 1.75 * 2^8 = 448.
 */
double oracle_e4m3_value(uint8_t byte)
{
    const int sign = byte >> 7, e = (byte >> 3) & 15, m = byte & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

/*
 * Attention of tq query rows against tk key/value rows, all in fp64.
 * Q is [tq][d], K and V are [tk][d], O is [tq][d], lse is [tq].
 * S is a caller-provided [tq][tk] buffer: the materialised score matrix.
 */
static void attend_rows(const double *Q, const double *K, const double *V,
                        int tq, int tk, int d, int causal, double scale,
                        double *S, double *O, double *lse)
{
    /* step 1: similarity, S = scale * Q K^T (summed in d order) */
    for (int i = 0; i < tq; i++) {
        for (int j = 0; j < tk; j++) {
            double acc = 0.0;
            for (int c = 0; c < d; c++)
                acc += Q[(size_t)i * d + c] * K[(size_t)j * d + c];
            S[(size_t)i * tk + j] = scale * acc;
        }
    }
    /* causal mask (bottom-right aligned) */
    if (causal) {
        for (int i = 0; i < tq; i++)
            for (int j = 0; j < tk; j++)
                if (j > i + (tk - tq))
                    S[(size_t)i * tk + j] = -INFINITY;
    }
    /* step 2: stable softmax per row; step 3: weighted sum with V */
    for (int i = 0; i < tq; i++) {
        double *row = S + (size_t)i * tk;
        double m = -INFINITY;
        for (int j = 0; j < tk; j++)
            if (row[j] > m)
                m = row[j];
        double *o = O + (size_t)i * d;
        if (m == -INFINITY) {          /* no key attended */
            for (int c = 0; c < d; c++)
                o[c] = 0.0;
            lse[i] = -INFINITY;
            continue;
        }
        double l = 0.0;
        for (int j = 0; j < tk; j++) {
            row[j] = exp(row[j] - m);
            l += row[j];
        }
        for (int c = 0; c < d; c++) {
            double acc = 0.0;
            for (int j = 0; j < tk; j++)
                acc += row[j] * V[(size_t)j * d + c];
            o[c] = acc / l;
        }
        lse[i] = m + log(l);
    }
}

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/*
 * Dense attention.  q is [B][Hq][Tq][D]; k, v are [B][Hkv][Tk][D];
 * o is fp64 [B][Hq][Tq][D]; lse is fp64 [B][Hq][Tq].
 * Returns 0, or -1 on a bad shape, -2 if memory runs out.
 */
int oracle_attention(const void *q, const void *k, const void *v, int dtype,
                     double *o, double *lse,
                     int B, int Hq, int Hkv, int Tq, int Tk, int D,
                     int causal, double scale, int nthreads)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || Tq < 0 || Tk < 0 || D <= 0)
        return -1;
    const int group = Hq / Hkv;
    int failed = 0;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic)
    for (long bh = 0; bh < (long)B * Hq; bh++) {
        const int b = (int)(bh / Hq), h = (int)(bh % Hq), kvh = h / group;
        double *Q = malloc(sizeof(double) * ((size_t)Tq * D + 1));
        double *K = malloc(sizeof(double) * ((size_t)Tk * D + 1));
        double *V = malloc(sizeof(double) * ((size_t)Tk * D + 1));
        double *S = malloc(sizeof(double) * ((size_t)Tq * Tk + 1));
        if (!Q || !K || !V || !S) {
#pragma omp atomic write
            failed = 1;
        } else {
            const size_t qbase = ((size_t)b * Hq + h) * Tq * D;
            const size_t kbase = ((size_t)b * Hkv + kvh) * Tk * D;
            for (size_t e = 0; e < (size_t)Tq * D; e++)
                Q[e] = load_elem(q, dtype, qbase + e);
            for (size_t e = 0; e < (size_t)Tk * D; e++) {
                K[e] = load_elem(k, dtype, kbase + e);
                V[e] = load_elem(v, dtype, kbase + e);
            }
            attend_rows(Q, K, V, Tq, Tk, D, causal, scale, S,
                        o + qbase, lse + ((size_t)b * Hq + h) * Tq);
        }
        free(Q); free(K); free(V); free(S);
    }
    return failed ? -2 : 0;
}

/*
 * Decode over a paged cache: one query row per (sequence, query head).
 * q is [B][Hq][D]; k_pages, v_pages are [num_pages][Hkv][page_size][D];
 * block_table is int32 [B][max_pages]; kv_lens is int32 [B].
 * The query of sequence b attends exactly its kv_lens[b] cached tokens.
 * o is fp64 [B][Hq][D], lse fp64 [B][Hq].
 */
int oracle_decode_paged(const void *q, const void *k_pages, const void *v_pages,
                        int dtype, const int32_t *block_table,
                        const int32_t *kv_lens, double *o, double *lse,
                        int B, int Hq, int Hkv, int D, int page_size,
                        int max_pages, long num_pages, double scale, int nthreads)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || D <= 0 || page_size <= 0)
        return -1;
    for (int b = 0; b < B; b++) {
        const int L = kv_lens[b];
        if (L < 0 || (L + page_size - 1) / page_size > max_pages)
            return -1;
        for (int p = 0; p < (L + page_size - 1) / page_size; p++) {
            const int32_t pg = block_table[(size_t)b * max_pages + p];
            if (pg < 0 || pg >= num_pages)
                return -1;
        }
    }
    const int group = Hq / Hkv;
    int failed = 0;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic)
    for (long bk = 0; bk < (long)B * Hkv; bk++) {
        const int b = (int)(bk / Hkv), kvh = (int)(bk % Hkv);
        const int L = kv_lens[b];
        double *K = malloc(sizeof(double) * ((size_t)L * D + 1));
        double *V = malloc(sizeof(double) * ((size_t)L * D + 1));
        double *Q = malloc(sizeof(double) * ((size_t)D + 1));
        double *S = malloc(sizeof(double) * ((size_t)L + 1));
        if (!K || !V || !Q || !S) {
#pragma omp atomic write
            failed = 1;
        } else {
            /* gather the logical key/value rows through the block table */
            for (int t = 0; t < L; t++) {
                const size_t page = (size_t)block_table[(size_t)b * max_pages + t / page_size];
                const size_t src = ((page * Hkv + kvh) * page_size + t % page_size) * D;
                for (int c = 0; c < D; c++) {
                    K[(size_t)t * D + c] = load_elem(k_pages, dtype, src + c);
                    V[(size_t)t * D + c] = load_elem(v_pages, dtype, src + c);
                }
            }
            for (int g = 0; g < group; g++) {
                const int h = kvh * group + g;
                const size_t row = (size_t)b * Hq + h;
                for (int c = 0; c < D; c++)
                    Q[c] = load_elem(q, dtype, row * D + c);
                attend_rows(Q, K, V, 1, L, D, 0, scale, S, o + row * D, lse + row);
            }
        }
        free(K); free(V); free(Q); free(S);
    }
    return failed ? -2 : 0;
}

/*
 * Prefill against a paged cache (chunked prefill).  The Tq query tokens of
 * sequence b are its last Tq positions; they attend the sequence's
 * kv_lens[b] cached keys, which include themselves, so query i sits at
 * position kv_lens[b] - Tq + i and, under the causal mask, sees key j
 * exactly when j <= i + (kv_lens[b] - Tq): the bottom-right alignment of
 * attend_rows with tk = kv_lens[b].  (The xhh.club summary, "FlashAttention
 * and paged attention", says the tiled kernel and the paged cache can be
 * used together; the gather is the paged-cache reading above.)
 * q is [B][Hq][Tq][D]; k_pages, v_pages, block_table, kv_lens as
 * oracle_decode_paged; o is fp64 [B][Hq][Tq][D], lse fp64 [B][Hq][Tq].
 */
int oracle_prefill_paged(const void *q, const void *k_pages, const void *v_pages,
                         int dtype, const int32_t *block_table,
                         const int32_t *kv_lens, double *o, double *lse,
                         int B, int Hq, int Hkv, int Tq, int D, int page_size,
                         int max_pages, long num_pages, int causal, double scale,
                         int nthreads)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || Tq < 0 || D <= 0 || page_size <= 0)
        return -1;
    for (int b = 0; b < B; b++) {
        const int L = kv_lens[b];
        if (L < 0 || (L + page_size - 1) / page_size > max_pages)
            return -1;
        for (int p = 0; p < (L + page_size - 1) / page_size; p++) {
            const int32_t pg = block_table[(size_t)b * max_pages + p];
            if (pg < 0 || pg >= num_pages)
                return -1;
        }
    }
    const int group = Hq / Hkv;
    int failed = 0;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic)
    for (long bh = 0; bh < (long)B * Hq; bh++) {
        const int b = (int)(bh / Hq), h = (int)(bh % Hq), kvh = h / group;
        const int L = kv_lens[b];
        const int32_t *table = block_table + (size_t)b * max_pages;
        double *K = malloc(sizeof(double) * ((size_t)L * D + 1));
        double *V = malloc(sizeof(double) * ((size_t)L * D + 1));
        double *Q = malloc(sizeof(double) * ((size_t)Tq * D + 1));
        double *S = malloc(sizeof(double) * ((size_t)Tq * L + 1));
        if (!K || !V || !Q || !S) {
#pragma omp atomic write
            failed = 1;
        } else {
            /* the sequence's logical key/value rows, through its table */
            for (int t = 0; t < L; t++) {
                const size_t page = (size_t)table[t / page_size];
                const size_t src = ((page * Hkv + kvh) * page_size + t % page_size) * D;
                for (int c = 0; c < D; c++) {
                    K[(size_t)t * D + c] = load_elem(k_pages, dtype, src + c);
                    V[(size_t)t * D + c] = load_elem(v_pages, dtype, src + c);
                }
            }
            const size_t qbase = (size_t)bh * Tq * D;
            for (size_t e = 0; e < (size_t)Tq * D; e++)
                Q[e] = load_elem(q, dtype, qbase + e);
            attend_rows(Q, K, V, Tq, L, D, causal, scale, S, o + qbase, lse + (size_t)bh * Tq);
        }
        free(K); free(V); free(Q); free(S);
    }
    return failed ? -2 : 0;
}

/*
 * Flat GEMM of the decode phase: C = A W^T with A [m][k] (the m tokens of a
 * decode step, m small) and W [n][k] (a layer's weight, n x k as the
 * FlashDecoding++ summary, section 5, writes the projections' shapes), so
 * C[i][j] = sum_t A[i][t] * W[j][t], summed in t order in fp64.  Inputs in
 * `dtype`, widened exactly; c is fp64 [m][n].
 */
int oracle_flat_gemm(const void *a, const void *w, int dtype, double *c,
                     int m, int n, int k, int nthreads)
{
    if (m < 0 || n < 0 || k < 0)
        return -1;
    set_threads(nthreads);
#pragma omp parallel for schedule(static)
    for (long ij = 0; ij < (long)m * n; ij++) {
        const int i = (int)(ij / n), j = (int)(ij % n);
        double acc = 0.0;
        for (int t = 0; t < k; t++)
            acc += load_elem(a, dtype, (size_t)i * k + t) * load_elem(w, dtype, (size_t)j * k + t);
        c[ij] = acc;
    }
    return 0;
}

/*
 * Paged decode over an FP8 cache: k_pages and v_pages are E4M3 bytes
 * [num_pages][Hkv][page_size][D], dequantised as k_scale * e4m3(byte) and
 * v_scale * e4m3(byte); q is in dtype q_dtype.  Everything else as
 * oracle_decode_paged (the same gather, then the plain attention of one
 * query row over the dequantised keys and values).
 */
int oracle_decode_paged_fp8(const void *q, int q_dtype, const uint8_t *k_pages,
                            const uint8_t *v_pages, double k_scale, double v_scale,
                            const int32_t *block_table, const int32_t *kv_lens,
                            double *o, double *lse, int B, int Hq, int Hkv, int D,
                            int page_size, int max_pages, long num_pages, double scale,
                            int nthreads)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || D <= 0 || page_size <= 0)
        return -1;
    for (int b = 0; b < B; b++) {
        const int L = kv_lens[b];
        if (L < 0 || (L + page_size - 1) / page_size > max_pages)
            return -1;
        for (int p = 0; p < (L + page_size - 1) / page_size; p++) {
            const int32_t pg = block_table[(size_t)b * max_pages + p];
            if (pg < 0 || pg >= num_pages)
                return -1;
        }
    }
    const int group = Hq / Hkv;
    int failed = 0;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic)
    for (long bk = 0; bk < (long)B * Hkv; bk++) {
        const int b = (int)(bk / Hkv), kvh = (int)(bk % Hkv);
        const int L = kv_lens[b];
        double *K = malloc(sizeof(double) * ((size_t)L * D + 1));
        double *V = malloc(sizeof(double) * ((size_t)L * D + 1));
        double *Q = malloc(sizeof(double) * ((size_t)D + 1));
        double *S = malloc(sizeof(double) * ((size_t)L + 1));
        if (!K || !V || !Q || !S) {
#pragma omp atomic write
            failed = 1;
        } else {
            for (int t = 0; t < L; t++) {
                const size_t page = (size_t)block_table[(size_t)b * max_pages + t / page_size];
                const size_t src = ((page * Hkv + kvh) * page_size + t % page_size) * D;
                for (int c = 0; c < D; c++) {
                    K[(size_t)t * D + c] = k_scale * oracle_e4m3_value(k_pages[src + c]);
                    V[(size_t)t * D + c] = v_scale * oracle_e4m3_value(v_pages[src + c]);
                }
            }
            for (int g = 0; g < group; g++) {
                const int h = kvh * group + g;
                const size_t row = (size_t)b * Hq + h;
                for (int c = 0; c < D; c++)
                    Q[c] = load_elem(q, q_dtype, row * D + c);
                attend_rows(Q, K, V, 1, L, D, 0, scale, S, o + row * D, lse + row);
            }
        }
        free(K); free(V); free(Q); free(S);
    }
    return failed ? -2 : 0;
}

/*
 * Merge of two partial states over disjoint key sets, row by row.
 * o_a, o_b, o_out are fp64 [rows][D]; lse_* are fp64 [rows].
 * o_out/lse_out may alias either input.
 */
void oracle_merge_states(const double *o_a, const double *lse_a,
                         const double *o_b, const double *lse_b,
                         double *o_out, double *lse_out, long rows, int D)
{
    for (long r = 0; r < rows; r++) {
        const double la = lse_a[r], lb = lse_b[r];
        const double M = la > lb ? la : lb;
        if (M == -INFINITY) {
            for (int c = 0; c < D; c++)
                o_out[r * D + c] = 0.0;
            lse_out[r] = -INFINITY;
            continue;
        }
        const double wa = exp(la - M), wb = exp(lb - M);
        for (int c = 0; c < D; c++) {
            /* a side with weight 0 (lse = -inf) is absent, whatever its o */
            const double ta = wa > 0.0 ? wa * o_a[r * D + c] : 0.0;
            const double tb = wb > 0.0 ? wb * o_b[r * D + c] : 0.0;
            o_out[r * D + c] = (ta + tb) / (wa + wb);
        }
        lse_out[r] = M + log(wa + wb);
    }
}

/*
 * Fallback model of the unified-max softmax (FlashDecoding++ summary,
 * wenjunhu.com/d/2311396.html, sections 1 and 3: every partial softmax uses
 * one fixed maximum phi; a partial whose values leave the range the fixed
 * maximum can serve is recomputed).  The pages fix neither phi nor the test;
 * the reading adopted: with s = scale * q.k, the pair (query row, chunk of
 * split_tokens keys) falls back when max_chunk(s) - phi > window or
 * max_chunk(s) - phi < -window.  Returns the number of such pairs over all
 * (b, hq) rows and chunks c < ceil(kv_lens[b] / split_tokens), scores in
 * fp64, or a negative value on bad arguments.
 */
long oracle_unified_fallback_count(const void *q, const void *k_pages, int dtype,
                                   const int32_t *block_table, const int32_t *kv_lens,
                                   int B, int Hq, int Hkv, int D, int page_size,
                                   int max_pages, double scale, int split_tokens,
                                   double phi, double window)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || D <= 0 || page_size <= 0 ||
        split_tokens <= 0)
        return -1;
    const int group = Hq / Hkv;
    long count = 0;
    for (int b = 0; b < B; b++) {
        const int L = kv_lens[b];
        if (L < 0 || (L + page_size - 1) / page_size > max_pages)
            return -1;
        for (int h = 0; h < Hq; h++) {
            const int kvh = h / group;
            for (int c0 = 0; c0 < L; c0 += split_tokens) {
                const int c1 = c0 + split_tokens < L ? c0 + split_tokens : L;
                double m = -INFINITY;
                for (int t = c0; t < c1; t++) {
                    const size_t page = (size_t)block_table[(size_t)b * max_pages + t / page_size];
                    const size_t src = ((page * Hkv + kvh) * page_size + t % page_size) * D;
                    double dot = 0.0;
                    for (int d = 0; d < D; d++)
                        dot += load_elem(q, dtype, ((size_t)b * Hq + h) * D + d) *
                               load_elem(k_pages, dtype, src + d);
                    const double s = scale * dot;
                    if (s > m)
                        m = s;
                }
                if (m - phi > window || m - phi < -window)
                    count++;
            }
        }
    }
    return count;
}
