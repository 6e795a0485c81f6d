/*
 * oracle.c -- plain, slow float64 reference for gathered sparse attention with
 * per-head sink logits, and for indexer top-k selection.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library. It shares no code, header, table or
 * helper with the GPU library, and the GPU library never calls it.
 *
 * What is computed (the definition, not the tiled algorithm):
 *
 *   akol1/TensorFold pull request 4 ("DeepSeek V4.1: sparse attention on eight
 *   SIMD groups, the same bytes"), first commit message: the kernel scores the
 *   keys selected for a (head, row) in 64-key tiles, keeping a running maximum,
 *   a tile sum and a value sum, over a 512-wide head of sixteen 32-wide output
 *   column groups. The exact quantity such an online softmax reaches is gathered
 *   softmax attention, which is what this file evaluates in one pass.
 *   TensorFold pull request 1206, "What changes" (padding bullet): each head has
 *   a sink, and padded heads get zero sinks. Reading taken here: the sink is one
 *   extra logit in the softmax denominator that carries a zero value vector; it
 *   is not multiplied by the softmax scale.
 *
 * For a row r, head h, with n = nsel[r] selected cache rows i_0..i_{n-1}:
 *   s_j = scale * sum_e q[r,h,e] * K[c(r), i_j, e]          (e ascending)
 *   M   = sink_h, then M = s_j wherever s_j > M             (j ascending)
 *   Z   = exp(sink_h - M) + sum_j exp(s_j - M)
 *   o_e = (sum_j exp(s_j - M) * V[c(r), i_j, e]) / Z
 * c(r) = r when every row has its own cache (decode) and 0 when the rows share
 * one cache (prefill). Every operation is IEEE float64, so infinities and NaNs
 * propagate as IEEE arithmetic dictates. An index outside [0, n_ctx) makes the
 * whole output row of that (row, head) NaN.
 *
 * Top-k (the indexer's selection; pull request 4 names an indexer whose merge
 * and finish give "the same picks"; the problem statement asks for exact
 * selection with ties broken by the lower index):
 *   candidates j in [0, valid_len[r]); order them by score descending under a
 *   total order in which NaN ranks below -inf and -0 equals +0, equal scores by
 *   position ascending; keep the first min(k, valid_len[r]); write those
 *   positions ascending, pad the rest of the row with -1, store the count.
 *
 * Parity pins live in tests/oracle_pins.py (run by tests/test_oracle_pins.py);
 * tests/test_oracle_mutants.py checks that planted mistakes fail them.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_F32 0
#define ORC_BF16 1

#define ORC_OK 0
#define ORC_ERR_ARG 1
#define ORC_ERR_MEM 2

static double widen(const void *base, int dtype, int64_t i)
{
    if (dtype == ORC_F32)
        return (double)((const float *)base)[i];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* One (row, head) of gathered softmax attention with a sink; writes D doubles. */
static int attend_one(int dtype, const void *q, const void *kc, const void *vc,
                      int64_t n_ctx, int64_t cache_rows_stride, const int32_t *idx,
                      int64_t n, const float *sinks, double scale, int64_t H, int64_t D,
                      int64_t r, int64_t h, double *o)
{
    const int64_t cache_base = r * cache_rows_stride * D; /* element offset of cache c(r) */
    const int64_t q_base = (r * H + h) * D;
    double sink = (double)sinks[h];

    for (int64_t j = 0; j < n; j++) {
        if (idx[j] < 0 || (int64_t)idx[j] >= n_ctx) {
            for (int64_t e = 0; e < D; e++)
                o[e] = NAN;
            return ORC_OK;
        }
    }

    double *s = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    if (!s)
        return ORC_ERR_MEM;

    for (int64_t j = 0; j < n; j++) {
        const int64_t k_base = cache_base + (int64_t)idx[j] * D;
        double dot = 0.0;
        for (int64_t e = 0; e < D; e++)
            dot += widen(q, dtype, q_base + e) * widen(kc, dtype, k_base + e);
        s[j] = scale * dot;
    }

    double m = sink;
    for (int64_t j = 0; j < n; j++)
        if (s[j] > m)
            m = s[j];

    double z = exp(sink - m);
    for (int64_t j = 0; j < n; j++)
        z += exp(s[j] - m);

    for (int64_t e = 0; e < D; e++) {
        double num = 0.0;
        for (int64_t j = 0; j < n; j++)
            num += exp(s[j] - m) * widen(vc, dtype, cache_base + (int64_t)idx[j] * D + e);
        o[e] = num / z;
    }
    free(s);
    return ORC_OK;
}

/*
 * Gathered softmax attention with sinks for rows [row_begin, row_end).
 *   dtype           ORC_F32 (q, kc, vc are float) or ORC_BF16 (uint16 bit patterns)
 *   q               [rows, H, D]
 *   kc, vc          caches; cache c holds n_ctx rows of D elements
 *   shared_cache    0: row r reads cache r (decode); 1: every row reads cache 0 (prefill)
 *   idx             [rows, kmax]; row r uses idx[r, 0 .. nsel[r])
 *   nsel            [rows] or NULL (then every row uses kmax indices)
 *   sinks           [H] float
 *   out             [rows, H, D] double; only rows in [row_begin, row_end) are written
 *   threads         OpenMP threads for the independent (row, head) units; <= 0: default
 */
int oracle_attention(int dtype, const void *q, const void *kc, const void *vc,
                     int64_t n_ctx, int shared_cache, const int32_t *idx, const int32_t *nsel,
                     int64_t kmax, const float *sinks, double scale, int64_t rows, int64_t H,
                     int64_t D, double *out, int64_t row_begin, int64_t row_end, int threads)
{
    if (!q || !kc || !vc || !idx || !sinks || !out)
        return ORC_ERR_ARG;
    if ((dtype != ORC_F32 && dtype != ORC_BF16) || rows < 0 || H <= 0 || D <= 0 || kmax < 0 ||
        n_ctx <= 0 || row_begin < 0 || row_end > rows || row_begin > row_end)
        return ORC_ERR_ARG;
    const int64_t stride = shared_cache ? 0 : n_ctx;
    const int64_t units = (row_end - row_begin) * H;
    int err = ORC_OK;
#ifdef _OPENMP
    const int nthreads = threads > 0 ? threads : omp_get_max_threads();
#else
    (void)threads;
#endif

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t u = 0; u < units; u++) {
        const int64_t r = row_begin + u / H;
        const int64_t h = u % H;
        int64_t n = nsel ? (int64_t)nsel[r] : kmax;
        if (n < 0 || n > kmax) {
#pragma omp atomic write
            err = ORC_ERR_ARG;
            continue;
        }
        int e = attend_one(dtype, q, kc, vc, n_ctx, stride, idx + r * kmax, n, sinks, scale, H, D,
                           r, h, out + (r * H + h) * D);
        if (e) {
#pragma omp atomic write
            err = e;
        }
    }
    return err;
}

/* ---------------------------------------------------------------- top-k */

typedef struct {
    float v;
    int32_t j;
} cand_t;

/* Strict weak order: larger score first, NaN after everything, -0 == +0, then lower position. */
static int cand_cmp(const void *pa, const void *pb)
{
    const cand_t *a = (const cand_t *)pa, *b = (const cand_t *)pb;
    int an = isnan(a->v), bn = isnan(b->v);
    if (an != bn)
        return an ? 1 : -1;
    if (!an) {
        if (a->v > b->v)
            return -1;
        if (a->v < b->v)
            return 1;
    }
    return (a->j > b->j) - (a->j < b->j);
}

static int int_cmp(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

/*
 * Exact top-k per row.
 *   scores     [rows, ld] float; row r's candidates are scores[r, 0 .. valid_len[r])
 *   valid_len  [rows] or NULL (then n for every row); each value is clamped to [0, n]
 *   idx_out    [rows, k] int32: selected positions ascending, then -1
 *   count_out  [rows] or NULL: number of selected positions
 */
int oracle_topk(const float *scores, int64_t rows, int64_t n, int64_t ld, const int32_t *valid_len,
                int64_t k, int32_t *idx_out, int32_t *count_out)
{
    if (!scores || !idx_out || rows < 0 || n < 0 || ld < n || k <= 0)
        return ORC_ERR_ARG;
    cand_t *c = (cand_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof(cand_t));
    int32_t *sel = (int32_t *)malloc((size_t)k * sizeof(int32_t));
    if (!c || !sel) {
        free(c);
        free(sel);
        return ORC_ERR_MEM;
    }
    for (int64_t r = 0; r < rows; r++) {
        int64_t vl = valid_len ? (int64_t)valid_len[r] : n;
        if (vl < 0)
            vl = 0;
        if (vl > n)
            vl = n;
        for (int64_t j = 0; j < vl; j++) {
            c[j].v = scores[r * ld + j];
            c[j].j = (int32_t)j;
        }
        qsort(c, (size_t)vl, sizeof(cand_t), cand_cmp);
        int64_t cnt = vl < k ? vl : k;
        for (int64_t t = 0; t < cnt; t++)
            sel[t] = c[t].j;
        qsort(sel, (size_t)cnt, sizeof(int32_t), int_cmp);
        for (int64_t t = 0; t < k; t++)
            idx_out[r * k + t] = t < cnt ? sel[t] : -1;
        if (count_out)
            count_out[r] = (int32_t)cnt;
    }
    free(c);
    free(sel);
    return ORC_OK;
}
