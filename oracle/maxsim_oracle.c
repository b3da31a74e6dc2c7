/*
 * Plain fp64 CPU oracle for Flash-MaxSim reranking.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
 * baseline use this file. The GPU library neither links it nor shares any code,
 * header, table or constant with it.
 *
 * What it computes (Flash-MaxSim rerank page, docs.vllm.ai,
 * vllm.v1.pool.flash_maxsim.flash_maxsim_rerank: the module description and the
 * `flash_maxsim_rerank_direct` parameter and return descriptions): one query Q with
 * Lq token rows of width d is scored against B docs. Doc i is the run of
 * lengths[i] consecutive rows of a packed row tensor X that starts at row
 * offsets[i]; docs may sit anywhere in X. Its score is
 *
 *     score_i = sum over q < Lq of ( max over t < len_i of  sum over k < d of
 *               Q[q][k] * X[offsets[i] + t][k] )
 *
 * i.e. each query row takes its best-matching doc row by dot product and the
 * per-row bests are added up, one float per doc.
 *
 * Readings of the page, stated where they apply below:
 *   - The page's kernel (section `_maxsim_rerank_kernel`) starts each query
 *     row's running max at minus infinity and only lets valid doc rows raise it,
 *     so a doc with no rows scores minus infinity; with Lq = 0 the sum is empty
 *     and the score is 0. Both fall out of the definition as written here.
 *   - The page computes in fp16 with fp32 accumulation; the oracle decodes the
 *     stored fp16 or bf16 bits exactly and does every product and sum in fp64,
 *     sequentially in k, then t, then q.
 *   - Rows are `stride` elements apart (stride >= d); columns d..stride-1 and
 *     rows outside every doc are never read.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (no fused multiply-add,
 * so each product is rounded to fp64 before it is added).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Format codes shared with the Python wrapper of this oracle. */
#define ORACLE_FMT_F16 0
#define ORACLE_FMT_BF16 1

/*
 * IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 *   exponent 0      -> subnormal (or zero):  fraction * 2^-24
 *   exponent 1..30  -> normal: (1024 + fraction) * 2^(exponent - 25)
 *   exponent 31     -> infinity (fraction 0) or NaN
 */
double oracle_decode_f16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1F;
    int frac = h & 0x3FF;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), expo - 25);
    return sign ? -v : v;
}

/*
 * bfloat16: the upper half of an IEEE 754 binary32 word, i.e. 1 sign bit,
 * 8 exponent bits (bias 127), 7 fraction bits.
 *   exponent 0       -> subnormal (or zero):  fraction * 2^-133
 *   exponent 1..254  -> normal: (128 + fraction) * 2^(exponent - 134)
 *   exponent 255     -> infinity (fraction 0) or NaN
 */
double oracle_decode_bf16(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int expo = (b >> 7) & 0xFF;
    int frac = b & 0x7F;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -133);
    else if (expo == 255)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + frac), expo - 134);
    return sign ? -v : v;
}

/* Decoded value of every 16-bit pattern of one format (out has 65536 entries). */
int oracle_decode_table(int fmt, double *out)
{
    if (fmt != ORACLE_FMT_F16 && fmt != ORACLE_FMT_BF16)
        return 1;
    for (uint32_t u = 0; u < 65536u; ++u)
        out[u] = fmt == ORACLE_FMT_F16 ? oracle_decode_f16((uint16_t)u)
                                       : oracle_decode_bf16((uint16_t)u);
    return 0;
}

/*
 * MaxSim scores of B docs against one query, in fp64 (definition above).
 *
 * Q        [Lq * d] raw bits, row q at Q + q*d
 * X        raw bits, doc row t of doc i at X + (offsets[i] + t) * stride
 * offsets  [B] first row of each doc (the 64-bit product offset*stride is formed
 *          in int64, as the page's kernel widens the offset before it multiplies)
 * lengths  [B] rows per doc
 * scores   [B] output
 * nthreads OpenMP threads over docs (<= 0: the OpenMP default)
 *
 * Returns 0, or 1 for an unknown format or a negative size. Offsets and lengths
 * are trusted to stay inside X.
 */
int maxsim_oracle_f64(int fmt, const uint16_t *Q, int32_t Lq, int32_t d,
                      const uint16_t *X, int64_t stride,
                      const int32_t *offsets, const int32_t *lengths, int32_t B,
                      double *scores, int nthreads)
{
    if (fmt != ORACLE_FMT_F16 && fmt != ORACLE_FMT_BF16)
        return 1;
    if (Lq < 0 || d < 0 || B < 0 || stride < d)
        return 1;

    double *tab = (double *)malloc(65536 * sizeof(double));
    double *Qd = (double *)malloc(((size_t)Lq * (size_t)d + 1) * sizeof(double));
    if (!tab || !Qd) {
        free(tab);
        free(Qd);
        return 1;
    }
    oracle_decode_table(fmt, tab);
    for (int64_t e = 0; e < (int64_t)Lq * d; ++e)
        Qd[e] = tab[Q[e]];

#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int32_t i = 0; i < B; ++i) {
        const int64_t off = (int64_t)offsets[i];
        const int64_t len = (int64_t)lengths[i];
        double s = 0.0;
        for (int32_t q = 0; q < Lq; ++q) {
            double m = -INFINITY;
            for (int64_t t = 0; t < len; ++t) {
                const uint16_t *row = X + (off + t) * stride;
                double dot = 0.0;
                for (int32_t k = 0; k < d; ++k)
                    dot += Qd[(int64_t)q * d + k] * tab[row[k]];
                if (dot > m)
                    m = dot;
            }
            s += m;
        }
        scores[i] = s;
    }

    free(tab);
    free(Qd);
    return 0;
}

/*
 * FP8 E4M3 ("e4m3fn" of the OCP 8-bit floating point formats): 1 sign bit, 4 exponent
 * bits (bias 7), 3 fraction bits, no infinities.
 *   exponent 0                   -> subnormal (or zero):  fraction * 2^-9
 *   exponent 1..15 (not S.1111.111) -> normal: (8 + fraction) * 2^(exponent - 10)
 *   S.1111.111                   -> NaN
 * Largest finite magnitude 448 (S.1111.110).
 */
double oracle_decode_e4m3(uint8_t b)
{
    int sign = (b >> 7) & 1;
    int expo = (b >> 3) & 0xF;
    int frac = b & 0x7;
    double v;
    if (expo == 15 && frac == 7)
        return NAN;
    if (expo == 0)
        v = ldexp((double)frac, -9);
    else
        v = ldexp((double)(8 + frac), expo - 10);
    return sign ? -v : v;
}

/* Decoded value of every 8-bit E4M3 pattern (out has 256 entries). */
void oracle_decode_e4m3_table(double *out)
{
    for (uint32_t u = 0; u < 256u; ++u)
        out[u] = oracle_decode_e4m3((uint8_t)u);
}

/*
 * Docs stored as FP8 E4M3 bits with one scale for the whole doc tensor: doc element
 * = doc_scale * e4m3(bits), as FP8 caches are dequantised with a per-tensor scale
 * (sparse prefill pages page, docs.vllm.ai, `stage_prefill_pages`: FP8 E4M3 pages
 * with k/v scales). The query stays fp16 or bf16 (qfmt). Same definition and loop
 * order as maxsim_oracle_f64.
 *
 * X  raw bytes, doc row t of doc i at X + (offsets[i] + t) * stride (stride in
 *    elements = bytes)
 */
int maxsim_oracle_fp8_f64(int qfmt, const uint16_t *Q, int32_t Lq, int32_t d,
                          const uint8_t *X, int64_t stride,
                          const int32_t *offsets, const int32_t *lengths, int32_t B,
                          double doc_scale, double *scores, int nthreads)
{
    if (qfmt != ORACLE_FMT_F16 && qfmt != ORACLE_FMT_BF16)
        return 1;
    if (Lq < 0 || d < 0 || B < 0 || stride < d)
        return 1;

    double *tab = (double *)malloc(65536 * sizeof(double));
    double *Qd = (double *)malloc(((size_t)Lq * (size_t)d + 1) * sizeof(double));
    if (!tab || !Qd) {
        free(tab);
        free(Qd);
        return 1;
    }
    oracle_decode_table(qfmt, tab);
    for (int64_t e = 0; e < (int64_t)Lq * d; ++e)
        Qd[e] = tab[Q[e]];
    double xtab[256];
    for (uint32_t u = 0; u < 256u; ++u)
        xtab[u] = doc_scale * oracle_decode_e4m3((uint8_t)u);

#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int32_t i = 0; i < B; ++i) {
        const int64_t off = (int64_t)offsets[i];
        const int64_t len = (int64_t)lengths[i];
        double s = 0.0;
        for (int32_t q = 0; q < Lq; ++q) {
            double m = -INFINITY;
            for (int64_t t = 0; t < len; ++t) {
                const uint8_t *row = X + (off + t) * stride;
                double dot = 0.0;
                for (int32_t k = 0; k < d; ++k)
                    dot += Qd[(int64_t)q * d + k] * xtab[row[k]];
                if (dot > m)
                    m = dot;
            }
            s += m;
        }
        scores[i] = s;
    }

    free(tab);
    free(Qd);
    return 0;
}

/* Threads an OpenMP parallel region of this library would use by default. */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
