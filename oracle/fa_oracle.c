/*
 * fa_oracle.c -- plain fp64 CPU reference for exact attention.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the package's
 * smoke check and the benchmark's CPU-baseline leg may load this library.
 * It shares no code with the HIP path and must never be called by it.
 *
 * What it computes (the plain definition, written out):
 *   For batch b, head h and query row i,
 *     s_j   = scale * sum_c q[b,h,i,c] * k[b,h,j,c]                   for every key j
 *     valid(j) = (kv_limit == NULL or j < kv_limit[b,i]) and (!causal or j <= i)
 *     m     = max over valid j of s_j
 *     w_j   = exp(s_j - m) for valid j, 0 otherwise
 *     l     = sum_j w_j
 *     o[i]  = sum_j w_j * v[b,h,j,:] / l
 *     lse[i]= m + ln(l)
 *   A row with no valid key gets o = 0 and lse = -inf.
 *
 * Sources on the pages:
 *   - O = softmax(Q K^T / sqrt(d) + M) V with an additive mask M that is -inf
 *     at future positions, Q/K/V shaped [b, h, seq, d]:
 *     "谁偷走了 5090 的算力和显存", attention section (the equation for O and
 *     the five eager steps that follow it).
 *   - Standard attention as S = Q K^T / sqrt(d), P = softmax(S), O = P V:
 *     "FlashAttention 1–4: How IO-Awareness Reshaped the Attention Kernel",
 *     section "Why attention is memory-bound, not compute-bound".
 *   - Subtracting the row max before exp so it cannot overflow: the same
 *     "5090" page, softmax paragraph after the roofline figure (Fig. 3-5).
 *   - The per-row log-sum-exp L = m + log(l) as the saved statistic:
 *     "FlashAttention 1–4 ...", section "FlashAttention-2" (fewer non-matmul
 *     FLOPs), and "GPU 与 TPU：让硬件不再是黑魔法" §11.4.
 *   - The result is exact attention; a tiled method differs only in the
 *     order of floating-point summation: "FlashAttention 1–4 ...", the
 *     exactness paragraph of section "FlashAttention (v1)".
 *   - A fully masked row must not compute -inf minus -inf:
 *     "07 GPU、资源估算与 FlashAttention" §7.8.  The pages do not say what such
 *     a row outputs; this oracle reads it as the empty sum: o = 0, lse = -inf.
 *
 * This is a two-pass row softmax (max, then exp-and-sum), not the online
 * recurrence the GPU kernel uses.  Inputs are fp64 copies of the exact
 * bf16/fp32 values; all arithmetic is fp64.  No BLAS.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static int key_is_valid(int64_t j, int64_t i, int causal, int64_t limit)
{
    if (causal && j > i) return 0;
    return j < limit;
}

/* One query row: fills o_row[0..d) and *lse_row.  s is scratch of length N. */
static void one_row(const double *q, const double *k, const double *v,
                    double *o_row, double *lse_row,
                    int64_t H, int64_t N, int64_t d, int causal, double scale,
                    const int32_t *kv_limit, int64_t b, int64_t h, int64_t i,
                    double *s)
{
    const double *qi = q + ((b * H + h) * N + i) * d;
    const double *kh = k + (b * H + h) * N * d;
    const double *vh = v + (b * H + h) * N * d;
    int64_t limit = kv_limit ? (int64_t)kv_limit[b * N + i] : N;
    if (limit > N) limit = N;

    /* 1. scores */
    for (int64_t j = 0; j < N; ++j) {
        double acc = 0.0;
        for (int64_t c = 0; c < d; ++c) {
            acc += qi[c] * kh[j * d + c];
        }
        s[j] = scale * acc;
    }

    /* 2. max over the valid keys */
    double m = -INFINITY;
    int64_t n_valid = 0;
    for (int64_t j = 0; j < N; ++j) {
        if (!key_is_valid(j, i, causal, limit)) continue;
        ++n_valid;
        if (s[j] > m) m = s[j];
    }
    if (n_valid == 0) {
        for (int64_t c = 0; c < d; ++c) o_row[c] = 0.0;
        *lse_row = -INFINITY;
        return;
    }

    /* 3. weights, their sum, and the weighted sum of value rows */
    double l = 0.0;
    for (int64_t c = 0; c < d; ++c) o_row[c] = 0.0;
    for (int64_t j = 0; j < N; ++j) {
        if (!key_is_valid(j, i, causal, limit)) continue;
        double w = exp(s[j] - m);
        l += w;
        for (int64_t c = 0; c < d; ++c) o_row[c] += w * vh[j * d + c];
    }
    for (int64_t c = 0; c < d; ++c) o_row[c] /= l;
    *lse_row = m + log(l);
}

/* Every row of a [B, H, N, d] problem.  o is [B, H, N, d], lse is [B, H, N].
 * nthreads <= 0 uses the OpenMP default.  Returns 0, or -1 on bad arguments
 * or an allocation failure. */
int fa_oracle_fwd(const double *q, const double *k, const double *v,
                  double *o, double *lse,
                  int64_t B, int64_t H, int64_t N, int64_t d,
                  int causal, double scale, const int32_t *kv_limit, int nthreads)
{
    if (!q || !k || !v || !o || !lse || B < 0 || H < 0 || N < 0 || d <= 0) return -1;
    const int64_t rows = B * H * N;
    int failed = 0;
#ifdef _OPENMP
    const int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
#endif
#pragma omp parallel num_threads(nt)
    {
        double *s = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        if (!s) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < rows; ++r) {
                int64_t i = r % N, bh = r / N;
                one_row(q, k, v, o + r * d, lse + r, H, N, d, causal, scale, kv_limit,
                        bh / H, bh % H, i, s);
            }
            free(s);
        }
    }
    return failed ? -1 : 0;
}

/* Selected rows only: row_ids[t] = (b * H + h) * N + i.  o is [nrows, d],
 * lse is [nrows].  Used for full-size checks on sampled outputs. */
int fa_oracle_rows(const double *q, const double *k, const double *v,
                   double *o, double *lse,
                   int64_t B, int64_t H, int64_t N, int64_t d,
                   int causal, double scale, const int32_t *kv_limit,
                   int64_t nrows, const int64_t *row_ids, int nthreads)
{
    if (!q || !k || !v || !o || !lse || !row_ids || d <= 0 || N <= 0) return -1;
    for (int64_t t = 0; t < nrows; ++t)
        if (row_ids[t] < 0 || row_ids[t] >= B * H * N) return -1;
    int failed = 0;
#ifdef _OPENMP
    const int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
#endif
#pragma omp parallel num_threads(nt)
    {
        double *s = (double *)malloc((size_t)N * sizeof(double));
        if (!s) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t t = 0; t < nrows; ++t) {
                int64_t r = row_ids[t];
                int64_t i = r % N, bh = r / N;
                one_row(q, k, v, o + t * d, lse + t, H, N, d, causal, scale, kv_limit,
                        bh / H, bh % H, i, s);
            }
            free(s);
        }
    }
    return failed ? -1 : 0;
}

/* Threads an OpenMP parallel region would use (for reporting). */
int fa_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
