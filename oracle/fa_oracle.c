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

/* ------------------------------------------------------------------------
 * Backward pass (gradients of the forward above).
 *
 * Given the upstream gradient dO (same shape as O), the gradients of the
 * scalar sum_i <dO_i, O_i> with respect to Q, K and V.  Written out with the
 * chain rule through the row softmax, all in fp64 from the exact inputs:
 *   P_ij  = exp(s_ij - lse_i) on valid keys, 0 elsewhere (0 for a row with no
 *           valid key);
 *   dV_j  = sum_i P_ij dO_i
 *   dP_ij = <dO_i, V_j>
 *   D_i   = sum_j P_ij dP_ij
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i  = scale * sum_j dS_ij K_j
 *   dK_j  = scale * sum_i dS_ij Q_i
 * Sources on the pages: the backward pass recomputes S and P = exp(S - L)
 * block by block from the saved Q, K, V, O and L, without an online softmax
 * ("GPU 与 TPU：让硬件不再是黑魔法" §11.5, part 3); the saved statistic is
 * L = m + log(l) ("FlashAttention 1–4 ...", section "FlashAttention-2").  The
 * pages do not print the gradient formulas; the lines above are the chain
 * rule, pinned in the tests against central finite differences of
 * fa_oracle_fwd.  Here D_i is formed from P and dP, the definition.  Since
 * O_i = sum_j P_ij V_j, D_i also equals <dO_i, O_i>; a backward pass that is
 * handed a stored O (rounded to the storage type) forms D_i from it.  When the
 * caller passes such an O (o_given, non-null), D_i = <dO_i, o_given_i> instead,
 * so that the result is exactly the gradient that a pass consuming that O
 * computes.
 * ------------------------------------------------------------------------ */

/* lse and D of every row of one head: lse_h[N], dd_h[N]. s scratch of N. */
static void head_row_stats(const double *q, const double *k, const double *v, const double *dout,
                           const double *o_given, int64_t H, int64_t N, int64_t d, int causal, double scale,
                           const int32_t *kv_limit, int64_t b, int64_t h,
                           double *lse_h, double *dd_h, double *s, double *orow)
{
    const double *vh = v + (b * H + h) * N * d;
    const double *dh = dout + (b * H + h) * N * d;
    for (int64_t i = 0; i < N; ++i) {
        one_row(q, k, v, orow, &lse_h[i], H, N, d, causal, scale, kv_limit, b, h, i, s);
        int64_t limit = kv_limit ? (int64_t)kv_limit[b * N + i] : N;
        if (limit > N) limit = N;
        double acc = 0.0;
        if (lse_h[i] != -INFINITY && !o_given) {
            /* one_row left the scores in s */
            for (int64_t j = 0; j < N; ++j) {
                if (!key_is_valid(j, i, causal, limit)) continue;
                double p = exp(s[j] - lse_h[i]);
                double dp = 0.0;
                for (int64_t c = 0; c < d; ++c) dp += dh[i * d + c] * vh[j * d + c];
                acc += p * dp;
            }
        } else if (lse_h[i] != -INFINITY) {
            const double *oh = o_given + (b * H + h) * N * d;
            for (int64_t c = 0; c < d; ++c) acc += dh[i * d + c] * oh[i * d + c];
        }
        dd_h[i] = acc;
    }
}

/* Full gradients.  dq, dk, dv are [B, H, N, d]; o_given is null or a
 * [B, H, N, d] output to form D from.  Heads run in parallel, rows of a head in
 * order (dK and dV accumulate over rows).  Returns 0 or -1. */
int fa_oracle_bwd(const double *q, const double *k, const double *v, const double *dout,
                  const double *o_given, double *dq, double *dk, double *dv,
                  int64_t B, int64_t H, int64_t N, int64_t d,
                  int causal, double scale, const int32_t *kv_limit, int nthreads)
{
    if (!q || !k || !v || !dout || !dq || !dk || !dv || B < 0 || H < 0 || N < 0 || d <= 0) return -1;
    int failed = 0;
#ifdef _OPENMP
    const int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
#endif
#pragma omp parallel num_threads(nt)
    {
        const size_t n1 = (size_t)(N > 0 ? N : 1);
        double *s = (double *)malloc(n1 * sizeof(double));
        double *lse_h = (double *)malloc(n1 * sizeof(double));
        double *dd_h = (double *)malloc(n1 * sizeof(double));
        double *orow = (double *)malloc((size_t)d * sizeof(double));
        if (!s || !lse_h || !dd_h || !orow) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t bh = 0; bh < B * H; ++bh) {
                const int64_t b = bh / H, h = bh % H;
                const double *qh = q + bh * N * d, *kh = k + bh * N * d, *vh = v + bh * N * d;
                const double *dh = dout + bh * N * d;
                double *dqh = dq + bh * N * d, *dkh = dk + bh * N * d, *dvh = dv + bh * N * d;
                head_row_stats(q, k, v, dout, o_given, H, N, d, causal, scale, kv_limit, b, h, lse_h, dd_h, s,
                               orow);
                for (int64_t e = 0; e < N * d; ++e) { dqh[e] = 0.0; dkh[e] = 0.0; dvh[e] = 0.0; }
                for (int64_t i = 0; i < N; ++i) {
                    if (lse_h[i] == -INFINITY) continue;
                    int64_t limit = kv_limit ? (int64_t)kv_limit[b * N + i] : N;
                    if (limit > N) limit = N;
                    for (int64_t j = 0; j < N; ++j) {
                        if (!key_is_valid(j, i, causal, limit)) continue;
                        double sij = 0.0, dp = 0.0;
                        for (int64_t c = 0; c < d; ++c) {
                            sij += qh[i * d + c] * kh[j * d + c];
                            dp += dh[i * d + c] * vh[j * d + c];
                        }
                        const double p = exp(scale * sij - lse_h[i]);
                        const double ds = p * (dp - dd_h[i]);
                        for (int64_t c = 0; c < d; ++c) {
                            dvh[j * d + c] += p * dh[i * d + c];
                            dqh[i * d + c] += scale * ds * kh[j * d + c];
                            dkh[j * d + c] += scale * ds * qh[i * d + c];
                        }
                    }
                }
            }
        }
        free(s); free(lse_h); free(dd_h); free(orow);
    }
    return failed ? -1 : 0;
}

/* Sampled gradients of one head (b, h): dq for nq query rows, dk and dv for nk
 * key rows.  Rows are head-local indices.  dq_out [nq, d], dk_out and dv_out
 * [nk, d]; o_head is null or the head's [N, d] output to form D from.  Cost: the
 * head's row statistics (two passes over all rows) plus the sampled sums.
 * Returns 0 or -1. */
int fa_oracle_bwd_sample(const double *q, const double *k, const double *v, const double *dout,
                         const double *o_head, int64_t B, int64_t H, int64_t N, int64_t d,
                         int causal, double scale, const int32_t *kv_limit,
                         int64_t b, int64_t h, int64_t nq, const int64_t *q_rows,
                         int64_t nk, const int64_t *k_rows,
                         double *dq_out, double *dk_out, double *dv_out, int nthreads)
{
    if (!q || !k || !v || !dout || b < 0 || b >= B || h < 0 || h >= H || N <= 0 || d <= 0) return -1;
    for (int64_t t = 0; t < nq; ++t) if (q_rows[t] < 0 || q_rows[t] >= N) return -1;
    for (int64_t t = 0; t < nk; ++t) if (k_rows[t] < 0 || k_rows[t] >= N) return -1;
    const int64_t bh = b * H + h;
    const double *qh = q + bh * N * d, *kh = k + bh * N * d, *vh = v + bh * N * d, *dh = dout + bh * N * d;
    double *lse_h = (double *)malloc((size_t)N * sizeof(double));
    double *dd_h = (double *)malloc((size_t)N * sizeof(double));
    if (!lse_h || !dd_h) { free(lse_h); free(dd_h); return -1; }
    int failed = 0;
#ifdef _OPENMP
    const int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
#endif
    /* row statistics, rows in parallel */
#pragma omp parallel num_threads(nt)
    {
        double *s = (double *)malloc((size_t)N * sizeof(double));
        double *orow = (double *)malloc((size_t)d * sizeof(double));
        if (!s || !orow) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 8)
            for (int64_t i = 0; i < N; ++i) {
                one_row(q, k, v, orow, &lse_h[i], H, N, d, causal, scale, kv_limit, b, h, i, s);
                int64_t limit = kv_limit ? (int64_t)kv_limit[b * N + i] : N;
                if (limit > N) limit = N;
                double acc = 0.0;
                if (lse_h[i] != -INFINITY && !o_head) {
                    for (int64_t j = 0; j < N; ++j) {
                        if (!key_is_valid(j, i, causal, limit)) continue;
                        double dp = 0.0;
                        for (int64_t c = 0; c < d; ++c) dp += dh[i * d + c] * vh[j * d + c];
                        acc += exp(s[j] - lse_h[i]) * dp;
                    }
                } else if (lse_h[i] != -INFINITY) {
                    for (int64_t c = 0; c < d; ++c) acc += dh[i * d + c] * o_head[i * d + c];
                }
                dd_h[i] = acc;
            }
        }
        free(s); free(orow);
    }
    if (failed) { free(lse_h); free(dd_h); return -1; }
    /* dq rows: sum over keys */
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1)
    for (int64_t t = 0; t < nq; ++t) {
        const int64_t i = q_rows[t];
        double *out = dq_out + t * d;
        for (int64_t c = 0; c < d; ++c) out[c] = 0.0;
        if (lse_h[i] == -INFINITY) continue;
        int64_t limit = kv_limit ? (int64_t)kv_limit[b * N + i] : N;
        if (limit > N) limit = N;
        for (int64_t j = 0; j < N; ++j) {
            if (!key_is_valid(j, i, causal, limit)) continue;
            double sij = 0.0, dp = 0.0;
            for (int64_t c = 0; c < d; ++c) {
                sij += qh[i * d + c] * kh[j * d + c];
                dp += dh[i * d + c] * vh[j * d + c];
            }
            const double ds = exp(scale * sij - lse_h[i]) * (dp - dd_h[i]);
            for (int64_t c = 0; c < d; ++c) out[c] += scale * ds * kh[j * d + c];
        }
    }
    /* dk, dv rows: sums over queries */
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1)
    for (int64_t t = 0; t < nk; ++t) {
        const int64_t j = k_rows[t];
        double *ok = dk_out + t * d, *ov = dv_out + t * d;
        for (int64_t c = 0; c < d; ++c) { ok[c] = 0.0; ov[c] = 0.0; }
        for (int64_t i = 0; i < N; ++i) {
            if (lse_h[i] == -INFINITY) continue;
            int64_t limit = kv_limit ? (int64_t)kv_limit[b * N + i] : N;
            if (limit > N) limit = N;
            if (!key_is_valid(j, i, causal, limit)) continue;
            double sij = 0.0, dp = 0.0;
            for (int64_t c = 0; c < d; ++c) {
                sij += qh[i * d + c] * kh[j * d + c];
                dp += dh[i * d + c] * vh[j * d + c];
            }
            const double p = exp(scale * sij - lse_h[i]);
            const double ds = p * (dp - dd_h[i]);
            for (int64_t c = 0; c < d; ++c) {
                ov[c] += p * dh[i * d + c];
                ok[c] += scale * ds * qh[i * d + c];
            }
        }
    }
    free(lse_h); free(dd_h);
    return 0;
}

/* ------------------------------------------------------------------------
 * Decode over a paged key/value cache.
 *
 * One query per sequence (N_q = 1, the token being generated), attending to
 * every cached key of its own sequence.  The cache is cut into fixed-size
 * pages; a per-sequence block table maps logical page p (keys p*page_size ..
 * p*page_size + page_size - 1) to a physical page of the pool, so that a
 * sequence's pages may lie anywhere ("CS336 第五讲 · GPU 与 GPU 优化", the
 * PagedAttention section: pages of 16 tokens and the block table).  The
 * result is the attention of the plain definition above over those keys:
 *   key j of sequence b, head h, is k_cache[page, h, j % page_size, :] with
 *   page = block_table[b, j / page_size], for 0 <= j < seq_lens[b];
 *   s_j = scale * <q[b,h,:], key j>, m = max_j s_j, w_j = exp(s_j - m),
 *   o[b,h,:] = sum_j w_j v_j / sum_j w_j, lse[b,h] = m + ln(sum_j w_j);
 *   a sequence with no key gets o = 0 and lse = -inf.
 * Layouts: q, o [B, H, d]; k_cache, v_cache [num_pages, H, page_size, d];
 * block_table [B, max_pages]; seq_lens [B]; lse [B, H].  A length outside
 * [0, max_pages * page_size] or a referenced page outside [0, num_pages) is
 * an error (-1): the oracle only defines valid caches.
 * ------------------------------------------------------------------------ */
int fa_oracle_decode_paged(const double *q, const double *k_cache, const double *v_cache,
                           const int32_t *block_table, const int32_t *seq_lens,
                           double *o, double *lse,
                           int64_t B, int64_t H, int64_t d, int64_t page_size,
                           int64_t max_pages, int64_t num_pages, double scale, int nthreads)
{
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !o || !lse) return -1;
    if (B < 0 || H < 0 || d <= 0 || page_size <= 0 || max_pages < 0 || num_pages < 0) return -1;
    int64_t max_len = 0;
    for (int64_t b = 0; b < B; ++b) {
        const int64_t len = seq_lens[b];
        if (len < 0 || len > max_pages * page_size) return -1;
        for (int64_t p = 0; p * page_size < len; ++p) {
            const int64_t page = block_table[b * max_pages + p];
            if (page < 0 || page >= num_pages) return -1;
        }
        if (len > max_len) max_len = len;
    }
    int failed = 0;
#ifdef _OPENMP
    const int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
#endif
#pragma omp parallel num_threads(nt)
    {
        double *s = (double *)malloc((size_t)(max_len > 0 ? max_len : 1) * sizeof(double));
        if (!s) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t bh = 0; bh < B * H; ++bh) {
                const int64_t b = bh / H, h = bh % H, len = seq_lens[b];
                const double *qv = q + bh * d;
                double *ov = o + bh * d;
                for (int64_t c = 0; c < d; ++c) ov[c] = 0.0;
                if (len == 0) {
                    lse[bh] = -INFINITY;
                    continue;
                }
                /* scores over the sequence's keys, gathered through the block table */
                double m = -INFINITY;
                for (int64_t j = 0; j < len; ++j) {
                    const int64_t page = block_table[b * max_pages + j / page_size];
                    const double *kj = k_cache + ((page * H + h) * page_size + j % page_size) * d;
                    double acc = 0.0;
                    for (int64_t c = 0; c < d; ++c) acc += qv[c] * kj[c];
                    s[j] = scale * acc;
                    if (s[j] > m) m = s[j];
                }
                double l = 0.0;
                for (int64_t j = 0; j < len; ++j) {
                    const int64_t page = block_table[b * max_pages + j / page_size];
                    const double *vj = v_cache + ((page * H + h) * page_size + j % page_size) * d;
                    const double w = exp(s[j] - m);
                    l += w;
                    for (int64_t c = 0; c < d; ++c) ov[c] += w * vj[c];
                }
                for (int64_t c = 0; c < d; ++c) ov[c] /= l;
                lse[bh] = m + log(l);
            }
            free(s);
        }
    }
    return failed ? -1 : 0;
}

/* ------------------------------------------------------------------------
 * FP8 forward: quantisation of Q and K, and attention on the quantised values.
 *
 * "FlashAttention 1–4 ...", section "FlashAttention-3" (FP8 with block
 * quantization and incoherent processing): one FP8 scale per tile of rows
 * instead of one per tensor, and Q and K both multiplied by the same random
 * orthogonal matrix before quantising -- random sign flips followed by a
 * Hadamard transform, O(d log d) per row -- which leaves Q K^T unchanged while
 * spreading an outlier over every coordinate.
 *
 * The encoding, step by step (the plainest reading where the page is silent):
 *   1. rotate each row x (length d, a power of two) of Q or K:
 *        y = H (s * x)   with s[c] in {+1, -1} given by the caller and H the
 *        unnormalised Sylvester-Hadamard matrix (entries +-1, H H^T = d I),
 *        computed in fp32 as the butterfly: for h = 1, 2, 4, ..., d/2, every
 *        pair (i, i + h) with i & h == 0 becomes (y_i + y_{i+h}, y_i - y_{i+h});
 *   2. per tile of `tile_rows` consecutive rows of one head (the last tile may
 *      be short), amax = max |y| and the exponent e = the smallest integer with
 *      amax <= 448 * 2^e (448 is the largest E4M3 value), clamped to
 *      [-127, 127]; e = 0 for an all-zero tile;
 *   3. code = E4M3(y * 2^-e), rounding to nearest, ties to even.
 * E4M3 (OCP FP8): 1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no
 * infinities; subnormals m * 2^-9; largest value 448.
 * Since (H s q) . (H s k) = d (q . k), attention on the quantised values uses
 *   s_ij = (scale / d) * sum_c deq(q_i)_c deq(k_j)_c,  deq(code) = E4M3 value * 2^e,
 * and otherwise the plain definition above (V unchanged).
 * ------------------------------------------------------------------------ */

/* E4M3 value of a code (codes 0x7F and 0xFF, the NaNs, are never produced). */
static double e4m3_value(uint8_t code)
{
    const int s = code >> 7, E = (code >> 3) & 15, m = code & 7;
    const double v = E == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, E - 7);
    return s ? -v : v;
}

/* E4M3 code of x, |x| <= 448: nearest representable value, ties to the even code. */
static uint8_t e4m3_encode(float x)
{
    const uint8_t sign = signbit(x) ? 0x80 : 0;
    double a = fabs((double)x);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);
    int E = e - 1;                    /* a in [2^E, 2^(E+1)) */
    if (E < -6) E = -6;               /* subnormals share the step of the lowest binade */
    const double step = ldexp(1.0, E - 3);
    const double r = nearbyint(a / step);   /* exact quotient; current mode rounds ties to even */
    const double v = r * step;
    if (v == 0.0) return sign;
    int e2;
    frexp(v, &e2);
    const int E2 = e2 - 1;
    if (E2 < -6) return sign | (uint8_t)(int)(v / ldexp(1.0, -9));
    const int mant = (int)(v / ldexp(1.0, E2 - 3)) - 8;
    return sign | (uint8_t)(((E2 + 7) << 3) | mant);
}

/* Smallest e with amax <= 448 * 2^e, clamped to [-127, 127]; 0 for amax == 0. */
static int tile_exponent(float amax)
{
    if (!(amax > 0.0f)) return 0;
    int k;
    const double m = frexp((double)amax, &k);   /* amax = m 2^k, m in [0.5, 1); 448 = 0.875 2^9 */
    int e = (m <= 0.875) ? k - 9 : k - 8;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* One row: y = H (s * x) in fp32, butterfly stages h = 1, 2, ..., d/2. */
static void rotate_row(const double *x, const int8_t *signs, int64_t d, float *y)
{
    for (int64_t c = 0; c < d; ++c) y[c] = (float)x[c] * (float)signs[c];
    for (int64_t h = 1; h < d; h <<= 1)
        for (int64_t i = 0; i < d; ++i) {
            if (i & h) continue;
            const float a = y[i], b = y[i + h];
            y[i] = a + b;
            y[i + h] = a - b;
        }
}

/* Quantise x [B, H, N, d] (exact bf16 values as fp64): codes [B, H, N, d],
 * exps [B, H, ceil(N / tile_rows)].  rotate = 0 skips step 1 (for the
 * per-tensor baseline below).  Returns 0 or -1. */
int fa_oracle_fp8_quantize(const double *x, const int8_t *signs, int rotate,
                           uint8_t *codes, int32_t *exps,
                           int64_t B, int64_t H, int64_t N, int64_t d, int64_t tile_rows, int nthreads)
{
    if (!x || !codes || !exps || (rotate && !signs) || B < 0 || H < 0 || N < 0 || tile_rows <= 0) return -1;
    if (d <= 0 || (d & (d - 1))) return -1;
    const int64_t nt = (N + tile_rows - 1) / tile_rows;
    int failed = 0;
#ifdef _OPENMP
    const int nth = nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
#endif
#pragma omp parallel num_threads(nth)
    {
        float *y = (float *)malloc((size_t)(tile_rows * d) * sizeof(float));
        if (!y) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t t = 0; t < B * H * nt; ++t) {
                const int64_t bh = t / nt, tile = t % nt;
                const int64_t r0 = tile * tile_rows;
                const int64_t nr = (r0 + tile_rows <= N) ? tile_rows : N - r0;
                float amax = 0.0f;
                for (int64_t r = 0; r < nr; ++r) {
                    const double *xr = x + (bh * N + r0 + r) * d;
                    float *yr = y + r * d;
                    if (rotate) {
                        rotate_row(xr, signs, d, yr);
                    } else {
                        for (int64_t c = 0; c < d; ++c) yr[c] = (float)xr[c];
                    }
                    for (int64_t c = 0; c < d; ++c) {
                        const float a = fabsf(yr[c]);
                        if (a > amax) amax = a;
                    }
                }
                const int e = tile_exponent(amax);
                exps[t] = e;
                const float inv = (float)ldexp(1.0, -e);   /* exact power of two */
                for (int64_t r = 0; r < nr; ++r)
                    for (int64_t c = 0; c < d; ++c)
                        codes[(bh * N + r0 + r) * d + c] = e4m3_encode(y[r * d + c] * inv);
            }
            free(y);
        }
    }
    return failed ? -1 : 0;
}

/* Attention on quantised q and k (codes with per-tile exponents as produced
 * above: q tiles of q_tile rows, k tiles of k_tile rows) and fp64 v.  With
 * score_div = d for rotated inputs (1 for unrotated ones).  o [B, H, N, d],
 * lse [B, H, N].  Masks as in fa_oracle_fwd.  Returns 0 or -1. */
int fa_oracle_fwd_fp8(const uint8_t *qc, const int32_t *qe, int64_t q_tile,
                      const uint8_t *kc, const int32_t *ke, int64_t k_tile,
                      const double *v, double *o, double *lse,
                      int64_t B, int64_t H, int64_t N, int64_t d,
                      int causal, double scale, double score_div, const int32_t *kv_limit, int nthreads)
{
    if (!qc || !qe || !kc || !ke || !v || !o || !lse || B < 0 || H < 0 || N < 0 || d <= 0) return -1;
    if (q_tile <= 0 || k_tile <= 0 || !(score_div > 0.0)) return -1;
    const int64_t nqt = (N + q_tile - 1) / q_tile, nkt = (N + k_tile - 1) / k_tile;
    double *qd = (double *)malloc((size_t)(B * H * N * d > 0 ? B * H * N * d : 1) * sizeof(double));
    double *kd = (double *)malloc((size_t)(B * H * N * d > 0 ? B * H * N * d : 1) * sizeof(double));
    if (!qd || !kd) { free(qd); free(kd); return -1; }
    for (int64_t bh = 0; bh < B * H; ++bh)
        for (int64_t r = 0; r < N; ++r)
            for (int64_t c = 0; c < d; ++c) {
                const int64_t i = (bh * N + r) * d + c;
                qd[i] = ldexp(e4m3_value(qc[i]), qe[bh * nqt + r / q_tile]);
                kd[i] = ldexp(e4m3_value(kc[i]), ke[bh * nkt + r / k_tile]);
            }
    const int rc = fa_oracle_fwd(qd, kd, v, o, lse, B, H, N, d, causal, scale / score_div, kv_limit, nthreads);
    free(qd);
    free(kd);
    return rc;
}

/* The rotation of step 1 alone, for checking: y [rows, d] = H (s * x) in fp32. */
int fa_oracle_fp8_rotate(const double *x, const int8_t *signs, float *y, int64_t rows, int64_t d)
{
    if (!x || !signs || !y || rows < 0 || d <= 0 || (d & (d - 1))) return -1;
    for (int64_t r = 0; r < rows; ++r) rotate_row(x + r * d, signs, d, y + r * d);
    return 0;
}
