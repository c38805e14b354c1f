/*
 * attn_oracle.c -- CPU reference for the fused attention forward.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, the smoke check
 * and the CPU-baseline leg of the benchmark may load this library.  It
 * shares no source, header, table or helper with the GPU library.
 *
 * What it computes (page 4, "FlashAttention (TR)", section on the problems
 * of standard attention, the attention formula): for every requested row
 * (b, h, i), in fp64, on the exact values of the (already rounded) inputs:
 *
 *   s_j  = scale * sum_c Q[b,h,i,c] * K[b,h,j,c]  +  bias[b,h,i/64,j/64]
 *          for every key j the mask allows (causal: j <= i, else all j)
 *   m    = max_j s_j,   p_j = exp(s_j - m),   l = sum_j p_j
 *   O[c] = sum_j p_j * V[b,h,j,c] / l,        LSE = m + ln l
 *
 * This is the naive algorithm the pages contrast the fused kernel with
 * (page 4, same section; page 3, the glossary paragraph): the whole score
 * row is formed, then normalised, then multiplied by V.  Subtracting the
 * row maximum is exact in real arithmetic because softmax is invariant to a
 * constant shift (page 1, "claim vs reality" section).  The bias is the
 * additive log-gate of page 5 ("SAS" section, log-form gate inside the
 * softmax), one scalar per 64-query x 64-key block, in natural-log units,
 * added after the scale.  A row with no visible key (possible only through
 * a -inf bias) returns O = 0 and LSE = -inf.
 *
 * Inputs are float32 arrays holding the exact values of the fp16/bf16
 * tensors (float32 represents every fp16 and bf16 value exactly).
 * Layout [B,H,N,d], d innermost; bias [B,H,nb,nb] with nb = ceil(N/64).
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_BIAS_BLOCK 64

/* Scores of one row into s[0..N): masked keys get -inf.  Returns the max. */
static double row_scores(const float* q, const float* k, const float* bias,
                         int64_t H, int64_t N, int64_t d, int causal,
                         double scale, int64_t b, int64_t h, int64_t i,
                         double* s)
{
    const int64_t nb = (N + ORACLE_BIAS_BLOCK - 1) / ORACLE_BIAS_BLOCK;
    const float* qi = q + ((b * H + h) * N + i) * d;
    const float* kb = k + (b * H + h) * N * d;
    double m = -INFINITY;
    for (int64_t j = 0; j < N; ++j) {
        if (causal && j > i) {
            s[j] = -INFINITY;
            continue;
        }
        const float* kj = kb + j * d;
        double acc = 0.0;
        for (int64_t c = 0; c < d; ++c)
            acc += (double)qi[c] * (double)kj[c];
        double sj = scale * acc;
        if (bias)
            sj += (double)bias[((b * H + h) * nb + i / ORACLE_BIAS_BLOCK) * nb +
                               j / ORACLE_BIAS_BLOCK];
        s[j] = sj;
        if (sj > m)
            m = sj;
    }
    return m;
}

/* Probabilities of one row: p[j] = exp(s_j - m) / l (0 for masked keys). */
int attn_oracle_row_probs(const float* q, const float* k, const float* bias,
                          int64_t B, int64_t H, int64_t N, int64_t d,
                          int causal, double scale, int64_t b, int64_t h,
                          int64_t i, double* p)
{
    if (!q || !k || !p || B <= 0 || H <= 0 || N <= 0 || d <= 0)
        return 1;
    if (b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= N)
        return 2;
    double m = row_scores(q, k, bias, H, N, d, causal, scale, b, h, i, p);
    double l = 0.0;
    for (int64_t j = 0; j < N; ++j) {
        p[j] = (m == -INFINITY) ? 0.0 : exp(p[j] - m);
        l += p[j];
    }
    for (int64_t j = 0; j < N; ++j)
        p[j] = (l > 0.0) ? p[j] / l : 0.0;
    return 0;
}

/*
 * Attention rows.  rows holds nrows triplets (b, h, i).  out is [nrows, d]
 * fp64, lse is [nrows] fp64 (nullable).  nthreads <= 0 uses the OpenMP
 * default.  Returns 0 on success.
 */
int attn_oracle_rows(const float* q, const float* k, const float* v,
                     const float* bias, int64_t B, int64_t H, int64_t N,
                     int64_t d, int causal, double scale, const int64_t* rows,
                     int64_t nrows, double* out, double* lse, int nthreads)
{
    if (!q || !k || !v || !rows || !out || B <= 0 || H <= 0 || N <= 0 ||
        d <= 0 || nrows < 0)
        return 1;
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
        if (b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= N)
            return 2;
    }
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int failed = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc((size_t)N * sizeof(double));
        if (!s) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            if (!s)
                continue;
            const int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
            const double m = row_scores(q, k, bias, H, N, d, causal, scale, b, h, i, s);
            double* o = out + r * d;
            for (int64_t c = 0; c < d; ++c)
                o[c] = 0.0;
            double l = 0.0;
            const float* vb = v + (b * H + h) * N * d;
            for (int64_t j = 0; j < N; ++j) {
                const double pj = (m == -INFINITY) ? 0.0 : exp(s[j] - m);
                if (pj == 0.0)
                    continue;
                l += pj;
                const float* vj = vb + j * d;
                for (int64_t c = 0; c < d; ++c)
                    o[c] += pj * (double)vj[c];
            }
            for (int64_t c = 0; c < d; ++c)
                o[c] = (l > 0.0) ? o[c] / l : 0.0;
            if (lse)
                lse[r] = (l > 0.0) ? m + log(l) : -INFINITY;
        }
        free(s);
    }
    return failed ? 3 : 0;
}

/* Number of OpenMP threads a parallel region would use (for reporting). */
int attn_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Gradients of the attention above (page 3, "FlashAttention", the glossary
 * paragraph: the backward pass recomputes the small intermediate quantities
 * instead of storing the score matrix; page 5, "SAS": the log-form gate sits
 * inside the softmax so that the loss's gradient reaches it).  For a loss L
 * with dO = dL/dO, per row (b,h,i), with P the probability row of the
 * definition above and s the (scaled, biased) score row:
 *
 *   dV[j]  += P_ij * dO_i                      (O_i = sum_j P_ij V_j)
 *   dp_ij   = dO_i . V_j                       (dL/dP_ij)
 *   ds_ij   = P_ij * (dp_ij - sum_k P_ik dp_ik)  (softmax Jacobian: dL/ds_ij)
 *   dQ_i   += scale * ds_ij * K_j,   dK_j += scale * ds_ij * Q_i
 *   dbias[b,h,i/64,j/64] += ds_ij               (the bias enters s unscaled)
 *
 * Everything in fp64 from the exact input values; the forward quantities
 * are recomputed here, nothing is taken from a GPU run.  Outputs are fp64
 * [B,H,N,d] (dq, dk, dv) and [B,H,nb,nb] (dbias, nullable), overwritten.
 * OpenMP runs over (b,h) heads.  Returns 0 on success.
 */
int attn_oracle_bwd(const float* q, const float* k, const float* v,
                    const float* dout, const float* bias, int64_t B,
                    int64_t H, int64_t N, int64_t d, int causal, double scale,
                    double* dq, double* dk, double* dv, double* dbias,
                    int nthreads)
{
    if (!q || !k || !v || !dout || !dq || !dk || !dv || B <= 0 || H <= 0 ||
        N <= 0 || d <= 0)
        return 1;
    const int64_t nb = (N + ORACLE_BIAS_BLOCK - 1) / ORACLE_BIAS_BLOCK;
    memset(dq, 0, (size_t)(B * H * N * d) * sizeof(double));
    memset(dk, 0, (size_t)(B * H * N * d) * sizeof(double));
    memset(dv, 0, (size_t)(B * H * N * d) * sizeof(double));
    if (dbias)
        memset(dbias, 0, (size_t)(B * H * nb * nb) * sizeof(double));
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int failed = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc((size_t)N * sizeof(double));
        double* dp = (double*)malloc((size_t)N * sizeof(double));
        if (!s || !dp) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t bh = 0; bh < B * H; ++bh) {
            if (!s || !dp)
                continue;
            const int64_t b = bh / H, h = bh % H;
            const float* kb = k + bh * N * d;
            const float* vb = v + bh * N * d;
            for (int64_t i = 0; i < N; ++i) {
                /* a row with dO_i = 0 contributes nothing (dp = 0, so ds = 0) */
                const float* doz = dout + (bh * N + i) * d;
                int64_t nz = 0;
                for (int64_t c = 0; c < d; ++c)
                    nz |= (doz[c] != 0.0f);
                if (!nz)
                    continue;
                const double m = row_scores(q, k, bias, H, N, d, causal, scale, b, h, i, s);
                if (m == -INFINITY)
                    continue; /* no visible key: O = 0, no gradient */
                double l = 0.0;
                for (int64_t j = 0; j < N; ++j) {
                    s[j] = exp(s[j] - m); /* s now holds unnormalised P */
                    l += s[j];
                }
                const float* doi = dout + (bh * N + i) * d;
                const float* qi = q + (bh * N + i) * d;
                double pdp = 0.0; /* sum_k P_ik dp_ik */
                for (int64_t j = 0; j < N; ++j) {
                    s[j] /= l;
                    dp[j] = 0.0;
                    if (s[j] == 0.0)
                        continue;
                    const float* vj = vb + j * d;
                    for (int64_t c = 0; c < d; ++c)
                        dp[j] += (double)doi[c] * (double)vj[c];
                    pdp += s[j] * dp[j];
                }
                double* dqi = dq + (bh * N + i) * d;
                for (int64_t j = 0; j < N; ++j) {
                    const double pj = s[j];
                    if (pj == 0.0)
                        continue;
                    const double dsj = pj * (dp[j] - pdp);
                    double* dvj = dv + (bh * N + j) * d;
                    double* dkj = dk + (bh * N + j) * d;
                    const float* kj = kb + j * d;
                    for (int64_t c = 0; c < d; ++c) {
                        dvj[c] += pj * (double)doi[c];
                        dkj[c] += scale * dsj * (double)qi[c];
                        dqi[c] += scale * dsj * (double)kj[c];
                    }
                    if (dbias)
                        dbias[(bh * nb + i / ORACLE_BIAS_BLOCK) * nb + j / ORACLE_BIAS_BLOCK] += dsj;
                }
            }
        }
        free(s);
        free(dp);
    }
    return failed ? 3 : 0;
}
