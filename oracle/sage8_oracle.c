/*
 * sage8_oracle.c -- CPU reference for the 8-bit (SageAttention-style) path.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, the smoke check
 * and the CPU-baseline leg of the benchmark may load this library.  It
 * shares no source, header, table or helper with the GPU library.
 *
 * The method (page 1, "SageAttention" newsletter, "claim vs reality"
 * section): the first product Q K^T runs in INT8; before quantising, K is
 * mean-centred ("smoothing"), which changes no output because softmax is
 * shift-invariant; the softmax output P lies in [0, 1] and goes to FP8 for
 * the second product P V; the two products are combined with a two-level
 * accumulation.  The pages name these ingredients only.  The readings used
 * here (plainest reading, stated so the GPU side can follow them exactly):
 *
 *  1. K smoothing: kmean[b,h,c] = mean over all N tokens of K[b,h,:,c].
 *     The sum is taken in fp64 over the exact input values, divided by N in
 *     fp64 and rounded once to fp32.  Smoothed K = fp32(K) - kmean (one fp32
 *     subtraction).
 *  2. INT8 Q and smoothed K: symmetric, one scale per 64-row block of each
 *     (b,h).  amax = max |x| over the block (fp32), scale = amax / 127 and
 *     inv = 127 / amax (each one correctly rounded fp32 division; amax = 0
 *     gives scale = inv = 1), code = clamp(rne(x * inv), -127, 127) with the
 *     product in fp32 and round-half-to-even.
 *  3. V in FP8 e4m3 (OCP "e4m3fn": bias 7, max 448, no infinities) with one
 *     scale per (b,h,channel) over all N: scale = amax / 448, inv = 448 /
 *     amax (fp32 divisions, amax = 0 gives 1), code = e4m3(v * inv) with
 *     round-half-to-even and saturation at 448.
 *  4. P in FP8: P^ = e4m3(448 * P) where P = exp(s - m) with m the running
 *     maximum after the current key block, so 448 * P <= 448 never
 *     saturates.  The pages do not say which P the row sum l adds up; here
 *     it is the unquantised P, as in the full-precision online softmax.
 *  5. Two-level accumulation: the products of one key block are summed into
 *     a fresh partial (level 1), which is then added to the running output
 *     after the running output is rescaled (level 2).
 *
 * Steps 1-3 are integer/byte results and are reproduced bit for bit by the
 * GPU prep.  sage8_oracle_emulate_rows models steps 4-5 in fp64 as read
 * above.  sage8_oracle_emulate_rows_fp32 runs the same algorithm with the
 * GPU kernel's own fp32 decisions (its lazily raised running maximum and P
 * scale, see there); it agrees with the GPU up to summation order and rare
 * one-code FP8 rounding differences from the hardware exponential.
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

#define SAGE_QK_BLOCK 64
#define SAGE_BIAS_BLOCK 64
#define E4M3_MAX 448.0

/* ---- OCP FP8 E4M3 ("e4m3fn") from its definition ----------------------- */

/* Encode with round-half-to-even; finite values beyond 448 saturate to 448;
 * NaN encodes as 0x7F. */
uint8_t sage8_e4m3_encode(double x)
{
    if (isnan(x))
        return 0x7F;
    const uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double a = fabs(x);
    if (a >= E4M3_MAX)
        return sign | 0x7E; /* 1.110b x 2^8 = 448 */
    if (a < ldexp(1.0, -6)) {
        /* subnormal: multiples of 2^-9; a code of 8 is the smallest normal */
        const double m = rint(a * 512.0); /* RNE in the default mode */
        return sign | (uint8_t)m;
    }
    int e2;
    const double f = frexp(a, &e2); /* a = f * 2^e2, f in [0.5, 1) */
    int e = e2 - 1;                 /* a = (2f) * 2^e, 2f in [1, 2) */
    double mant = rint((2.0 * f - 1.0) * 8.0);
    if (mant == 8.0) {
        mant = 0.0;
        e += 1;
    }
    if (e > 8 || (e == 8 && mant > 6.0))
        return sign | 0x7E;
    return sign | (uint8_t)(((e + 7) << 3) | (int)mant);
}

double sage8_e4m3_decode(uint8_t c)
{
    const int e = (c >> 3) & 0xF, m = c & 7;
    const double s = (c & 0x80) ? -1.0 : 1.0;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        return s * ldexp((double)m, -9);
    return s * ldexp(1.0 + m / 8.0, e - 7);
}

/* ---- step 1: K mean over tokens --------------------------------------- */

int sage8_oracle_kmean(const float* k, int64_t B, int64_t H, int64_t N,
                       int64_t d, float* kmean)
{
    if (!k || !kmean || B <= 0 || H <= 0 || N <= 0 || d <= 0)
        return 1;
    for (int64_t bh = 0; bh < B * H; ++bh)
        for (int64_t c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n)
                acc += (double)k[(bh * N + n) * d + c];
            kmean[bh * d + c] = (float)(acc / (double)N);
        }
    return 0;
}

/* ---- step 2: per-64-row-block symmetric INT8 ---------------------------- */

/* center (nullable, [B,H,d]) is subtracted first in fp32.  codes [B,H,N,d],
 * scales [B,H,ceil(N/64)]. */
int sage8_oracle_quant_int8(const float* x, const float* center, int64_t B,
                            int64_t H, int64_t N, int64_t d, int8_t* codes,
                            float* scales)
{
    if (!x || !codes || !scales || B <= 0 || H <= 0 || N <= 0 || d <= 0)
        return 1;
    const int64_t nb = (N + SAGE_QK_BLOCK - 1) / SAGE_QK_BLOCK;
    for (int64_t bh = 0; bh < B * H; ++bh)
        for (int64_t blk = 0; blk < nb; ++blk) {
            const int64_t n0 = blk * SAGE_QK_BLOCK;
            const int64_t n1 = (n0 + SAGE_QK_BLOCK < N) ? n0 + SAGE_QK_BLOCK : N;
            float amax = 0.0f;
            for (int64_t n = n0; n < n1; ++n)
                for (int64_t c = 0; c < d; ++c) {
                    float y = x[(bh * N + n) * d + c];
                    if (center)
                        y = y - center[bh * d + c];
                    const float ay = fabsf(y);
                    if (ay > amax)
                        amax = ay;
                }
            float scale = 1.0f, inv = 1.0f;
            if (amax > 0.0f) {
                scale = amax / 127.0f;
                inv = 127.0f / amax;
            }
            scales[bh * nb + blk] = scale;
            for (int64_t n = n0; n < n1; ++n)
                for (int64_t c = 0; c < d; ++c) {
                    float y = x[(bh * N + n) * d + c];
                    if (center)
                        y = y - center[bh * d + c];
                    const float t = y * inv;
                    float r = rintf(t);
                    if (r > 127.0f)
                        r = 127.0f;
                    if (r < -127.0f)
                        r = -127.0f;
                    codes[(bh * N + n) * d + c] = (int8_t)r;
                }
        }
    return 0;
}

/* ---- step 2, FP8 variant: per-64-row-block e4m3 Q and smoothed K ------- */

/* The FP8-QK variant (page 2, "FlashAttention-3" bulletin, claim vs reality
 * section: FP8 for the products needs block-wise dynamic scaling): the same
 * blocks as step 2, amax over the block (fp32), scale = amax / 448 and
 * inv = 448 / amax (correctly rounded fp32 divisions; amax = 0 gives 1),
 * code = e4m3(x * inv) with the product in fp32, round-half-to-even and
 * saturation at 448.  center (nullable) is subtracted first, as for K in
 * step 2.  codes [B,H,N,d] (e4m3 bytes), scales [B,H,ceil(N/64)]. */
int sage8_oracle_quant_fp8(const float* x, const float* center, int64_t B,
                           int64_t H, int64_t N, int64_t d, uint8_t* codes,
                           float* scales)
{
    if (!x || !codes || !scales || B <= 0 || H <= 0 || N <= 0 || d <= 0)
        return 1;
    const int64_t nb = (N + SAGE_QK_BLOCK - 1) / SAGE_QK_BLOCK;
    for (int64_t bh = 0; bh < B * H; ++bh)
        for (int64_t blk = 0; blk < nb; ++blk) {
            const int64_t n0 = blk * SAGE_QK_BLOCK;
            const int64_t n1 = (n0 + SAGE_QK_BLOCK < N) ? n0 + SAGE_QK_BLOCK : N;
            float amax = 0.0f;
            for (int64_t n = n0; n < n1; ++n)
                for (int64_t c = 0; c < d; ++c) {
                    float y = x[(bh * N + n) * d + c];
                    if (center)
                        y = y - center[bh * d + c];
                    const float ay = fabsf(y);
                    if (ay > amax)
                        amax = ay;
                }
            float scale = 1.0f, inv = 1.0f;
            if (amax > 0.0f) {
                scale = amax / 448.0f;
                inv = 448.0f / amax;
            }
            scales[bh * nb + blk] = scale;
            for (int64_t n = n0; n < n1; ++n)
                for (int64_t c = 0; c < d; ++c) {
                    float y = x[(bh * N + n) * d + c];
                    if (center)
                        y = y - center[bh * d + c];
                    const float t = y * inv;
                    codes[(bh * N + n) * d + c] = sage8_e4m3_encode((double)t);
                }
        }
    return 0;
}

/* ---- step 3: V to e4m3 with a per-channel scale ------------------------- */

/* codes [B,H,N,d] (logical layout), scales [B,H,d]. */
int sage8_oracle_quant_v(const float* v, int64_t B, int64_t H, int64_t N,
                         int64_t d, uint8_t* codes, float* scales)
{
    if (!v || !codes || !scales || B <= 0 || H <= 0 || N <= 0 || d <= 0)
        return 1;
    for (int64_t bh = 0; bh < B * H; ++bh)
        for (int64_t c = 0; c < d; ++c) {
            float amax = 0.0f;
            for (int64_t n = 0; n < N; ++n) {
                const float a = fabsf(v[(bh * N + n) * d + c]);
                if (a > amax)
                    amax = a;
            }
            float scale = 1.0f, inv = 1.0f;
            if (amax > 0.0f) {
                scale = amax / (float)E4M3_MAX;
                inv = (float)E4M3_MAX / amax;
            }
            scales[bh * d + c] = scale;
            for (int64_t n = 0; n < N; ++n) {
                const float t = v[(bh * N + n) * d + c] * inv;
                codes[(bh * N + n) * d + c] = sage8_e4m3_encode((double)t);
            }
        }
    return 0;
}

/* Q.K of two quantised rows, exactly: INT8 codes (qk_fp8 = 0) as integers,
 * or e4m3 codes (qk_fp8 = 1) decoded through dec[]; the e4m3 products and
 * their sum over d <= 128 terms are exact in fp64. */
static double qk_dot(const void* qq, const void* kq, int64_t qoff, int64_t koff,
                     int64_t d, int qk_fp8, const double* dec)
{
    if (qk_fp8) {
        const uint8_t* a = (const uint8_t*)qq + qoff;
        const uint8_t* b = (const uint8_t*)kq + koff;
        double acc = 0.0;
        for (int64_t c = 0; c < d; ++c)
            acc += dec[a[c]] * dec[b[c]];
        return acc;
    }
    const int8_t* a = (const int8_t*)qq + qoff;
    const int8_t* b = (const int8_t*)kq + koff;
    int64_t acc = 0;
    for (int64_t c = 0; c < d; ++c)
        acc += (int64_t)a[c] * (int64_t)b[c];
    return (double)acc;
}

/* The value of quantised Q element idx (before its block scale). */
static double q_value(const void* qq, int64_t idx, int qk_fp8, const double* dec)
{
    return qk_fp8 ? dec[((const uint8_t*)qq)[idx]] : (double)((const int8_t*)qq)[idx];
}

/* ---- steps 4-5: the blocked 8-bit attention, modelled in fp64 ----------- */

/*
 * Emulates the quantised forward on rows (b,h,i) from the quantised data of
 * steps 1-3.  kv_block is the number of keys per online-softmax update.
 * p_mode 1 rounds 448*P to e4m3 as the method does; p_mode 0 keeps P exact
 * (used to pin the blocked algebra against the plain oracle).  out [nrows,d]
 * and lse [nrows] (nullable) are fp64; LSE is in natural-log units.
 */
int sage8_oracle_emulate_rows(const void* qq, const void* kq,
                              const uint8_t* vq, const float* sq,
                              const float* sk, const float* sv,
                              const float* kmean, const float* bias, int64_t B, int64_t H,
                              int64_t N, int64_t d, int causal, double scale,
                              int64_t kv_block, int p_mode,
                              const int64_t* rows, int64_t nrows, double* out,
                              double* lse, int qk_fp8, int nthreads)
{
    if (!qq || !kq || !vq || !sq || !sk || !sv || !rows || !out || B <= 0 ||
        H <= 0 || N <= 0 || d <= 0 || kv_block <= 0 || nrows < 0)
        return 1;
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
        if (b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= N)
            return 2;
    }
    const int64_t nqk = (N + SAGE_QK_BLOCK - 1) / SAGE_QK_BLOCK;
    const int64_t nbb = (N + SAGE_BIAS_BLOCK - 1) / SAGE_BIAS_BLOCK;
    double vdec[256];
    for (int c = 0; c < 256; ++c)
        vdec[c] = sage8_e4m3_decode((uint8_t)c);
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int failed = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc((size_t)kv_block * sizeof(double));
        double* blk = (double*)malloc((size_t)d * sizeof(double));
        if (!s || !blk) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            if (!s || !blk)
                continue;
            const int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
            const int64_t bh = b * H + h;
            const int64_t qoff = (bh * N + i) * d;
            const double sqi = (double)sq[bh * nqk + i / SAGE_QK_BLOCK];
            double* o = out + r * d;
            for (int64_t c = 0; c < d; ++c)
                o[c] = 0.0;
            double m = -INFINITY, l = 0.0;
            const int64_t jend = causal ? i + 1 : N;
            for (int64_t j0 = 0; j0 < jend; j0 += kv_block) {
                const int64_t j1 = (j0 + kv_block < jend) ? j0 + kv_block : jend;
                double mb = -INFINITY;
                for (int64_t j = j0; j < j1; ++j) {
                    const double acc = qk_dot(qq, kq, qoff, (bh * N + j) * d, d, qk_fp8, vdec);
                    double sj = acc * sqi *
                                (double)sk[bh * nqk + j / SAGE_QK_BLOCK] * scale;
                    if (bias)
                        sj += (double)bias[(bh * nbb + i / SAGE_BIAS_BLOCK) * nbb +
                                           j / SAGE_BIAS_BLOCK];
                    s[j - j0] = sj;
                    if (sj > mb)
                        mb = sj;
                }
                const double mnew = (mb > m) ? mb : m;
                if (mnew == -INFINITY)
                    continue; /* nothing visible yet */
                const double alpha = (m == -INFINITY) ? 0.0 : exp(m - mnew);
                for (int64_t c = 0; c < d; ++c)
                    blk[c] = 0.0;
                double lb = 0.0;
                for (int64_t j = j0; j < j1; ++j) {
                    const double p = exp(s[j - j0] - mnew);
                    lb += p;
                    const double ph = p_mode ? vdec[sage8_e4m3_encode(E4M3_MAX * p)]
                                             : E4M3_MAX * p;
                    if (ph == 0.0)
                        continue;
                    const uint8_t* vj = vq + (bh * N + j) * d;
                    for (int64_t c = 0; c < d; ++c)
                        blk[c] += ph * vdec[vj[c]]; /* level 1 */
                }
                for (int64_t c = 0; c < d; ++c)
                    o[c] = o[c] * alpha + blk[c]; /* level 2 */
                l = l * alpha + lb;
                m = mnew;
            }
            for (int64_t c = 0; c < d; ++c)
                o[c] = (l > 0.0) ? o[c] * (double)sv[bh * d + c] / (E4M3_MAX * l) : 0.0;
            if (lse) {
                /* the centring of K shifted every score of the row by
                 * scale * (dequantised q) . kmean; add it back to the LSE */
                double shift = 0.0;
                if (kmean)
                    for (int64_t c = 0; c < d; ++c)
                        shift += q_value(qq, qoff + c, qk_fp8, vdec) * (double)kmean[bh * d + c];
                lse[r] = (l > 0.0) ? m + log(l) + scale * sqi * shift : -INFINITY;
            }
        }
        free(s);
        free(blk);
    }
    return failed ? 3 : 0;
}

/* ---- the blocked 8-bit forward with the GPU kernel's fp32 decisions ------ */

/*
 * Same algorithm as sage8_oracle_emulate_rows, but every quantity that
 * decides an FP8 code or a rescale is formed in fp32 with the operations and
 * the order the GPU kernel uses (the pages leave these choices open; where
 * floating point decides a quantised code, both sides take the decision in
 * the kernel's precision):
 *   c = fp32(scale * log2(e)) (the smallest normal float if that is 0),
 *   f = (sq * sk) * c; the integer score S enters as s = M + S with
 *   M = 12582912 = 1.5 * 2^23 (exact in fp32 for |S| < 2^22) and the offset
 *   is folded into g = fmaf(-M, f, bias * log2(e)),
 *   the block maximum is m_blk = fmaf(M + S_max, f, g) (S_min when f < 0),
 *   the running maximum m (log2 units) is raised only when a block maximum
 *   exceeds it by more than 2, kc = (g - m) + (log2(448) - 2),
 *   P^ = e4m3(fp32(2^fmaf(M + S, f, kc))) <= 448, l = sum of the fp32 values.
 * Exponentials are evaluated in fp64 and rounded to fp32 (the kernel's
 * hardware exp2 is within about one fp32 ulp of that); sums are in fp64.
 * kv_block is 64, as in the kernel.
 */
int sage8_oracle_emulate_rows_fp32(const void* qq, const void* kq,
                                   const uint8_t* vq, const float* sq,
                                   const float* sk, const float* sv,
                                   const float* kmean, const float* bias, int64_t B, int64_t H,
                                   int64_t N, int64_t d, int causal,
                                   float scale, const int64_t* rows,
                                   int64_t nrows, double* out, double* lse,
                                   int qk_fp8, int nthreads)
{
    if (!qq || !kq || !vq || !sq || !sk || !sv || !rows || !out || B <= 0 ||
        H <= 0 || N <= 0 || d <= 0 || nrows < 0)
        return 1;
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
        if (b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= N)
            return 2;
    }
    const int64_t kvb = 64;
    const int64_t nqk = (N + SAGE_QK_BLOCK - 1) / SAGE_QK_BLOCK;
    const int64_t nbb = (N + SAGE_BIAS_BLOCK - 1) / SAGE_BIAS_BLOCK;
    const float log2e_f = 1.4426950408889634f;
    const float tau = 2.0f;
    const float plog = (float)6.807354922057604; /* log2(448) - 2 */
    /* INT8 scores leave the matrix unit offset by 1.5 * 2^23; FP8 scores do not */
    const float magic = qk_fp8 ? 0.0f : 12582912.0f;
    float c = (float)((double)scale * 1.4426950408889634);
    if (c == 0.0f)
        c = 1.17549435e-38f;
    double vdec[256];
    for (int cc = 0; cc < 256; ++cc)
        vdec[cc] = sage8_e4m3_decode((uint8_t)cc);
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int failed = 0;
#pragma omp parallel
    {
        float* s = (float*)malloc((size_t)kvb * sizeof(float));
        double* blk = (double*)malloc((size_t)d * sizeof(double));
        if (!s || !blk) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            if (!s || !blk)
                continue;
            const int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
            const int64_t bh = b * H + h;
            const int64_t qoff = (bh * N + i) * d;
            const float sqi = sq[bh * nqk + i / SAGE_QK_BLOCK];
            double* o = out + r * d;
            for (int64_t cc = 0; cc < d; ++cc)
                o[cc] = 0.0;
            float m = -INFINITY;
            double l = 0.0;
            const int64_t jend = causal ? i + 1 : N;
            for (int64_t j0 = 0; j0 < jend; j0 += kvb) {
                const int64_t j1 = (j0 + kvb < jend) ? j0 + kvb : jend;
                const float f = (sqi * sk[bh * nqk + j0 / SAGE_QK_BLOCK]) * c;
                const float bl = bias ? bias[(bh * nbb + i / SAGE_BIAS_BLOCK) * nbb +
                                             j0 / SAGE_BIAS_BLOCK] * log2e_f
                                      : 0.0f;
                float ext = (f > 0.0f) ? -INFINITY : INFINITY;
                for (int64_t j = j0; j < j1; ++j) {
                    /* exact for INT8 (|acc| < 2^24); one fp32 rounding for FP8 */
                    s[j - j0] = (float)qk_dot(qq, kq, qoff, (bh * N + j) * d, d, qk_fp8, vdec);
                    if (f > 0.0f ? s[j - j0] > ext : s[j - j0] < ext)
                        ext = s[j - j0];
                }
                const float g = fmaf(-magic, f, bl);
                const float m_blk = fmaf(magic + ext, f, g);
                if (m_blk > m + tau) {
                    const double alpha = (m == -INFINITY) ? 0.0 : exp2((double)m - (double)m_blk);
                    for (int64_t cc = 0; cc < d; ++cc)
                        o[cc] *= alpha;
                    l *= alpha;
                    m = m_blk;
                }
                const float base = (m == -INFINITY) ? 0.0f : m;
                const float kc = (g - base) + plog;
                for (int64_t cc = 0; cc < d; ++cc)
                    blk[cc] = 0.0;
                for (int64_t j = j0; j < j1; ++j) {
                    const float p = (float)exp2((double)fmaf(magic + s[j - j0], f, kc));
                    l += (double)p;
                    const double ph = vdec[sage8_e4m3_encode((double)p)];
                    if (ph == 0.0)
                        continue;
                    const uint8_t* vj = vq + (bh * N + j) * d;
                    for (int64_t cc = 0; cc < d; ++cc)
                        blk[cc] += ph * vdec[vj[cc]]; /* level 1 */
                }
                for (int64_t cc = 0; cc < d; ++cc)
                    o[cc] += blk[cc]; /* level 2 */
            }
            for (int64_t cc = 0; cc < d; ++cc)
                o[cc] = (l > 0.0) ? o[cc] * (double)sv[bh * d + cc] / l : 0.0;
            if (lse) {
                double shift = 0.0;
                if (kmean)
                    for (int64_t cc = 0; cc < d; ++cc)
                        shift += q_value(qq, qoff + cc, qk_fp8, vdec) * (double)kmean[bh * d + cc];
                lse[r] = (l > 0.0) ? ((double)m + log2(l) - (double)plog) * 0.6931471805599453 +
                                         (double)scale * (double)sqi * shift
                                   : -INFINITY;
            }
        }
        free(s);
        free(blk);
    }
    return failed ? 3 : 0;
}

/* ---- INT8 scores with the 16-bit P V product, modelled in fp64 ---------- */

/*
 * The variant of the 8-bit recipe that quantises only the first product
 * (page 1, "SageAttention", claim vs reality section: INT8 for Q K^T after
 * K is mean-centred; the page puts P and V in FP8 as the second ingredient,
 * this variant keeps them in the inputs' 16-bit format).  For every row
 * (b,h,i), in fp64, from the quantised data of steps 1-2 and the exact V:
 *
 *   s_j  = scale * sq[i/64] * sk[j/64] * sum_c Qq[i,c] Kq[j,c]
 *          + bias[b,h,i/64,j/64]          for the keys the mask allows
 *   m    = max_j s_j,  p_j = exp(s_j - m),  l = sum_j p_j
 *   O[c] = sum_j p_j V[j,c] / l
 *   LSE  = m + ln l + scale * sq[i/64] * sum_c Qq[i,c] kmean[c]
 *
 * The scores are exact attention scores of the dequantised Q and centred K
 * (the integer dot product is exact); centring K shifts every score of a row
 * by the same amount, which leaves O unchanged and is added back to the LSE
 * so that it refers to the original scores.  Everything after the scores is
 * the exact softmax(.)V of the plain oracle: the row is formed whole, then
 * normalised, then multiplied by V.  v holds the exact values of the 16-bit
 * V ([B,H,N,d] float32); qq, kq are INT8 [B,H,N,d]; sq, sk [B,H,ceil(N/64)];
 * kmean [B,H,d] (nullable: no LSE shift).  out [nrows,d], lse [nrows]
 * (nullable), fp64.  A row with no visible key gives O = 0, LSE = -inf.
 */
int sage8_oracle_qk8_rows(const int8_t* qq, const int8_t* kq, const float* sq,
                          const float* sk, const float* v, const float* kmean,
                          const float* bias, int64_t B, int64_t H, int64_t N,
                          int64_t d, int causal, double scale,
                          const int64_t* rows, int64_t nrows, double* out,
                          double* lse, int nthreads)
{
    if (!qq || !kq || !sq || !sk || !v || !rows || !out || B <= 0 || H <= 0 ||
        N <= 0 || d <= 0 || nrows < 0)
        return 1;
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
        if (b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= N)
            return 2;
    }
    const int64_t nqk = (N + SAGE_QK_BLOCK - 1) / SAGE_QK_BLOCK;
    const int64_t nbb = (N + SAGE_BIAS_BLOCK - 1) / SAGE_BIAS_BLOCK;
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
            const int64_t bh = b * H + h;
            const int8_t* qi = qq + (bh * N + i) * d;
            const double sqi = (double)sq[bh * nqk + i / SAGE_QK_BLOCK];
            double m = -INFINITY;
            for (int64_t j = 0; j < N; ++j) {
                if (causal && j > i) {
                    s[j] = -INFINITY;
                    continue;
                }
                const int8_t* kj = kq + (bh * N + j) * d;
                int64_t acc = 0;
                for (int64_t c = 0; c < d; ++c)
                    acc += (int64_t)qi[c] * (int64_t)kj[c];
                double sj = scale * (sqi * (double)sk[bh * nqk + j / SAGE_QK_BLOCK] * (double)acc);
                if (bias)
                    sj += (double)bias[(bh * nbb + i / SAGE_BIAS_BLOCK) * nbb + j / SAGE_BIAS_BLOCK];
                s[j] = sj;
                if (sj > m)
                    m = sj;
            }
            double l = 0.0;
            for (int64_t j = 0; j < N; ++j) {
                s[j] = (m == -INFINITY) ? 0.0 : exp(s[j] - m);
                l += s[j];
            }
            double* o = out + r * d;
            for (int64_t c = 0; c < d; ++c)
                o[c] = 0.0;
            for (int64_t j = 0; j < N; ++j) {
                if (s[j] == 0.0)
                    continue;
                const float* vj = v + (bh * N + j) * d;
                for (int64_t c = 0; c < d; ++c)
                    o[c] += s[j] * (double)vj[c];
            }
            for (int64_t c = 0; c < d; ++c)
                o[c] = (l > 0.0) ? o[c] / l : 0.0;
            if (lse) {
                double shift = 0.0;
                if (kmean)
                    for (int64_t c = 0; c < d; ++c)
                        shift += (double)qi[c] * (double)kmean[bh * d + c];
                lse[r] = (l > 0.0) ? m + log(l) + scale * sqi * shift : -INFINITY;
            }
        }
        free(s);
    }
    return failed ? 3 : 0;
}
