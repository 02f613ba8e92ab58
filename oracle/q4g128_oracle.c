/*
 * q4g128_oracle.c -- plain, slow, fp64 CPU oracle for the group-wise
 * asymmetric int4 weight-streaming product y = x . dequant(W).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant
 * with the HIP library.
 *
 * What it computes follows the Token Rush README (github.com/zyhector/
 * token-rush):
 *   - its weight format paragraph: asymmetric int4 by groups, every 128
 *     consecutive weights sharing one bf16 scale and one bf16 minimum, 4.25
 *     bits per weight;
 *   - its list of constraints, which gives the same format;
 *   - its bandwidth paragraph: a decode step multiplies the activation by
 *     every streamed weight matrix;
 *   - its steps table, rows 13-14 and 28: a verify step is the same product
 *     with M activation rows.
 * and the bw24 article (wpnews.pro), exactness paragraph: verify must agree
 * with plain decode exactly, and the order of summation is part of that
 * contract.
 *
 * Readings taken where the pages leave a step open (all listed in the design
 * notes): a weight is w = q*s + m (q = 0 maps to the minimum); the 128-weight
 * group runs along the contraction axis k within one output column n; codes
 * are packed as W[n][k/8] uint32 with nibble (k mod 8) of that word holding
 * code k, low nibble first; scale and minimum are stored [n][k/128].
 *
 * Arithmetic: every bf16 is decoded exactly from its bit fields; w is formed
 * in fp64 and checked to be exact (a 4-bit code times an 8-bit significand
 * plus an 8-bit significand); y[m][n] = sum over k ascending of x[m][k]*w in
 * fp64; a[m][n] = sum of |x[m][k]*w| is the tolerance scale.  Each (m, n) is
 * summed by one thread, so results do not depend on the thread count.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (no fast-math).  Compiling with
 * -DORACLE_PLANT=<n> plants one deliberate mistake; the test suite uses that
 * to show that its pins catch each kind of mistake.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef ORACLE_PLANT
#define ORACLE_PLANT 0
#endif

enum { ORC_OK = 0, ORC_EINVAL = 1, ORC_EINEXACT = 2, ORC_ENONFINITE = 3 };

/* bf16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits.  Decoded
 * from the fields, not by reinterpreting memory. */
static int bf16_decode(uint16_t b, double *out)
{
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xFF;
    int f = b & 0x7F;
    double v;
    if (e == 0xFF)
        return ORC_ENONFINITE;
    if (e == 0)
        v = ldexp((double)f, -126 - 7);           /* subnormal: f/128 * 2^-126 */
    else
        v = ldexp((double)(128 + f), e - 127 - 7); /* (1 + f/128) * 2^(e-127) */
    *out = sign ? -v : v;
    return ORC_OK;
}

/* Code k of output column n. */
static int code_at(const uint32_t *W, long K, long n, long k)
{
    uint32_t word = W[n * (K / 8) + k / 8];
#if ORACLE_PLANT == 3
    return (int)((word >> (4 * (7 - k % 8))) & 0xFu); /* planted: high nibble first */
#else
    return (int)((word >> (4 * (k % 8))) & 0xFu);
#endif
}

/* Index of the (n, group-of-k) entry in a [N][K/128] scale or minimum array. */
static long group_index(long K, long N, long n, long k)
{
    long G = K / 128;
#if ORACLE_PLANT == 4
    (void)N;
    return n * G + (k / 64) % G;      /* planted: groups of 64 */
#elif ORACLE_PLANT == 5
    (void)G;
    return (k / 128) * N + n;         /* planted: scale array read transposed */
#else
    (void)N;
    return n * G + k / 128;
#endif
}

/* Knuth's two-sum: err is the exact rounding error of s = a + b. */
static double two_sum_err(double a, double b, double s)
{
    double bb = s - a;
    return (a - (s - bb)) + (b - bb);
}

/* Exact fp64 weight w = q*s + m of column n, position k. */
static int weight_f64(const uint32_t *W, const uint16_t *S, const uint16_t *Mn,
                      long K, long N, long n, long k, double *w)
{
    double s, m, qs, v;
    int q = code_at(W, K, n, k);
    long gi = group_index(K, N, n, k);
    if (bf16_decode(S[gi], &s) || bf16_decode(Mn[gi], &m))
        return ORC_ENONFINITE;
    qs = (double)q * s;               /* <= 12 significant bits: exact */
#if ORACLE_PLANT == 1
    m = 0.0;                          /* planted: minimum dropped */
#elif ORACLE_PLANT == 2
    m = -m;                           /* planted: minimum subtracted */
#endif
    v = qs + m;
    if (two_sum_err(qs, m, v) != 0.0)
        return ORC_EINEXACT;
    *w = v;
    return ORC_OK;
}

static int shape_ok(long M, long K, long N)
{
    return M >= 1 && K >= 128 && K % 128 == 0 && N >= 1;
}

int q4o_abi_version(void) { return 1; }

int q4o_plant(void) { return ORACLE_PLANT; }

/* Codes as bytes, [N][K]. */
int q4o_codes(const uint32_t *W, long K, long N, uint8_t *q)
{
    if (!shape_ok(1, K, N) || !W || !q)
        return ORC_EINVAL;
    for (long n = 0; n < N; ++n)
        for (long k = 0; k < K; ++k)
            q[n * K + k] = (uint8_t)code_at(W, K, n, k);
    return ORC_OK;
}

/* Decoded weights, fp64, [N][K] (w_nk; the product uses its transpose). */
int q4o_dequant_f64(const uint32_t *W, const uint16_t *S, const uint16_t *Mn,
                    long K, long N, double *w)
{
    if (!shape_ok(1, K, N) || !W || !S || !Mn || !w)
        return ORC_EINVAL;
    for (long n = 0; n < N; ++n)
        for (long k = 0; k < K; ++k) {
            int rc = weight_f64(W, S, Mn, K, N, n, k, &w[n * K + k]);
            if (rc)
                return rc;
        }
    return ORC_OK;
}

/* Decoded weights rounded once to fp32 (round to nearest, ties to even),
 * [N][K].  A one-rounding fp32 dequant must equal this bit for bit. */
int q4o_dequant_f32(const uint32_t *W, const uint16_t *S, const uint16_t *Mn,
                    long K, long N, float *w32)
{
    if (!shape_ok(1, K, N) || !W || !S || !Mn || !w32)
        return ORC_EINVAL;
    for (long n = 0; n < N; ++n)
        for (long k = 0; k < K; ++k) {
            double w;
            int rc = weight_f64(W, S, Mn, K, N, n, k, &w);
            if (rc)
                return rc;
            w32[n * K + k] = (float)w;
        }
    return ORC_OK;
}

/* y[m][c] and a[m][c] for the listed output columns cols[c] (all columns
 * when cols is NULL, then ncols must equal N).  x is bf16 [M][K].  Each
 * column's weights are decoded once into a scratch vector, x once into
 * doubles; the sums then run over k in ascending order. */
int q4o_gemm_cols(const uint16_t *x, long M, long K, const uint32_t *W,
                  const uint16_t *S, const uint16_t *Mn, long N,
                  const long *cols, long ncols, double *y, double *a,
                  int nthreads)
{
    int status = ORC_OK;
    double *xd;
    if (!shape_ok(M, K, N) || !x || !W || !S || !Mn || !y || !a || ncols < 0)
        return ORC_EINVAL;
    if (!cols && ncols != N)
        return ORC_EINVAL;
    for (long c = 0; cols && c < ncols; ++c)
        if (cols[c] < 0 || cols[c] >= N)
            return ORC_EINVAL;
    xd = (double *)malloc((size_t)M * (size_t)K * sizeof(double));
    if (!xd)
        return ORC_EINVAL;
    for (long e = 0; e < M * K; ++e)
        if (bf16_decode(x[e], &xd[e])) {
            free(xd);
            return ORC_ENONFINITE;
        }
#ifdef _OPENMP
    if (nthreads < 1)
        nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#else
    (void)nthreads;
#endif
    {
        double *wcol = (double *)malloc((size_t)K * sizeof(double));
#ifdef _OPENMP
#pragma omp for schedule(static)
#endif
        for (long c = 0; c < ncols; ++c) {
            long n = cols ? cols[c] : c;
            int rc = wcol ? ORC_OK : ORC_EINVAL;
            for (long k = 0; k < K && !rc; ++k)
                rc = weight_f64(W, S, Mn, K, N, n, k, &wcol[k]);
            if (rc) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
                status = rc;
                continue;
            }
            for (long m = 0; m < M; ++m) {
                double acc = 0.0, mag = 0.0;
#if ORACLE_PLANT == 6
                long kend = K - 1;        /* planted: last k dropped */
#else
                long kend = K;
#endif
                long xrow = m;
#if ORACLE_PLANT == 7
                xrow = 0;                 /* planted: every output row reads x row 0 */
#endif
                for (long k = 0; k < kend; ++k) {
                    double p = xd[xrow * K + k] * wcol[k];
                    acc += p;
                    mag += fabs(p);
                }
                y[m * ncols + c] = acc;
                a[m * ncols + c] = mag;
            }
        }
        free(wcol);
    }
    free(xd);
    return status;
}

/* Whole product: y, a are [M][N]. */
int q4o_gemm(const uint16_t *x, long M, long K, const uint32_t *W,
             const uint16_t *S, const uint16_t *Mn, long N, double *y,
             double *a, int nthreads)
{
    return q4o_gemm_cols(x, M, K, W, S, Mn, N, NULL, N, y, a, nthreads);
}

/* ---- quantizer ---------------------------------------------------------------
 *
 * Producing the format from bf16 weights (Token Rush README, quantization
 * section): codes, scale and minimum are chosen per group of 128 weights;
 * plain round-to-nearest is the baseline there, and a per-group search over
 * narrowed ranges, scored by squared error, gives up accuracy on the extreme
 * values for a finer step on the rest.  The pages give no formula; the reading
 * taken
 * (one candidate = round-to-nearest):
 *
 *   v_k        the 128 weights of the group, decoded exactly to fp64
 *   lo, hi     min and max of v;  c = (lo + hi) * 0.5
 *   candidates (i, j), i = 0 .. ncand-1 outer, j = 0 .. ncand-1 inner:
 *     l = lo + (i / 20.0) * (c - lo),  h = hi - (j / 20.0) * (hi - c)
 *                                                        (each end clipped toward c)
 *     s = (h - l) / 15
 *     s_b = bf16(fp32(s)), m_b = bf16(fp32(l))            (round to nearest even, twice)
 *     q_k = 0 if s_b == 0, else min(15, max(0, rint((v_k - m_b) / s_b)))
 *     e   = sum over k ascending of ((q_k * s_b + m_b) - v_k)^2
 *   keep the first candidate with the smallest e.
 *
 * Every step is one IEEE fp64 operation in the order written (no fused
 * multiply-add), so an fp64 implementation that follows the same steps makes
 * the same choices bit for bit.
 */

static uint16_t bf16_of_f32(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    u = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;      /* round to nearest, ties to even */
    return (uint16_t)u;
}

static double f64_of_bf16_bits(uint16_t b)
{
    double v = 0.0;
    bf16_decode(b, &v);
    return v;
}

/* One group: v[128] -> codes q[128], scale/minimum bits; returns the error. */
static double quantize_group(const double *v, int ncand, uint8_t *q, uint16_t *sb, uint16_t *mb)
{
    double lo = v[0], hi = v[0];
    for (int k = 1; k < 128; ++k) {
        if (v[k] < lo) lo = v[k];
        if (v[k] > hi) hi = v[k];
    }
    const double c = (lo + hi) * 0.5;
    double best = INFINITY;
    uint8_t qc[128];
    for (int ij = 0; ij < ncand * ncand; ++ij) {
        const double bl = (double)(ij / ncand) / 20.0;
        const double bh = (double)(ij % ncand) / 20.0;
        const double l = lo + bl * (c - lo);
        const double h = hi - bh * (hi - c);
        const double sv = (h - l) / 15.0;
        const uint16_t s16 = bf16_of_f32((float)sv);
        const uint16_t m16 = bf16_of_f32((float)l);
        const double sd = f64_of_bf16_bits(s16);
        const double md = f64_of_bf16_bits(m16);
        double e = 0.0;
        for (int k = 0; k < 128; ++k) {
            double code = 0.0;
            if (sd != 0.0) {
#if ORACLE_PLANT == 9
                code = floor((v[k] - md) / sd);               /* planted: truncation */
#elif ORACLE_PLANT == 10
                code = rint((v[k] - md) / (sd * 15.0 / 16.0)); /* planted: 16 steps */
#else
                code = rint((v[k] - md) / sd);
#endif
                if (code < 0.0) code = 0.0;
#if ORACLE_PLANT == 8
                if (code > 14.0) code = 14.0;                 /* planted: top code lost */
#else
                if (code > 15.0) code = 15.0;
#endif
            }
            qc[k] = (uint8_t)code;
            const double r = (code * sd + md) - v[k];
            e = e + r * r;
        }
        if (e < best) {
            best = e;
            memcpy(q, qc, 128);
            *sb = s16;
            *mb = m16;
        }
    }
    return best;
}

/* Quantize w [N][K] bf16 (K a multiple of 128) into W [N][K/8] (code k of
 * column n in nibble k % 8 of word k / 8, low nibble first), scale and
 * minimum [N][K/128] bf16; err [N][K/128] (may be NULL) gets each group's
 * squared error.  ncand in 1..16 (ncand * ncand candidates per group). */
int q4o_quantize(const uint16_t *w, long K, long N, int ncand, uint32_t *W, uint16_t *S,
                 uint16_t *Mn, double *err, int nthreads)
{
    if (!w || !W || !S || !Mn || K <= 0 || K % 128 || N <= 0 || ncand < 1 || ncand > 16)
        return ORC_EINVAL;
    const long G = K / 128;
    int status = ORC_OK;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(static) num_threads(nthreads)
#else
    (void)nthreads;
#endif
    for (long gi = 0; gi < N * G; ++gi) {
        const long n = gi / G, g = gi % G;
        double v[128];
        uint8_t q[128];
        uint16_t sb = 0, mb = 0;
        int bad = 0;
        for (int k = 0; k < 128; ++k)
            if (bf16_decode(w[n * K + g * 128 + k], &v[k]) != ORC_OK) bad = 1;
        if (bad) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            status = ORC_ENONFINITE;
            continue;
        }
        const double e = quantize_group(v, ncand, q, &sb, &mb);
        for (int j = 0; j < 16; ++j) {
            uint32_t word = 0;
            for (int i = 0; i < 8; ++i) word |= (uint32_t)q[8 * j + i] << (4 * i);
            W[n * (K / 8) + g * 16 + j] = word;
        }
        S[n * G + g] = sb;
        Mn[n * G + g] = mb;
        if (err) err[n * G + g] = e;
    }
    return status;
}

/* Threads the OpenMP runtime would use by default (for reporting). */
/* ---- epilogues after the product ---------------------------------------------
 *
 * Token Rush README, steps table: the projections are fused side by side
 * along N (row 3), and split-K partial sums are added inside the following
 * norm (rows 8-9).  The pages name neither the activation nor the norm's
 * formula; the readings taken are those of the gated MLP and the RMSNorm of
 * the model family both pages run:
 *
 *   SwiGLU on a fused gate/up product y [M][N], N = 2I, gate = columns
 *   0..I-1, up = columns I..2I-1:
 *       act[m][i] = silu(g) * u,  silu(g) = g / (1 + exp(-g)),
 *       g = y[m][i], u = y[m][I + i];
 *
 *   residual add + RMSNorm of a product y [M][N] with residual r [M][N],
 *   bf16 gain gamma [N] and eps:
 *       h[m][n]   = r[m][n] + y[m][n]
 *       ms[m]     = (sum over n ascending of h[m][n]^2) / N
 *       out[m][n] = h[m][n] / sqrt(ms[m] + eps) * gamma[n].
 *
 * Both in fp64, on fp64 inputs (the oracle's own product), one row at a time.
 */
int q4o_swiglu(const double *y, long M, long N, double *act)
{
    if (!y || !act || M <= 0 || N <= 0 || N % 2) return ORC_EINVAL;
    const long I = N / 2;
    for (long m = 0; m < M; ++m)
        for (long i = 0; i < I; ++i) {
#if ORACLE_PLANT == 12
            const double g = y[m * N + I + i], u = y[m * N + i];   /* planted: halves swapped */
#else
            const double g = y[m * N + i], u = y[m * N + I + i];
#endif
#if ORACLE_PLANT == 11
            act[m * I + i] = g / (1.0 + exp(g)) * u;              /* planted: wrong sign in exp */
#else
            act[m * I + i] = g / (1.0 + exp(-g)) * u;
#endif
        }
    return ORC_OK;
}

int q4o_residual_rmsnorm(const double *y, const double *r, const uint16_t *gamma, double eps, long M, long N,
                         double *h, double *out)
{
    if (!y || !r || !gamma || !h || !out || M <= 0 || N <= 0 || !(eps >= 0.0)) return ORC_EINVAL;
    for (long m = 0; m < M; ++m) {
        double ss = 0.0;
        for (long n = 0; n < N; ++n) {
            h[m * N + n] = r[m * N + n] + y[m * N + n];
            ss += h[m * N + n] * h[m * N + n];
        }
#if ORACLE_PLANT == 13
        const double ms = ss;                                    /* planted: sum, not mean */
#else
        const double ms = ss / (double)N;
#endif
#if ORACLE_PLANT == 14
        const double inv = 1.0 / sqrt(ms);                       /* planted: eps dropped */
#else
        const double inv = 1.0 / sqrt(ms + eps);
#endif
        for (long n = 0; n < N; ++n) {
            double gm;
            if (bf16_decode(gamma[n], &gm) != ORC_OK) return ORC_ENONFINITE;
            out[m * N + n] = h[m * N + n] * inv * gm;
        }
    }
    return ORC_OK;
}

int q4o_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
