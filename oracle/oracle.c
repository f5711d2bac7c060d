/*
 * oracle.c - CPU parity oracle for the block-scaled linear layer.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h).  Shares nothing with the HIP
 * library.  Built with plain gcc, -std=c11 -O2 -ffp-contract=off, no
 * fast-math; every FP operation below is an IEEE operation in the precision
 * written.
 */
#include "oracle.h"

#include <float.h>
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#if FLT_EVAL_METHOD != 0
#error "the oracle needs float and double arithmetic evaluated in their own precision"
#endif

/* ------------------------------------------------------------------------ */
/* Decoders                                                                  */
/* ------------------------------------------------------------------------ */

/* OCP E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; exponent field 0 is
 * the subnormal range with step 0.5.  Positive values {0,.5,1,1.5,2,3,4,6}. */
double orc_e2m1_value(unsigned code)
{
    unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
    double mag = (e == 0) ? 0.5 * (double)m : (1.0 + 0.5 * (double)m) * ldexp(1.0, (int)e - 1);
    return s ? -mag : mag;
}

/* OCP E8M0: unsigned biased exponent, value 2^(code-127); 0xFF encodes NaN. */
double orc_e8m0_value(unsigned code)
{
    code &= 0xFFu;
    if (code == 0xFFu) return NAN;
    return ldexp(1.0, (int)code - 127);
}

/* OCP E4M3 "fn": 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0 is
 * subnormal (step 2^-9); S.1111.111 is NaN; there is no infinity; max 448. */
double orc_e4m3fn_value(unsigned code)
{
    unsigned s = (code >> 7) & 1u, e = (code >> 3) & 15u, m = code & 7u;
    double mag;
    if (e == 15u && m == 7u) return NAN;
    if (e == 0) mag = (double)m * ldexp(1.0, -9);
    else mag = (1.0 + (double)m / 8.0) * ldexp(1.0, (int)e - 7);
    return s ? -mag : mag;
}

/* bfloat16 is the upper half of an IEEE binary32. */
double orc_bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------------------ */
/* Encoders: nearest representable value, ties to the even code (the code's  */
/* last bit is the mantissa's last bit, so this is round-half-to-even),       */
/* magnitudes beyond the largest finite value clamp to it (saturation).       */
/* ------------------------------------------------------------------------ */

/* Magnitude code 0..7 for t >= 0. */
unsigned orc_e2m1_encode(double t)
{
    unsigned best = 0, c;
    double bestd = fabs(t - orc_e2m1_value(0));
    for (c = 1; c < 8; ++c) {
        double d = fabs(t - orc_e2m1_value(c));
        if (d < bestd || (d == bestd && (c & 1u) == 0)) {
            best = c;
            bestd = d;
        }
    }
    return best; /* t > 6 is nearest to 6 (code 7): saturation */
}

unsigned orc_e4m3fn_encode(double r)
{
    unsigned sign, lo = 0, hi = 0x7E, c;
    double m, dl, dh;
    if (isnan(r)) return 0x7F;
    sign = signbit(r) ? 0x80u : 0u;
    m = fabs(r);
    if (m >= orc_e4m3fn_value(0x7E)) return sign | 0x7Eu; /* saturate at 448 */
    /* largest code lo with value(lo) <= m; finite positive codes 0..0x7E are
     * increasing in value */
    while (lo < hi) {
        unsigned mid = (lo + hi + 1u) / 2u;
        if (orc_e4m3fn_value(mid) <= m) lo = mid;
        else hi = mid - 1u;
    }
    dl = m - orc_e4m3fn_value(lo);
    dh = orc_e4m3fn_value(lo + 1u) - m;
    if (dl < dh) c = lo;
    else if (dh < dl) c = lo + 1u;
    else c = (lo & 1u) ? lo + 1u : lo;
    return sign | c;
}

/* ------------------------------------------------------------------------ */
/* MX block (32 consecutive K values -> 32 E2M1 codes + one E8M0 scale)       */
/*   shared exponent e = floor(log2(max|v|)) - 2  (2 = largest E2M1 exponent), */
/*   clamped to the E8M0 range [-127, 127]; an all-zero block gets e = -127;  */
/*   a block holding NaN or +-Inf gets the NaN scale 0xFF and codes 0.        */
/*   Elements: v / 2^e rounded to E2M1, sign kept (so -0 and small negatives   */
/*   encode as 0x8).                                                         */
/* ------------------------------------------------------------------------ */
void orc_mx_block(const double v[32], uint8_t codes[32], uint8_t *scale)
{
    double amax = 0.0;
    int i, e;
    for (i = 0; i < 32; ++i) {
        if (!isfinite(v[i])) {
            *scale = 0xFF;
            memset(codes, 0, 32);
            return;
        }
        if (fabs(v[i]) > amax) amax = fabs(v[i]);
    }
    if (amax == 0.0) {
        e = -127;
    } else {
        int x;
        (void)frexp(amax, &x);   /* amax = f * 2^x, f in [0.5, 1)  =>  floor(log2 amax) = x - 1 */
        e = (x - 1) - 2;
        if (e < -127) e = -127;
        if (e > 127) e = 127;
    }
    *scale = (uint8_t)(e + 127);
    for (i = 0; i < 32; ++i) {
        double t = ldexp(fabs(v[i]), -e); /* exact: power-of-two scaling in FP64 */
        codes[i] = (uint8_t)((signbit(v[i]) ? 8u : 0u) | orc_e2m1_encode(t));
    }
}

/* ------------------------------------------------------------------------ */
/* Row-parallel driver: [0, n) is cut into nthreads contiguous ranges; range */
/* t runs on its own thread and is told its slot number t.                  */
/* ------------------------------------------------------------------------ */
typedef void (*range_fn)(void *ctx, int64_t r0, int64_t r1, int slot);

struct range_job {
    range_fn fn;
    void *ctx;
    int64_t r0, r1;
    int slot;
};

static void *range_thread(void *p)
{
    struct range_job *j = (struct range_job *)p;
    j->fn(j->ctx, j->r0, j->r1, j->slot);
    return NULL;
}

static void parallel_ranges(int64_t n, int nthreads, range_fn fn, void *ctx)
{
    pthread_t tid[256];
    struct range_job job[256];
    int t, started = 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > n) nthreads = (int)(n > 0 ? n : 1);
    if (nthreads == 1) {
        fn(ctx, 0, n, 0);
        return;
    }
    for (t = 0; t < nthreads; ++t) {
        job[t].fn = fn;
        job[t].ctx = ctx;
        job[t].r0 = n * t / nthreads;
        job[t].r1 = n * (t + 1) / nthreads;
        job[t].slot = t;
    }
    for (t = 1; t < nthreads; ++t) {
        if (pthread_create(&tid[t], NULL, range_thread, &job[t]) != 0) break;
        started = t;
    }
    fn(ctx, job[0].r0, job[0].r1, 0);
    for (t = 1; t <= started; ++t) pthread_join(tid[t], NULL);
    for (t = started + 1; t < nthreads; ++t) fn(ctx, job[t].r0, job[t].r1, t); /* thread creation failed */
}

/* ------------------------------------------------------------------------ */
/* MX row quantizers                                                         */
/* ------------------------------------------------------------------------ */
struct mx_ctx {
    const uint16_t *xb;
    const float *xf;
    int64_t K;
    uint8_t *q, *s;
};

static void mx_rows(void *p, int64_t r0, int64_t r1, int slot)
{
    (void)slot;
    struct mx_ctx *c = (struct mx_ctx *)p;
    int64_t r, b, i;
    double v[32];
    uint8_t codes[32];
    for (r = r0; r < r1; ++r) {
        for (b = 0; b < c->K / 32; ++b) {
            for (i = 0; i < 32; ++i) {
                int64_t k = b * 32 + i;
                v[i] = c->xb ? orc_bf16_value(c->xb[r * c->K + k]) : (double)c->xf[r * c->K + k];
            }
            orc_mx_block(v, codes, &c->s[r * (c->K / 32) + b]);
            for (i = 0; i < 16; ++i)
                c->q[r * (c->K / 2) + b * 16 + i] = (uint8_t)(codes[2 * i] | (codes[2 * i + 1] << 4));
        }
    }
}

static int mx_quant(const uint16_t *xb, const float *xf, int64_t rows, int64_t K,
                    uint8_t *q, uint8_t *s, int nthreads)
{
    struct mx_ctx c;
    if (rows < 0 || K <= 0 || K % 32 != 0) return ORC_EARG;
    if (rows == 0) return ORC_OK;
    if ((!xb && !xf) || !q || !s) return ORC_EARG;
    c.xb = xb; c.xf = xf; c.K = K; c.q = q; c.s = s;
    parallel_ranges(rows, nthreads, mx_rows, &c);
    return ORC_OK;
}

int orc_mx_quant_bf16(const uint16_t *x, int64_t rows, int64_t K, uint8_t *q, uint8_t *s, int nthreads)
{
    if (rows > 0 && !x) return ORC_EARG;
    return mx_quant(x, NULL, rows, K, q, s, nthreads);
}

int orc_mx_quant_f32(const float *x, int64_t rows, int64_t K, uint8_t *q, uint8_t *s, int nthreads)
{
    if (rows > 0 && !x) return ORC_EARG;
    return mx_quant(NULL, x, rows, K, q, s, nthreads);
}

/* ------------------------------------------------------------------------ */
/* PTPC (per-token / per-channel) FP8 row quantizer                           */
/*   a = max_k |x_k|;  s = fl32(a / 448)  (448 = largest E4M3fn value);       */
/*   a == 0 gives s = 1;  a row holding NaN or +-Inf gives s = NaN and every  */
/*   code the NaN code 0x7F;  q_k = E4M3fn(fl32(x_k / s)), both divisions     */
/*   IEEE binary32 with round-to-nearest-even.                               */
/* ------------------------------------------------------------------------ */
struct ptpc_ctx {
    const uint16_t *xb;
    const float *xf;
    int64_t K;
    uint8_t *q;
    float *s;
};

static float row_elem(const struct ptpc_ctx *c, int64_t r, int64_t k)
{
    return c->xb ? (float)orc_bf16_value(c->xb[r * c->K + k]) : c->xf[r * c->K + k];
}

static void ptpc_rows(void *p, int64_t r0, int64_t r1, int slot)
{
    (void)slot;
    struct ptpc_ctx *c = (struct ptpc_ctx *)p;
    int64_t r, k;
    for (r = r0; r < r1; ++r) {
        float a = 0.0f, sc;
        int nonfinite = 0;
        for (k = 0; k < c->K; ++k) {
            float x = row_elem(c, r, k);
            if (!isfinite(x)) nonfinite = 1;
            else if (fabsf(x) > a) a = fabsf(x);
        }
        if (nonfinite) {
            c->s[r] = NAN;
            memset(c->q + r * c->K, 0x7F, (size_t)c->K);
            continue;
        }
        sc = (a == 0.0f) ? 1.0f : a / 448.0f;
        c->s[r] = sc;
        for (k = 0; k < c->K; ++k) {
            float t = row_elem(c, r, k) / sc;
            c->q[r * c->K + k] = (uint8_t)orc_e4m3fn_encode((double)t);
        }
    }
}

static int ptpc_quant(const uint16_t *xb, const float *xf, int64_t rows, int64_t K,
                      uint8_t *q, float *s, int nthreads)
{
    struct ptpc_ctx c;
    if (rows < 0 || K <= 0) return ORC_EARG;
    if (rows == 0) return ORC_OK;
    if ((!xb && !xf) || !q || !s) return ORC_EARG;
    c.xb = xb; c.xf = xf; c.K = K; c.q = q; c.s = s;
    parallel_ranges(rows, nthreads, ptpc_rows, &c);
    return ORC_OK;
}

int orc_ptpc_quant_bf16(const uint16_t *x, int64_t rows, int64_t K, uint8_t *q, float *s, int nthreads)
{
    if (rows > 0 && !x) return ORC_EARG;
    return ptpc_quant(x, NULL, rows, K, q, s, nthreads);
}

int orc_ptpc_quant_f32(const float *x, int64_t rows, int64_t K, uint8_t *q, float *s, int nthreads)
{
    if (rows > 0 && !x) return ORC_EARG;
    return ptpc_quant(NULL, x, rows, K, q, s, nthreads);
}

/* ------------------------------------------------------------------------ */
/* Exact A4W4 GEMM                                                           */
/*   Every E2M1 value is an integer multiple of 1/2, so with ia = 2*a and     */
/*   iw = 2*w (integers, |.| <= 12) the dot product of one 32-block is the    */
/*   integer I_b = sum ia*iw (|I_b| <= 32*144 < 2^13), and                    */
/*     Y[m,n] = sum_b I_b * 2^(sA[m,b] + sW[n,b] - 254 - 2).                  */
/*   All terms are integer multiples of 2^(min exponent), so when             */
/*   span + 13 + ceil(log2(#terms)) <= 53 every partial sum is exact in FP64  */
/*   and the order of summation does not matter.  The check is made for each  */
/*   output; ORC_EINEXACT is returned if it ever fails.  A NaN scale (0xFF)   */
/*   on either side makes the output NaN.                                     */
/* ------------------------------------------------------------------------ */
static int ceil_log2_i64(int64_t n)
{
    int b = 0;
    while (((int64_t)1 << b) < n) ++b;
    return b;
}

struct a4_ctx {
    const uint8_t *qa, *sa, *qw, *sw;
    int64_t K;
    const int64_t *rows, *cols;
    int64_t n_cols;
    const int8_t *wdec; /* [n_cols, K] decoded 2*w */
    double *y, *absdot;
    int span[256];
    int inexact[256];   /* per worker slot */
};

static int8_t e2m1_twice(unsigned code)
{
    return (int8_t)(2.0 * orc_e2m1_value(code & 15u));
}

static void a4_rows(void *p, int64_t i0, int64_t i1, int slot)
{
    struct a4_ctx *c = (struct a4_ctx *)p;
    int64_t nb = c->K / 32, i, j, b, k;
    int8_t *adec = (int8_t *)malloc((size_t)c->K);
    for (i = i0; i < i1; ++i) {
        int64_t m = c->rows[i];
        int a_nan = 0;
        for (k = 0; k < c->K; ++k) {
            uint8_t byte = c->qa[m * (c->K / 2) + k / 2];
            adec[k] = e2m1_twice((k & 1) ? (unsigned)(byte >> 4) : (unsigned)(byte & 15u));
        }
        for (b = 0; b < nb; ++b)
            if (c->sa[m * nb + b] == 0xFF) a_nan = 1;
        for (j = 0; j < c->n_cols; ++j) {
            int64_t n = c->cols[j];
            const int8_t *wd = c->wdec + j * c->K;
            double acc = 0.0, accabs = 0.0;
            int emin = 1 << 20, emax = -(1 << 20), nz = 0, w_nan = 0;
            for (b = 0; b < nb; ++b)
                if (c->sw[n * nb + b] == 0xFF) w_nan = 1;
            if (a_nan || w_nan) {
                c->y[i * c->n_cols + j] = NAN;
                if (c->absdot) c->absdot[i * c->n_cols + j] = NAN;
                continue;
            }
            for (b = 0; b < nb; ++b) {
                int32_t I = 0, Iabs = 0;
                int e = (int)c->sa[m * nb + b] + (int)c->sw[n * nb + b] - 256;
                for (k = b * 32; k < b * 32 + 32; ++k) {
                    int32_t prod = (int32_t)adec[k] * (int32_t)wd[k];
                    I += prod;
                    Iabs += prod < 0 ? -prod : prod;
                }
                if (I != 0) {
                    acc += ldexp((double)I, e);
                    if (e < emin) emin = e;
                    if (e > emax) emax = e;
                    ++nz;
                }
                if (Iabs != 0) accabs += ldexp((double)Iabs, e);
            }
            if (nz > 0) {
                int span = emax - emin;
                if (span > c->span[slot]) c->span[slot] = span;
                if (span + 13 + ceil_log2_i64(nz) > 53) c->inexact[slot] = 1;
            }
            c->y[i * c->n_cols + j] = acc;
            if (c->absdot) c->absdot[i * c->n_cols + j] = accabs;
        }
    }
    free(adec);
}

struct wdec_ctx {
    const uint8_t *qw;
    int64_t K;
    const int64_t *cols;
    int8_t *wdec;
};

static void wdec_rows(void *p, int64_t j0, int64_t j1, int slot)
{
    (void)slot;
    struct wdec_ctx *c = (struct wdec_ctx *)p;
    int64_t j, k;
    for (j = j0; j < j1; ++j) {
        int64_t n = c->cols[j];
        for (k = 0; k < c->K; ++k) {
            uint8_t byte = c->qw[n * (c->K / 2) + k / 2];
            c->wdec[j * c->K + k] = e2m1_twice((k & 1) ? (unsigned)(byte >> 4) : (unsigned)(byte & 15u));
        }
    }
}

static int check_grid(int64_t M, int64_t N, int64_t K, const int64_t *rows, int64_t n_rows,
                      const int64_t *cols, int64_t n_cols)
{
    int64_t i;
    if (M < 0 || N < 0 || K <= 0 || n_rows < 0 || n_cols < 0) return ORC_EARG;
    for (i = 0; i < n_rows; ++i)
        if (rows[i] < 0 || rows[i] >= M) return ORC_EARG;
    for (i = 0; i < n_cols; ++i)
        if (cols[i] < 0 || cols[i] >= N) return ORC_EARG;
    return ORC_OK;
}

int orc_gemm_a4w4_at(const uint8_t *qa, const uint8_t *sa, const uint8_t *qw, const uint8_t *sw,
                     int64_t M, int64_t N, int64_t K,
                     const int64_t *rows, int64_t n_rows, const int64_t *cols, int64_t n_cols,
                     double *y, double *absdot, int *max_span, int nthreads)
{
    struct a4_ctx c;
    struct wdec_ctx w;
    int t, rc = ORC_OK, ms = 0;
    if (K % 32 != 0) return ORC_EARG;
    if (check_grid(M, N, K, rows, n_rows, cols, n_cols) != ORC_OK) return ORC_EARG;
    if (max_span) *max_span = 0;
    if (n_rows == 0 || n_cols == 0) return ORC_OK;
    if (!qa || !sa || !qw || !sw || !y) return ORC_EARG;
    memset(&c, 0, sizeof c);
    c.wdec = (int8_t *)malloc((size_t)(n_cols * K));
    if (!c.wdec) return ORC_EARG;
    w.qw = qw; w.K = K; w.cols = cols; w.wdec = (int8_t *)c.wdec;
    parallel_ranges(n_cols, nthreads, wdec_rows, &w);
    c.qa = qa; c.sa = sa; c.qw = qw; c.sw = sw; c.K = K;
    c.rows = rows; c.cols = cols; c.n_cols = n_cols;
    c.y = y; c.absdot = absdot;
    parallel_ranges(n_rows, nthreads, a4_rows, &c);
    for (t = 0; t < 256; ++t) {
        if (c.span[t] > ms) ms = c.span[t];
        if (c.inexact[t]) rc = ORC_EINEXACT;
    }
    if (max_span) *max_span = ms;
    free((void *)c.wdec);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Exact A8W8 GEMM                                                           */
/*   Every finite E4M3fn value is an integer multiple of 2^-9 below 2^9, so   */
/*   with ia = 512*a, iw = 512*w (|.| <= 229376 < 2^18) the dot product is    */
/*   the int64 S = sum ia*iw (|S| < K*2^36 < 2^53 for K < 2^17, so S is exact */
/*   in FP64), and Y[m,n] = (sA[m]*sW[n]) * S * 2^-18, where the scale      */
/*   product is exact in FP64 and the last multiply rounds once.  A NaN code  */
/*   in either operand row or a NaN scale makes the output NaN.               */
/* ------------------------------------------------------------------------ */
struct a8_ctx {
    const uint8_t *qa, *qw;
    const float *sa, *sw;
    int64_t K;
    const int64_t *rows, *cols;
    int64_t n_cols;
    const int32_t *wdec; /* [n_cols, K] 512*w, INT32_MIN marks NaN */
    double *y, *absdot;
};

static int32_t e4m3_times512(unsigned code)
{
    double v = orc_e4m3fn_value(code & 0xFFu);
    if (isnan(v)) return INT32_MIN;
    return (int32_t)(v * 512.0);
}

static void a8_rows(void *p, int64_t i0, int64_t i1, int slot)
{
    (void)slot;
    struct a8_ctx *c = (struct a8_ctx *)p;
    int64_t i, j, k;
    int32_t *adec = (int32_t *)malloc((size_t)c->K * sizeof(int32_t));
    for (i = i0; i < i1; ++i) {
        int64_t m = c->rows[i];
        int a_nan = 0;
        for (k = 0; k < c->K; ++k) {
            adec[k] = e4m3_times512(c->qa[m * c->K + k]);
            if (adec[k] == INT32_MIN) a_nan = 1;
        }
        for (j = 0; j < c->n_cols; ++j) {
            int64_t n = c->cols[j];
            const int32_t *wd = c->wdec + j * c->K;
            int64_t S = 0, Sabs = 0;
            int w_nan = 0;
            double sc = (double)c->sa[m] * (double)c->sw[n];
            for (k = 0; k < c->K; ++k) {
                int64_t prod;
                if (wd[k] == INT32_MIN) { w_nan = 1; continue; }
                prod = (int64_t)adec[k] * (int64_t)wd[k];
                S += prod;
                Sabs += prod < 0 ? -prod : prod;
            }
            if (a_nan || w_nan) {
                c->y[i * c->n_cols + j] = NAN;
                if (c->absdot) c->absdot[i * c->n_cols + j] = NAN;
                continue;
            }
            c->y[i * c->n_cols + j] = sc * ldexp((double)S, -18);
            if (c->absdot) c->absdot[i * c->n_cols + j] = fabs(sc) * ldexp((double)Sabs, -18);
        }
    }
    free(adec);
}

struct w8dec_ctx {
    const uint8_t *qw;
    int64_t K;
    const int64_t *cols;
    int32_t *wdec;
};

static void w8dec_rows(void *p, int64_t j0, int64_t j1, int slot)
{
    (void)slot;
    struct w8dec_ctx *c = (struct w8dec_ctx *)p;
    int64_t j, k;
    for (j = j0; j < j1; ++j)
        for (k = 0; k < c->K; ++k)
            c->wdec[j * c->K + k] = e4m3_times512(c->qw[c->cols[j] * c->K + k]);
}

int orc_gemm_a8w8_at(const uint8_t *qa, const float *sa, const uint8_t *qw, const float *sw,
                     int64_t M, int64_t N, int64_t K,
                     const int64_t *rows, int64_t n_rows, const int64_t *cols, int64_t n_cols,
                     double *y, double *absdot, int nthreads)
{
    struct a8_ctx c;
    struct w8dec_ctx w;
    if (K >= ((int64_t)1 << 17)) return ORC_EARG; /* keeps |S| < 2^53 */
    if (check_grid(M, N, K, rows, n_rows, cols, n_cols) != ORC_OK) return ORC_EARG;
    if (n_rows == 0 || n_cols == 0) return ORC_OK;
    if (!qa || !sa || !qw || !sw || !y) return ORC_EARG;
    c.wdec = (int32_t *)malloc((size_t)(n_cols * K) * sizeof(int32_t));
    if (!c.wdec) return ORC_EARG;
    w.qw = qw; w.K = K; w.cols = cols; w.wdec = (int32_t *)c.wdec;
    parallel_ranges(n_cols, nthreads, w8dec_rows, &w);
    c.qa = qa; c.sa = sa; c.qw = qw; c.sw = sw; c.K = K;
    c.rows = rows; c.cols = cols; c.n_cols = n_cols;
    c.y = y; c.absdot = absdot;
    parallel_ranges(n_rows, nthreads, a8_rows, &c);
    free((void *)c.wdec);
    return ORC_OK;
}
