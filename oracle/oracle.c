/*
 * oracle.c — fp64 CPU reference (see oracle.h for the page legend).
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the test suite, the smoke check and the
 * benchmark's CPU-baseline leg, never by the GPU library.  It shares no code,
 * header, table or constant with the GPU path.
 *
 * Each routine is the plain definition written out: no blocking, no fusion,
 * no reordering of any sum.  Sums run over the reduction index in ascending
 * order, in double.  The loop nest of the GEMM puts the reduction index
 * outside the column loop, but every output element is still accumulated
 * k = 0, 1, …, K-1 in that order, so the rounding sequence is the one of the
 * textbook inner-product loop.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -fPIC -shared (no -ffast-math).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- exact decoders ---------------------------------------------------- */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double orc_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);    /* (1.m) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16: the upper 16 bits of a binary32 — 1 sign, 8 exponent (bias 127),
 * 7 fraction bits. */
double orc_bf16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 0xff;
    int m = h & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)m, -133);                /* subnormal: m * 2^-133 */
    else if (e == 255)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + m), e - 134);    /* (1.m) * 2^(e-127) */
    return sign ? -v : v;
}

/* binary32: 1 sign, 8 exponent (bias 127), 23 fraction bits. */
double orc_f32_to_f64(uint32_t u)
{
    int sign = (u >> 31) & 1;
    int e = (u >> 23) & 0xff;
    uint32_t m = u & 0x7fffffu;
    double v;
    if (e == 0)
        v = ldexp((double)m, -149);
    else if (e == 255)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(8388608u + m), e - 150);
    return sign ? -v : v;
}

int orc_decode(int dtype, const void *src, int64_t n, double *dst)
{
    if (!src || !dst || n < 0)
        return -1;
    if (dtype == ORC_F16) {
        const uint16_t *s = (const uint16_t *)src;
        for (int64_t i = 0; i < n; ++i) dst[i] = orc_f16_to_f64(s[i]);
    } else if (dtype == ORC_BF16) {
        const uint16_t *s = (const uint16_t *)src;
        for (int64_t i = 0; i < n; ++i) dst[i] = orc_bf16_to_f64(s[i]);
    } else if (dtype == ORC_F32) {
        const uint32_t *s = (const uint32_t *)src;
        for (int64_t i = 0; i < n; ++i) dst[i] = orc_f32_to_f64(s[i]);
    } else if (dtype == ORC_I8) {
        /* two's complement: bit 7 weighs -128 */
        const uint8_t *s = (const uint8_t *)src;
        for (int64_t i = 0; i < n; ++i) dst[i] = (double)(s[i] & 0x7f) - ((s[i] & 0x80) ? 128.0 : 0.0);
    } else if (dtype == ORC_I32) {
        /* two's complement: bit 31 weighs -2^31 */
        const uint32_t *s = (const uint32_t *)src;
        for (int64_t i = 0; i < n; ++i)
            dst[i] = (double)(s[i] & 0x7fffffffu) - ((s[i] & 0x80000000u) ? 2147483648.0 : 0.0);
    } else {
        return -1;
    }
    return 0;
}

/* ---- activation -------------------------------------------------------- */

/* LeakyReLU: non-negative values pass unchanged, negative values are scaled
 * by alpha ([MLR] 概述 and the leaky_relu row of 核心接口).  ReLU keeps
 * positive values and maps the rest to +0 ([FMR] host loop).  tanh is the
 * hyperbolic tangent ([FCT] K2 chain: (e^z - e^-z) / (e^z + e^-z)); libm's
 * tanh is used because the quotient form overflows for |z| > ~709.
 * GELU and Sigmoid are the other element-wise activations of the matmul +
 * activation family ([FMR] ops-nn的融合算子分类与适用场景, first class; Sigmoid
 * is also the activation of [FCT]'s twin ConvSigmoid operator).  The pages
 * name them without a formula; the plain definitions are taken:
 * GELU(z) = z * Phi(z) with Phi the standard normal CDF, Phi(z) =
 * (1 + erf(z / sqrt 2)) / 2 = erfc(-z / sqrt 2) / 2 (the exact form, not the
 * tanh approximation; the erfc form keeps Phi's relative accuracy in the
 * negative tail, where 1 + erf cancels),
 * and Sigmoid(z) = 1 / (1 + e^-z), written for z < 0 as e^z / (1 + e^z) so
 * that e^-z never overflows. */
double orc_act(int act, double z, double alpha)
{
    switch (act) {
    case ORC_ACT_NONE:
        return z;
    case ORC_ACT_RELU:
        return z > 0.0 ? z : 0.0;
    case ORC_ACT_LEAKY:
        return z >= 0.0 ? z : alpha * z;
    case ORC_ACT_TANH:
        return tanh(z);
    case ORC_ACT_GELU:
        return z * 0.5 * erfc(-z / sqrt(2.0));
    case ORC_ACT_SIGMOID:
        if (z >= 0.0) return 1.0 / (1.0 + exp(-z));
        return exp(z) / (1.0 + exp(z));
    default:
        return NAN;
    }
}

void orc_act_array(int act, double alpha, const double *z, double *y, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) y[i] = orc_act(act, z[i], alpha);
}

static int act_ok(int act)
{
    return act >= ORC_ACT_NONE && act <= ORC_ACT_SIGMOID;
}

/* The residual joins the sum before the activation: act(A.B + bias + R). */
int orc_residual_act(const double *z, const double *r, double *y, int64_t n, int act,
                     double alpha)
{
    if (!z || !r || !y || n < 0 || !act_ok(act))
        return -1;
    for (int64_t i = 0; i < n; ++i) y[i] = orc_act(act, z[i] + r[i], alpha);
    return 0;
}

/* ---- GEMM -------------------------------------------------------------- */

int orc_gemm_bias_act(const double *A, const double *B, const double *bias,
                      double *C, int64_t M, int64_t N, int64_t K,
                      int act, double alpha)
{
    if (!A || !B || !C || M < 0 || N < 0 || K < 0 || !act_ok(act))
        return -1;
    int err = 0;
#pragma omp parallel
    {
        double *acc = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        if (!acc) {
#pragma omp atomic write
            err = -1;
        } else {
#pragma omp for schedule(static)
            for (int64_t i = 0; i < M; ++i) {
                for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    double a = A[i * K + k];
                    const double *brow = B + k * N;
                    for (int64_t j = 0; j < N; ++j) acc[j] += a * brow[j];
                }
                for (int64_t j = 0; j < N; ++j) {
                    double z = acc[j] + (bias ? bias[j] : 0.0);
                    C[i * N + j] = orc_act(act, z, alpha);
                }
            }
            free(acc);
        }
    }
    return err;
}

int orc_gemm_bias_act_elems(const double *A, const double *B, const double *bias,
                            int64_t M, int64_t N, int64_t K,
                            const int64_t *ii, const int64_t *jj, int64_t n,
                            int act, double alpha, double *out)
{
    if (!A || !B || !ii || !jj || !out || n < 0 || !act_ok(act))
        return -1;
    for (int64_t t = 0; t < n; ++t)
        if (ii[t] < 0 || ii[t] >= M || jj[t] < 0 || jj[t] >= N)
            return -1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        int64_t i = ii[t], j = jj[t];
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k) s += A[i * K + k] * B[k * N + j];
        out[t] = orc_act(act, s + (bias ? bias[j] : 0.0), alpha);
    }
    return 0;
}

int orc_gemm_bias_fold(const double *A, const double *B, const double *bias,
                       double *C, int64_t M, int64_t N, int64_t K,
                       int act, double alpha)
{
    if (!A || !B || !C || M < 0 || N < 0 || K < 0 || !act_ok(act))
        return -1;
    const int64_t K1 = K + 1;
    double *Af = (double *)malloc((size_t)(M * K1 > 0 ? M * K1 : 1) * sizeof(double));
    double *Bf = (double *)malloc((size_t)(K1 * N > 0 ? K1 * N : 1) * sizeof(double));
    if (!Af || !Bf) {
        free(Af);
        free(Bf);
        return -1;
    }
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t k = 0; k < K; ++k) Af[i * K1 + k] = A[i * K + k];
        Af[i * K1 + K] = 1.0;                       /* the all-ones column */
    }
    memcpy(Bf, B, (size_t)(K * N) * sizeof(double));
    for (int64_t j = 0; j < N; ++j) Bf[K * N + j] = bias ? bias[j] : 0.0;  /* bias row */
    int rc = orc_gemm_bias_act(Af, Bf, NULL, C, M, N, K1, act, alpha);
    free(Af);
    free(Bf);
    return rc;
}

/* ---- conv2d ------------------------------------------------------------ */

int64_t orc_conv_out_dim(int64_t in, int64_t k, int64_t stride,
                         int64_t pad_lo, int64_t pad_hi, int64_t dil)
{
    if (stride <= 0 || dil <= 0 || k <= 0)
        return 0;
    int64_t span = in + pad_lo + pad_hi - dil * (k - 1) - 1;
    if (span < 0)
        return 0;
    return span / stride + 1;
}

typedef struct {
    int64_t N, C, H, W, Co, kh, kw, sh, sw, pt, pb, pl, pr, dh, dw, Ho, Wo;
} conv_shape;

static int conv_setup(conv_shape *s, int64_t N, int64_t C, int64_t H, int64_t W,
                      int64_t Co, int64_t kh, int64_t kw, const int64_t strides[2],
                      const int64_t pads[4], const int64_t dils[2])
{
    if (!strides || !pads || !dils)
        return -1;
    s->N = N; s->C = C; s->H = H; s->W = W; s->Co = Co; s->kh = kh; s->kw = kw;
    s->sh = strides[0]; s->sw = strides[1];
    s->pt = pads[0]; s->pb = pads[1]; s->pl = pads[2]; s->pr = pads[3];
    s->dh = dils[0]; s->dw = dils[1];
    if (N < 0 || C <= 0 || H <= 0 || W <= 0 || Co <= 0 || kh <= 0 || kw <= 0 ||
        s->sh <= 0 || s->sw <= 0 || s->dh <= 0 || s->dw <= 0 ||
        s->pt < 0 || s->pb < 0 || s->pl < 0 || s->pr < 0)
        return -1;
    s->Ho = orc_conv_out_dim(H, kh, s->sh, s->pt, s->pb, s->dh);
    s->Wo = orc_conv_out_dim(W, kw, s->sw, s->pl, s->pr, s->dw);
    if (s->Ho <= 0 || s->Wo <= 0)
        return -1;
    return 0;
}

/* One output value of the direct convolution: the seven-loop definition with
 * the (n, co, oh, ow) loops fixed. */
static double conv_point(const conv_shape *s, const double *x, const double *w,
                         const double *bias, int64_t n, int64_t co,
                         int64_t oh, int64_t ow)
{
    double acc = 0.0;
    for (int64_t c = 0; c < s->C; ++c)
        for (int64_t r = 0; r < s->kh; ++r) {
            int64_t ih = oh * s->sh - s->pt + r * s->dh;
            if (ih < 0 || ih >= s->H)
                continue;                                   /* zero padding */
            for (int64_t q = 0; q < s->kw; ++q) {
                int64_t iw = ow * s->sw - s->pl + q * s->dw;
                if (iw < 0 || iw >= s->W)
                    continue;                               /* zero padding */
                acc += x[((n * s->C + c) * s->H + ih) * s->W + iw] *
                       w[((co * s->C + c) * s->kh + r) * s->kw + q];
            }
        }
    return acc + (bias ? bias[co] : 0.0);
}

int orc_conv2d_bias_act(const double *x, const double *w, const double *bias,
                        double *y, int64_t N, int64_t C, int64_t H, int64_t W,
                        int64_t Co, int64_t kh, int64_t kw,
                        const int64_t strides[2], const int64_t pads[4],
                        const int64_t dils[2], int act, double alpha)
{
    conv_shape s;
    if (!x || !w || !y || !act_ok(act) ||
        conv_setup(&s, N, C, H, W, Co, kh, kw, strides, pads, dils))
        return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t nc = 0; nc < N * Co; ++nc) {
        int64_t n = nc / Co, co = nc % Co;
        for (int64_t oh = 0; oh < s.Ho; ++oh)
            for (int64_t ow = 0; ow < s.Wo; ++ow) {
                double z = conv_point(&s, x, w, bias, n, co, oh, ow);
                y[((n * Co + co) * s.Ho + oh) * s.Wo + ow] = orc_act(act, z, alpha);
            }
    }
    return 0;
}

int orc_conv2d_bias_act_elems(const double *x, const double *w, const double *bias,
                              int64_t N, int64_t C, int64_t H, int64_t W,
                              int64_t Co, int64_t kh, int64_t kw,
                              const int64_t strides[2], const int64_t pads[4],
                              const int64_t dils[2], const int64_t *idx, int64_t n,
                              int act, double alpha, double *out)
{
    conv_shape s;
    if (!x || !w || !idx || !out || n < 0 || !act_ok(act) ||
        conv_setup(&s, N, C, H, W, Co, kh, kw, strides, pads, dils))
        return -1;
    const int64_t total = N * Co * s.Ho * s.Wo;
    for (int64_t t = 0; t < n; ++t)
        if (idx[t] < 0 || idx[t] >= total)
            return -1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        int64_t f = idx[t];
        int64_t ow = f % s.Wo; f /= s.Wo;
        int64_t oh = f % s.Ho; f /= s.Ho;
        int64_t co = f % Co;
        int64_t nn = f / Co;
        out[t] = orc_act(act, conv_point(&s, x, w, bias, nn, co, oh, ow), alpha);
    }
    return 0;
}

int orc_conv2d_im2col(const double *x, const double *w, const double *bias,
                      double *y, int64_t N, int64_t C, int64_t H, int64_t W,
                      int64_t Co, int64_t kh, int64_t kw,
                      const int64_t strides[2], const int64_t pads[4],
                      const int64_t dils[2], int act, double alpha, int fold_bias)
{
    conv_shape s;
    if (!x || !w || !y || !act_ok(act) ||
        conv_setup(&s, N, C, H, W, Co, kh, kw, strides, pads, dils))
        return -1;
    const int64_t K = C * kh * kw, P = N * s.Ho * s.Wo;
    double *cols = (double *)calloc((size_t)(K * P > 0 ? K * P : 1), sizeof(double));
    double *ym = (double *)malloc((size_t)(Co * P > 0 ? Co * P : 1) * sizeof(double));
    if (!cols || !ym) {
        free(cols);
        free(ym);
        return -1;
    }
    /* cols[k][p]: k = (c*kh + r)*kw + q, p = (n*Ho + oh)*Wo + ow; taps that
     * fall in the padding stay 0. */
    for (int64_t c = 0; c < C; ++c)
        for (int64_t r = 0; r < kh; ++r)
            for (int64_t q = 0; q < kw; ++q) {
                int64_t k = (c * kh + r) * kw + q;
                for (int64_t n = 0; n < N; ++n)
                    for (int64_t oh = 0; oh < s.Ho; ++oh)
                        for (int64_t ow = 0; ow < s.Wo; ++ow) {
                            int64_t ih = oh * s.sh - s.pt + r * s.dh;
                            int64_t iw = ow * s.sw - s.pl + q * s.dw;
                            int64_t p = (n * s.Ho + oh) * s.Wo + ow;
                            if (ih >= 0 && ih < H && iw >= 0 && iw < W)
                                cols[k * P + p] = x[((n * C + c) * H + ih) * W + iw];
                        }
            }
    /* The weight tensor [Co, C, kh, kw] is already the row-major [Co, K]
     * matrix with the same k order. */
    int rc;
    if (fold_bias) {
        /* w' = [w | bias] (Co x (K+1)), cols' = [cols ; 1...1] ((K+1) x P):
         * the bias is one more reduction index, with no separate add. */
        const int64_t K1 = K + 1;
        double *wf = (double *)malloc((size_t)(Co * K1) * sizeof(double));
        double *cf = (double *)malloc((size_t)(K1 * P > 0 ? K1 * P : 1) * sizeof(double));
        if (!wf || !cf) {
            free(wf); free(cf); free(cols); free(ym);
            return -1;
        }
        for (int64_t co = 0; co < Co; ++co) {
            for (int64_t k = 0; k < K; ++k) wf[co * K1 + k] = w[co * K + k];
            wf[co * K1 + K] = bias ? bias[co] : 0.0;
        }
        memcpy(cf, cols, (size_t)(K * P) * sizeof(double));
        for (int64_t p = 0; p < P; ++p) cf[K * P + p] = 1.0;
        rc = orc_gemm_bias_act(wf, cf, NULL, ym, Co, P, K1, act, alpha);
        free(wf);
        free(cf);
    } else {
        /* bias is per row co here: add it after the plain GEMM. */
        rc = orc_gemm_bias_act(w, cols, NULL, ym, Co, P, K, ORC_ACT_NONE, 0.0);
        if (rc == 0)
            for (int64_t co = 0; co < Co; ++co)
                for (int64_t p = 0; p < P; ++p)
                    ym[co * P + p] = orc_act(act, ym[co * P + p] + (bias ? bias[co] : 0.0), alpha);
    }
    if (rc == 0)
        for (int64_t co = 0; co < Co; ++co)
            for (int64_t n = 0; n < N; ++n)
                for (int64_t q = 0; q < s.Ho * s.Wo; ++q)
                    y[(n * Co + co) * s.Ho * s.Wo + q] = ym[co * P + n * s.Ho * s.Wo + q];
    free(cols);
    free(ym);
    return rc;
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Thread count of the following parallel loops (timing only; results do not
 * depend on it: every output is summed by one thread in index order). */
void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
