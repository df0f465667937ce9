/*
 * oracle.c -- plain, slow, CPU reference for the fused operator chains.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * includes this file; only the test suite, the smoke check and the bench's
 * CPU-baseline leg load it.  It shares no code, header or table with the HIP
 * path.
 *
 * What it computes (the method, restated):
 *   - BOLT persistent kernel fusion ("BOLT" reading notes, section "Persistent
 *     kernel (GEMM/Conv) fusion", threadblock residence) fuses two GEMMs
 *     D1 = act(A*W0 + b0)*W1 + b1 into one kernel.  Fusion only changes where
 *     the intermediate lives, never the mathematics, so this oracle evaluates
 *     the plain UNFUSED composition.
 *   - Welder's tile graph ("Welder" reading notes, sections "Operator-tile and
 *     Tile-graph" and "Tile-graph Scheduling", Figure 5) chains Conv -> ReLU ->
 *     MaxPool; again the oracle is the unfused composition.
 *   - Epilogue operations (BOLT notes, "Prerequisite: Epilogue fusion"):
 *     element-wise activation, fp16 conversion, broadcast bias along rows,
 *     partial reduction (max-pool).
 *   - 1x1 convolution is a GEMM (interview page, "Conv optimisation", item 5).
 *
 * Arithmetic: every fp16 input is decoded exactly to fp64; products of two
 * fp16 values are exact in fp64; sums run sequentially in the stated index
 * order; the bias is added after the sum; the activation is applied in fp64;
 * the intermediate is rounded ONCE to fp16 (round-to-nearest-even) where the
 * fused GPU chain rounds it.  The fp16 codec below is written from the IEEE
 * 754 binary16 definition (1 sign, 5 exponent bits with bias 15, 10 fraction
 * bits, subnormals with quantum 2^-24).
 *
 * Parallelism: OpenMP over independent output rows only; each output element
 * is summed in a fixed order, so results do not depend on the thread count.
 *
 * GELU: the tanh form 0.5*s*(1 + tanh(sqrt(2/pi)*(s + 0.044715*s^3))) from
 * Hendrycks & Gimpel, "Gaussian Error Linear Units" (the pages never define
 * GELU; the workload names its tanh form).
 * Hardswish: s * min(max(s + 3, 0), 6) / 6, as defined in Howard et al.,
 * "Searching for MobileNetV3" (BOLT notes, "Enabling deeper operator
 * fusion", name Conv2D + BiasAdd + Hardswish as the fused epilogue but do not
 * define it).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_ACT_NONE 0
#define ORC_ACT_RELU 1
#define ORC_ACT_GELU_TANH 2
#define ORC_ACT_HARDSWISH 3

/* ------------------------------------------------------------------ */
/* fp16 codec (IEEE 754 binary16)                                      */
/* ------------------------------------------------------------------ */

double orc_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);                 /* subnormal: f * 2^-24 */
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + f), e - 25);     /* (1.f) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* Round an fp64 value to the nearest binary16 value, ties to even. */
uint16_t orc_f64_to_f16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v)) return (uint16_t)(sign | 0x7e00);
    /* 65520 = 65504 + half an ulp: it and anything above round to infinity */
    if (a >= 65520.0) return (uint16_t)(sign | 0x7c00);
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: representable values are integer multiples of
         * 2^-24; the scaling below is exact, nearbyint rounds ties to even
         * in the default rounding mode.  A result of 1024 is the smallest
         * normal number, whose bit pattern is also 1024 (0x0400). */
        double q = nearbyint(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)q);
    }
    int e2;
    frexp(a, &e2);               /* a = m * 2^e2, m in [0.5, 1) */
    int E = e2 - 1;              /* a in [2^E, 2^(E+1)), E in [-14, 15] */
    double q = nearbyint(ldexp(a, 10 - E));   /* in [1024, 2048] */
    if (q >= 2048.0) { q = 1024.0; E += 1; }
    if (E > 15) return (uint16_t)(sign | 0x7c00);
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)((int)q - 1024));
}

void orc_f16_to_f64_array(const uint16_t *h, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_to_f64(h[i]);
}

void orc_f64_to_f16_array(const double *v, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f64_to_f16(v[i]);
}

/* ------------------------------------------------------------------ */
/* activations                                                         */
/* ------------------------------------------------------------------ */

double orc_act(int act, double s)
{
    if (act == ORC_ACT_RELU) return s > 0.0 ? s : 0.0;
    if (act == ORC_ACT_GELU_TANH) {
        double c = sqrt(2.0 / M_PI);
        return 0.5 * s * (1.0 + tanh(c * (s + 0.044715 * s * s * s)));
    }
    if (act == ORC_ACT_HARDSWISH) {
        double r6 = s + 3.0;
        r6 = r6 < 0.0 ? 0.0 : (r6 > 6.0 ? 6.0 : r6);
        return s * r6 / 6.0;
    }
    return s;
}

void orc_act_array(int act, const double *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_act(act, in[i]);
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

static double *decode_all(const uint16_t *h, int64_t n)
{
    double *d = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    orc_f16_to_f64_array(h, d, n);
    return d;
}

/* ------------------------------------------------------------------ */
/* GEMM + bias + activation                                            */
/*   Y[m,n] = act( sum_{k=0}^{K-1} X[m,k]*W[k,n]  + b[n] )              */
/* X [M,K], W [K,N] row-major fp16 bit patterns; b [N] fp16 (nullable = 0) */
/* Y [M,N] fp64, unrounded.                                             */
/* ------------------------------------------------------------------ */

void orc_gemm_bias_act(const uint16_t *X, const uint16_t *W, const uint16_t *b, int act,
                       int64_t M, int64_t K, int64_t N, double *Y)
{
    double *Wd = decode_all(W, K * N);
    double *bd = (double *)calloc((size_t)(N > 0 ? N : 1), sizeof(double));
    if (b) orc_f16_to_f64_array(b, bd, N);
#pragma omp parallel
    {
        double *acc = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
#pragma omp for schedule(static)
        for (int64_t m = 0; m < M; ++m) {
            for (int64_t n = 0; n < N; ++n) acc[n] = 0.0;
            /* for every (m,n) the sum runs over k = 0, 1, ..., K-1 in order */
            for (int64_t k = 0; k < K; ++k) {
                double xv = orc_f16_to_f64(X[m * K + k]);
                const double *wr = Wd + k * N;
                for (int64_t n = 0; n < N; ++n) acc[n] += xv * wr[n];
            }
            for (int64_t n = 0; n < N; ++n) Y[m * N + n] = orc_act(act, acc[n] + bd[n]);
        }
        free(acc);
    }
    free(Wd);
    free(bd);
}

/* ------------------------------------------------------------------ */
/* Direct convolution (deep-learning cross-correlation, no kernel flip), */
/* zero padding, NHWC input, HWIO weights, + bias, + activation.        */
/*   P = floor((H + 2*pad - R)/stride) + 1, Q likewise                   */
/*   y[n,p,q,k] = act( sum_{r,s,c} x[n, p*st+r-pad, q*st+s-pad, c] *     */
/*                                  w[r,s,c,k]   + b[k] )               */
/* sum order: r, then s, then c (c fastest); out-of-range x is zero.    */
/* ------------------------------------------------------------------ */

void orc_conv_bias_act(const uint16_t *x, const uint16_t *w, const uint16_t *b, int act,
                       int64_t NB, int64_t H, int64_t Wd_, int64_t C, int64_t K,
                       int64_t R, int64_t S, int64_t stride, int64_t pad, double *y)
{
    int64_t P = (H + 2 * pad - R) / stride + 1;
    int64_t Q = (Wd_ + 2 * pad - S) / stride + 1;
    double *wd = decode_all(w, R * S * C * K);
    double *bd = (double *)calloc((size_t)(K > 0 ? K : 1), sizeof(double));
    if (b) orc_f16_to_f64_array(b, bd, K);
#pragma omp parallel
    {
        double *acc = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
#pragma omp for schedule(static) collapse(2)
        for (int64_t n = 0; n < NB; ++n)
            for (int64_t p = 0; p < P; ++p)
                for (int64_t q = 0; q < Q; ++q) {
                    for (int64_t k = 0; k < K; ++k) acc[k] = 0.0;
                    for (int64_t r = 0; r < R; ++r) {
                        int64_t ih = p * stride + r - pad;
                        if (ih < 0 || ih >= H) continue;      /* zero row */
                        for (int64_t s = 0; s < S; ++s) {
                            int64_t iw = q * stride + s - pad;
                            if (iw < 0 || iw >= Wd_) continue; /* zero column */
                            const uint16_t *xp = x + ((n * H + ih) * Wd_ + iw) * C;
                            const double *wp = wd + (r * S + s) * C * K;
                            for (int64_t c = 0; c < C; ++c) {
                                double xv = orc_f16_to_f64(xp[c]);
                                const double *wr = wp + c * K;
                                for (int64_t k = 0; k < K; ++k) acc[k] += xv * wr[k];
                            }
                        }
                    }
                    double *yo = y + ((n * P + p) * Q + q) * K;
                    for (int64_t k = 0; k < K; ++k) yo[k] = orc_act(act, acc[k] + bd[k]);
                }
        free(acc);
    }
    free(wd);
    free(bd);
}

/* ------------------------------------------------------------------ */
/* 2x2 stride-2 max pool over fp16 values v [n,P,Q,K].                  */
/*   y[n,i,j,k] = max_{dy,dx in {0,1}} v[n,2i+dy,2j+dx,k]                */
/* output size floor(P/2) x floor(Q/2); argmax = 2*dy+dx of the FIRST    */
/* maximal element in the order (0,0),(0,1),(1,0),(1,1).  argmax may be  */
/* NULL.                                                                */
/* ------------------------------------------------------------------ */

void orc_maxpool2x2(const uint16_t *v, int64_t NB, int64_t P, int64_t Q, int64_t K,
                    uint16_t *y, uint8_t *argmax)
{
    int64_t PO = P / 2, QO = Q / 2;
#pragma omp parallel for schedule(static) collapse(2)
    for (int64_t n = 0; n < NB; ++n)
        for (int64_t i = 0; i < PO; ++i)
            for (int64_t j = 0; j < QO; ++j)
                for (int64_t k = 0; k < K; ++k) {
                    int best = 0;
                    uint16_t bh = 0;
                    double bv = 0.0;
                    for (int e = 0; e < 4; ++e) {
                        int dy = e >> 1, dx = e & 1;
                        uint16_t h = v[((n * P + 2 * i + dy) * Q + 2 * j + dx) * K + k];
                        double val = orc_f16_to_f64(h);
                        if (e == 0 || val > bv) { bv = val; bh = h; best = e; }
                    }
                    int64_t o = ((n * PO + i) * QO + j) * K + k;
                    y[o] = bh;
                    if (argmax) argmax[o] = (uint8_t)best;
                }
}

/* ------------------------------------------------------------------ */
/* Chains: the unfused compositions.                                    */
/* ------------------------------------------------------------------ */

/* D1 = act(A*W0 + b0) * W1 + b1.  H (fp16 [M,N0]) = the rounded          */
/* intermediate; ref (fp64 [M,N1]) = the unrounded final value.           */
void orc_chain_gemm2(const uint16_t *A, const uint16_t *W0, const uint16_t *b0, int act,
                     const uint16_t *W1, const uint16_t *b1,
                     int64_t M, int64_t K0, int64_t N0, int64_t N1,
                     uint16_t *H, double *ref)
{
    double *h64 = (double *)malloc(sizeof(double) * (size_t)(M * N0 > 0 ? M * N0 : 1));
    orc_gemm_bias_act(A, W0, b0, act, M, K0, N0, h64);
    orc_f64_to_f16_array(h64, H, M * N0);
    free(h64);
    orc_gemm_bias_act(H, W1, b1, ORC_ACT_NONE, M, N0, N1, ref);
}

/* conv RxS (stride, pad) + b0 + act -> fp16 H -> 1x1 conv (= GEMM over    */
/* the N*P*Q pixels) + b1.  H [n,P,Q,K0] fp16, ref [n,P,Q,K1] fp64.        */
void orc_chain_conv2(const uint16_t *x, const uint16_t *w0, const uint16_t *b0, int act,
                     const uint16_t *w1, const uint16_t *b1,
                     int64_t NB, int64_t Hh, int64_t Ww, int64_t C, int64_t K0,
                     int64_t R, int64_t S, int64_t stride, int64_t pad, int64_t K1,
                     uint16_t *H, double *ref)
{
    int64_t P = (Hh + 2 * pad - R) / stride + 1;
    int64_t Q = (Ww + 2 * pad - S) / stride + 1;
    int64_t npix = NB * P * Q;
    double *h64 = (double *)malloc(sizeof(double) * (size_t)(npix * K0 > 0 ? npix * K0 : 1));
    orc_conv_bias_act(x, w0, b0, act, NB, Hh, Ww, C, K0, R, S, stride, pad, h64);
    orc_f64_to_f16_array(h64, H, npix * K0);
    free(h64);
    orc_gemm_bias_act(H, w1, b1, ORC_ACT_NONE, npix, K0, K1, ref);
}

/* conv + b + act -> fp16 v -> maxpool 2x2/2 (+argmax).  conv64 (nullable) */
/* receives the unrounded post-activation conv values for tie analysis.    */
void orc_chain_conv_pool(const uint16_t *x, const uint16_t *w, const uint16_t *b, int act,
                         int64_t NB, int64_t Hh, int64_t Ww, int64_t C, int64_t K,
                         int64_t R, int64_t S, int64_t stride, int64_t pad,
                         uint16_t *v, double *conv64, uint16_t *y, uint8_t *argmax)
{
    int64_t P = (Hh + 2 * pad - R) / stride + 1;
    int64_t Q = (Ww + 2 * pad - S) / stride + 1;
    int64_t nv = NB * P * Q * K;
    double *c64 = conv64 ? conv64 : (double *)malloc(sizeof(double) * (size_t)(nv > 0 ? nv : 1));
    orc_conv_bias_act(x, w, b, act, NB, Hh, Ww, C, K, R, S, stride, pad, c64);
    orc_f64_to_f16_array(c64, v, nv);
    if (!conv64) free(c64);
    orc_maxpool2x2(v, NB, P, Q, K, y, argmax);
}
