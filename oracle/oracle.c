/*
 * oracle.c -- plain, slow, fp64 CPU reference for the fused convolution hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or calls
 * this file; only the test suite, the smoke check and the benchmark's CPU-baseline
 * leg use it.  It shares no code, header, table or helper with the HIP kernels.
 *
 * Every function computes the plain definition of its operation in the order the
 * definition states, with fp64 accumulation over fp32 inputs:
 *   - conv3d / conv3d_mish_tanh: page "Kimi-K2.6 l2_p47 (Conv3d + Mish + Tanh)",
 *     the naive one-thread-per-output kernel (cross-correlation, no flip, weight
 *     layout [Cout][Cin][kD][kH][kW]) and the softplus-threshold paragraph
 *     (softplus(v) = v when v > 20, else log1p(exp(v)); mish = v*tanh(softplus);
 *     out = tanh(mish)).  Padding/stride generalisation from the same page's
 *     stride/padding paragraph: in = out*s - p + k, reads outside are zero.
 *   - conv3d_div_maxpool_gap_bias_sum: page "Kimi-K2.6 l2_p8 (Conv3d, divide,
 *     MaxPool3d, AdaptiveAvgPool3d, bias, sum)", the opening shape walk-through:
 *     conv (+conv bias) -> /divisor -> max over non-overlapping pool^3 windows
 *     (floor mode) -> mean over the pooled volume -> + bias[c] -> sum over c.
 *   - dwsep_conv2d: page "Kimi-K2.6 l1_p86 (depthwise-separable Conv2d)", the
 *     fused-definition pseudocode: depthwise KxK per channel (stride, padding,
 *     dilation, zero padding) then pointwise 1x1 over channels, each with an
 *     optional bias.
 *
 * OpenMP is used only across independent output elements; each element's sum is
 * taken in the definitional loop order.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Output length of one spatial dimension: floor((in + 2p - d(k-1) - 1)/s) + 1.
 * Page l1_p86, output-size formula; for d = 1 it is the l2_p47 form (in+2p-k)/s+1.
 * Returns 0 when the kernel does not fit. */
static int64_t or_out_len(int64_t in, int64_t k, int64_t s, int64_t p, int64_t d)
{
    int64_t span = in + 2 * p - d * (k - 1) - 1;
    if (span < 0 || s <= 0) return 0;
    return span / s + 1;
}

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

int64_t oracle_out_len(int64_t in, int64_t k, int64_t s, int64_t p, int64_t d)
{
    return or_out_len(in, k, s, p, d);
}

/* One pre-activation output of a cubic-kernel Conv3d: bias + sum over c, kd, kh, kw
 * of w[o,c,kd,kh,kw] * x[n,c,od*s-p+kd, oh*s-p+kh, ow*s-p+kw]. */
static double or_conv3d_point(const float *x, const float *w, const float *b,
                              int64_t C, int64_t D, int64_t H, int64_t W, int64_t k,
                              int64_t s, int64_t p, int64_t n, int64_t o,
                              int64_t od, int64_t oh, int64_t ow)
{
    double acc = b ? (double)b[o] : 0.0;
    for (int64_t c = 0; c < C; ++c)
        for (int64_t kd = 0; kd < k; ++kd) {
            int64_t id = od * s - p + kd;
            if (id < 0 || id >= D) continue;
            for (int64_t kh = 0; kh < k; ++kh) {
                int64_t ih = oh * s - p + kh;
                if (ih < 0 || ih >= H) continue;
                for (int64_t kw = 0; kw < k; ++kw) {
                    int64_t iw = ow * s - p + kw;
                    if (iw < 0 || iw >= W) continue;
                    double wv = w[(((o * C + c) * k + kd) * k + kh) * k + kw];
                    double xv = x[(((n * C + c) * D + id) * H + ih) * W + iw];
                    acc += wv * xv;
                }
            }
        }
    return acc;
}

/* Full Conv3d (+ optional bias) into y [N,O,OD,OH,OW] as fp64. */
int oracle_conv3d(const float *x, const float *w, const float *b, double *y,
                  int64_t N, int64_t C, int64_t D, int64_t H, int64_t W,
                  int64_t O, int64_t k, int64_t s, int64_t p)
{
    if (!x || !w || !y || N < 0 || C <= 0 || O <= 0 || k <= 0) return -1;
    int64_t OD = or_out_len(D, k, s, p, 1), OH = or_out_len(H, k, s, p, 1),
            OW = or_out_len(W, k, s, p, 1);
    if (OD <= 0 || OH <= 0 || OW <= 0) return -2;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t o = 0; o < O; ++o) {
            double *yo = y + (n * O + o) * OD * OH * OW;
            for (int64_t od = 0; od < OD; ++od)
                for (int64_t oh = 0; oh < OH; ++oh)
                    for (int64_t ow = 0; ow < OW; ++ow)
                        yo[(od * OH + oh) * OW + ow] =
                            or_conv3d_point(x, w, b, C, D, H, W, k, s, p, n, o, od, oh, ow);
        }
    return 0;
}

/* softplus with PyTorch's default beta = 1, threshold = 20 (page l2_p47,
 * softplus-threshold paragraph), then mish, then tanh. */
static double or_mish_tanh(double v)
{
    double sp = v > 20.0 ? v : log1p(exp(v));
    double m = v * tanh(sp);
    return tanh(m);
}

int oracle_mish_tanh(const double *v, double *out, int64_t count)
{
    if (count < 0 || (count > 0 && (!v || !out))) return -1;
    for (int64_t i = 0; i < count; ++i) out[i] = or_mish_tanh(v[i]);
    return 0;
}

/* y = tanh(mish(conv3d(x) + b)), all of y. */
int oracle_conv3d_mish_tanh(const float *x, const float *w, const float *b, double *y,
                            int64_t N, int64_t C, int64_t D, int64_t H, int64_t W,
                            int64_t O, int64_t k, int64_t s, int64_t p)
{
    int rc = oracle_conv3d(x, w, b, y, N, C, D, H, W, O, k, s, p);
    if (rc) return rc;
    int64_t total = N * O * or_out_len(D, k, s, p, 1) * or_out_len(H, k, s, p, 1) *
                    or_out_len(W, k, s, p, 1);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < total; ++i) y[i] = or_mish_tanh(y[i]);
    return 0;
}

/* The same, only at the flat output indices idx[0..count) of y [N,O,OD,OH,OW]. */
int oracle_conv3d_mish_tanh_at(const float *x, const float *w, const float *b,
                               const int64_t *idx, int64_t count, double *out,
                               int64_t N, int64_t C, int64_t D, int64_t H, int64_t W,
                               int64_t O, int64_t k, int64_t s, int64_t p)
{
    if (!x || !w || (count > 0 && (!idx || !out))) return -1;
    int64_t OD = or_out_len(D, k, s, p, 1), OH = or_out_len(H, k, s, p, 1),
            OW = or_out_len(W, k, s, p, 1);
    if (OD <= 0 || OH <= 0 || OW <= 0) return -2;
    int64_t total = N * O * OD * OH * OW;
    for (int64_t i = 0; i < count; ++i)
        if (idx[i] < 0 || idx[i] >= total) return -3;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < count; ++i) {
        int64_t r = idx[i];
        int64_t ow = r % OW; r /= OW;
        int64_t oh = r % OH; r /= OH;
        int64_t od = r % OD; r /= OD;
        int64_t o = r % O;   r /= O;
        int64_t n = r;
        out[i] = or_mish_tanh(or_conv3d_point(x, w, b, C, D, H, W, k, s, p, n, o, od, oh, ow));
    }
    return 0;
}

/* out[n] = sum_c ( mean_{pooled}( maxpool_{pool, stride pool, floor}( (conv3d(x)+cb)/divisor ) )
 *                  + bias[c] ),  valid conv (stride 1, no padding), in exactly that order.
 * Page l2_p8, opening shape walk-through.  out has N entries (the [N,1,1,1] result). */
int oracle_conv3d_div_maxpool_gap_bias_sum(const float *x, const float *w, const float *cb,
                                           double divisor, int64_t pool, const float *bias,
                                           double *out, int64_t N, int64_t C, int64_t D,
                                           int64_t H, int64_t W, int64_t O, int64_t k)
{
    if (!x || !w || !bias || !out || N < 0 || C <= 0 || O <= 0 || k <= 0 || pool <= 0)
        return -1;
    if (divisor == 0.0) return -1;
    int64_t OD = or_out_len(D, k, 1, 0, 1), OH = or_out_len(H, k, 1, 0, 1),
            OW = or_out_len(W, k, 1, 0, 1);
    if (OD <= 0 || OH <= 0 || OW <= 0) return -2;
    int64_t PD = or_out_len(OD, pool, pool, 0, 1), PH = or_out_len(OH, pool, pool, 0, 1),
            PW = or_out_len(OW, pool, pool, 0, 1);
    if (PD <= 0 || PH <= 0 || PW <= 0) return -2;
    double count = (double)(PD * PH * PW);

    /* g[n][o] = mean of the pooled maxima + bias[o], one independent (n, o) pair per
     * task; the channel sum is then taken in order c = 0..O-1. */
    double *g = (double *)malloc((size_t)(N * O > 0 ? N * O : 1) * sizeof(double));
    if (!g) return -4;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t o = 0; o < O; ++o) {
            double ssum = 0.0;
            for (int64_t pd = 0; pd < PD; ++pd)
                for (int64_t ph = 0; ph < PH; ++ph)
                    for (int64_t pw = 0; pw < PW; ++pw) {
                        double m = 0.0;
                        int first = 1;
                        for (int64_t a = 0; a < pool; ++a)
                            for (int64_t bb = 0; bb < pool; ++bb)
                                for (int64_t cc = 0; cc < pool; ++cc) {
                                    double v = or_conv3d_point(x, w, cb, C, D, H, W, k, 1, 0, n, o,
                                                               pd * pool + a, ph * pool + bb,
                                                               pw * pool + cc);
                                    v = v / divisor;
                                    if (first || v > m) m = v;
                                    first = 0;
                                }
                        ssum += m;
                    }
            g[n * O + o] = ssum / count + (double)bias[o];
        }
    for (int64_t n = 0; n < N; ++n) {
        double total = 0.0;
        for (int64_t o = 0; o < O; ++o) total += g[n * O + o];
        out[n] = total;
    }
    free(g);
    return 0;
}

/* y[n,o,pd,ph,pw] = max over the pool^3 window (stride pool, floor mode) of
 * (conv3d(x)+cb)/divisor, valid conv (stride 1, no padding): the pooled tensor before the
 * global mean (page l2_p8, the "Option A" output of the fused conv + divide + max-pool).
 * y has N*O*PD*PH*PW entries. */
int oracle_conv3d_div_maxpool(const float *x, const float *w, const float *cb, double divisor,
                              int64_t pool, double *y, int64_t N, int64_t C, int64_t D,
                              int64_t H, int64_t W, int64_t O, int64_t k)
{
    if (!x || !w || !y || N < 0 || C <= 0 || O <= 0 || k <= 0 || pool <= 0) return -1;
    if (divisor == 0.0) return -1;
    int64_t OD = or_out_len(D, k, 1, 0, 1), OH = or_out_len(H, k, 1, 0, 1),
            OW = or_out_len(W, k, 1, 0, 1);
    if (OD <= 0 || OH <= 0 || OW <= 0) return -2;
    int64_t PD = or_out_len(OD, pool, pool, 0, 1), PH = or_out_len(OH, pool, pool, 0, 1),
            PW = or_out_len(OW, pool, pool, 0, 1);
    if (PD <= 0 || PH <= 0 || PW <= 0) return -2;
    int64_t total = N * O * PD * PH * PW;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < total; ++i) {
        int64_t t = i;
        int64_t pw = t % PW; t /= PW;
        int64_t ph = t % PH; t /= PH;
        int64_t pd = t % PD; t /= PD;
        int64_t o = t % O, n = t / O;
        double m = 0.0;
        int first = 1;
        for (int64_t a = 0; a < pool; ++a)
            for (int64_t bb = 0; bb < pool; ++bb)
                for (int64_t cc = 0; cc < pool; ++cc) {
                    double v = or_conv3d_point(x, w, cb, C, D, H, W, k, 1, 0, n, o,
                                               pd * pool + a, ph * pool + bb, pw * pool + cc);
                    v = v / divisor;
                    if (first || v > m) m = v;
                    first = 0;
                }
        y[i] = m;
    }
    return 0;
}

/* One depthwise output: bd[c] + sum_{kh,kw} wd[c,0,kh,kw] * x[n,c,h*s-p+kh*d, w*s-p+kw*d]. */
static double or_depthwise_point(const float *x, const float *wd, const float *bd,
                                 int64_t C, int64_t H, int64_t W, int64_t K, int64_t s,
                                 int64_t p, int64_t dil, int64_t n, int64_t c, int64_t h,
                                 int64_t ww)
{
    double acc = bd ? (double)bd[c] : 0.0;
    for (int64_t kh = 0; kh < K; ++kh) {
        int64_t ih = h * s - p + kh * dil;
        if (ih < 0 || ih >= H) continue;
        for (int64_t kw = 0; kw < K; ++kw) {
            int64_t iw = ww * s - p + kw * dil;
            if (iw < 0 || iw >= W) continue;
            acc += (double)wd[(c * K + kh) * K + kw] * (double)x[((n * C + c) * H + ih) * W + iw];
        }
    }
    return acc;
}

/* y[n,o,h,w] = bp[o] + sum_c wp[o,c] * dw[n,c,h,w]; dw held in fp64 (the intermediate
 * never leaves fp64).  Full output; the depthwise intermediate is built first. */
int oracle_dwsep_conv2d(const float *x, const float *wd, const float *bd, const float *wp,
                        const float *bp, double *y, double *dw_scratch, int64_t N, int64_t C,
                        int64_t H, int64_t W, int64_t O, int64_t K, int64_t s, int64_t p,
                        int64_t dil)
{
    if (!x || !wd || !wp || !y || !dw_scratch || N < 0 || C <= 0 || O <= 0 || K <= 0)
        return -1;
    int64_t Ho = or_out_len(H, K, s, p, dil), Wo = or_out_len(W, K, s, p, dil);
    if (Ho <= 0 || Wo <= 0) return -2;
    int64_t plane = Ho * Wo;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t c = 0; c < C; ++c)
            for (int64_t h = 0; h < Ho; ++h)
                for (int64_t ww = 0; ww < Wo; ++ww)
                    dw_scratch[(n * C + c) * plane + h * Wo + ww] =
                        or_depthwise_point(x, wd, bd, C, H, W, K, s, p, dil, n, c, h, ww);
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t o = 0; o < O; ++o)
            for (int64_t q = 0; q < plane; ++q) {
                double acc = bp ? (double)bp[o] : 0.0;
                for (int64_t c = 0; c < C; ++c)
                    acc += (double)wp[o * C + c] * dw_scratch[(n * C + c) * plane + q];
                y[(n * O + o) * plane + q] = acc;
            }
    return 0;
}

/* The same at flat output indices idx[0..count) of y [N,O,Ho,Wo]; each sample recomputes
 * the depthwise values it needs. */
int oracle_dwsep_conv2d_at(const float *x, const float *wd, const float *bd, const float *wp,
                           const float *bp, const int64_t *idx, int64_t count, double *out,
                           int64_t N, int64_t C, int64_t H, int64_t W, int64_t O, int64_t K,
                           int64_t s, int64_t p, int64_t dil)
{
    if (!x || !wd || !wp || (count > 0 && (!idx || !out))) return -1;
    int64_t Ho = or_out_len(H, K, s, p, dil), Wo = or_out_len(W, K, s, p, dil);
    if (Ho <= 0 || Wo <= 0) return -2;
    int64_t total = N * O * Ho * Wo;
    for (int64_t i = 0; i < count; ++i)
        if (idx[i] < 0 || idx[i] >= total) return -3;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < count; ++i) {
        int64_t r = idx[i];
        int64_t ww = r % Wo; r /= Wo;
        int64_t h = r % Ho;  r /= Ho;
        int64_t o = r % O;   r /= O;
        int64_t n = r;
        double acc = bp ? (double)bp[o] : 0.0;
        for (int64_t c = 0; c < C; ++c)
            acc += (double)wp[o * C + c] *
                   or_depthwise_point(x, wd, bd, C, H, W, K, s, p, dil, n, c, h, ww);
        out[i] = acc;
    }
    return 0;
}
