/*
 * convfuse.h -- C ABI of the fused fp32 convolution library (libconvfuse.so, gfx950).
 *
 * Three entry points, each one fused GPU pass whose intermediate tensors never reach
 * HBM:
 *   conv3d_mish_tanh                 y = tanh(mish(conv3d(x) + b))
 *   conv3d_div_maxpool_gap_bias_sum  out[n] = sum_c(mean(maxpool(conv3d(x)/divisor)) + bias[c])
 *   dwsep_conv2d                     y = pointwise1x1(depthwise(x))
 *
 * Conventions shared by every entry point
 *   - Tensors are contiguous fp32 in PyTorch's layouts: activations NCDHW / NCHW,
 *     Conv3d weights [Cout][Cin][k][k][k], depthwise weights [Cin][1][K][K],
 *     pointwise weights [Cout][Cin][1][1].  All tensor pointers are DEVICE pointers
 *     on the current HIP device.
 *   - Convolutions are cross-correlations (no kernel flip) with zero padding.
 *   - The caller owns every buffer, outputs included; no call allocates memory.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the default
 *     stream).  Inputs must stay valid and unmodified until the stream reaches the call.
 *     Calls that share no output buffer may run concurrently on different streams.
 *   - Return value: CONVFUSE_OK, or an error code.  Arguments are validated before
 *     anything is launched, so a non-OK return from validation has no side effects.
 *     convfuse_last_error() returns a message for the calling thread's last failure.
 *   - Output sizes follow floor((in + 2*pad - dilation*(k-1) - 1)/stride) + 1
 *     (convfuse_conv_out_len; whole shapes: convfuse_out_dims_conv3d / _conv2d).
 *   - Outputs are written only where they exist; ragged tiles never write past them.
 */
#ifndef CONVFUSE_H
#define CONVFUSE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    CONVFUSE_OK = 0,
    CONVFUSE_ERR_NULL = 1,        /* a required pointer is NULL */
    CONVFUSE_ERR_SHAPE = 2,       /* a size is non-positive, too large, or the output is empty */
    CONVFUSE_ERR_UNSUPPORTED = 3, /* valid convolution parameters the GPU path does not implement */
    CONVFUSE_ERR_DEVICE = 4       /* a HIP call or kernel launch failed */
};

/*
 * y = tanh(mish(conv3d(x, w) + b)),  mish(v) = v * tanh(softplus(v)).
 * Page "Kimi-K2.6 l2_p47" (Conv3d + Mish + Tanh): problem statement and the
 * softplus-threshold paragraph (softplus(v) = v for v > 20).
 *
 *   x  [N][Cin][D][H][W]            device, read-only
 *   w  [Cout][Cin][k][k][k]         device, read-only
 *   b  [Cout] or NULL (no bias)     device, read-only
 *   y  [N][Cout][OD][OH][OW]        device, written; OD = (D + 2*pad - k)/stride + 1, etc.
 * Any k, stride >= 1 and pad >= 0 that give a non-empty output, any N, Cin, Cout >= 1
 * (page l2_p47's generalised stride/padding).  k = 3, stride = 1, pad <= 2 run the tuned
 * kernel; other values a general kernel.  k^3 above 2^30 returns CONVFUSE_ERR_UNSUPPORTED.
 * Accumulation is fp32 on fp32 matrix cores; the epilogue runs in registers.
 */
int conv3d_mish_tanh(const float *x, const float *w, const float *b, float *y,
                     int64_t N, int64_t Cin, int64_t D, int64_t H, int64_t W,
                     int64_t Cout, int64_t k, int64_t stride, int64_t pad, void *stream);

/*
 * out[n] = sum_c ( mean_{pd,ph,pw} maxpool_pool( (conv3d(x, w) + conv_b) / divisor )[n,c]
 *                  + bias[c] )
 * with a valid (stride 1, no padding) conv and a pool^3 max-pool of stride pool, floor
 * mode.  Page "Kimi-K2.6 l2_p8" (Conv3d, /2, MaxPool3d, AdaptiveAvgPool3d, +bias, sum over
 * channels): the opening shape walk-through and the rewrite as a sum of channel means
 * plus the bias sum.
 *
 *   x       [N][Cin][D][H][W]       device, read-only
 *   w       [Cout][Cin][k][k][k]    device, read-only
 *   conv_b  [Cout] or NULL          device, read-only
 *   divisor finite and non-zero (negative divisors turn the max into a min of the conv)
 *   bias    [Cout] (the [Cout,1,1,1] tensor)  device, read-only
 *   out     [N] (the [N,1,1,1] result)        device, written; the call initialises it,
 *           so the caller need not clear it.
 * The whole reduction happens on the device; nothing is synchronised with the host.  The
 * channel/window partial sums meet through float atomics, so the last bits of out[n]
 * may differ from run to run.
 * Any k; pool from 1 to 32 (k = 3, pool = 2 run the tuned kernel).  pool > 32 or k^3 above
 * 2^30 return CONVFUSE_ERR_UNSUPPORTED.
 */
int conv3d_div_maxpool_gap_bias_sum(const float *x, const float *w, const float *conv_b,
                                    float divisor, int64_t pool, const float *bias, float *out,
                                    int64_t N, int64_t Cin, int64_t D, int64_t H, int64_t W,
                                    int64_t Cout, int64_t k, void *stream);

/*
 * y = maxpool_pool( (conv3d(x, w) + conv_b) / divisor ): the pooled tensor of the fused
 * conv + divide + max-pool, before the global mean (page "Kimi-K2.6 l2_p8", the option
 * that writes the [N,C,7,31,31] pooled output for callers that need it).  Valid conv
 * (stride 1, no padding), pool^3 windows of stride pool, floor mode.
 *
 *   x       [N][Cin][D][H][W]       device, read-only
 *   w       [Cout][Cin][k][k][k]    device, read-only
 *   conv_b  [Cout] or NULL          device, read-only
 *   divisor finite and non-zero
 *   y       [N][Cout][PD][PH][PW]   device, written; PD = (D - k + 1 - pool)/pool + 1, etc.
 * The conv output never reaches memory.  Any k; pool from 1 to 32 (k = 3, pool = 2 run the
 * tuned kernel); pool > 32 or k^3 above 2^30 return CONVFUSE_ERR_UNSUPPORTED.
 */
int conv3d_div_maxpool(const float *x, const float *w, const float *conv_b, float divisor,
                       int64_t pool, float *y, int64_t N, int64_t Cin, int64_t D, int64_t H,
                       int64_t W, int64_t Cout, int64_t k, void *stream);

/*
 * y = pointwise(depthwise(x)):
 *   dw[n,c,h,w] = dw_b[c] + sum_{kh,kw} dw_w[c,0,kh,kw] * x[n,c,h*s-p+kh*d, w*s-p+kw*d]
 *   y[n,o,h,w]  = pw_b[o] + sum_c pw_w[o,c,0,0] * dw[n,c,h,w]
 * Page "Kimi-K2.6 l1_p86" (depthwise-separable Conv2d): the fused-definition pseudocode.
 *
 *   x     [N][Cin][H][W]       device, read-only
 *   dw_w  [Cin][1][K][K]       device, read-only
 *   dw_b  [Cin] or NULL        device, read-only
 *   pw_w  [Cout][Cin][1][1]    device, read-only
 *   pw_b  [Cout] or NULL       device, read-only
 *   y     [N][Cout][Ho][Wo]    device, written; Ho = (H + 2p - d(K-1) - 1)/s + 1
 * The depthwise result stays on chip; only y is written.
 * Any K, stride, pad, dilation that give a non-empty output (page l1_p86's generalised
 * kernel).  K = 3, stride = 1, dilation = 1, pad <= 2 run the tuned kernels; other values a
 * general kernel.  K^2 above 2^30 returns CONVFUSE_ERR_UNSUPPORTED.
 */
int dwsep_conv2d(const float *x, const float *dw_w, const float *dw_b, const float *pw_w,
                 const float *pw_b, float *y, int64_t N, int64_t Cin, int64_t H, int64_t W,
                 int64_t Cout, int64_t K, int64_t stride, int64_t pad, int64_t dilation,
                 void *stream);

/*
 * conv3d_mish_tanh with the implicit GEMM on bf16 matrix cores (opt-in precision mode, the
 * same three-term split of fp32 as dwsep_conv2d_split_bf16 below: v*w taken as
 * hi*hi + hi*lo + lo*hi with fp32 accumulation; bias and tanh(mish) in fp32).
 * Error contract (a separate one from the fp32 entry points): each product is off by at
 * most 3 * 2^-16 |x*w|, and tanh(mish(.)) changes by at most 1.1 times a change of its
 * argument, so
 *     |y - y_exact| <= 1e-4 + 1e-4 |y_exact| + 2^-13 * sum over taps and channels |x * w|.
 * Same arguments, layouts and errors as conv3d_mish_tanh.  Applies to k = 3, stride 1,
 * pad <= 2; every other case runs the fp32 kernels (which meet the tighter fp32 contract).
 */
int conv3d_mish_tanh_split_bf16(const float *x, const float *w, const float *b, float *y,
                                int64_t N, int64_t Cin, int64_t D, int64_t H, int64_t W,
                                int64_t Cout, int64_t k, int64_t stride, int64_t pad,
                                void *stream);

/*
 * conv3d_div_maxpool_gap_bias_sum with the Conv3d on bf16 matrix cores (opt-in precision
 * mode, the same three-term split of fp32; divide, max-pool, mean, bias and sum in fp32).
 * Error contract: each conv output v is off by at most 2^-14 * S(v), S(v) = the sum over taps
 * and input channels of |x * w| (3 * 2^-16 per product).  A window maximum moves by at most
 * the largest change in its window, a mean by at most the largest of its terms, so with
 * M_o[n] = the largest S(v) over the pooled voxels of image n and output channel o,
 *     |out[n] - out_exact[n]| <= 1e-4 |out_exact[n]| + 2^-14 * sum_o M_o[n] / |divisor|.
 * Same arguments, layouts and errors as conv3d_div_maxpool_gap_bias_sum.  Applies to k = 3
 * and pool 2; every other case runs the fp32 kernels.
 */
int conv3d_div_maxpool_gap_bias_sum_split_bf16(const float *x, const float *w,
                                               const float *conv_b, float divisor, int64_t pool,
                                               const float *bias, float *out, int64_t N,
                                               int64_t Cin, int64_t D, int64_t H, int64_t W,
                                               int64_t Cout, int64_t k, void *stream);

/*
 * dwsep_conv2d with the pointwise GEMM on bf16 matrix cores (opt-in precision mode).  The
 * pages weigh reduced-precision tensor-core formats (TF32) against true fp32 for these layers
 * (page "Kimi-K2.6 l2_p47", the roofline estimate and the mma-precision paragraph); gfx950 has
 * no TF32-like format, so fp32 is emulated: each operand v splits into hi = bf16(v) and
 * lo = bf16(v - hi), and v*w is taken as hi*hi + hi*lo + lo*hi with fp32 accumulation.  The
 * depthwise step, the biases and the accumulation stay fp32.
 * Error contract (a separate one from the fp32 entry points): with bf16 rounding to nearest,
 * |v - hi - lo| <= 2^-16 |v| and |lo| <= 2^-8 |v|, so each product is off by at most
 * 3 * 2^-16 |v*w|.  Hence, with d[c] the depthwise output at the pixel,
 *     |y[o] - y_exact[o]| <= 1e-4 + 1e-4 |y_exact[o]| + 2^-14 * sum_c |d[c] * pw[o,c]|.
 * Same arguments, layouts and errors as dwsep_conv2d.  Applies to K = 3, stride 1,
 * dilation 1, pad <= 2 when the layer's weights fit on chip; every other case runs the fp32
 * kernels (which meet the tighter fp32 contract).
 */
int dwsep_conv2d_split_bf16(const float *x, const float *dw_w, const float *dw_b,
                            const float *pw_w, const float *pw_b, float *y, int64_t N,
                            int64_t Cin, int64_t H, int64_t W, int64_t Cout, int64_t K,
                            int64_t stride, int64_t pad, int64_t dilation, void *stream);

/*
 * ---- Unfused path: the separate steps the fused entry points replace ----
 * The pages' alternative to fusion runs the convolution as its own kernel, writes its output
 * to memory, then applies the epilogue or the reduction in further kernels (page "Kimi-K2.6
 * l2_p47": library conv + elementwise Mish/tanh; page "Kimi-K2.6 l2_p8": library conv +
 * reduction kernel over its 441 MB output; page "Kimi-K2.6 l1_p86": separate depthwise and
 * pointwise passes).  These entry points are those steps, built from the same kernels, so
 * the saving of fusion can be measured.  Same conventions: device pointers, caller-owned
 * buffers, the caller's stream, validation before any launch.
 */

/* y = conv3d(x, w) + b (b may be NULL), y [N][Cout][OD][OH][OW]; any k, stride, pad. */
int conv3d_bias(const float *x, const float *w, const float *b, float *y,
                int64_t N, int64_t Cin, int64_t D, int64_t H, int64_t W,
                int64_t Cout, int64_t k, int64_t stride, int64_t pad, void *stream);

/* y[i] = tanh(mish(v[i])) for i < count (v may equal y). */
int mish_tanh(const float *v, float *y, int64_t count, void *stream);

/* out[n] = sum_c ( mean(maxpool_pool(conv[n,c] / divisor)) + bias[c] ) from a stored conv
 * output conv [N][C][OD][OH][OW] that already includes the conv bias; out [N] is
 * initialised by the call.  Float atomics: the last bits may vary from run to run. */
int div_maxpool_gap_bias_sum(const float *conv, float divisor, int64_t pool, const float *bias,
                             float *out, int64_t N, int64_t C, int64_t OD, int64_t OH,
                             int64_t OW, void *stream);

/* y = depthwise K x K conv of x (+ dw_b), y [N][C][Ho][Wo] (the intermediate the fused
 * dwsep_conv2d never writes). */
int depthwise_conv2d(const float *x, const float *dw_w, const float *dw_b, float *y,
                     int64_t N, int64_t C, int64_t H, int64_t W, int64_t K, int64_t stride,
                     int64_t pad, int64_t dilation, void *stream);

/* y = pointwise 1x1 conv of x (+ pw_b), x [N][Cin][H][W] -> y [N][Cout][H][W]. */
int pointwise_conv2d(const float *x, const float *pw_w, const float *pw_b, float *y,
                     int64_t N, int64_t Cin, int64_t H, int64_t W, int64_t Cout, void *stream);

/* Output length of one spatial dimension, floor((in + 2*pad - dilation*(k-1) - 1)/stride)+1
 * (page l1_p86 output-size formula).  Pure host function.  Writes *out and returns
 * CONVFUSE_OK, or CONVFUSE_ERR_NULL / CONVFUSE_ERR_SHAPE (non-positive in, k, stride or
 * dilation, negative pad, or an empty output). */
int convfuse_conv_out_len(int64_t in, int64_t k, int64_t stride, int64_t pad, int64_t dilation,
                          int64_t *out);

/*
 * Output sizes of the valid/padded Conv3d of conv3d_mish_tanh: OD = (D + 2*pad - k)/stride + 1,
 * and likewise OH, OW (page "Kimi-K2.6 l2_p47", the output-size line of the generalised
 * stride/padding kernel; 32 x 64 x 64 with k = 3 gives 30 x 62 x 62).  Pure host function, no
 * device is touched.  Writes *OD, *OH, *OW and returns CONVFUSE_OK; CONVFUSE_ERR_NULL for a
 * NULL output pointer; CONVFUSE_ERR_SHAPE (outputs untouched) for a non-positive size, k or
 * stride, a negative pad, a size above 2^24, or an empty output.
 */
int convfuse_out_dims_conv3d(int64_t D, int64_t H, int64_t W, int64_t k, int64_t stride,
                             int64_t pad, int64_t *OD, int64_t *OH, int64_t *OW);

/*
 * Output sizes of the depthwise step of dwsep_conv2d (and of the whole layer):
 * Ho = (H + 2*pad - dilation*(K-1) - 1)/stride + 1, likewise Wo (page "Kimi-K2.6 l1_p86", the
 * output-size formula; 512 x 512 at K = 3, pad 1 stays 512 x 512).  Pure host function.
 * Writes *Ho, *Wo and returns CONVFUSE_OK; CONVFUSE_ERR_NULL for a NULL output pointer;
 * CONVFUSE_ERR_SHAPE (outputs untouched) for a non-positive size, K, stride or dilation, a
 * negative pad, a size above 2^24, or an empty output.
 */
int convfuse_out_dims_conv2d(int64_t H, int64_t W, int64_t K, int64_t stride, int64_t pad,
                             int64_t dilation, int64_t *Ho, int64_t *Wo);

/* Name of the last kernel the calling thread launched through the library (the main kernel
 * of its last successful launching call, e.g. "dwsep_persistent_kernel"; "" before any), so a
 * caller or a benchmark can see which kernel the dispatch chose.  Static string. */
const char *convfuse_last_kernel(void);

/* Hash of the kernel and ABI sources this library was compiled from (16 hex digits, or
 * "unknown" for a build that did not stamp it), so a caller can tell which sources a loaded
 * binary was built from.  Static string. */
const char *convfuse_build_id(void);

/* Message describing the calling thread's most recent failed call ("" if none).  The
 * pointer stays valid until the thread's next failing call. */
const char *convfuse_last_error(void);

/*
 * Diagnostic, outside the convolution path: launches `workgroups` workgroups of 4 waves,
 * each wave running iters x 16 independent fp32 16x16x4 MFMAs with no memory traffic, so
 * the launch's rate (workgroups * 4 * iters * 16 * 2048 FLOP over its duration) is the
 * practical fp32 matrix-core ceiling that the kernels' roofline fractions are compared
 * with.  Writes iters * 2^-14 to out[0] (a device pointer), exactly.  Errors: SHAPE for
 * iters outside [1, 2^22) or workgroups outside [1, 2^20], NULL for a null out.
 */
int convfuse_measure_mfma(float *out, int64_t iters, int64_t workgroups, void *stream);

/* ABI version (major * 100 + minor).  A caller built against this header can compare
 * CONVFUSE_ABI_VERSION with what the loaded library returns; minor versions only add entry
 * points (1.01 added the unfused steps', the split-bf16 and the diagnostic entry points;
 * 1.02 the whole-shape helpers convfuse_out_dims_conv3d / _conv2d, convfuse_build_id and
 * convfuse_last_kernel). */
#define CONVFUSE_ABI_VERSION 102
int convfuse_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CONVFUSE_H */
