// abi.hip -- the extern "C" entry points of libconvfuse.so: argument validation, output
// shapes, and dispatch to the gfx950 kernels on the caller's stream.  Every check runs
// before anything is launched; no entry point allocates memory or synchronises.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/convfuse.h"
#include "kernels.hpp"

namespace {

thread_local char g_err[512];
thread_local const char *g_last_kernel = "";

int fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

// Largest size accepted for one dimension or channel count: keeps every in-kernel
// 32-bit local index and the per-dimension arithmetic far from overflow.
constexpr int64_t kMaxDim = 1LL << 24;
// Largest element count of one tensor: byte offsets stay below 2^62.
constexpr int64_t kMaxElems = 1LL << 60;

bool out_len(int64_t in, int64_t k, int64_t s, int64_t p, int64_t d, int64_t *out)
{
    if (in <= 0 || k <= 0 || s <= 0 || p < 0 || d <= 0) return false;
    if (in > kMaxDim || k > kMaxDim || s > kMaxDim || p > kMaxDim || d > kMaxDim) return false;
    const int64_t span = in + 2 * p - d * (k - 1) - 1;
    if (span < 0) return false;
    *out = span / s + 1;
    return true;
}

// Taps of a k^dims kernel: the general kernels index them with 32-bit integers.
constexpr int64_t kMaxTaps = 1LL << 30;
bool taps_ok(int64_t k, int dims)
{
    int64_t t = 1;
    for (int i = 0; i < dims; ++i) {
        t *= k;
        if (t > kMaxTaps) return false;
    }
    return true;
}

bool elems_ok(std::initializer_list<int64_t> dims)
{
    int64_t total = 1;
    for (int64_t v : dims) {
        if (v < 0 || v > kMaxDim * 64) return false;
        if (v != 0 && total > kMaxElems / v) return false;
        total *= v;
    }
    return true;
}

int device_status(hipError_t e, const char *what)
{
    if (e == hipSuccess) return CONVFUSE_OK;
    return fail(CONVFUSE_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

namespace convfuse {
void note_kernel(const char *name) { g_last_kernel = name; }
}  // namespace convfuse

extern "C" {

int convfuse_abi_version(void) { return CONVFUSE_ABI_VERSION; }

const char *convfuse_last_kernel(void) { return g_last_kernel; }

int convfuse_measure_mfma(float *out, int64_t iters, int64_t workgroups, void *stream)
{
    const char *fn = "convfuse_measure_mfma";
    if (iters < 1 || iters >= ((int64_t)1 << 22) || workgroups < 1 || workgroups > (1 << 20))
        return fail(CONVFUSE_ERR_SHAPE, "%s: iters must be in [1, 2^22), workgroups in [1, 2^20]",
                    fn);
    if (!out) return fail(CONVFUSE_ERR_NULL, "%s: out is required", fn);
    return device_status(
        convfuse::launch_mfma_loop(out, (int)iters, (int)workgroups, (hipStream_t)stream),
        "convfuse_measure_mfma launch");
}

const char *convfuse_last_error(void) { return g_err; }

int convfuse_conv_out_len(int64_t in, int64_t k, int64_t stride, int64_t pad, int64_t dilation,
                          int64_t *out)
{
    if (!out) return fail(CONVFUSE_ERR_NULL, "convfuse_conv_out_len: out is NULL");
    int64_t v;
    if (!out_len(in, k, stride, pad, dilation, &v) || v <= 0)
        return fail(CONVFUSE_ERR_SHAPE,
                    "convfuse_conv_out_len: in=%lld k=%lld stride=%lld pad=%lld dilation=%lld "
                    "gives no output",
                    (long long)in, (long long)k, (long long)stride, (long long)pad,
                    (long long)dilation);
    *out = v;
    return CONVFUSE_OK;
}

int convfuse_out_dims_conv3d(int64_t D, int64_t H, int64_t W, int64_t k, int64_t stride,
                             int64_t pad, int64_t *OD, int64_t *OH, int64_t *OW)
{
    const char *fn = "convfuse_out_dims_conv3d";
    if (!OD || !OH || !OW) return fail(CONVFUSE_ERR_NULL, "%s: OD, OH and OW are required", fn);
    int64_t od, oh, ow;
    if (!out_len(D, k, stride, pad, 1, &od) || !out_len(H, k, stride, pad, 1, &oh) ||
        !out_len(W, k, stride, pad, 1, &ow) || od <= 0 || oh <= 0 || ow <= 0)
        return fail(CONVFUSE_ERR_SHAPE,
                    "%s: D=%lld H=%lld W=%lld k=%lld stride=%lld pad=%lld give no output", fn,
                    (long long)D, (long long)H, (long long)W, (long long)k, (long long)stride,
                    (long long)pad);
    *OD = od;
    *OH = oh;
    *OW = ow;
    return CONVFUSE_OK;
}

int convfuse_out_dims_conv2d(int64_t H, int64_t W, int64_t K, int64_t stride, int64_t pad,
                             int64_t dilation, int64_t *Ho, int64_t *Wo)
{
    const char *fn = "convfuse_out_dims_conv2d";
    if (!Ho || !Wo) return fail(CONVFUSE_ERR_NULL, "%s: Ho and Wo are required", fn);
    int64_t ho, wo;
    if (!out_len(H, K, stride, pad, dilation, &ho) || !out_len(W, K, stride, pad, dilation, &wo) ||
        ho <= 0 || wo <= 0)
        return fail(CONVFUSE_ERR_SHAPE,
                    "%s: H=%lld W=%lld K=%lld stride=%lld pad=%lld dilation=%lld give no output",
                    fn, (long long)H, (long long)W, (long long)K, (long long)stride,
                    (long long)pad, (long long)dilation);
    *Ho = ho;
    *Wo = wo;
    return CONVFUSE_OK;
}

#ifndef CONVFUSE_SOURCE_SHA
#define CONVFUSE_SOURCE_SHA "unknown"
#endif
const char *convfuse_build_id(void) { return CONVFUSE_SOURCE_SHA; }

// Validation and dispatch shared by conv3d_mish_tanh and its split-bf16 mode.
static int conv3d_act_entry(const char *fn, bool split, const float *x, const float *w,
                            const float *b, float *y, int64_t N, int64_t Cin, int64_t D,
                            int64_t H, int64_t W, int64_t Cout, int64_t k, int64_t stride,
                            int64_t pad, void *stream)
{
    if (N < 0 || N > kMaxDim || Cin <= 0 || Cin > kMaxDim || Cout <= 0 || Cout > kMaxDim)
        return fail(CONVFUSE_ERR_SHAPE, "%s: bad N=%lld Cin=%lld Cout=%lld", fn, (long long)N,
                    (long long)Cin, (long long)Cout);
    int64_t OD, OH, OW;
    if (!out_len(D, k, stride, pad, 1, &OD) || !out_len(H, k, stride, pad, 1, &OH) ||
        !out_len(W, k, stride, pad, 1, &OW) || OD <= 0 || OH <= 0 || OW <= 0)
        return fail(CONVFUSE_ERR_SHAPE,
                    "%s: D=%lld H=%lld W=%lld k=%lld stride=%lld pad=%lld give no output", fn,
                    (long long)D, (long long)H, (long long)W, (long long)k, (long long)stride,
                    (long long)pad);
    if (!elems_ok({N, Cin, D, H, W}) || !elems_ok({N, Cout, OD, OH, OW}) ||
        !elems_ok({Cout, Cin, k, k, k}))
        return fail(CONVFUSE_ERR_SHAPE, "%s: tensor too large", fn);
    if (!taps_ok(k, 3))
        return fail(CONVFUSE_ERR_UNSUPPORTED, "%s: k=%lld: more than 2^30 taps", fn, (long long)k);
    if (N == 0) return CONVFUSE_OK;
    if (!x || !w || !y) return fail(CONVFUSE_ERR_NULL, "%s: x, w and y are required", fn);
    convfuse::Conv3dDims d{N, Cin, D, H, W, Cout, OD, OH, OW, (int)pad};
    if (k == 3 && stride == 1 && pad <= 2) {
        if (split)
            return device_status(convfuse::launch_conv3d_mish_tanh_split_bf16(
                                     x, w, b, y, d, (hipStream_t)stream),
                                 "conv3d_mish_tanh_split_bf16 launch");
        return device_status(
            convfuse::launch_conv3d_mish_tanh(x, w, b, y, d, (hipStream_t)stream),
            "conv3d_mish_tanh launch");
    }
    // other geometries run the fp32 kernels (more accurate than the split contract)
    const convfuse::GenConv g{(int)k, (int)stride, 1};
    return device_status(
        convfuse::launch_conv3d_mish_tanh_generic(x, w, b, y, d, g, (hipStream_t)stream),
        split ? "conv3d_mish_tanh_split_bf16 launch" : "conv3d_mish_tanh launch");
}

int conv3d_mish_tanh(const float *x, const float *w, const float *b, float *y, int64_t N,
                     int64_t Cin, int64_t D, int64_t H, int64_t W, int64_t Cout, int64_t k,
                     int64_t stride, int64_t pad, void *stream)
{
    return conv3d_act_entry("conv3d_mish_tanh", false, x, w, b, y, N, Cin, D, H, W, Cout, k,
                            stride, pad, stream);
}

int conv3d_mish_tanh_split_bf16(const float *x, const float *w, const float *b, float *y,
                                int64_t N, int64_t Cin, int64_t D, int64_t H, int64_t W,
                                int64_t Cout, int64_t k, int64_t stride, int64_t pad,
                                void *stream)
{
    return conv3d_act_entry("conv3d_mish_tanh_split_bf16", true, x, w, b, y, N, Cin, D, H, W,
                            Cout, k, stride, pad, stream);
}

// Validation and dispatch shared by conv3d_div_maxpool_gap_bias_sum and its split-bf16 mode.
static int pool_sum_entry(const char *fn, bool split, const float *x, const float *w,
                          const float *conv_b, float divisor, int64_t pool, const float *bias,
                          float *out, int64_t N, int64_t Cin, int64_t D, int64_t H, int64_t W,
                          int64_t Cout, int64_t k, void *stream)
{
    if (N < 0 || N > kMaxDim || Cin <= 0 || Cin > kMaxDim || Cout <= 0 || Cout > kMaxDim)
        return fail(CONVFUSE_ERR_SHAPE, "%s: bad N=%lld Cin=%lld Cout=%lld", fn, (long long)N,
                    (long long)Cin, (long long)Cout);
    if (!std::isfinite(divisor) || divisor == 0.0f)
        return fail(CONVFUSE_ERR_SHAPE, "%s: divisor must be finite and non-zero", fn);
    int64_t OD, OH, OW, PD, PH, PW;
    if (!out_len(D, k, 1, 0, 1, &OD) || !out_len(H, k, 1, 0, 1, &OH) ||
        !out_len(W, k, 1, 0, 1, &OW) || OD <= 0 || OH <= 0 || OW <= 0)
        return fail(CONVFUSE_ERR_SHAPE, "%s: D=%lld H=%lld W=%lld k=%lld give no conv output", fn,
                    (long long)D, (long long)H, (long long)W, (long long)k);
    if (!out_len(OD, pool, pool, 0, 1, &PD) || !out_len(OH, pool, pool, 0, 1, &PH) ||
        !out_len(OW, pool, pool, 0, 1, &PW) || PD <= 0 || PH <= 0 || PW <= 0)
        return fail(CONVFUSE_ERR_SHAPE, "%s: pool=%lld does not fit the %lldx%lldx%lld conv output",
                    fn, (long long)pool, (long long)OD, (long long)OH, (long long)OW);
    if (!elems_ok({N, Cin, D, H, W}) || !elems_ok({N, Cout, OD, OH, OW}) ||
        !elems_ok({Cout, Cin, k, k, k}))
        return fail(CONVFUSE_ERR_SHAPE, "%s: tensor too large", fn);
    if (!taps_ok(k, 3))
        return fail(CONVFUSE_ERR_UNSUPPORTED, "%s: k=%lld: more than 2^30 taps", fn,
                    (long long)k);
    if (pool > convfuse::kGenericMaxPool)
        return fail(CONVFUSE_ERR_UNSUPPORTED, "%s: GPU path implements pool<=%d (got pool=%lld)",
                    fn, convfuse::kGenericMaxPool, (long long)pool);
    if (N == 0) return CONVFUSE_OK;
    if (!x || !w || !bias || !out)
        return fail(CONVFUSE_ERR_NULL, "%s: x, w, bias and out are required", fn);
    convfuse::PoolDims p{{N, Cin, D, H, W, Cout, OD, OH, OW, 0}, PD, PH, PW, divisor};
    const char *what = split ? "conv3d_div_maxpool_gap_bias_sum_split_bf16 launch"
                             : "conv3d_div_maxpool_gap_bias_sum launch";
    if (k == 3 && pool == 2) {
        if (split)
            return device_status(convfuse::launch_conv3d_pool_sum_split_bf16(
                                     x, w, conv_b, bias, out, p, (hipStream_t)stream),
                                 what);
        return device_status(
            convfuse::launch_conv3d_pool_sum(x, w, conv_b, bias, out, p, (hipStream_t)stream),
            what);
    }
    // other parameters run the fp32 kernels (more accurate than the split contract)
    const convfuse::GenConv g{(int)k, 1, 1};
    return device_status(convfuse::launch_conv3d_pool_sum_generic(x, w, conv_b, bias, out, p, g,
                                                                  (int)pool, (hipStream_t)stream),
                         what);
}

int conv3d_div_maxpool_gap_bias_sum(const float *x, const float *w, const float *conv_b,
                                    float divisor, int64_t pool, const float *bias, float *out,
                                    int64_t N, int64_t Cin, int64_t D, int64_t H, int64_t W,
                                    int64_t Cout, int64_t k, void *stream)
{
    return pool_sum_entry("conv3d_div_maxpool_gap_bias_sum", false, x, w, conv_b, divisor, pool,
                          bias, out, N, Cin, D, H, W, Cout, k, stream);
}

int conv3d_div_maxpool_gap_bias_sum_split_bf16(const float *x, const float *w,
                                               const float *conv_b, float divisor, int64_t pool,
                                               const float *bias, float *out, int64_t N,
                                               int64_t Cin, int64_t D, int64_t H, int64_t W,
                                               int64_t Cout, int64_t k, void *stream)
{
    return pool_sum_entry("conv3d_div_maxpool_gap_bias_sum_split_bf16", true, x, w, conv_b,
                          divisor, pool, bias, out, N, Cin, D, H, W, Cout, k, stream);
}

int conv3d_div_maxpool(const float *x, const float *w, const float *conv_b, float divisor,
                       int64_t pool, float *y, int64_t N, int64_t Cin, int64_t D, int64_t H,
                       int64_t W, int64_t Cout, int64_t k, void *stream)
{
    const char *fn = "conv3d_div_maxpool";
    if (N < 0 || N > kMaxDim || Cin <= 0 || Cin > kMaxDim || Cout <= 0 || Cout > kMaxDim)
        return fail(CONVFUSE_ERR_SHAPE, "%s: bad N=%lld Cin=%lld Cout=%lld", fn, (long long)N,
                    (long long)Cin, (long long)Cout);
    if (!std::isfinite(divisor) || divisor == 0.0f)
        return fail(CONVFUSE_ERR_SHAPE, "%s: divisor must be finite and non-zero", fn);
    int64_t OD, OH, OW, PD, PH, PW;
    if (!out_len(D, k, 1, 0, 1, &OD) || !out_len(H, k, 1, 0, 1, &OH) ||
        !out_len(W, k, 1, 0, 1, &OW) || OD <= 0 || OH <= 0 || OW <= 0)
        return fail(CONVFUSE_ERR_SHAPE, "%s: D=%lld H=%lld W=%lld k=%lld give no conv output", fn,
                    (long long)D, (long long)H, (long long)W, (long long)k);
    if (!out_len(OD, pool, pool, 0, 1, &PD) || !out_len(OH, pool, pool, 0, 1, &PH) ||
        !out_len(OW, pool, pool, 0, 1, &PW) || PD <= 0 || PH <= 0 || PW <= 0)
        return fail(CONVFUSE_ERR_SHAPE, "%s: pool=%lld does not fit the %lldx%lldx%lld conv output",
                    fn, (long long)pool, (long long)OD, (long long)OH, (long long)OW);
    if (!elems_ok({N, Cin, D, H, W}) || !elems_ok({N, Cout, OD, OH, OW}) ||
        !elems_ok({Cout, Cin, k, k, k}))
        return fail(CONVFUSE_ERR_SHAPE, "%s: tensor too large", fn);
    if (!taps_ok(k, 3))
        return fail(CONVFUSE_ERR_UNSUPPORTED, "%s: k=%lld: more than 2^30 taps", fn,
                    (long long)k);
    if (pool > convfuse::kGenericMaxPool)
        return fail(CONVFUSE_ERR_UNSUPPORTED, "%s: GPU path implements pool<=%d (got pool=%lld)",
                    fn, convfuse::kGenericMaxPool, (long long)pool);
    if (N == 0) return CONVFUSE_OK;
    if (!x || !w || !y) return fail(CONVFUSE_ERR_NULL, "%s: x, w and y are required", fn);
    convfuse::PoolDims p{{N, Cin, D, H, W, Cout, OD, OH, OW, 0}, PD, PH, PW, divisor};
    if (k == 3 && pool == 2)
        return device_status(
            convfuse::launch_conv3d_div_maxpool(x, w, conv_b, y, p, (hipStream_t)stream),
            "conv3d_div_maxpool launch");
    const convfuse::GenConv g{(int)k, 1, 1};
    return device_status(convfuse::launch_conv3d_div_maxpool_generic(x, w, conv_b, y, p, g,
                                                                     (int)pool,
                                                                     (hipStream_t)stream),
                         "conv3d_div_maxpool launch");
}

int dwsep_conv2d(const float *x, const float *dw_w, const float *dw_b, const float *pw_w,
                 const float *pw_b, float *y, int64_t N, int64_t Cin, int64_t H, int64_t W,
                 int64_t Cout, int64_t K, int64_t stride, int64_t pad, int64_t dilation,
                 void *stream)
{
    if (N < 0 || N > kMaxDim || Cin <= 0 || Cin > kMaxDim || Cout <= 0 || Cout > kMaxDim)
        return fail(CONVFUSE_ERR_SHAPE, "dwsep_conv2d: bad N=%lld Cin=%lld Cout=%lld",
                    (long long)N, (long long)Cin, (long long)Cout);
    int64_t Ho, Wo;
    if (!out_len(H, K, stride, pad, dilation, &Ho) || !out_len(W, K, stride, pad, dilation, &Wo) ||
        Ho <= 0 || Wo <= 0)
        return fail(CONVFUSE_ERR_SHAPE,
                    "dwsep_conv2d: H=%lld W=%lld K=%lld stride=%lld pad=%lld dilation=%lld give "
                    "no output",
                    (long long)H, (long long)W, (long long)K, (long long)stride, (long long)pad,
                    (long long)dilation);
    if (!elems_ok({N, Cin, H, W}) || !elems_ok({N, Cout, Ho, Wo}) || !elems_ok({Cin, K, K}))
        return fail(CONVFUSE_ERR_SHAPE, "dwsep_conv2d: tensor too large");
    if (!taps_ok(K, 2))
        return fail(CONVFUSE_ERR_UNSUPPORTED, "dwsep_conv2d: K=%lld: more than 2^30 taps",
                    (long long)K);
    if (N == 0) return CONVFUSE_OK;
    if (!x || !dw_w || !pw_w || !y)
        return fail(CONVFUSE_ERR_NULL, "dwsep_conv2d: x, dw_w, pw_w and y are required");
    convfuse::DwsepDims d{N, Cin, H, W, Cout, Ho, Wo, (int)pad};
    if (K == 3 && stride == 1 && dilation == 1 && pad <= 2)
        return device_status(
            convfuse::launch_dwsep_conv2d(x, dw_w, dw_b, pw_w, pw_b, y, d, (hipStream_t)stream),
            "dwsep_conv2d launch");
    const convfuse::GenConv g{(int)K, (int)stride, (int)dilation};
    return device_status(convfuse::launch_dwsep_conv2d_generic(x, dw_w, dw_b, pw_w, pw_b, y, d, g,
                                                               (hipStream_t)stream),
                         "dwsep_conv2d launch");
}

int dwsep_conv2d_split_bf16(const float *x, const float *dw_w, const float *dw_b,
                            const float *pw_w, const float *pw_b, float *y, int64_t N,
                            int64_t Cin, int64_t H, int64_t W, int64_t Cout, int64_t K,
                            int64_t stride, int64_t pad, int64_t dilation, void *stream)
{
    const char *fn = "dwsep_conv2d_split_bf16";
    if (N < 0 || N > kMaxDim || Cin <= 0 || Cin > kMaxDim || Cout <= 0 || Cout > kMaxDim)
        return fail(CONVFUSE_ERR_SHAPE, "%s: bad N=%lld Cin=%lld Cout=%lld", fn, (long long)N,
                    (long long)Cin, (long long)Cout);
    int64_t Ho, Wo;
    if (!out_len(H, K, stride, pad, dilation, &Ho) || !out_len(W, K, stride, pad, dilation, &Wo) ||
        Ho <= 0 || Wo <= 0)
        return fail(CONVFUSE_ERR_SHAPE, "%s: H=%lld W=%lld K=%lld stride=%lld pad=%lld "
                    "dilation=%lld give no output", fn, (long long)H, (long long)W, (long long)K,
                    (long long)stride, (long long)pad, (long long)dilation);
    if (!elems_ok({N, Cin, H, W}) || !elems_ok({N, Cout, Ho, Wo}) || !elems_ok({Cin, K, K}))
        return fail(CONVFUSE_ERR_SHAPE, "%s: tensor too large", fn);
    if (!taps_ok(K, 2))
        return fail(CONVFUSE_ERR_UNSUPPORTED, "%s: K=%lld: more than 2^30 taps", fn, (long long)K);
    if (N == 0) return CONVFUSE_OK;
    if (!x || !dw_w || !pw_w || !y)
        return fail(CONVFUSE_ERR_NULL, "%s: x, dw_w, pw_w and y are required", fn);
    convfuse::DwsepDims d{N, Cin, H, W, Cout, Ho, Wo, (int)pad};
    if (K == 3 && stride == 1 && dilation == 1 && pad <= 2)
        return device_status(convfuse::launch_dwsep_conv2d_split_bf16(x, dw_w, dw_b, pw_w, pw_b,
                                                                      y, d, (hipStream_t)stream),
                             "dwsep_conv2d_split_bf16 launch");
    // other geometries run the fp32 general kernel (more accurate than the split contract)
    const convfuse::GenConv g{(int)K, (int)stride, (int)dilation};
    return device_status(convfuse::launch_dwsep_conv2d_generic(x, dw_w, dw_b, pw_w, pw_b, y, d, g,
                                                               (hipStream_t)stream),
                         "dwsep_conv2d_split_bf16 launch");
}

// ------------------------------------------------------------------ unfused path steps

int conv3d_bias(const float *x, const float *w, const float *b, float *y, int64_t N,
                int64_t Cin, int64_t D, int64_t H, int64_t W, int64_t Cout, int64_t k,
                int64_t stride, int64_t pad, void *stream)
{
    const char *fn = "conv3d_bias";
    if (N < 0 || N > kMaxDim || Cin <= 0 || Cin > kMaxDim || Cout <= 0 || Cout > kMaxDim)
        return fail(CONVFUSE_ERR_SHAPE, "%s: bad N=%lld Cin=%lld Cout=%lld", fn, (long long)N,
                    (long long)Cin, (long long)Cout);
    int64_t OD, OH, OW;
    if (!out_len(D, k, stride, pad, 1, &OD) || !out_len(H, k, stride, pad, 1, &OH) ||
        !out_len(W, k, stride, pad, 1, &OW) || OD <= 0 || OH <= 0 || OW <= 0)
        return fail(CONVFUSE_ERR_SHAPE, "%s: D=%lld H=%lld W=%lld k=%lld stride=%lld pad=%lld "
                    "give no output", fn, (long long)D, (long long)H, (long long)W, (long long)k,
                    (long long)stride, (long long)pad);
    if (!elems_ok({N, Cin, D, H, W}) || !elems_ok({N, Cout, OD, OH, OW}) ||
        !elems_ok({Cout, Cin, k, k, k}))
        return fail(CONVFUSE_ERR_SHAPE, "%s: tensor too large", fn);
    if (!taps_ok(k, 3))
        return fail(CONVFUSE_ERR_UNSUPPORTED, "%s: k=%lld: more than 2^30 taps", fn, (long long)k);
    if (N == 0) return CONVFUSE_OK;
    if (!x || !w || !y) return fail(CONVFUSE_ERR_NULL, "%s: x, w and y are required", fn);
    convfuse::Conv3dDims d{N, Cin, D, H, W, Cout, OD, OH, OW, (int)pad};
    if (k == 3 && stride == 1 && pad <= 2)
        return device_status(convfuse::launch_conv3d_bias(x, w, b, y, d, (hipStream_t)stream),
                             "conv3d_bias launch");
    const convfuse::GenConv g{(int)k, (int)stride, 1};
    return device_status(
        convfuse::launch_conv3d_bias_generic(x, w, b, y, d, g, (hipStream_t)stream),
        "conv3d_bias launch");
}

int mish_tanh(const float *v, float *y, int64_t count, void *stream)
{
    if (count < 0 || count > kMaxElems)
        return fail(CONVFUSE_ERR_SHAPE, "mish_tanh: bad count=%lld", (long long)count);
    if (count == 0) return CONVFUSE_OK;
    if (!v || !y) return fail(CONVFUSE_ERR_NULL, "mish_tanh: v and y are required");
    return device_status(convfuse::launch_mish_tanh(v, y, count, (hipStream_t)stream),
                         "mish_tanh launch");
}

int div_maxpool_gap_bias_sum(const float *conv, float divisor, int64_t pool, const float *bias,
                             float *out, int64_t N, int64_t C, int64_t OD, int64_t OH,
                             int64_t OW, void *stream)
{
    const char *fn = "div_maxpool_gap_bias_sum";
    if (N < 0 || N > kMaxDim || C <= 0 || C > kMaxDim)
        return fail(CONVFUSE_ERR_SHAPE, "%s: bad N=%lld C=%lld", fn, (long long)N, (long long)C);
    if (!std::isfinite(divisor) || divisor == 0.0f)
        return fail(CONVFUSE_ERR_SHAPE, "%s: divisor must be finite and non-zero", fn);
    int64_t PD, PH, PW;
    if (!out_len(OD, pool, pool, 0, 1, &PD) || !out_len(OH, pool, pool, 0, 1, &PH) ||
        !out_len(OW, pool, pool, 0, 1, &PW) || PD <= 0 || PH <= 0 || PW <= 0)
        return fail(CONVFUSE_ERR_SHAPE, "%s: pool=%lld does not fit %lldx%lldx%lld", fn,
                    (long long)pool, (long long)OD, (long long)OH, (long long)OW);
    if (!elems_ok({N, C, OD, OH, OW}) || !taps_ok(pool, 3))
        return fail(CONVFUSE_ERR_SHAPE, "%s: tensor too large", fn);
    if (N == 0) return CONVFUSE_OK;
    if (!conv || !bias || !out)
        return fail(CONVFUSE_ERR_NULL, "%s: conv, bias and out are required", fn);
    convfuse::PoolDims p{{N, 0, 0, 0, 0, C, OD, OH, OW, 0}, PD, PH, PW, divisor};
    return device_status(convfuse::launch_div_maxpool_gap_bias_sum(conv, bias, out, p, (int)pool,
                                                                   (hipStream_t)stream),
                         "div_maxpool_gap_bias_sum launch");
}

int depthwise_conv2d(const float *x, const float *dw_w, const float *dw_b, float *y, int64_t N,
                     int64_t C, int64_t H, int64_t W, int64_t K, int64_t stride, int64_t pad,
                     int64_t dilation, void *stream)
{
    const char *fn = "depthwise_conv2d";
    if (N < 0 || N > kMaxDim || C <= 0 || C > kMaxDim)
        return fail(CONVFUSE_ERR_SHAPE, "%s: bad N=%lld C=%lld", fn, (long long)N, (long long)C);
    int64_t Ho, Wo;
    if (!out_len(H, K, stride, pad, dilation, &Ho) || !out_len(W, K, stride, pad, dilation, &Wo) ||
        Ho <= 0 || Wo <= 0)
        return fail(CONVFUSE_ERR_SHAPE, "%s: H=%lld W=%lld K=%lld stride=%lld pad=%lld "
                    "dilation=%lld give no output", fn, (long long)H, (long long)W, (long long)K,
                    (long long)stride, (long long)pad, (long long)dilation);
    if (!elems_ok({N, C, H, W}) || !elems_ok({N, C, Ho, Wo}) || !elems_ok({C, K, K}))
        return fail(CONVFUSE_ERR_SHAPE, "%s: tensor too large", fn);
    if (!taps_ok(K, 2))
        return fail(CONVFUSE_ERR_UNSUPPORTED, "%s: K=%lld: more than 2^30 taps", fn, (long long)K);
    if (N == 0) return CONVFUSE_OK;
    if (!x || !dw_w || !y) return fail(CONVFUSE_ERR_NULL, "%s: x, dw_w and y are required", fn);
    convfuse::DwsepDims d{N, C, H, W, C, Ho, Wo, (int)pad};
    const convfuse::GenConv g{(int)K, (int)stride, (int)dilation};
    return device_status(
        convfuse::launch_depthwise_conv2d(x, dw_w, dw_b, y, d, g, (hipStream_t)stream),
        "depthwise_conv2d launch");
}

int pointwise_conv2d(const float *x, const float *pw_w, const float *pw_b, float *y, int64_t N,
                     int64_t Cin, int64_t H, int64_t W, int64_t Cout, void *stream)
{
    const char *fn = "pointwise_conv2d";
    if (N < 0 || N > kMaxDim || Cin <= 0 || Cin > kMaxDim || Cout <= 0 || Cout > kMaxDim ||
        H <= 0 || H > kMaxDim || W <= 0 || W > kMaxDim)
        return fail(CONVFUSE_ERR_SHAPE, "%s: bad N=%lld Cin=%lld H=%lld W=%lld Cout=%lld", fn,
                    (long long)N, (long long)Cin, (long long)H, (long long)W, (long long)Cout);
    if (!elems_ok({N, Cin, H, W}) || !elems_ok({N, Cout, H, W}))
        return fail(CONVFUSE_ERR_SHAPE, "%s: tensor too large", fn);
    if (N == 0) return CONVFUSE_OK;
    if (!x || !pw_w || !y) return fail(CONVFUSE_ERR_NULL, "%s: x, pw_w and y are required", fn);
    convfuse::DwsepDims d{N, Cin, H, W, Cout, H, W, 1};
    return device_status(
        convfuse::launch_pointwise_conv2d(x, pw_w, pw_b, y, d, (hipStream_t)stream),
        "pointwise_conv2d launch");
}

}  // extern "C"
