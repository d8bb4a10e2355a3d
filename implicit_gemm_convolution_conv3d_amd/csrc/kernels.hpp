// kernels.hpp -- host-side launchers of the gfx950 kernels (internal to libconvfuse.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convfuse {

// Records, for the calling thread, the name of the kernel it is about to launch (a string
// literal); convfuse_last_kernel() returns it.
void note_kernel(const char *name);

// Shape of a Conv3d with a cubic kernel; O* are the output sizes, pad the zero padding on
// every side.  Kernel size and stride are implied (3 and 1) for the tuned kernels and given
// by GenConv for the general ones.
struct Conv3dDims {
    int64_t N, C, D, H, W, O;
    int64_t OD, OH, OW;
    int pad;
};

struct PoolDims {
    Conv3dDims conv;   // valid conv: pad 0
    int64_t PD, PH, PW;
    float divisor;
};

struct DwsepDims {
    int64_t N, C, H, W, O;
    int64_t Ho, Wo;
    int pad;
};

// Kernel size, stride and dilation of the general-parameter kernels.
struct GenConv {
    int k, stride, dilation;
};

// Tuned kernels: k = 3, stride 1, pad <= 2 (pool 2; dwsep dilation 1).
hipError_t launch_conv3d_mish_tanh(const float *x, const float *w, const float *b, float *y,
                                   const Conv3dDims &d, hipStream_t stream);

hipError_t launch_conv3d_pool_sum(const float *x, const float *w, const float *conv_b,
                                  const float *bias, float *out, const PoolDims &d,
                                  hipStream_t stream);

hipError_t launch_dwsep_conv2d(const float *x, const float *dw_w, const float *dw_b,
                               const float *pw_w, const float *pw_b, float *y,
                               const DwsepDims &d, hipStream_t stream);

// The pooled tensor y [N][O][PD][PH][PW] = maxpool((conv + conv_b) / divisor) (k = 3, pool 2).
hipError_t launch_conv3d_div_maxpool(const float *x, const float *w, const float *conv_b,
                                     float *y, const PoolDims &d, hipStream_t stream);

// Unfused path: conv + bias written to y (tuned k = 3 / general), tanh(mish) elementwise,
// the pooled channel sum from a stored conv output, depthwise alone, pointwise alone.
hipError_t launch_conv3d_bias(const float *x, const float *w, const float *b, float *y,
                              const Conv3dDims &d, hipStream_t stream);
hipError_t launch_mish_tanh(const float *v, float *y, int64_t count, hipStream_t stream);
hipError_t launch_div_maxpool_gap_bias_sum(const float *conv, const float *bias, float *out,
                                           const PoolDims &d, int pool, hipStream_t stream);
hipError_t launch_depthwise_conv2d(const float *x, const float *dw_w, const float *dw_b,
                                   float *y, const DwsepDims &d, const GenConv &g,
                                   hipStream_t stream);
hipError_t launch_pointwise_conv2d(const float *x, const float *pw_w, const float *pw_b, float *y,
                                   const DwsepDims &d, hipStream_t stream);

// dwsep with the pointwise GEMM on bf16 matrix cores as a three-term split of each fp32
// operand (opt-in precision mode; k = 3, stride 1, dilation 1, pad <= 2).
// Diagnostic: workgroups x 4 waves, each running iters x 16 independent fp32 MFMAs.
hipError_t launch_mfma_loop(float *out, int iters, int workgroups, hipStream_t stream);

// Split-bf16 mode of conv3d_div_maxpool_gap_bias_sum (k = 3, pool 2).
hipError_t launch_conv3d_pool_sum_split_bf16(const float *x, const float *w,
                                             const float *conv_b, const float *bias, float *out,
                                             const PoolDims &p, hipStream_t stream);

// Split-bf16 mode of conv3d_mish_tanh (k = 3, stride 1, pad <= 2).
hipError_t launch_conv3d_mish_tanh_split_bf16(const float *x, const float *w, const float *b,
                                              float *y, const Conv3dDims &d, hipStream_t stream);

hipError_t launch_dwsep_conv2d_split_bf16(const float *x, const float *dw_w, const float *dw_b,
                                          const float *pw_w, const float *pw_b, float *y,
                                          const DwsepDims &d, hipStream_t stream);

// out[n] = sum_c bias[c] (the constant term of the pooled channel sum), on the stream.
hipError_t launch_pool_sum_init(const float *bias, float *out, int64_t N, int64_t O,
                                hipStream_t stream);

// General-parameter kernels (any k, stride, padding, dilation; pooled sum: pool <= 32).
hipError_t launch_conv3d_mish_tanh_generic(const float *x, const float *w, const float *b,
                                           float *y, const Conv3dDims &d, const GenConv &g,
                                           hipStream_t stream);

hipError_t launch_conv3d_pool_sum_generic(const float *x, const float *w, const float *conv_b,
                                          const float *bias, float *out, const PoolDims &d,
                                          const GenConv &g, int pool, hipStream_t stream);

hipError_t launch_conv3d_div_maxpool_generic(const float *x, const float *w,
                                             const float *conv_b, float *y, const PoolDims &d,
                                             const GenConv &g, int pool, hipStream_t stream);

hipError_t launch_conv3d_bias_generic(const float *x, const float *w, const float *b, float *y,
                                      const Conv3dDims &d, const GenConv &g, hipStream_t stream);

hipError_t launch_dwsep_conv2d_generic(const float *x, const float *dw_w, const float *dw_b,
                                       const float *pw_w, const float *pw_b, float *y,
                                       const DwsepDims &d, const GenConv &g, hipStream_t stream);

constexpr int kGenericMaxPool = 32;  // largest pooling window of the general kernel

}  // namespace convfuse
