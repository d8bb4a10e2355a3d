// kernels.hpp -- host-side launchers of the gfx950 kernels (internal to libconvfuse.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convfuse {

// Shape of a cubic-kernel (k = 3), stride-1 Conv3d; O* are the output sizes.
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

hipError_t launch_conv3d_mish_tanh(const float *x, const float *w, const float *b, float *y,
                                   const Conv3dDims &d, hipStream_t stream);

hipError_t launch_conv3d_pool_sum(const float *x, const float *w, const float *conv_b,
                                  const float *bias, float *out, const PoolDims &d,
                                  hipStream_t stream);

hipError_t launch_dwsep_conv2d(const float *x, const float *dw_w, const float *dw_b,
                               const float *pw_w, const float *pw_b, float *y,
                               const DwsepDims &d, hipStream_t stream);

}  // namespace convfuse
