// diag.hip -- a diagnostic kernel outside the convolution path: an fp32 matrix-core issue
// loop with no memory traffic, whose rate is the practical ceiling the roofline fractions
// are compared with (the spec peak assumes the full clock, which MFMA-heavy work does not
// sustain).
#include "common.hpp"
#include "kernels.hpp"

namespace convfuse {

namespace {

constexpr int kLoopAcc = 16;  // independent accumulators per wave: no MFMA waits on another

// Every wave runs iters x kLoopAcc 16x16x4 fp32 MFMAs on operands a = b = 2^-10, so each
// accumulator element ends at iters * 4 * 2^-20 (exact in fp32 for iters < 2^22).  Lane 0 of
// wave 0 of workgroup 0 writes the sum of its first elements to out[0].
__global__ __launch_bounds__(256) void mfma_loop_kernel(float *out, int iters)
{
    const float a = 1.0f / 1024.0f;
    floatx4 acc[kLoopAcc];
#pragma unroll
    for (int i = 0; i < kLoopAcc; ++i) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < kLoopAcc; ++i) acc[i] = mfma_16x16x4(a, a, acc[i]);
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < kLoopAcc; ++i) s += acc[i][0];
    if (blockIdx.x == 0 && threadIdx.x == 0) out[0] = s;
}

}  // namespace

hipError_t launch_mfma_loop(float *out, int iters, int workgroups, hipStream_t s)
{
    note_kernel("mfma_loop_kernel");
    hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)workgroups), dim3(256), 0, s, out,
                       iters);
    return hipGetLastError();
}

}  // namespace convfuse
