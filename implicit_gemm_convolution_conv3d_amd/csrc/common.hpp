// common.hpp -- device helpers shared by the gfx950 convolution kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convfuse {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;   // CDNA wavefront width
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, one L2 each

// D(16x16) += A(16x4) * B(4x16) on the fp32 matrix cores.
// Lane l supplies A[l%16][l/16] and B[l/16][l%16]; it receives D[4*(l/16)+r][l%16] in
// element r of the result.
__device__ __forceinline__ floatx4 mfma_16x16x4(float a, float b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Workgroups are dispatched round-robin over the XCDs (workgroup i lands on XCD i % 8).
// Remap the linear workgroup id so that each XCD processes one contiguous run of tiles:
// neighbouring tiles then share their halo rows in the same L2.  Bijective on [0, total).
__device__ __forceinline__ int64_t xcd_tile(int64_t bid, int64_t total)
{
    int64_t q = total / kNumXcd, r = total % kNumXcd;
    int64_t xcd = bid % kNumXcd, idx = bid / kNumXcd;
    return xcd * q + (xcd < r ? xcd : r) + idx;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

template <int V>
struct IntC {
    static constexpr int value = V;
};

constexpr int round_up(int v, int m) { return (v + m - 1) / m * m; }

// LDS channel stride for halo tiles: a multiple of 4 floats (16-byte rows) that is
// congruent to 16 (mod 64) words, so the four 16-lane groups of a wave that read four
// consecutive channels at the same offset land in four disjoint 16-bank groups.
constexpr int halo_channel_stride(int plane_floats)
{
    int s = round_up(plane_floats, 16);
    while (s % 64 != 16 && s % 64 != 48) s += 16;
    return s;
}

}  // namespace convfuse
