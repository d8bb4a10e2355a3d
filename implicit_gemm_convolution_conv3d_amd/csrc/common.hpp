// common.hpp -- device helpers shared by the gfx950 convolution kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convfuse {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;   // CDNA wavefront width
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, one L2 each

// D(16x16) += A(16x4) * B(4x16) on the fp32 matrix cores.
// Lane l supplies A[l%16][l/16] and B[l/16][l%16]; it receives D[4*(l/16)+r][l%16] in
// element r of the result.
__device__ __forceinline__ floatx4 mfma_16x16x4(float a, float b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// D(16x16) += A(16x32) * B(32x16) on the bf16 matrix cores, fp32 accumulation.  Lane l
// supplies A[l%16][8*(l/16) + i] and B[8*(l/16) + i][l%16] in element i; it receives
// D[4*(l/16)+r][l%16] in element r of the result (the fp32 16x16x4 layout).
__device__ __forceinline__ floatx4 mfma_16x16x32_bf16(bf16x8 a, bf16x8 b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Three-term split of fp32 values for bf16 matrix cores: hi = bf16(v) (nearest), lo =
// bf16(v - hi); v*w is then taken as hi_v*hi_w + hi_v*lo_w + lo_v*hi_w.
__device__ __forceinline__ void split_bf16(const float (&v)[8], bf16x8 &hi, bf16x8 &lo)
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const __bf16 h = (__bf16)v[i];
        hi[i] = h;
        lo[i] = (__bf16)(v[i] - (float)h);
    }
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

// tanh(mish(v)), mish(v) = v * tanh(softplus(v)), softplus(v) = v for v > 20 (PyTorch's
// threshold).  For v <= 20, tanh(log(1 + e^v)) = n / (n + 2) with n = e^v (e^v + 2); for
// v > 20, tanh(v) rounds to 1 in fp32, so mish(v) = v.  The outer tanh(m) = 1 - 2/(e^2m + 1);
// m >= -0.31 keeps e^2m away from 0, and its overflow to +inf gives exactly 1.
// Both quotients use the hardware reciprocal (v_rcp_f32, 1 ulp) instead of an IEEE division,
// whose scale/fixup sequence is about ten vector instructions that issue from the same SIMDs
// as the matrix work: t then carries about 2 ulp of relative error and the result under
// 1e-6 absolute.
__device__ __forceinline__ float mish_tanh(float v)
{
    float t = 1.0f;
    if (v <= 20.0f) {
        const float e = __expf(v);
        const float n = e * (e + 2.0f);
        t = n * __builtin_amdgcn_rcpf(n + 2.0f);
    }
    const float m = v * t;
    return 1.0f - 2.0f * __builtin_amdgcn_rcpf(__expf(2.0f * m) + 1.0f);
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

namespace convfuse {

// Global -> register -> LDS staging of a halo box stored as ROWS rows.  Each row is MAIN
// contiguous floats starting at global column col0 (a multiple of 4), plus two edge
// columns (the halo: `pad` columns left of col0 and 2 - pad right of col0 + MAIN).  In
// LDS, column 4 of a row holds global column col0, so the main part is 16-byte aligned.
// load() issues every global load of the box before any is waited on; store() writes the
// registers to LDS.  Columns outside [0, W) and rows the source marks as absent read as 0.
// VEC: W % 4 == 0 and 16-byte aligned rows, so the main part moves as float4.
template <int ROWS, int MAIN, int NT, bool VEC>
struct HaloRows {
    static constexpr int TPR = MAIN / 4;                 // threads per row, one float4 each
    static constexpr int RPP = NT / TPR;                 // rows per pass
    static constexpr int P = (ROWS + RPP - 1) / RPP;     // passes over the rows
    static constexpr int PE = (2 * ROWS + NT - 1) / NT;  // edge values per thread
    static_assert(MAIN % 4 == 0 && NT % TPR == 0, "row split");
    floatx4 m[P];
    float e[PE];

    // src(row): global pointer to column 0 of the row, or nullptr for an all-zero row.
    template <class Src>
    __device__ __forceinline__ void load(const Src &src, int col0, int pad, int W)
    {
        const int t = threadIdx.x;
        const int c = col0 + 4 * (t % TPR);
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int row = t / TPR + p * RPP;
            floatx4 v = {0.f, 0.f, 0.f, 0.f};
            const float *base = row < ROWS ? src(row) : nullptr;
            if (base) {
                if constexpr (VEC) {
                    if (c < W) v = *reinterpret_cast<const floatx4 *>(base + c);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (c + i < W) v[i] = base[c + i];
                }
            }
            m[p] = v;
        }
#pragma unroll
        for (int p = 0; p < PE; ++p) {
            const int idx = t + p * NT;
            const int row = idx >> 1, j = idx & 1;
            float v = 0.f;
            if (row < ROWS) {
                const float *base = src(row);
                const int col = j < pad ? col0 - pad + j : col0 + MAIN + j - pad;
                if (base && (unsigned)col < (unsigned)W) v = base[col];
            }
            e[p] = v;
        }
    }

    // dst(row): LDS pointer of the row (its column 0 = global column col0 - 4).
    template <class Dst>
    __device__ __forceinline__ void store(const Dst &dst, int pad) const
    {
        const int t = threadIdx.x;
        const int q = t % TPR;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int row = t / TPR + p * RPP;
            if (row < ROWS) *reinterpret_cast<floatx4 *>(dst(row) + 4 + 4 * q) = m[p];
        }
#pragma unroll
        for (int p = 0; p < PE; ++p) {
            const int idx = t + p * NT;
            const int row = idx >> 1, j = idx & 1;
            if (row < ROWS) dst(row)[j < pad ? 4 - pad + j : 4 + MAIN + j - pad] = e[p];
        }
    }
};

// Buffer-resource access.  An offset at or past the resource's range is dropped by the
// hardware (loads return 0, stores write nothing), so padding and ragged edges need no
// branches, and a tile issues the same memory instructions on every path.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kBufferWord3 = 0x00020000;  // buffer resource word 3: raw 32-bit access
constexpr int kDropOffset = 0x80000000;   // >= kBufRange: the access is dropped
constexpr int kBufRange = 0x7fffffff;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const float *base)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0, kBufRange,
                                             kBufferWord3);
}

// HaloRows through a buffer resource: roff(row) is the byte offset of the row's column 0
// from the resource base, or a negative value for an all-zero row (byte offsets of present
// columns stay below 2^31).  Absent rows and columns outside [0, W) read as zero without
// branches.
template <int ROWS, int MAIN, int NT, bool VEC>
struct BufHaloRows {
    static constexpr int TPR = MAIN / 4;
    static constexpr int RPP = NT / TPR;
    static constexpr int P = (ROWS + RPP - 1) / RPP;
    static constexpr int PE = (2 * ROWS + NT - 1) / NT;
    static_assert(MAIN % 4 == 0 && NT % TPR == 0, "row split");
    floatx4 m[P];
    float e[PE];

    template <class Roff>
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, const Roff &roff, int col0,
                                         int pad, int W)
    {
        const int t = threadIdx.x;
        const int c = col0 + 4 * (t % TPR);
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int row = t / TPR + p * RPP;
            const int ro = row < ROWS ? roff(row) : -1;
            if constexpr (VEC) {
                const int off = ro >= 0 && c < W ? ro + 4 * c : kDropOffset;
                m[p] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int off = ro >= 0 && c + i < W ? ro + 4 * (c + i) : kDropOffset;
                    m[p][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
                }
            }
        }
#pragma unroll
        for (int p = 0; p < PE; ++p) {
            const int idx = t + p * NT;
            const int row = idx >> 1, j = idx & 1;
            const int ro = row < ROWS ? roff(row) : -1;
            const int col = j < pad ? col0 - pad + j : col0 + MAIN + j - pad;
            const int off = ro >= 0 && (unsigned)col < (unsigned)W ? ro + 4 * col : kDropOffset;
            e[p] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
        }
    }

    template <class Dst>
    __device__ __forceinline__ void store(const Dst &dst, int pad) const
    {
        const int t = threadIdx.x;
        const int q = t % TPR;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int row = t / TPR + p * RPP;
            if (row < ROWS) *reinterpret_cast<floatx4 *>(dst(row) + 4 + 4 * q) = m[p];
        }
#pragma unroll
        for (int p = 0; p < PE; ++p) {
            const int idx = t + p * NT;
            const int row = idx >> 1, j = idx & 1;
            if (row < ROWS) dst(row)[j < pad ? 4 - pad + j : 4 + MAIN + j - pad] = e[p];
        }
    }
};

}  // namespace convfuse

namespace convfuse {

// Workgroup barrier for data exchanged through LDS only: waits for this wave's LDS accesses
// (lgkmcnt) and synchronises the workgroup, but leaves its global loads and stores in
// flight.  __syncthreads also orders global memory and so waits for every outstanding
// vector-memory operation, stores included.  Register operands of pending loads are still
// waited for by the compiler where they are used.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace convfuse
