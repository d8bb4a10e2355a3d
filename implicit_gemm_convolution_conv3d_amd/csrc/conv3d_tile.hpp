// conv3d_tile.hpp -- pieces shared by the LDS-staged Conv3d implicit-GEMM kernels: weight
// staging in MFMA fragment order, fragment loads, and the tanh(mish) / bias row epilogue.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace convfuse {

// Weights of output channels [o0, o0 + 16*MB) x input channels [c0, c0 + CC), TAPS taps per
// (output, input) channel pair, held in registers between the global load and the LDS
// store.  In memory a pair's taps start at ((o*C + c)*KT + toff) (KT taps per pair in all:
// the staged taps are a contiguous run of them).
// LDS layout (A-fragment order): ws[((tap*CC/4 + cg)*64 + lane)*MB + mb] holds
// w[o0 + 16*mb + lane%16][c0 + 4*cg + lane/16][toff + tap].  Missing channels are zero.
// Pair p = (cl*16 + j)*MB + mb names output channel 16*mb + j and input channel cl; its slot
// at tap t is t*(CC/4)*64*MB + p, so threads holding consecutive pairs write consecutive LDS
// words.  With at least as many pairs as threads, thread t owns the pairs t, t + NT, ...;
// with fewer, pair t % PAIRS is split over TPP threads, TPT taps each.
template <int MB, int CC, int NT, int TAPS>
struct WeightChunk {
    static constexpr int PAIRS = 16 * MB * CC;
    static constexpr int TPP = PAIRS >= NT ? 1 : NT / PAIRS;  // threads per pair
    static constexpr int TPT = (TAPS + TPP - 1) / TPP;        // taps per thread
    static constexpr int PP = (PAIRS * TPP + NT - 1) / NT;
    static constexpr int TAPSTRIDE = (CC / 4) * 64 * MB;
    static_assert(PAIRS >= NT || NT % PAIRS == 0, "pair split");
    float v[PP][TPT];

    __device__ __forceinline__ static void decode(int idx, int &pair, int &t0)
    {
        if constexpr (TPP == 1) {
            pair = idx;
            t0 = 0;
        } else {
            pair = idx % PAIRS;
            t0 = (idx / PAIRS) * TPT;
        }
    }

    __device__ __forceinline__ void load(const float *__restrict__ w, const Conv3dDims &d, int o0,
                                         int c0, int KT, int toff)
    {
#pragma unroll
        for (int p = 0; p < PP; ++p) {
            int pair, t0;
            decode(threadIdx.x + p * NT, pair, t0);
            const int mb = pair % MB, jj = (pair / MB) % 16, cl = pair / (16 * MB);
            const int o = o0 + 16 * mb + jj, c = c0 + cl;
            const bool ok = pair < PAIRS && o < d.O && c < d.C;
            const float *src = w + ((int64_t)o * d.C + c) * KT + toff + t0;
#pragma unroll
            for (int i = 0; i < TPT; ++i) v[p][i] = ok && t0 + i < TAPS ? src[i] : 0.0f;
        }
    }

    __device__ __forceinline__ void store(float *__restrict__ ws) const
    {
#pragma unroll
        for (int p = 0; p < PP; ++p) {
            int pair, t0;
            decode(threadIdx.x + p * NT, pair, t0);
            if (pair >= PAIRS) continue;
#pragma unroll
            for (int i = 0; i < TPT; ++i)
                if (t0 + i < TAPS) ws[(t0 + i) * TAPSTRIDE + pair] = v[p][i];
        }
    }
};

template <int MB>
__device__ __forceinline__ void load_afrag(const float *p, float (&a)[MB])
{
    if constexpr (MB % 4 == 0) {
#pragma unroll
        for (int i = 0; i < MB / 4; ++i) {
            const floatx4 v = *reinterpret_cast<const floatx4 *>(p + 4 * i);
            a[4 * i + 0] = v[0];
            a[4 * i + 1] = v[1];
            a[4 * i + 2] = v[2];
            a[4 * i + 3] = v[3];
        }
    } else {
#pragma unroll
        for (int i = 0; i < MB; ++i) a[i] = p[i];
    }
}

// Store one wave's output row (n, od, oh), columns [ow0, ow0 + 16*NBW), output channels
// [o0, o0 + 16*MB): acc[mb][nb] element r is column ow0 + 16*nb + 4*(lane/16) + r of output
// channel o0 + 16*mb + lane%16 (the voxels were the MFMA rows).  ACT: y = tanh(mish(v + b)),
// else y = v + b.  SW-float stores (SW = 2 needs 8-byte aligned output rows, SW = 4 16-byte
// aligned ones); the row's last partial quad is stored one float at a time.
template <int MB, int NBW, bool ACT, int SW>
__device__ __forceinline__ void store_conv_row(float *__restrict__ y, const float *__restrict__ b,
                                               const Conv3dDims &d, int64_t n, int od, int oh,
                                               int ow0, int o0, const floatx4 (&acc)[MB][NBW])
{
    const int lane = threadIdx.x & 63;
    const int j = lane & 15, q = 4 * (lane >> 4);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int o = o0 + 16 * mb + j;
        if (o >= d.O) continue;
        const float bias = b ? b[o] : 0.0f;
        float *yrow = y + (((n * d.O + o) * d.OD + od) * d.OH + oh) * d.OW;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
            const int ow = ow0 + 16 * nb + q;
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float a = acc[mb][nb][r] + bias;
                v[r] = ACT ? mish_tanh(a) : a;
            }
            if (ow + 3 < d.OW) {
                if constexpr (SW == 4) {
                    *reinterpret_cast<floatx4 *>(yrow + ow) = floatx4{v[0], v[1], v[2], v[3]};
                } else if constexpr (SW == 2) {
                    *reinterpret_cast<floatx2 *>(yrow + ow) = floatx2{v[0], v[1]};
                    *reinterpret_cast<floatx2 *>(yrow + ow + 2) = floatx2{v[2], v[3]};
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) yrow[ow + r] = v[r];
                }
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (ow + r < d.OW) yrow[ow + r] = v[r];
            }
        }
    }
}

// Widest output store the rows' alignment allows (see store_conv_row).
inline int conv_store_width(const float *y, int64_t OW)
{
    const uintptr_t a = (uintptr_t)y;
    return (OW % 4 == 0 && (a & 15) == 0) ? 4 : (OW % 2 == 0 && (a & 7) == 0) ? 2 : 1;
}

}  // namespace convfuse
