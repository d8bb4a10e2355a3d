// dwsep.hip -- fused depthwise 3x3 + pointwise 1x1 Conv2d on gfx950
// (page "Kimi-K2.6 l1_p86", depthwise-separable Conv2d: the fused definition and the
// implicit-GEMM view of the pointwise step, with the depthwise computed while the GEMM
// operand is formed).
//
// GEMM view: output pixels x output channels, reduced over input channels.  For a 16x16x4
// MFMA k-step, lane l forms the pixel-side operand as the depthwise output of channel
// (4*cg + l/16) at pixel column (l%16): nine reads of the staged input halo and nine FMAs,
// so the depthwise tile never leaves registers.  The pointwise weights of a channel chunk
// are staged in LDS in fragment order.
//
// Workgroup = WGW waves side by side along W; each wave owns R consecutive output rows of
// one 16-pixel column block and every output channel of its channel group, so the input is
// read once per channel group.  The next chunk's global loads are issued into registers
// before the current chunk's MFMAs.
//
// PIXROWS selects which MFMA operand carries the pixels.  With pixels as the A operand each
// lane ends with 4 consecutive pixels of one output channel and stores them as one float4
// (rows 16-byte aligned); otherwise each lane holds 4 output channels of one pixel and the
// 16 lanes of a row group store 64 contiguous bytes.
#include "common.hpp"
#include "kernels.hpp"

namespace convfuse {

namespace {

// Pointwise weights of output channels [o0, o0 + 16*MB) x input channels [c0, c0 + CC),
// stored as ps[(cg*64 + lane)*MB + mb] = pw_w[o0 + 16*mb + lane%16][c0 + 4*cg + lane/16].
// Thread t loads the float4 quads t, t + NT, ... (quad = 4 consecutive input channels).
template <int MB, int CC, int NT, bool VEC>
struct PwChunk {
    static constexpr int QUADS = 16 * MB * CC / 4;
    static constexpr int PQ = (QUADS + NT - 1) / NT;
    floatx4 v[PQ];

    __device__ __forceinline__ void load(const float *__restrict__ pw, const DwsepDims &d, int o0,
                                         int c0)
    {
#pragma unroll
        for (int p = 0; p < PQ; ++p) {
            const int qd = threadIdx.x + p * NT;
            const int o = o0 + qd / (CC / 4), c = c0 + 4 * (qd % (CC / 4));
            floatx4 r = {0.f, 0.f, 0.f, 0.f};
            if (qd < QUADS && o < d.O) {
                const float *src = pw + (int64_t)o * d.C + c;
                if constexpr (VEC) {
                    if (c < d.C) r = *reinterpret_cast<const floatx4 *>(src);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (c + i < d.C) r[i] = src[i];
                }
            }
            v[p] = r;
        }
    }

    __device__ __forceinline__ void store(float *__restrict__ ps) const
    {
#pragma unroll
        for (int p = 0; p < PQ; ++p) {
            const int qd = threadIdx.x + p * NT;
            if (qd >= QUADS) continue;
            const int ol = qd / (CC / 4), cg = qd % (CC / 4);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ps[(cg * 64 + i * 16 + (ol & 15)) * MB + (ol >> 4)] = v[p][i];
        }
    }
};

template <int MB, int R, int WGW, int CC, bool VEC, bool PIXROWS>
__global__ __launch_bounds__(64 * WGW, 2) void dwsep_kernel(
    const float *__restrict__ x, const float *__restrict__ dw_w, const float *__restrict__ dw_b,
    const float *__restrict__ pw_w, const float *__restrict__ pw_b, float *__restrict__ y,
    DwsepDims d, int64_t tiles, int tiles_w, int tiles_h)
{
    constexpr int NT = 64 * WGW;
    constexpr int MAIN = 16 * WGW;
    constexpr int HR = R + 2;
    constexpr int RS = MAIN + 8;
    constexpr int CS = halo_channel_stride(HR * RS);
    constexpr int XS = CC * CS;
    constexpr int PS = CC * 16 * MB;  // pointwise fragments of one chunk
    constexpr int DS = CC * 12;       // depthwise weights (9) + bias, padded to 12
    static_assert(DS <= NT, "one depthwise value per thread");
    __shared__ __attribute__((aligned(16))) float lds[XS + PS + DS];
    float *xs = lds;
    float *ps = lds + XS;
    float *ds = lds + XS + PS;

    int64_t t = xcd_tile(blockIdx.x, tiles);
    const int tw = (int)(t % tiles_w); t /= tiles_w;
    const int th = (int)(t % tiles_h); t /= tiles_h;
    const int64_t n = t % d.N;
    const int og = (int)(t / d.N);

    const int h0 = th * R, w0 = tw * MAIN, o0 = og * 16 * MB;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // LDS column of pixel column v at tap kw is v + kw + 4 - pad.
    const int xlane = (lane >> 4) * CS + 16 * wave + (lane & 15) + 4 - d.pad;
    const int ih0 = h0 - d.pad;

    HaloRows<CC * HR, MAIN, NT, VEC> halo;
    PwChunk<MB, CC, NT, VEC> pwc;
    float dwv = 0.0f;
    auto load = [&](int c0) {
        auto src = [&](int row) -> const float * {
            const int hr = row % HR, c = row / HR;
            const int ci = c0 + c, ih = ih0 + hr;
            if (ci >= d.C || (unsigned)ih >= (unsigned)d.H) return nullptr;
            return x + ((n * d.C + ci) * d.H + ih) * d.W;
        };
        halo.load(src, w0, d.pad, (int)d.W);
        pwc.load(pw_w, d, o0, c0);
        const int k = threadIdx.x % 12, ci = c0 + threadIdx.x / 12;
        dwv = 0.0f;
        if (threadIdx.x < DS && ci < d.C) {
            if (k < 9) dwv = dw_w[(int64_t)ci * 9 + k];
            else if (k == 9 && dw_b) dwv = dw_b[ci];
        }
    };
    auto store = [&]() {
        auto dst = [&](int row) -> float * {
            const int hr = row % HR, c = row / HR;
            return xs + c * CS + hr * RS;
        };
        halo.store(dst, d.pad);
        pwc.store(ps);
        if (threadIdx.x < DS) ds[threadIdx.x] = dwv;
    };

    load(0);
    if (w0 + 16 * wave < d.Wo) {
        floatx4 acc[MB][R];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int r = 0; r < R; ++r) acc[mb][r] = floatx4{0.f, 0.f, 0.f, 0.f};
        for (int c0 = 0; c0 < d.C; c0 += CC) {
            __syncthreads();
            store();
            __syncthreads();
            if (c0 + CC < d.C) load(c0 + CC);
#pragma unroll
            for (int cg = 0; cg < CC / 4; ++cg) {
                const float *dwp = ds + (4 * cg + (lane >> 4)) * 12;
                const floatx4 k0 = *reinterpret_cast<const floatx4 *>(dwp);
                const floatx4 k1 = *reinterpret_cast<const floatx4 *>(dwp + 4);
                const floatx4 k2 = *reinterpret_cast<const floatx4 *>(dwp + 8);
                const float kw9[9] = {k0[0], k0[1], k0[2], k0[3], k1[0],
                                      k1[1], k1[2], k1[3], k2[0]};
                const float dbias = k2[1];
                float pwf[MB];
#pragma unroll
                for (int i = 0; i < MB / 4; ++i) {
                    const floatx4 v =
                        *reinterpret_cast<const floatx4 *>(ps + (cg * 64 + lane) * MB + 4 * i);
                    pwf[4 * i + 0] = v[0];
                    pwf[4 * i + 1] = v[1];
                    pwf[4 * i + 2] = v[2];
                    pwf[4 * i + 3] = v[3];
                }
                float xv[HR][3];
#pragma unroll
                for (int hr = 0; hr < HR; ++hr)
#pragma unroll
                    for (int kw = 0; kw < 3; ++kw)
                        xv[hr][kw] = xs[xlane + 4 * cg * CS + hr * RS + kw];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float v = dbias;
#pragma unroll
                    for (int kh = 0; kh < 3; ++kh)
#pragma unroll
                        for (int kw = 0; kw < 3; ++kw)
                            v = fmaf(kw9[kh * 3 + kw], xv[r + kh][kw], v);
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        if constexpr (PIXROWS)
                            acc[mb][r] = mfma_16x16x4(v, pwf[mb], acc[mb][r]);
                        else
                            acc[mb][r] = mfma_16x16x4(pwf[mb], v, acc[mb][r]);
                    }
                }
            }
        }

        if constexpr (PIXROWS) {
            // lane holds pixels w0 + 16*wave + 4*(lane/16) + 0..3 of channel 16*mb + lane%16
            const int wcol = w0 + 16 * wave + 4 * (lane >> 4);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int o = o0 + 16 * mb + (lane & 15);
                if (o >= d.O) continue;
                const float bias = pw_b ? pw_b[o] : 0.0f;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if (h0 + r >= d.Ho) continue;
                    float *yp = y + ((n * d.O + o) * d.Ho + h0 + r) * d.Wo + wcol;
                    const floatx4 v = acc[mb][r] + bias;
                    if (wcol + 3 < d.Wo) {
                        *reinterpret_cast<floatx4 *>(yp) = v;
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (wcol + i < d.Wo) yp[i] = v[i];
                    }
                }
            }
        } else {
            // lane holds channels 16*mb + 4*(lane/16) + 0..3 of pixel w0 + 16*wave + lane%16
            const int wcol = w0 + 16 * wave + (lane & 15);
            if (wcol < d.Wo) {
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        const int o = o0 + 16 * mb + 4 * (lane >> 4) + r4;
                        if (o >= d.O) continue;
                        const float bias = pw_b ? pw_b[o] : 0.0f;
                        float *yp = y + ((n * d.O + o) * d.Ho + h0) * d.Wo + wcol;
#pragma unroll
                        for (int r = 0; r < R; ++r)
                            if (h0 + r < d.Ho) yp[(int64_t)r * d.Wo] = acc[mb][r][r4] + bias;
                    }
            }
        }
    } else {
        // This wave's columns lie past the output: it only helps stage the shared tiles.
        for (int c0 = 0; c0 < d.C; c0 += CC) {
            __syncthreads();
            store();
            __syncthreads();
            if (c0 + CC < d.C) load(c0 + CC);
        }
    }
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

template <int MB, int R, int WGW, int CC, bool VEC, bool PIXROWS>
hipError_t launch_t(const float *x, const float *dw_w, const float *dw_b, const float *pw_w,
                    const float *pw_b, float *y, const DwsepDims &d, hipStream_t s)
{
    const int64_t tw = cdiv(d.Wo, 16 * WGW), th = cdiv(d.Ho, R), og = cdiv(d.O, 16 * MB);
    const int64_t tiles = tw * th * d.N * og;
    if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((dwsep_kernel<MB, R, WGW, CC, VEC, PIXROWS>), dim3((unsigned)tiles),
                       dim3(64 * WGW), 0, s, x, dw_w, dw_b, pw_w, pw_b, y, d, tiles, (int)tw,
                       (int)th);
    return hipGetLastError();
}

template <int MB, int R, int WGW, int CC>
hipError_t launch(const float *x, const float *dw_w, const float *dw_b, const float *pw_w,
                  const float *pw_b, float *y, const DwsepDims &d, hipStream_t s)
{
    // Loads move as float4 when input rows and pointwise rows are 16-byte aligned; stores
    // do when output rows are.
    const bool vin = d.W % 4 == 0 && d.C % 4 == 0 && ((uintptr_t)x & 15) == 0 &&
                     ((uintptr_t)pw_w & 15) == 0;
    const bool vout = d.Wo % 4 == 0 && ((uintptr_t)y & 15) == 0;
    if (vin && vout) return launch_t<MB, R, WGW, CC, true, true>(x, dw_w, dw_b, pw_w, pw_b, y, d, s);
    if (vin) return launch_t<MB, R, WGW, CC, true, false>(x, dw_w, dw_b, pw_w, pw_b, y, d, s);
    if (vout) return launch_t<MB, R, WGW, CC, false, true>(x, dw_w, dw_b, pw_w, pw_b, y, d, s);
    return launch_t<MB, R, WGW, CC, false, false>(x, dw_w, dw_b, pw_w, pw_b, y, d, s);
}

}  // namespace

hipError_t launch_dwsep_conv2d(const float *x, const float *dw_w, const float *dw_b,
                               const float *pw_w, const float *pw_b, float *y,
                               const DwsepDims &d, hipStream_t s)
{
    if (d.O <= 64) return launch<4, 4, 4, 16>(x, dw_w, dw_b, pw_w, pw_b, y, d, s);
    if (d.O <= 128) return launch<8, 4, 4, 16>(x, dw_w, dw_b, pw_w, pw_b, y, d, s);
    return launch<12, 2, 4, 16>(x, dw_w, dw_b, pw_w, pw_b, y, d, s);
}

}  // namespace convfuse
