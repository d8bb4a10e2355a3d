// dwsep.hip -- fused depthwise 3x3 + pointwise 1x1 Conv2d on gfx950
// (page "Kimi-K2.6 l1_p86", depthwise-separable Conv2d: the fused definition and the
// implicit-GEMM view of the pointwise step, with the depthwise computed while the GEMM
// operand is formed).
//
// GEMM view: rows = output channels (16*MB per workgroup), columns = output pixels,
// reduction over input channels.  For a 16x16x4 MFMA k-step, lane l forms its B operand
// as the depthwise output of channel (4*cg + l/16) at pixel column (l%16): nine LDS reads
// of the staged input halo and nine FMAs, so the depthwise tile never leaves registers.
// The pointwise weights of a channel chunk are staged in A-fragment order.
//
// Workgroup = WGW waves side by side along W; each wave owns R consecutive output rows of
// one 16-pixel column block and every output channel of its channel group, so the input
// is read once per channel group.
#include "common.hpp"
#include "kernels.hpp"

namespace convfuse {

namespace {

template <int MB, int R, int WGW, int CC>
__global__ __launch_bounds__(64 * WGW) void dwsep_kernel(
    const float *__restrict__ x, const float *__restrict__ dw_w, const float *__restrict__ dw_b,
    const float *__restrict__ pw_w, const float *__restrict__ pw_b, float *__restrict__ y,
    DwsepDims d, int64_t tiles, int tiles_w, int tiles_h)
{
    constexpr int NT = 64 * WGW;
    constexpr int HR = R + 2, HWD = 16 * WGW + 2;
    constexpr int RS = round_up(HWD, 4);
    constexpr int CS = halo_channel_stride(HR * RS);
    constexpr int XS = CC * CS;
    constexpr int PS = CC * 16 * MB;  // pointwise fragments of one chunk
    constexpr int DS = CC * 12;       // depthwise weights (9) + bias, padded to 12
    __shared__ __attribute__((aligned(16))) float lds[XS + PS + DS];
    float *xs = lds;
    float *ps = lds + XS;
    float *ds = lds + XS + PS;

    int64_t t = xcd_tile(blockIdx.x, tiles);
    const int tw = (int)(t % tiles_w); t /= tiles_w;
    const int th = (int)(t % tiles_h); t /= tiles_h;
    const int64_t n = t % d.N;
    const int og = (int)(t / d.N);

    const int h0 = th * R, w0 = tw * 16 * WGW, o0 = og * 16 * MB;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int xlane = (lane >> 4) * CS + 16 * wave + (lane & 15);
    const int ih0 = h0 - d.pad, iw0 = w0 - d.pad;

    floatx4 acc[MB][R];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[mb][r] = floatx4{0.f, 0.f, 0.f, 0.f};

    const bool active = w0 + 16 * wave < d.Wo;
    for (int c0 = 0; c0 < d.C; c0 += CC) {
        __syncthreads();
        // input halo rows [ih0, ih0 + HR) x columns [iw0, iw0 + HWD), zero outside
        for (int e = threadIdx.x; e < CC * HR * HWD; e += NT) {
            const int col = e % HWD;
            const int row = e / HWD;
            const int hr = row % HR;
            const int c = row / HR;
            const int ci = c0 + c, ih = ih0 + hr, iw = iw0 + col;
            float v = 0.0f;
            if (ci < d.C && (unsigned)ih < (unsigned)d.H && (unsigned)iw < (unsigned)d.W)
                v = x[((n * d.C + ci) * d.H + ih) * d.W + iw];
            xs[c * CS + hr * RS + col] = v;
        }
        // pointwise weights in A-fragment order: ps[(cg*64 + lane)*MB + mb] =
        // pw_w[o0 + 16*mb + lane%16][c0 + 4*cg + lane/16]
        for (int e = threadIdx.x; e < 16 * MB * CC; e += NT) {
            const int cl = e % CC;
            const int ol = e / CC;
            const int o = o0 + ol, c = c0 + cl;
            float v = 0.0f;
            if (o < d.O && c < d.C) v = pw_w[(int64_t)o * d.C + c];
            ps[((cl >> 2) * 64 + (cl & 3) * 16 + (ol & 15)) * MB + (ol >> 4)] = v;
        }
        for (int e = threadIdx.x; e < CC * 12; e += NT) {
            const int k = e % 12;
            const int c = e / 12;
            const int ci = c0 + c;
            float v = 0.0f;
            if (ci < d.C) {
                if (k < 9) v = dw_w[(int64_t)ci * 9 + k];
                else if (k == 9 && dw_b) v = dw_b[ci];
            }
            ds[e] = v;
        }
        __syncthreads();
        if (!active) continue;
#pragma unroll
        for (int cg = 0; cg < CC / 4; ++cg) {
            const float *dwp = ds + (4 * cg + (lane >> 4)) * 12;
            const floatx4 k0 = *reinterpret_cast<const floatx4 *>(dwp);
            const floatx4 k1 = *reinterpret_cast<const floatx4 *>(dwp + 4);
            const floatx4 k2 = *reinterpret_cast<const floatx4 *>(dwp + 8);
            const float kw9[9] = {k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3], k2[0]};
            const float dbias = k2[1];
            float a[MB];
#pragma unroll
            for (int i = 0; i < MB / 4; ++i) {
                const floatx4 v = *reinterpret_cast<const floatx4 *>(ps + (cg * 64 + lane) * MB + 4 * i);
                a[4 * i + 0] = v[0];
                a[4 * i + 1] = v[1];
                a[4 * i + 2] = v[2];
                a[4 * i + 3] = v[3];
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
                    for (int kw = 0; kw < 3; ++kw) v = fmaf(kw9[kh * 3 + kw], xv[r + kh][kw], v);
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) acc[mb][r] = mfma_16x16x4(a[mb], v, acc[mb][r]);
            }
        }
    }
    if (!active) return;

    const int wcol = w0 + 16 * wave + (lane & 15);
    if (wcol >= d.Wo) return;
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

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

template <int MB, int R, int WGW, int CC>
hipError_t launch(const float *x, const float *dw_w, const float *dw_b, const float *pw_w,
                  const float *pw_b, float *y, const DwsepDims &d, hipStream_t s)
{
    const int64_t tw = cdiv(d.Wo, 16 * WGW), th = cdiv(d.Ho, R), og = cdiv(d.O, 16 * MB);
    const int64_t tiles = tw * th * d.N * og;
    if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((dwsep_kernel<MB, R, WGW, CC>), dim3((unsigned)tiles), dim3(64 * WGW), 0,
                       s, x, dw_w, dw_b, pw_w, pw_b, y, d, tiles, (int)tw, (int)th);
    return hipGetLastError();
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
