// unfused.hip -- the separate steps of the unfused path (the pages' main alternative to
// fusion: a convolution that writes its output to memory, then separate epilogue and
// reduction kernels; page "Kimi-K2.6 l2_p47", the library-conv + elementwise split; page
// "Kimi-K2.6 l2_p8", the hybrid of a library conv and a reduction kernel; page "Kimi-K2.6
// l1_p86", separate depthwise and pointwise passes).  Together with the identity epilogue
// of the conv kernels and the pointwise-only mode of the dwsep kernels they measure what
// the fused kernels save.
#include "common.hpp"
#include "kernels.hpp"

namespace convfuse {

namespace {

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Grid of at most this many workgroups for the grid-stride loops.
inline unsigned stride_grid(int64_t items, int per_block)
{
    int64_t g = cdiv(items, per_block);
    if (g > 65536) g = 65536;
    return (unsigned)(g > 0 ? g : 1);
}

// y[i] = tanh(mish(v[i])) (v may alias y).  VEC: both 16-byte aligned; quads first, then the
// tail.
template <bool VEC>
__global__ __launch_bounds__(256) void mish_tanh_kernel(const float *v, float *y, int64_t count)
{
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
    int64_t done = 0;
    if constexpr (VEC) {
        const int64_t quads = count / 4;
        for (int64_t q = i0; q < quads; q += stride) {
            const floatx4 a = reinterpret_cast<const floatx4 *>(v)[q];
            reinterpret_cast<floatx4 *>(y)[q] =
                floatx4{mish_tanh(a[0]), mish_tanh(a[1]), mish_tanh(a[2]), mish_tanh(a[3])};
        }
        done = quads * 4;
    }
    for (int64_t i = done + i0; i < count; i += stride) y[i] = mish_tanh(v[i]);
}

// From a stored conv output c [N][C][OD][OH][OW]: out[n] += sum over channel c and windows
// of max((c + 0) / divisor) / count, one workgroup per (n, c) pair, one atomicAdd each.  The
// divide comes before the max (the definition's order).  out[n] must hold sum_c bias[c].
__global__ __launch_bounds__(256) void pool_reduce_kernel(const float *__restrict__ conv,
                                                          float *__restrict__ out, PoolDims p,
                                                          int pool, float inv_count)
{
    const Conv3dDims &d = p.conv;
    const int64_t nc = blockIdx.x;
    const int64_t n = nc / d.O;
    const float *cp = conv + nc * d.OD * d.OH * d.OW;
    const int64_t windows = p.PD * p.PH * p.PW;
    float part = 0.0f;
    for (int64_t wi = threadIdx.x; wi < windows; wi += 256) {
        const int64_t pw = wi % p.PW, t = wi / p.PW;
        const int64_t ph = t % p.PH, pd = t / p.PH;
        float m = -INFINITY;
        for (int a = 0; a < pool; ++a)
            for (int b = 0; b < pool; ++b) {
                const float *row = cp + ((pd * pool + a) * d.OH + ph * pool + b) * d.OW + pw * pool;
                for (int e = 0; e < pool; ++e) m = fmaxf(m, row[e] / p.divisor);
            }
        part += m;
    }
    __shared__ float red[4];
    part = wave_sum(part);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = part;
    __syncthreads();
    if (threadIdx.x == 0) atomicAdd(out + n, (red[0] + red[1] + red[2] + red[3]) * inv_count);
}

// Depthwise K x K (stride, padding, dilation, optional bias): thread t computes the 4
// consecutive outputs of row (n, c, oh) starting at column 4*q; rows of the input it needs
// come from L1/L2.  VEC: Wo % 4 == 0 and y 16-byte aligned (float4 stores).
template <bool VEC>
__global__ __launch_bounds__(256) void depthwise_kernel(const float *__restrict__ x,
                                                        const float *__restrict__ dw_w,
                                                        const float *__restrict__ dw_b,
                                                        float *__restrict__ y, DwsepDims d,
                                                        GenConv g)
{
    const int64_t quads = (d.Wo + 3) / 4;
    const int64_t total = d.N * d.C * d.Ho * quads;
    const int64_t stride = (int64_t)gridDim.x * 256;
    const int K = g.k;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += stride) {
        const int64_t q = i % quads, t = i / quads;
        const int64_t oh = t % d.Ho, nc = t / d.Ho;
        const int64_t c = nc % d.C;
        const float *xc = x + nc * d.H * d.W;
        const float *wc = dw_w + c * K * K;
        const float bias = dw_b ? dw_b[c] : 0.0f;
        float acc[4] = {bias, bias, bias, bias};
        const int64_t ow0 = 4 * q;
        for (int kh = 0; kh < K; ++kh) {
            const int64_t ih = oh * g.stride - d.pad + kh * g.dilation;
            if (ih < 0 || ih >= d.H) continue;
            const float *xr = xc + ih * d.W;
            for (int kw = 0; kw < K; ++kw) {
                const float wv = wc[kh * K + kw];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t iw = (ow0 + e) * g.stride - d.pad + kw * g.dilation;
                    if (ow0 + e < d.Wo && iw >= 0 && iw < d.W) acc[e] = fmaf(wv, xr[iw], acc[e]);
                }
            }
        }
        float *yr = y + (nc * d.Ho + oh) * d.Wo + ow0;
        if (VEC) {
            *reinterpret_cast<floatx4 *>(yr) = floatx4{acc[0], acc[1], acc[2], acc[3]};
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (ow0 + e < d.Wo) yr[e] = acc[e];
        }
    }
}

}  // namespace

hipError_t launch_mish_tanh(const float *v, float *y, int64_t count, hipStream_t s)
{
    const bool vec = ((uintptr_t)v & 15) == 0 && ((uintptr_t)y & 15) == 0;
    const unsigned grid = stride_grid(vec ? cdiv(count, 4) : count, 256);
    note_kernel("mish_tanh_kernel");
    if (vec)
        hipLaunchKernelGGL(mish_tanh_kernel<true>, dim3(grid), dim3(256), 0, s, v, y, count);
    else
        hipLaunchKernelGGL(mish_tanh_kernel<false>, dim3(grid), dim3(256), 0, s, v, y, count);
    return hipGetLastError();
}

hipError_t launch_div_maxpool_gap_bias_sum(const float *conv, const float *bias, float *out,
                                           const PoolDims &p, int pool, hipStream_t s)
{
    const Conv3dDims &d = p.conv;
    hipError_t e = launch_pool_sum_init(bias, out, d.N, d.O, s);
    if (e != hipSuccess) return e;
    const int64_t blocks = d.N * d.O;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const float inv_count = (float)(1.0 / ((double)p.PD * (double)p.PH * (double)p.PW));
    note_kernel("pool_reduce_kernel");
    hipLaunchKernelGGL(pool_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, s, conv, out, p,
                       pool, inv_count);
    return hipGetLastError();
}

hipError_t launch_depthwise_conv2d(const float *x, const float *dw_w, const float *dw_b,
                                   float *y, const DwsepDims &d, const GenConv &g, hipStream_t s)
{
    const int64_t total = d.N * d.C * d.Ho * ((d.Wo + 3) / 4);
    const unsigned grid = stride_grid(total, 256);
    note_kernel("depthwise_kernel");
    if (d.Wo % 4 == 0 && ((uintptr_t)y & 15) == 0)
        hipLaunchKernelGGL(depthwise_kernel<true>, dim3(grid), dim3(256), 0, s, x, dw_w, dw_b, y,
                           d, g);
    else
        hipLaunchKernelGGL(depthwise_kernel<false>, dim3(grid), dim3(256), 0, s, x, dw_w, dw_b,
                           y, d, g);
    return hipGetLastError();
}

}  // namespace convfuse
