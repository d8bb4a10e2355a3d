// conv3d_split.hip -- Conv3d + Mish + tanh (k = 3, stride 1, pad <= 2) and the Conv3d +
// divide + max-pool + channel-sum layer (k = 3, pool 2) with the implicit GEMM on bf16 matrix
// cores as a three-term split of fp32: the opt-in reduced-precision mode the
// pages weigh against true fp32 (page "Kimi-K2.6 l2_p47", the roofline estimate and the
// mma-precision paragraph; gfx950 has no TF32-like format, so fp32 is emulated).  Each fp32
// operand v splits into hi = bf16(v) and lo = bf16(v - hi); v*w is taken as
// hi*hi + hi*lo + lo*hi with fp32 accumulation.  The bias and the tanh(mish) epilogue are fp32.
//
// GEMM view as in the fp32 kernel (rows = output voxels, columns = output channels), with a
// 16x16x32 k-step of 8 input channels x 4 taps: lane group g holds taps 4s + g of k-step s
// (s < 7; the 28th tap has zero weights), element i input channel c0 + i.  The input halo is
// staged in LDS already split and channel-interleaved -- per halo position 8 channels of hi
// (16 bytes) and 8 of lo -- so each operand fragment is one 16-byte LDS read; the weights are
// staged split in fragment order.  Workgroup = 2 x 2 waves, each wave one output row of 64
// voxels x 16*MB output channels; chunks of 8 input channels, the next one prefetched into
// registers while the current one computes.
#include "common.hpp"
#include "conv3d_tile.hpp"
#include "kernels.hpp"

namespace convfuse {

namespace {

constexpr int kSpCC = 8;     // input channels per chunk: the 8 elements of a fragment
constexpr int kSpSteps = 7;  // k-steps per chunk: 28 taps (27 + one with zero weights)

// Split halo of NT threads: HD x HH rows of RSX positions, each 8 channels of hi and of lo.
template <int NT_, int HD_, int HH_, int RSX_>
struct SpHalo {
    static constexpr int NT = NT_, HD = HD_, HH = HH_, RSX = RSX_;
    static constexpr int POS = HD * HH * RSX;                // halo positions
    static constexpr int PPT = (POS + NT - 1) / NT;          // positions per thread
};

// Conv3d tile: WD x WH waves, each one output row of 64 voxels; halo column c holds input
// column ow0 - 4 + c.
template <int WD_, int WH_>
struct SpGeom : SpHalo<64 * WD_ * WH_, WD_ + 2, WH_ + 2, 72> {
    static constexpr int WD = WD_, WH = WH_, NBW = 4;
};

// One chunk in registers between the global loads and the split LDS stores.
// x: position p = tid + NT*u, 8 channels each.  w: (output, input channel) pair
// q = tid + NT*u, numbered q = (m*MB + mb)*8 + i for output channel o0 + 16*mb + m and input
// channel c0 + i; its 27 taps are contiguous in memory.
template <int MB, class G>
struct SpStage {
    static constexpr int PAIRS = 16 * MB * kSpCC;
    static constexpr int PPQ = (PAIRS + G::NT - 1) / G::NT;
    float xv[G::PPT][8];
    float wv[PPQ][27];

    __device__ __forceinline__ void load(const float *__restrict__ x, const float *__restrict__ w,
                                         const Conv3dDims &d, int64_t n, int c0, int o0, int id0,
                                         int ih0, int iw0)
    {
        const int tid = threadIdx.x;
        const int64_t plane = d.D * d.H * d.W;
#pragma unroll
        for (int u = 0; u < G::PPT; ++u) {
            const int p = tid + G::NT * u;
            const int hd = p / (G::HH * G::RSX), rem = p % (G::HH * G::RSX);
            const int hh = rem / G::RSX, col = rem % G::RSX;
            const int id = id0 + hd, ih = ih0 + hh, iw = iw0 + col;
            const bool ok = p < G::POS && (unsigned)id < (unsigned)d.D &&
                            (unsigned)ih < (unsigned)d.H && (unsigned)iw < (unsigned)d.W;
            const float *src =
                x + (n * d.C + c0) * plane + ok * (((int64_t)id * d.H + ih) * d.W + iw);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                xv[u][i] = ok && c0 + i < d.C ? src[i * plane] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < PPQ; ++u) {
            const int q = tid + G::NT * u;
            const int i = q & 7, mb = (q >> 3) % MB, m = (q >> 3) / MB;
            const int o = o0 + 16 * mb + m, c = c0 + i;
            const bool ok = q < PAIRS && o < d.O && c < d.C;
            const float *src = w + ((int64_t)(ok ? o : 0) * d.C + (ok ? c : 0)) * 27;
#pragma unroll
            for (int t = 0; t < 27; ++t) wv[u][t] = ok ? src[t] : 0.0f;
        }
    }

    // xs_hi / xs_lo: [POS] fragments; ws_hi / ws_lo: [7][64][MB] fragments (entry of k-step s,
    // lane 16*g + m, block mb holds taps 4s + g of output channel 16*mb + m).
    __device__ __forceinline__ void store(bf16x8 *xs_hi, bf16x8 *xs_lo, __bf16 *ws_hi,
                                          __bf16 *ws_lo) const
    {
        const int tid = threadIdx.x;
#pragma unroll
        for (int u = 0; u < G::PPT; ++u) {
            const int p = tid + G::NT * u;
            if (p >= G::POS) continue;
            bf16x8 hi, lo;
            split_bf16(xv[u], hi, lo);
            xs_hi[p] = hi;
            xs_lo[p] = lo;
        }
#pragma unroll
        for (int u = 0; u < PPQ; ++u) {
            const int q = tid + G::NT * u;
            if (q >= PAIRS) continue;
            const int i = q & 7, mb = (q >> 3) % MB, m = (q >> 3) / MB;
#pragma unroll
            for (int t = 0; t < 27; ++t) {
                const int s = t >> 2, g = t & 3;
                const int e = ((s * 64 + 16 * g + m) * MB + mb) * 8 + i;
                const __bf16 h = (__bf16)wv[u][t];
                ws_hi[e] = h;
                ws_lo[e] = (__bf16)(wv[u][t] - (float)h);
            }
        }
    }
};

template <int MB, int WD, int WH, bool ACT, int SW>
__global__ __launch_bounds__(64 * WD * WH, 8 / (WD * WH)) void conv3d_split_kernel(
    const float *__restrict__ x, const float *__restrict__ w, const float *__restrict__ b,
    float *__restrict__ y, Conv3dDims d, int64_t tiles, int tiles_w, int tiles_h, int tiles_d)
{
    using G = SpGeom<WD, WH>;
    constexpr int NBW = G::NBW;
    constexpr int WENT = kSpSteps * 64 * MB;  // weight fragments per chunk
    __shared__ bf16x8 xs_hi[G::POS], xs_lo[G::POS];
    __shared__ bf16x8 ws_hi[WENT], ws_lo[WENT];

    int64_t t = xcd_tile(blockIdx.x, tiles);
    const int tw = (int)(t % tiles_w); t /= tiles_w;
    const int th = (int)(t % tiles_h); t /= tiles_h;
    const int td = (int)(t % tiles_d); t /= tiles_d;
    const int64_t n = t % d.N;
    const int o0 = (int)(t / d.N) * 16 * MB;
    const int od0 = td * G::WD, oh0 = th * G::WH, ow0 = tw * 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wd = wave / G::WH, wh = wave % G::WH, g = lane >> 4;

    // the 28th tap (k-step 6, lane group 3) has zero weights; they are never restaged
    if (threadIdx.x < 16 * MB) {
        const int m = threadIdx.x / MB, mb = threadIdx.x % MB;
        const int e = (6 * 64 + 48 + m) * MB + mb;
        ws_hi[e] = bf16x8{};
        ws_lo[e] = bf16x8{};
    }
    // B-fragment position of lane (g, j) at k-step s: halo (wd + kd, wh + kh, j + kw + 4 - pad)
    // for tap 4s + g = (kd, kh, kw); the zero-weight 28th tap reads tap 26's position.
    int toff[kSpSteps];
#pragma unroll
    for (int s = 0; s < kSpSteps; ++s) {
        const int tp = 4 * s + g < 27 ? 4 * s + g : 26;
        const int kd = tp / 9, kh = (tp / 3) % 3, kw = tp % 3;
        toff[s] = ((wd + kd) * G::HH + wh + kh) * G::RSX + (lane & 15) + kw + 4 - d.pad;
    }

    SpStage<MB, G> stage;
    const int id0 = od0 - d.pad, ih0 = oh0 - d.pad, iw0 = ow0 - 4;
    stage.load(x, w, d, n, 0, o0, id0, ih0, iw0);
    const int od = od0 + wd, oh = oh0 + wh;
    const bool active = od < d.OD && oh < d.OH;
    floatx4 acc[MB][NBW];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < d.C; c0 += kSpCC) {
        __syncthreads();
        stage.store(xs_hi, xs_lo, reinterpret_cast<__bf16 *>(ws_hi),
                    reinterpret_cast<__bf16 *>(ws_lo));
        __syncthreads();
        if (c0 + kSpCC < d.C) stage.load(x, w, d, n, c0 + kSpCC, o0, id0, ih0, iw0);
        if (!active) continue;  // (this wave only helps stage the shared tiles)
#pragma unroll
        for (int s = 0; s < kSpSteps; ++s) {
            bf16x8 wh_[MB], wl_[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                wh_[mb] = ws_hi[(s * 64 + lane) * MB + mb];
                wl_[mb] = ws_lo[(s * 64 + lane) * MB + mb];
            }
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const bf16x8 xh = xs_hi[toff[s] + 16 * nb], xl = xs_lo[toff[s] + 16 * nb];
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    acc[mb][nb] = mfma_16x16x32_bf16(xl, wh_[mb], acc[mb][nb]);
                    acc[mb][nb] = mfma_16x16x32_bf16(xh, wl_[mb], acc[mb][nb]);
                    acc[mb][nb] = mfma_16x16x32_bf16(xh, wh_[mb], acc[mb][nb]);
                }
            }
        }
    }
    if (active) store_conv_row<MB, NBW, ACT, SW>(y, b, d, n, od, oh, ow0, o0, acc);
}

// ------------------------------------------------------------------ pooling layer
// Conv3d (k = 3, no padding), divide, 2x2x2 max-pool, then the pooled channel sum (or, STORE,
// the pooled tensor), with the Conv3d on the split.  Workgroup = WH waves; wave w owns pooled
// row (n, pd0, ph0 + w), the 8*NBW pooled columns from pw0 and output channels
// [o0, o0 + 16).  Its conv voxels come in 4*NBW blocks (dd, dh, q): conv voxel
// (2*pd0 + dd, 2*(ph0 + w) + dh, 2*pw0 + 16*q + j) for MFMA row j.  Halo: 4 depth planes x
// (2*WH + 2) rows x (16*NBW + 2) columns (column c holds input column 2*pw0 + c).  The voxels
// are the MFMA rows, so a lane holds 4 consecutive conv columns of one channel: two whole
// windows, whose maximum needs no other lane.
template <int WH, int NBW>
using SpPoolGeom = SpHalo<64 * WH, 4, 2 * WH + 2, 16 * NBW + 2>;

template <int WH, int NBW, bool STORE>
__global__ __launch_bounds__(64 * WH, 8 / WH) void conv3d_pool_split_kernel(
    const float *__restrict__ x, const float *__restrict__ w, const float *__restrict__ cb,
    float *__restrict__ out, PoolDims p, int64_t tiles, int tiles_w, int tiles_h,
    float inv_count)
{
    using G = SpPoolGeom<WH, NBW>;
    constexpr int NB = 4 * NBW;
    constexpr int WENT = kSpSteps * 64;  // weight fragments per chunk (16 outputs)
    __shared__ bf16x8 xs_hi[G::POS], xs_lo[G::POS];
    __shared__ bf16x8 ws_hi[WENT], ws_lo[WENT];
    const Conv3dDims &d = p.conv;

    int64_t t = xcd_tile(blockIdx.x, tiles);
    const int tw = (int)(t % tiles_w); t /= tiles_w;
    const int th = (int)(t % tiles_h); t /= tiles_h;
    const int pd0 = (int)(t % p.PD); t /= p.PD;
    const int64_t n = t % d.N;
    const int o0 = (int)(t / d.N) * 16;
    const int ph0 = th * WH, pw0 = tw * 8 * NBW;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4;

    if (threadIdx.x < 16) {  // the 28th tap's weights are zero and never restaged
        const int e = 6 * 64 + 48 + threadIdx.x;
        ws_hi[e] = bf16x8{};
        ws_lo[e] = bf16x8{};
    }
    // lane (g, j) at k-step s: halo (kd + dd, 2*wave + dh + kh, 16*q + j + kw) for tap
    // 4s + g = (kd, kh, kw) of block (dd, dh, q); toff holds the part without (dd, dh, q)
    int toff[kSpSteps];
#pragma unroll
    for (int s = 0; s < kSpSteps; ++s) {
        const int tp = 4 * s + g < 27 ? 4 * s + g : 26;
        const int kd = tp / 9, kh = (tp / 3) % 3, kw = tp % 3;
        toff[s] = (kd * G::HH + 2 * wave + kh) * G::RSX + (lane & 15) + kw;
    }

    const int id0 = 2 * pd0, ih0 = 2 * ph0, iw0 = 2 * pw0;
    const int ph = ph0 + wave;
    const bool active = ph < p.PH;
    floatx4 acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = floatx4{0.f, 0.f, 0.f, 0.f};
    // Each chunk is loaded right before it is stored (no prefetch: its registers would stay
    // live through the MFMAs); the other resident workgroups cover the latency.
    for (int c0 = 0; c0 < d.C; c0 += kSpCC) {
        __syncthreads();
        {
            SpStage<1, G> stage;
            stage.load(x, w, d, n, c0, o0, id0, ih0, iw0);
            stage.store(xs_hi, xs_lo, reinterpret_cast<__bf16 *>(ws_hi),
                        reinterpret_cast<__bf16 *>(ws_lo));
        }
        __syncthreads();
        if (!active) continue;  // (this wave only helps stage the shared tiles)
#pragma unroll
        for (int s = 0; s < kSpSteps; ++s) {
            const bf16x8 wh_ = ws_hi[s * 64 + lane], wl_ = ws_lo[s * 64 + lane];
#pragma unroll
            for (int dd = 0; dd < 2; ++dd)
#pragma unroll
                for (int dh = 0; dh < 2; ++dh)
#pragma unroll
                    for (int q = 0; q < NBW; ++q) {
                        const int b = (dd * 2 + dh) * NBW + q;
                        const int pos = toff[s] + (dd * G::HH + dh) * G::RSX + 16 * q;
                        const bf16x8 xh = xs_hi[pos], xl = xs_lo[pos];
                        acc[b] = mfma_16x16x32_bf16(xl, wh_, acc[b]);
                        acc[b] = mfma_16x16x32_bf16(xh, wl_, acc[b]);
                        acc[b] = mfma_16x16x32_bf16(xh, wh_, acc[b]);
                    }
        }
    }
    if (!active) return;  // (no barrier follows)
    // (conv + cb) / divisor is monotone in conv: the window's extreme of the divided values is
    // (max conv + cb) / divisor for a positive divisor, (min conv + cb) / divisor otherwise.
    const bool use_min = p.divisor < 0.0f;
    const int o = o0 + (lane & 15);
    const float cbv = (cb && o < d.O) ? cb[o] : 0.0f;
    float part = 0.0f;
#pragma unroll
    for (int q = 0; q < NBW; ++q)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            float m = acc[q][2 * half];
#pragma unroll
            for (int b2 = 0; b2 < 4; ++b2)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const float v = acc[b2 * NBW + q][2 * half + e];
                    m = use_min ? fminf(m, v) : fmaxf(m, v);
                }
            const int pw = pw0 + 8 * q + 2 * g + half;
            if (o < d.O && pw < p.PW) {
                const float v = (m + cbv) / p.divisor;
                if constexpr (STORE)
                    out[(((n * d.O + o) * p.PD + pd0) * p.PH + ph) * p.PW + pw] = v;
                else
                    part += v;
            }
        }
    if constexpr (!STORE) {
        part = wave_sum(part);
        if (lane == 0) atomicAdd(out + n, part * inv_count);
    }
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

template <int MB, int WD, int WH, bool ACT>
hipError_t launch_split(const float *x, const float *w, const float *b, float *y,
                        const Conv3dDims &d, hipStream_t s)
{
    using G = SpGeom<WD, WH>;
    const int64_t tw = cdiv(d.OW, 64), th = cdiv(d.OH, G::WH), td = cdiv(d.OD, G::WD);
    const int64_t tiles = tw * th * td * d.N * cdiv(d.O, 16 * MB);
    if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const int sw = conv_store_width(y, d.OW);
    auto go = [&](auto kern) {
        note_kernel("conv3d_split_kernel");
        hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(G::NT), 0, s, x, w, b, y, d, tiles,
                           (int)tw, (int)th, (int)td);
    };
    if (sw == 4) go(conv3d_split_kernel<MB, WD, WH, ACT, 4>);
    else if (sw == 2) go(conv3d_split_kernel<MB, WD, WH, ACT, 2>);
    else go(conv3d_split_kernel<MB, WD, WH, ACT, 1>);
    return hipGetLastError();
}

}  // namespace

namespace {

template <bool STORE>
hipError_t launch_pool_split(const float *x, const float *w, const float *conv_b, float *out,
                             const PoolDims &p, hipStream_t s)
{
    constexpr int WH = 4, NBW = 1;
    const Conv3dDims &d = p.conv;
    const int64_t tw = cdiv(p.PW, 8 * NBW), th = cdiv(p.PH, WH);
    const int64_t tiles = tw * th * p.PD * d.N * cdiv(d.O, 16);
    if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const float inv_count = (float)(1.0 / ((double)p.PD * (double)p.PH * (double)p.PW));
    note_kernel("conv3d_pool_split_kernel");
    hipLaunchKernelGGL((conv3d_pool_split_kernel<WH, NBW, STORE>), dim3((unsigned)tiles),
                       dim3(64 * WH), 0, s, x, w, conv_b, out, p, tiles, (int)tw, (int)th,
                       inv_count);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_conv3d_pool_sum_split_bf16(const float *x, const float *w,
                                             const float *conv_b, const float *bias, float *out,
                                             const PoolDims &p, hipStream_t s)
{
    const hipError_t e = launch_pool_sum_init(bias, out, p.conv.N, p.conv.O, s);
    if (e != hipSuccess) return e;
    return launch_pool_split<false>(x, w, conv_b, out, p, s);
}

hipError_t launch_conv3d_mish_tanh_split_bf16(const float *x, const float *w, const float *b,
                                              float *y, const Conv3dDims &d, hipStream_t s)
{
    if (d.O > 16) return launch_split<2, 2, 2, true>(x, w, b, y, d, s);
    return launch_split<1, 2, 2, true>(x, w, b, y, d, s);
}

}  // namespace convfuse
