// generic.hip -- the three fused operations for any kernel size, stride, padding, dilation and
// pooling size, on gfx950 fp32 matrix cores.
//
// The tuned kernels (conv3d_igemm.hip, dwsep.hip) cover k = 3, stride 1, pad <= 2 (and, for
// the pooled sum, a 2x2x2 pool; for dwsep, dilation 1).  These kernels compute the same
// definitions for every other parameter set (page "Kimi-K2.6 l2_p47", generalised stride and
// padding of the Conv3d; page "Kimi-K2.6 l1_p86", stride/padding/dilation and kernel sizes
// 1/3/5/7 of the depthwise-separable Conv2d; page "Kimi-K2.6 l2_p8", the pooled channel sum).
//
// Conv3d with kernel size 3, 5 or 7 and stride 1 or 2 (any padding) runs an LDS-staged
// implicit GEMM with the tuned kernel's organisation (conv3d_staged_kernel).  Everything else
// is a direct implicit GEMM over global memory: one wave owns 16*MB output channels x 16*NB
// output positions along W, and each 16x16x4 MFMA k-step gathers its operands straight from
// global memory (L1/L2 serve the reuse) with zero padding by bounds checks; there is no LDS
// staging and no inter-wave synchronisation except the pooled sum's window reduction.
// The GEMM K order is tap-major, input-channel-minor: a k-step is four input channels at one
// tap, lane l supplying input channel 4*cg + l/16.
#include "common.hpp"
#include "conv3d_tile.hpp"
#include "kernels.hpp"

namespace convfuse {

namespace {

constexpr int kGenWaves = 4;  // waves per workgroup (independent tiles)

// Conv3d accumulators of one wave: output channels o0 + 16*mb + (4*(l/16) + r) at output
// voxel (n, od, oh, ow0 + 16*nb + l%16), before bias.
template <int MB, int NB>
__device__ __forceinline__ void conv3d_direct(const float *__restrict__ x,
                                              const float *__restrict__ w, const Conv3dDims &d,
                                              const GenConv &g, int64_t n, int od, int oh,
                                              int ow0, int o0, floatx4 (&acc)[MB][NB])
{
    const int lane = threadIdx.x & 63, j = lane & 15, cq = lane >> 4;
    const int k = g.k, k3 = k * k * k;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
    int iw[NB];
    bool owok[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int ow = ow0 + 16 * nb + j;
        owok[nb] = ow < d.OW;
        iw[nb] = ow * g.stride - d.pad;
    }
    for (int kd = 0; kd < k; ++kd) {
        const int id = od * g.stride - d.pad + kd;
        if ((unsigned)id >= (unsigned)d.D) continue;  // zero plane: no contribution
        for (int kh = 0; kh < k; ++kh) {
            const int ih = oh * g.stride - d.pad + kh;
            if ((unsigned)ih >= (unsigned)d.H) continue;
            for (int kw = 0; kw < k; ++kw) {
                const int tap = (kd * k + kh) * k + kw;
                for (int c4 = 0; c4 < d.C; c4 += 4) {
                    const int c = c4 + cq;
                    const bool cok = c < d.C;
                    float a[MB], b[NB];
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        const int o = o0 + 16 * mb + j;
                        a[mb] = cok && o < d.O ? w[((int64_t)o * d.C + c) * k3 + tap] : 0.0f;
                    }
                    const float *xrow = x + ((n * d.C + (cok ? c : 0)) * d.D + id) * d.H * d.W +
                                        (int64_t)ih * d.W;
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        const int col = iw[nb] + kw;
                        b[nb] = cok && owok[nb] && (unsigned)col < (unsigned)d.W ? xrow[col] : 0.0f;
                    }
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
                            acc[mb][nb] = mfma_16x16x4(a[mb], b[nb], acc[mb][nb]);
                }
            }
        }
    }
}

// ------------------------------------------------------------------ staged general Conv3d
// Workgroup = 2 x 2 waves; wave (wd, wh) owns output row (od0 + wd, oh0 + wh), columns
// [ow0, ow0 + 16*NBW) and output channels [o0, o0 + 16*MB).  The K loop runs over chunks of
// four input channels at one kernel depth kd.  Per channel and per output depth of the tile a
// chunk stages the HHR input rows that the tile's two output rows reach, COLS columns each
// (the columns its 16*NBW outputs reach), plus the chunk's K*K taps of weights in A-fragment
// order.  The next chunk is loaded into registers while the current one computes.
template <int K, int S, int NBW>
struct StagedGeom {
    static constexpr int WD = 2, WH = 2, NT = 64 * WD * WH;
    static constexpr int HHR = (WH - 1) * S + K;          // input rows per (channel, depth)
    static constexpr int COLS = (16 * NBW - 1) * S + K;   // input columns per row
    static constexpr int RS = round_up(COLS, 4);
    static constexpr int CS = halo_channel_stride(WD * HHR * RS);
    static constexpr int XS = 4 * CS;
    static constexpr int ROWS = 4 * WD * HHR;             // staged rows per chunk
    static constexpr int RPW = (ROWS + 3) / 4;            // rows per wave
    static constexpr int CPL = (COLS + 63) / 64;          // columns per lane
};

// Input rows of one chunk in registers between global load and LDS store.  Wave w handles
// rows r = w + 4i: channel r / (WD*HHR), tile depth (r / HHR) % WD, row r % HHR; lane l
// columns l + 64j.  LDS column c holds input column ow0*S - pad + c.
template <int K, int S, int NBW>
struct StagedHalo {
    using G = StagedGeom<K, S, NBW>;
    float v[G::RPW][G::CPL];

    __device__ __forceinline__ void load(const float *__restrict__ x, const Conv3dDims &d,
                                         int64_t n, int c0, int kd, int od0, int oh0, int ow0)
    {
        const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
        const int iw0 = ow0 * S - d.pad;
#pragma unroll
        for (int i = 0; i < G::RPW; ++i) {
            const int r = wave + 4 * i;
            const int cl = r / (G::WD * G::HHR), rem = r % (G::WD * G::HHR);
            const int wdp = rem / G::HHR, hr = rem % G::HHR;
            const int c = c0 + cl, id = (od0 + wdp) * S - d.pad + kd, ih = oh0 * S - d.pad + hr;
            const bool rowok = r < G::ROWS && c < d.C && (unsigned)id < (unsigned)d.D &&
                               (unsigned)ih < (unsigned)d.H;
            const float *src =
                x + (((n * d.C + (rowok ? c : 0)) * d.D + (rowok ? id : 0)) * d.H +
                     (rowok ? ih : 0)) * d.W;
#pragma unroll
            for (int jj = 0; jj < G::CPL; ++jj) {
                const int col = lane + 64 * jj, iw = iw0 + col;
                v[i][jj] = rowok && col < G::COLS && (unsigned)iw < (unsigned)d.W ? src[iw] : 0.0f;
            }
        }
    }

    __device__ __forceinline__ void store(float *__restrict__ xs) const
    {
        const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
        for (int i = 0; i < G::RPW; ++i) {
            const int r = wave + 4 * i;
            if (r >= G::ROWS) continue;
            const int cl = r / (G::WD * G::HHR), rem = r % (G::WD * G::HHR);
            const int wdp = rem / G::HHR, hr = rem % G::HHR;
            float *dst = xs + cl * G::CS + (wdp * G::HHR + hr) * G::RS;
#pragma unroll
            for (int jj = 0; jj < G::CPL; ++jj) {
                const int col = lane + 64 * jj;
                if (col < G::COLS) dst[col] = v[i][jj];
            }
        }
    }
};

// One chunk: K*K taps of one k-step each (four channels); voxels are the MFMA rows.
template <int MB, int NBW, int K, int S>
__device__ __forceinline__ void staged_chunk(const float *__restrict__ xs,
                                             const float *__restrict__ ws, int xlane,
                                             floatx4 (&acc)[MB][NBW])
{
    using G = StagedGeom<K, S, NBW>;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int kh = 0; kh < K; ++kh)
#pragma unroll
        for (int kw = 0; kw < K; ++kw) {
            float a[MB];
            load_afrag<MB>(ws + ((kh * K + kw) * 64 + lane) * MB, a);
            float bv[NBW];
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) bv[nb] = xs[xlane + kh * G::RS + kw + 16 * S * nb];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb)
                    acc[mb][nb] = mfma_16x16x4(bv[nb], a[mb], acc[mb][nb]);
        }
}

template <int MB, int NBW, int K, int S, bool ACT, int SW>
__global__ __launch_bounds__(256, 2) void conv3d_staged_kernel(
    const float *__restrict__ x, const float *__restrict__ w, const float *__restrict__ b,
    float *__restrict__ y, Conv3dDims d, int64_t tiles, int tiles_w, int tiles_h, int tiles_d)
{
    using G = StagedGeom<K, S, NBW>;
    extern __shared__ __attribute__((aligned(16))) float dyn[];
    float *xs = dyn;
    float *ws = dyn + G::XS;

    int64_t t = xcd_tile(blockIdx.x, tiles);
    const int tw = (int)(t % tiles_w); t /= tiles_w;
    const int th = (int)(t % tiles_h); t /= tiles_h;
    const int td = (int)(t % tiles_d); t /= tiles_d;
    const int64_t n = t % d.N;
    const int og = (int)(t / d.N);
    const int od0 = td * G::WD, oh0 = th * G::WH, ow0 = tw * 16 * NBW, o0 = og * 16 * MB;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wd = wave / G::WH, wh = wave % G::WH;
    const int xlane = (lane >> 4) * G::CS + (wd * G::HHR + wh * S) * G::RS + (lane & 15) * S;

    StagedHalo<K, S, NBW> halo;
    WeightChunk<MB, 4, G::NT, K * K> wts;
    const int chunks = (int)((d.C + 3) / 4) * K;  // chunk q: channels 4*(q/K).., depth q%K
    auto load = [&](int q) {
        const int c0 = (q / K) * 4, kd = q % K;
        halo.load(x, d, n, c0, kd, od0, oh0, ow0);
        wts.load(w, d, o0, c0, K * K * K, kd * K * K);
    };
    load(0);
    const int od = od0 + wd, oh = oh0 + wh;
    const bool active = od < d.OD && oh < d.OH;
    floatx4 acc[MB][NBW];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < chunks; ++q) {
        __syncthreads();
        halo.store(xs);
        wts.store(ws);
        __syncthreads();
        if (q + 1 < chunks) load(q + 1);
        // (a wave whose row lies past the output only helps stage the shared tiles)
        if (active) staged_chunk<MB, NBW, K, S>(xs, ws, xlane, acc);
    }
    if (active) store_conv_row<MB, NBW, ACT, SW>(y, b, d, n, od, oh, ow0, o0, acc);
}

// Wave tile t: (og, n, od, oh, owb) with owb fastest.  ACT: tanh(mish(conv + b)), else
// conv + b.
template <int MB, int NB, bool ACT>
__global__ __launch_bounds__(64 * kGenWaves) void conv3d_mish_tanh_generic_kernel(
    const float *__restrict__ x, const float *__restrict__ w, const float *__restrict__ b,
    float *__restrict__ y, Conv3dDims d, GenConv g, int64_t tiles, int tiles_w)
{
    const int64_t t0 = (int64_t)blockIdx.x * kGenWaves + (threadIdx.x >> 6);
    if (t0 >= tiles) return;  // whole wave: no barrier below
    int64_t t = t0;
    const int owb = (int)(t % tiles_w);
    t /= tiles_w;
    const int oh = (int)(t % d.OH);
    t /= d.OH;
    const int od = (int)(t % d.OD);
    t /= d.OD;
    const int64_t n = t % d.N;
    const int og = (int)(t / d.N);
    const int ow0 = owb * 16 * NB, o0 = og * 16 * MB;
    floatx4 acc[MB][NB];
    conv3d_direct<MB, NB>(x, w, d, g, n, od, oh, ow0, o0, acc);
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int o = o0 + 16 * mb + 4 * (lane >> 4) + r;
            if (o >= d.O) continue;
            const float bias = b ? b[o] : 0.0f;
            float *yrow = y + (((n * d.O + o) * d.OD + od) * d.OH + oh) * d.OW;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int ow = ow0 + 16 * nb + (lane & 15);
                if (ow < d.OW) {
                    const float v = acc[mb][nb][r] + bias;
                    yrow[ow] = ACT ? mish_tanh(v) : v;
                }
            }
        }
}

// Pooled channel sum for any window size P (<= 16*NB): a wave owns pooled row (n, pd, ph)
// and pooled columns [pw0, pw0 + TWP), TWP = floor(16*NB / P), and all output channels of
// its group.  For each of the P*P conv rows of the window row it computes the conv outputs
// of its P*TWP conv columns, divides (conv + cb) by the divisor (the definition's order)
// and keeps the running maximum per (channel, column); the column maxima of each window are
// then taken through LDS.  One atomicAdd per wave adds its windows' sum / count to out[n].
// STORE: write each window's maximum to the pooled tensor out [N][O][PD][PH][PW] instead.
template <int MB, int NB, bool STORE>
__global__ __launch_bounds__(64 * kGenWaves) void conv3d_pool_sum_generic_kernel(
    const float *__restrict__ x, const float *__restrict__ w, const float *__restrict__ cb,
    float *__restrict__ out, PoolDims p, GenConv g, int pool, int64_t tiles, int tiles_w,
    float inv_count)
{
    constexpr int OC = 16 * MB, COLS = 16 * NB;
    __shared__ float mx[kGenWaves][OC][COLS + 1];
    const Conv3dDims &d = p.conv;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t t0 = (int64_t)blockIdx.x * kGenWaves + wave;
    if (t0 >= tiles) return;  // whole wave; only wave-local LDS is used below
    const int twp = COLS / pool;
    int64_t t = t0;
    const int pwb = (int)(t % tiles_w);
    t /= tiles_w;
    const int ph = (int)(t % p.PH);
    t /= p.PH;
    const int pd = (int)(t % p.PD);
    t /= p.PD;
    const int64_t n = t % d.N;
    const int og = (int)(t / d.N);
    const int pw0 = pwb * twp, ow0 = pw0 * pool, o0 = og * OC;

    floatx4 m[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) m[mb][nb] = floatx4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    for (int dd = 0; dd < pool; ++dd)
        for (int dh = 0; dh < pool; ++dh) {
            floatx4 acc[MB][NB];
            conv3d_direct<MB, NB>(x, w, d, g, n, pd * pool + dd, ph * pool + dh, ow0, o0, acc);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int o = o0 + 16 * mb + 4 * (lane >> 4) + r;
                    const float cbv = (cb && o < d.O) ? cb[o] : 0.0f;
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        const float v = (acc[mb][nb][r] + cbv) / p.divisor;
                        m[mb][nb][r] = fmaxf(m[mb][nb][r], v);
                    }
                }
        }
    // column maxima of each window through this wave's LDS slice
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                mx[wave][16 * mb + 4 * (lane >> 4) + r][16 * nb + (lane & 15)] = m[mb][nb][r];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float part = 0.0f;
    for (int e = lane; e < OC * twp; e += 64) {
        const int ol = e / twp, q = e % twp;
        const int o = o0 + ol, pw = pw0 + q;
        if (o >= d.O || pw >= p.PW) continue;
        float v = mx[wave][ol][q * pool];
        for (int i = 1; i < pool; ++i) v = fmaxf(v, mx[wave][ol][q * pool + i]);
        if constexpr (STORE)
            out[(((n * d.O + o) * p.PD + pd) * p.PH + ph) * p.PW + pw] = v;
        else
            part += v;
    }
    if constexpr (STORE) return;
    part = wave_sum(part);
    if (lane == 0) atomicAdd(out + n, part * inv_count);
}

// Depthwise (K x K, stride, padding, dilation, optional bias) then pointwise: a wave owns
// output row (n, oh), columns [ow0, ow0 + 16) and output channels [o0, o0 + 16*MB).  Lane l
// forms the B operand of a k-step, the depthwise output of channel c4 + l/16 at column
// ow0 + l%16, from K*K gathered inputs; the pointwise weights are the A operand.
template <int MB>
__global__ __launch_bounds__(64 * kGenWaves) void dwsep_generic_kernel(
    const float *__restrict__ x, const float *__restrict__ dw_w, const float *__restrict__ dw_b,
    const float *__restrict__ pw_w, const float *__restrict__ pw_b, float *__restrict__ y,
    DwsepDims d, GenConv g, int64_t tiles, int tiles_w)
{
    const int64_t t0 = (int64_t)blockIdx.x * kGenWaves + (threadIdx.x >> 6);
    if (t0 >= tiles) return;
    int64_t t = t0;
    const int owb = (int)(t % tiles_w);
    t /= tiles_w;
    const int oh = (int)(t % d.Ho);
    t /= d.Ho;
    const int64_t n = t % d.N;
    const int og = (int)(t / d.N);
    const int ow0 = owb * 16, o0 = og * 16 * MB;
    const int lane = threadIdx.x & 63, j = lane & 15, cq = lane >> 4;
    const int K = g.k, KK = K * K;
    const int ow = ow0 + j;
    const bool owok = ow < d.Wo;
    const int iw0 = ow * g.stride - d.pad, ih0 = oh * g.stride - d.pad;

    floatx4 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int o = o0 + 16 * mb + 4 * cq + r;
            acc[mb][r] = (pw_b && o < d.O) ? pw_b[o] : 0.0f;
        }
    for (int c4 = 0; c4 < d.C; c4 += 4) {
        const int c = c4 + cq;
        const bool cok = c < d.C;
        float v = 0.0f;
        if (cok && owok) {
            v = dw_b ? dw_b[c] : 0.0f;
            const float *xc = x + (n * d.C + c) * d.H * d.W;
            const float *wc = dw_w + (int64_t)c * KK;
            for (int kh = 0; kh < K; ++kh) {
                const int ih = ih0 + kh * g.dilation;
                if ((unsigned)ih >= (unsigned)d.H) continue;
                for (int kw = 0; kw < K; ++kw) {
                    const int iw = iw0 + kw * g.dilation;
                    if ((unsigned)iw < (unsigned)d.W)
                        v = fmaf(wc[kh * K + kw], xc[(int64_t)ih * d.W + iw], v);
                }
            }
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int o = o0 + 16 * mb + j;
            const float a = cok && o < d.O ? pw_w[(int64_t)o * d.C + c] : 0.0f;
            acc[mb] = mfma_16x16x4(a, v, acc[mb]);
        }
    }
    if (!owok) return;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int o = o0 + 16 * mb + 4 * cq + r;
            if (o < d.O) y[((n * d.O + o) * d.Ho + oh) * d.Wo + ow] = acc[mb][r];
        }
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline hipError_t launch_waves(int64_t tiles, unsigned &grid)
{
    const int64_t g = cdiv(tiles, kGenWaves);
    if (g > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    grid = (unsigned)g;
    return hipSuccess;
}

}  // namespace

namespace {

template <int MB, int NBW, int K, int S, bool ACT, int SW>
hipError_t launch_staged_sw(const float *x, const float *w, const float *b, float *y,
                            const Conv3dDims &d, hipStream_t s)
{
    using G = StagedGeom<K, S, NBW>;
    auto kern = conv3d_staged_kernel<MB, NBW, K, S, ACT, SW>;
    const size_t lds = 4 * (size_t)(G::XS + K * K * 64 * MB);
    hipError_t e = hipFuncSetAttribute((const void *)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const int64_t tw = cdiv(d.OW, 16 * NBW), th = cdiv(d.OH, G::WH), td = cdiv(d.OD, G::WD);
    const int64_t tiles = tw * th * td * d.N * cdiv(d.O, 16 * MB);
    if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(G::NT), lds, s, x, w, b, y, d, tiles,
                       (int)tw, (int)th, (int)td);
    return hipGetLastError();
}

template <int K, int S, bool ACT>
hipError_t launch_staged(const float *x, const float *w, const float *b, float *y,
                         const Conv3dDims &d, hipStream_t s)
{
    constexpr int NBW = S == 1 ? 4 : 2;  // output columns per wave: 64 or 32
    const int sw = conv_store_width(y, d.OW);
    if (d.O > 16) {
        if (sw == 4) return launch_staged_sw<4, NBW, K, S, ACT, 4>(x, w, b, y, d, s);
        if (sw == 2) return launch_staged_sw<4, NBW, K, S, ACT, 2>(x, w, b, y, d, s);
        return launch_staged_sw<4, NBW, K, S, ACT, 1>(x, w, b, y, d, s);
    }
    if (sw == 4) return launch_staged_sw<1, NBW, K, S, ACT, 4>(x, w, b, y, d, s);
    if (sw == 2) return launch_staged_sw<1, NBW, K, S, ACT, 2>(x, w, b, y, d, s);
    return launch_staged_sw<1, NBW, K, S, ACT, 1>(x, w, b, y, d, s);
}

template <bool ACT>
hipError_t launch_conv3d_generic(const float *x, const float *w, const float *b, float *y,
                                 const Conv3dDims &d, const GenConv &g, hipStream_t s)
{
    if (g.stride == 1) {
        if (g.k == 3) return launch_staged<3, 1, ACT>(x, w, b, y, d, s);
        if (g.k == 5) return launch_staged<5, 1, ACT>(x, w, b, y, d, s);
        if (g.k == 7) return launch_staged<7, 1, ACT>(x, w, b, y, d, s);
    } else if (g.stride == 2) {
        if (g.k == 3) return launch_staged<3, 2, ACT>(x, w, b, y, d, s);
        if (g.k == 5) return launch_staged<5, 2, ACT>(x, w, b, y, d, s);
        if (g.k == 7) return launch_staged<7, 2, ACT>(x, w, b, y, d, s);
    }
    constexpr int NB = 2;
    const int64_t tw = cdiv(d.OW, 16 * NB);
    unsigned grid;
    if (d.O > 32) {
        const int64_t tiles = cdiv(d.O, 64) * d.N * d.OD * d.OH * tw;
        if (hipError_t e = launch_waves(tiles, grid)) return e;
        hipLaunchKernelGGL((conv3d_mish_tanh_generic_kernel<4, NB, ACT>), dim3(grid),
                           dim3(64 * kGenWaves), 0, s, x, w, b, y, d, g, tiles, (int)tw);
    } else {
        const int64_t tiles = cdiv(d.O, 16) * d.N * d.OD * d.OH * tw;
        if (hipError_t e = launch_waves(tiles, grid)) return e;
        hipLaunchKernelGGL((conv3d_mish_tanh_generic_kernel<1, NB, ACT>), dim3(grid),
                           dim3(64 * kGenWaves), 0, s, x, w, b, y, d, g, tiles, (int)tw);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_conv3d_mish_tanh_generic(const float *x, const float *w, const float *b,
                                           float *y, const Conv3dDims &d, const GenConv &g,
                                           hipStream_t s)
{
    return launch_conv3d_generic<true>(x, w, b, y, d, g, s);
}

hipError_t launch_conv3d_bias_generic(const float *x, const float *w, const float *b, float *y,
                                      const Conv3dDims &d, const GenConv &g, hipStream_t s)
{
    return launch_conv3d_generic<false>(x, w, b, y, d, g, s);
}

namespace {

template <bool STORE>
hipError_t launch_pool_generic(const float *x, const float *w, const float *conv_b, float *out,
                               const PoolDims &p, const GenConv &g, int pool, hipStream_t s)
{
    constexpr int MB = 1, NB = 2;
    const Conv3dDims &d = p.conv;
    if (pool < 1 || pool > 16 * NB || pool > kGenericMaxPool) return hipErrorInvalidValue;
    const int twp = 16 * NB / pool;
    const int64_t tw = cdiv(p.PW, twp);
    const int64_t tiles = cdiv(d.O, 16 * MB) * d.N * p.PD * p.PH * tw;
    unsigned grid;
    if (hipError_t e = launch_waves(tiles, grid)) return e;
    const float inv_count = (float)(1.0 / ((double)p.PD * (double)p.PH * (double)p.PW));
    hipLaunchKernelGGL((conv3d_pool_sum_generic_kernel<MB, NB, STORE>), dim3(grid),
                       dim3(64 * kGenWaves), 0, s, x, w, conv_b, out, p, g, pool, tiles, (int)tw,
                       inv_count);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_conv3d_pool_sum_generic(const float *x, const float *w, const float *conv_b,
                                          const float *bias, float *out, const PoolDims &p,
                                          const GenConv &g, int pool, hipStream_t s)
{
    if (pool < 1 || pool > kGenericMaxPool) return hipErrorInvalidValue;
    const hipError_t e = launch_pool_sum_init(bias, out, p.conv.N, p.conv.O, s);
    if (e != hipSuccess) return e;
    return launch_pool_generic<false>(x, w, conv_b, out, p, g, pool, s);
}

hipError_t launch_conv3d_div_maxpool_generic(const float *x, const float *w,
                                             const float *conv_b, float *y, const PoolDims &p,
                                             const GenConv &g, int pool, hipStream_t s)
{
    return launch_pool_generic<true>(x, w, conv_b, y, p, g, pool, s);
}

hipError_t launch_dwsep_conv2d_generic(const float *x, const float *dw_w, const float *dw_b,
                                       const float *pw_w, const float *pw_b, float *y,
                                       const DwsepDims &d, const GenConv &g, hipStream_t s)
{
    const int64_t tw = cdiv(d.Wo, 16);
    unsigned grid;
    if (d.O > 64) {
        const int64_t tiles = cdiv(d.O, 128) * d.N * d.Ho * tw;
        if (hipError_t e = launch_waves(tiles, grid)) return e;
        hipLaunchKernelGGL((dwsep_generic_kernel<8>), dim3(grid), dim3(64 * kGenWaves), 0, s, x,
                           dw_w, dw_b, pw_w, pw_b, y, d, g, tiles, (int)tw);
    } else {
        const int64_t tiles = cdiv(d.O, 16) * d.N * d.Ho * tw;
        if (hipError_t e = launch_waves(tiles, grid)) return e;
        hipLaunchKernelGGL((dwsep_generic_kernel<1>), dim3(grid), dim3(64 * kGenWaves), 0, s, x,
                           dw_w, dw_b, pw_w, pw_b, y, d, g, tiles, (int)tw);
    }
    return hipGetLastError();
}

}  // namespace convfuse
