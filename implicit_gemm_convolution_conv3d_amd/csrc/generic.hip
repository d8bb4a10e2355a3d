// generic.hip -- the three fused operations for any kernel size, stride, padding, dilation and
// pooling size, on gfx950 fp32 matrix cores.
//
// The tuned kernels (conv3d_igemm.hip, dwsep.hip) cover k = 3, stride 1, pad <= 2 (and, for
// the pooled sum, a 2x2x2 pool; for dwsep, dilation 1).  These kernels compute the same
// definitions for every other parameter set (page "Kimi-K2.6 l2_p47", generalised stride and
// padding of the Conv3d; page "Kimi-K2.6 l1_p86", stride/padding/dilation and kernel sizes
// 1/3/5/7 of the depthwise-separable Conv2d; page "Kimi-K2.6 l2_p8", the pooled channel sum).
//
// LDS-staged kernels cover the common cases: Conv3d with kernel size 3, 5 or 7 and stride 1
// or 2, any padding (conv3d_staged_kernel, the tuned kernel's organisation); the pooled layer
// with kernel size 1, 3 or 5 and pool 2, 3 or 4 (conv3d_pool_staged_kernel); the
// depthwise-separable conv with any kernel size up to 7, stride and dilation
// (dwsep_staged_kernel, input rows streamed straight into LDS).  Everything else is a
// direct implicit GEMM over global memory: one wave owns 16*MB output channels x 16*NB
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

// ------------------------------------------------------------------ staged general pool
// Conv3d (kernel K, stride 1, no padding), divide, P x P x P max-pool, then the pooled
// channel sum (or, STORE, the pooled tensor), for K in {1, 3, 5} and P in {2, 3, 4}.
// Workgroup = 4 waves; wave w owns pooled row (n, pd0, ph0 + w), TWP pooled columns from pw0,
// and output channels [o0, o0 + 16).  Its conv voxels come in NB = P*P*NBW blocks
// (dd, dh, q): conv voxel (P*pd0 + dd, P*(ph0 + w) + dh, P*pw0 + BW*q + j) for MFMA row j,
// BW = the largest multiple of P up to 16 (a block's last 16 - BW rows are not used).  The K
// loop runs over chunks of four input channels at one kernel depth kd, double-buffered in
// LDS: P depth planes x HHR rows x COLS columns per channel, streamed from global memory
// straight into LDS, and K*K taps of weights in A-fragment order (through registers).  The
// epilogue takes each window's extreme over (dd, dh) in registers and over its P columns
// through wave-private LDS.
template <int K, int P, int NBW>
struct PoolGeom {
    static constexpr int NT = 256;
    static constexpr int BW = 16 - 16 % P;                   // used columns per block
    static constexpr int TWP = NBW * BW / P;                 // pooled columns per wave
    static constexpr int NB = P * P * NBW;                   // voxel blocks per wave
    static constexpr int HHR = 4 * P + K - 1;                // input rows per (channel, plane)
    static constexpr int COLS = BW * (NBW - 1) + 16 + K - 1; // input columns per row (<= 64)
    static constexpr int RS = round_up(COLS, 4);
    static constexpr int CS = halo_channel_stride(P * HHR * RS);
    static constexpr int XS = 4 * CS;
    static constexpr int WSZ = K * K * 64;                   // weights per chunk (16 outputs)
    static constexpr int BUF = XS + WSZ;                     // one stage
    static constexpr int RED = 16 * (16 * NBW + 1);          // per-wave window buffer
    // (the window buffers reuse the stages once the K loop is over)
    static constexpr int LDS = 2 * BUF > 4 * RED ? 2 * BUF : 4 * RED;  // floats
    static_assert(COLS <= 64, "one load per staged row");
};

template <int K, int P, int NBW, bool STORE>
__global__ __launch_bounds__(256, 2) void conv3d_pool_staged_kernel(
    const float *__restrict__ x, const float *__restrict__ w, const float *__restrict__ cb,
    float *__restrict__ out, PoolDims p, int64_t tiles, int tiles_w, int tiles_h,
    float inv_count)
{
    using G = PoolGeom<K, P, NBW>;
    extern __shared__ __attribute__((aligned(16))) float dyn[];
    // (the wave index made explicitly uniform: the row copy's channel, buffer resources and
    // LDS addresses are then scalar work)
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const Conv3dDims &d = p.conv;
    const int D = (int)d.D, H = (int)d.H, W = (int)d.W;

    int64_t t = xcd_tile(blockIdx.x, tiles);
    const int tw = (int)(t % tiles_w); t /= tiles_w;
    const int th = (int)(t % tiles_h); t /= tiles_h;
    const int pd0 = (int)(t % p.PD); t /= p.PD;
    const int64_t n = t % d.N;
    const int o0 = (int)(t / d.N) * 16;
    const int ph0 = th * 4, pw0 = tw * G::TWP;
    const int xlane = (lane >> 4) * G::CS + wave * P * G::RS + (lane & 15);
    const int id0 = P * pd0, ih0 = P * ph0, iw0 = P * pw0;

    // Issue chunk q's input rows into buffer xsb: wave w copies the P*HHR rows of channel
    // c0 + w (plane pl, row hr at LDS row pl*HHR + hr); LDS column c holds input column
    // iw0 + c.  Each plane is read through a resource that starts at its row ih0 and ends
    // with the plane (no records for an absent channel or plane), so rows past H read as
    // zero by the range check; lanes past W carry a dropped offset.  The loops are unrolled:
    // a row costs an offset add and the load.  A plane's byte size is below 2^31 (the host
    // checks four channels' volume).
    const int lcol = iw0 + lane < W ? 4 * lane : kDropOffset;
    auto rows_dma = [&](int q, float *xsb) {
        const int c0 = (q / K) * 4, kd = q % K;
        const int cw = c0 + wave;
        float *dst = xsb + wave * G::CS;
        int rstep = 4 * W;
        asm volatile("" : "+s"(rstep));
        if (lane < G::COLS) {
#pragma unroll
            for (int pl = 0; pl < P; ++pl) {
                const int id = id0 + pl + kd;
                const bool plok = cw < d.C && id < D;
                // (an absent plane keeps the tensor's base: its resource has no records)
                const float *pbase =
                    plok ? x + (((n * d.C + cw) * D + id) * H + ih0) * (int64_t)W + iw0 : x;
                const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                    const_cast<float *>(pbase), (short)0, plok ? 4 * (H - ih0) * W : 0,
                    kBufferWord3);
                int off = lcol;
#pragma unroll
                for (int hr = 0; hr < G::HHR; ++hr) {
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rs,
                        (__attribute__((address_space(3))) void *)(dst +
                                                                   (pl * G::HHR + hr) * G::RS),
                        4, off, 0, 0, 0);
                    off += rstep;
                }
            }
        }
    };
    WeightChunk<1, 4, G::NT, K * K> wts;
    auto wload = [&](int q) { wts.load(w, d, o0, (q / K) * 4, K * K * K, (q % K) * K * K); };

    const int chunks = (int)((d.C + 3) / 4) * K;  // chunk q: channels 4*(q/K).., depth q%K
    rows_dma(0, dyn);
    wload(0);
    wts.store(dyn + G::XS);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int ph = ph0 + wave;
    const bool active = ph < p.PH;
    floatx4 acc[G::NB];
#pragma unroll
    for (int nb = 0; nb < G::NB; ++nb) acc[nb] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < chunks; ++q) {
        const float *xs = dyn + (q & 1) * G::BUF, *ws = xs + G::XS;
        float *nxt = dyn + ((q & 1) ^ 1) * G::BUF;
        const bool more = q + 1 < chunks;
        if (more) {
            rows_dma(q + 1, nxt);
            wload(q + 1);
        }
        if (active) {
#pragma unroll
            for (int kh = 0; kh < K; ++kh)
#pragma unroll
                for (int kw = 0; kw < K; ++kw) {
                    const float a = ws[(kh * K + kw) * 64 + lane];
#pragma unroll
                    for (int dd = 0; dd < P; ++dd)
#pragma unroll
                        for (int dh = 0; dh < P; ++dh)
#pragma unroll
                            for (int qb = 0; qb < NBW; ++qb) {
                                const int nb = (dd * P + dh) * NBW + qb;
                                const float bv = xs[xlane + (dd * G::HHR + dh + kh) * G::RS +
                                                    G::BW * qb + kw];
                                acc[nb] = mfma_16x16x4(bv, a, acc[nb]);
                            }
                }
        }
        if (more) wts.store(nxt + G::XS);
        __builtin_amdgcn_s_waitcnt(0);  // this wave's rows of the next chunk are in LDS
        __syncthreads();                // ... and every wave's; nobody reads this stage
    }
    if (!active) return;  // (no barrier follows)
    // Every wave is past the last barrier: no wave reads a stage and no load into one is in
    // flight, so the stages hold the per-wave window buffers now.
    float *red = dyn + wave * G::RED;
    // lane holds columns 4*(lane/16) + r of every block of output channel o0 + lane%16
    const bool use_min = p.divisor < 0.0f;
    const int j = lane & 15, g4 = 4 * (lane >> 4);
#pragma unroll
    for (int qb = 0; qb < NBW; ++qb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float m = acc[qb][r];
#pragma unroll
            for (int b2 = 1; b2 < P * P; ++b2) {
                const float v = acc[b2 * NBW + qb][r];
                m = use_min ? fminf(m, v) : fmaxf(m, v);
            }
            red[j * (16 * NBW + 1) + 16 * qb + g4 + r] = m;
        }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float part = 0.0f;
    for (int e = lane; e < 16 * G::TWP; e += 64) {
        const int ol = e / G::TWP, wq = e % G::TWP;
        const int o = o0 + ol, pw = pw0 + wq;
        if (o >= d.O || pw >= p.PW) continue;
        const int col = (wq / (G::BW / P)) * 16 + (wq % (G::BW / P)) * P;  // window's first
        const float *rp = red + ol * (16 * NBW + 1) + col;
        float m = rp[0];
#pragma unroll
        for (int i = 1; i < P; ++i) m = use_min ? fminf(m, rp[i]) : fmaxf(m, rp[i]);
        const float v = (m + (cb ? cb[o] : 0.0f)) / p.divisor;
        if constexpr (STORE)
            out[(((n * d.O + o) * p.PD + pd0) * p.PH + ph) * p.PW + pw] = v;
        else
            part += v;
    }
    if constexpr (!STORE) {
        part = wave_sum(part);
        if (lane == 0) atomicAdd(out + n, part * inv_count);
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

// Accumulators of a pixel-rows MFMA tile start at the pointwise bias: element r of
// acc[mb][.] is output channel 16*mb + lane%16.
template <int MB, int R>
__device__ __forceinline__ void acc_init_pixrows(floatx4 (&acc)[MB][R], const float *bs)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const float v = bs[16 * mb + (lane & 15)];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[mb][r] = floatx4{v, v, v, v};
    }
}

// ------------------------------------------------------------------ staged general dwsep
// Workgroup = 4 waves side by side; tile = R output rows x 64 output columns of image n,
// output channels [obase, obase + ocnt).  The K loop runs over chunks of 8 input channels,
// double-buffered in LDS: while a chunk computes, the next chunk's input rows stream from
// global memory straight into the other LDS buffer (buffer loads with an LDS destination: no
// registers held, zero padding from dropped offsets) and its weights pass through registers.
// A chunk holds the HR input rows and the input columns the tile reaches, per channel, the
// depthwise taps and bias, and the pointwise weights in fragment order.  Staged column c of
// a row is input column qa + c, qa = the tile's first input column rounded down to a multiple
// of 4 (so rows of a 4-aligned input can be staged 16 bytes per lane).  Lane l of wave w forms
// the MFMA operand of k-step cg, the depthwise output of chunk channel 4*cg + l/16 at output
// column 16*w + l%16 of each row, from K*K LDS reads; the pixels are the MFMA rows, so each
// lane ends with 4 consecutive pixels of one output channel.
constexpr int kDwsCC = 8;     // input channels per chunk
constexpr int kDwsCPL = 5;    // staged column blocks of 64 (staged row <= 320 floats)
constexpr int kDwsKT = 64;    // depthwise slots per channel (K*K taps + bias, K <= 7)

// Geometry with every size a run-time value (any K <= 7, stride, dilation).
struct DwStagedGeom {
    int K, S, dil;   // kernel size, stride, dilation
    int HR, COLS;    // input rows / columns the tile reaches
    int RS, CS, XS;  // LDS row stride (COLS + 3 rounded up to 4), channel stride, halo floats
    int vec, vin;    // output rows 16-byte aligned; input rows 16-byte aligned (W % 4 == 0)
};

// The same geometry fixed at compile time (kernel size, stride, dilation as template
// arguments), so that every LDS offset of the depthwise step is an immediate.
template <int R, int K_, int S_, int D_>
struct DwFixedGeom {
    static constexpr int K = K_, S = S_, dil = D_;
    static constexpr int HR = (R - 1) * S + (K - 1) * dil + 1;
    static constexpr int COLS = 63 * S + (K - 1) * dil + 1;
    static constexpr int RS = round_up(COLS + 3, 4);
    static constexpr int CS = halo_channel_stride(HR * RS);
    static constexpr int XS = kDwsCC * CS;
    int vec, vin;
};

template <int MB>
constexpr int dws_buffer_floats(int XS)
{
    return XS + kDwsCC * 16 * MB + kDwsCC * kDwsKT;
}

template <int MB, int R, int K, class GEO>
__global__ __launch_bounds__(256, 2) void dwsep_staged_kernel(
    const float *__restrict__ x, const float *__restrict__ dw_w, const float *__restrict__ dw_b,
    const float *__restrict__ pw_w, const float *__restrict__ pw_b, float *__restrict__ y,
    DwsepDims d, GEO g, int64_t tiles, int tiles_w, int tiles_h)
{
    // buffer b: halo [8][HR][RS] at channel stride CS, pointwise [2][64][MB] (fragment
    // order), depthwise [8][64] (taps, bias at K*K); then the pointwise bias [16*MB]
    extern __shared__ __attribute__((aligned(16))) float dyn[];
    constexpr int TAPS = K * K;
    const int BF = dws_buffer_floats<MB>(g.XS);
    float *bs = dyn + 2 * BF;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int C = (int)d.C, H = (int)d.H, W = (int)d.W;

    int64_t t = xcd_tile(blockIdx.x, tiles);
    const int tw = (int)(t % tiles_w);
    t /= tiles_w;
    const int th = (int)(t % tiles_h);
    t /= tiles_h;
    const int64_t n = t % d.N;
    const int obase = (int)(t / d.N) * 16 * MB;
    const int ocnt = (int)(d.O - obase < 16 * MB ? d.O - obase : 16 * MB);
    const int h0 = th * R, w0 = tw * 64;
    const int ih0 = h0 * g.S - d.pad, iw0 = w0 * g.S - d.pad;
    const int sh = iw0 & 3, qa = iw0 - sh;  // staged column c = input column qa + c
    const int span = g.COLS + sh;           // staged columns of a row
    const bool active = w0 + 16 * wave < d.Wo;

    // Per-lane part of the row loads, fixed for the tile: 16-byte quads (lane l: columns
    // qa + 4l ..) when the input rows are 16-byte aligned, else 4-byte columns l + 64j.
    const int nq = (span + 3) >> 2;
    const int qcol = qa + 4 * lane;
    const bool qok = lane < nq && (unsigned)qcol < (unsigned)W;

    // Issue the input rows of chunk c0 into buffer xsb: wave w copies every row of channels
    // CPW*w .. CPW*w + CPW-1.  The wave index is made explicitly uniform, so each row's global
    // offset and LDS address are scalar values and a row costs one vector select.
    // Byte offsets over the channels [c0, c0 + 8) of image n stay below 2^31 (host check).
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    auto rows_dma = [&](int c0, float *xsb) {
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(x + (n * C + c0) * (int64_t)H * W);
        constexpr int CPW = kDwsCC / 4;  // channels per wave (4 waves)
        static_assert(kDwsCC % 4 == 0, "whole channels per wave");
#pragma unroll
        for (int k = 0; k < CPW; ++k) {
#pragma unroll
            for (int hr = 0; hr < g.HR; ++hr) {
                const int cl = CPW * wv + k;
                const int ih = ih0 + hr;
                const bool rowok = c0 + cl < C && (unsigned)ih < (unsigned)H;
                const int rowoff = (cl * H + ih) * W;
                float *dst = xsb + cl * g.CS + hr * g.RS;
                if (g.vin) {
                    const int off = rowok && qok ? 4 * (rowoff + qcol) : kDropOffset;
                    if (lane < nq)
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            rs, (__attribute__((address_space(3))) void *)dst, 16, off, 0, 0, 0);
                } else {
#pragma unroll
                    for (int jj = 0; jj < kDwsCPL; ++jj) {
                        if (64 * jj >= span) break;
                        const int col = 64 * jj + lane, iw = qa + col;
                        const int off =
                            rowok && (unsigned)iw < (unsigned)W ? 4 * (rowoff + iw) : kDropOffset;
                        if (col < span)
                            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                                rs, (__attribute__((address_space(3))) void *)(dst + 64 * jj), 4,
                                off, 0, 0, 0);
                    }
                }
            }
        }
    };
    // Weights of chunk c0 in registers: pointwise element (ol, cl) = tid + 256u, depthwise
    // slot e = tid + 256u of [8][64].
    float wp[MB / 2], wd[2];
    auto wload = [&](int c0) {
#pragma unroll
        for (int u = 0; u < MB / 2; ++u) {
            const int e = tid + 256 * u, ol = e >> 3, cl = e & 7;
            wp[u] = (ol < ocnt && c0 + cl < C) ? pw_w[(int64_t)(obase + ol) * C + c0 + cl] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int e = tid + 256 * u, cl = e >> 6, k = e & 63, c = c0 + cl;
            float v = 0.0f;
            if (c < C && k <= TAPS)
                v = k < TAPS ? dw_w[(int64_t)c * TAPS + k] : (dw_b ? dw_b[c] : 0.0f);
            wd[u] = v;
        }
    };
    auto wstore = [&](float *buf) {
        float *ps = buf + g.XS, *dk = ps + kDwsCC * 16 * MB;
#pragma unroll
        for (int u = 0; u < MB / 2; ++u) {
            const int e = tid + 256 * u, ol = e >> 3, cl = e & 7;
            ps[((cl >> 2) * 64 + (cl & 3) * 16 + (ol & 15)) * MB + (ol >> 4)] = wp[u];
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) dk[tid + 256 * u] = wd[u];
    };

    if (tid < 16 * MB) bs[tid] = (pw_b && tid < ocnt) ? pw_b[obase + tid] : 0.0f;
    rows_dma(0, dyn);
    wload(0);
    wstore(dyn);
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
    floatx4 acc[MB][R];
    acc_init_pixrows<MB, R>(acc, bs);
    const int xoff = sh + (16 * wave + (lane & 15)) * g.S;
    for (int c0 = 0, b = 0; c0 < C; c0 += kDwsCC, b ^= 1) {
        float *cur = dyn + b * BF, *nxt = dyn + (b ^ 1) * BF;
        const bool more = c0 + kDwsCC < C;
        if (more) {
            rows_dma(c0 + kDwsCC, nxt);
            wload(c0 + kDwsCC);
        }
        if (active) {
            const float *ps = cur + g.XS, *dk = ps + kDwsCC * 16 * MB;
#pragma unroll
            for (int cg = 0; cg < 2; ++cg) {
                const int cl = 4 * cg + (lane >> 4);
                const float *xc = cur + cl * g.CS + xoff;
                const float *kc = dk + cl * kDwsKT;
                float pwf[MB];
                load_afrag<MB>(ps + (cg * 64 + lane) * MB, pwf);
                float tap[TAPS];
#pragma unroll
                for (int k = 0; k < TAPS; ++k) tap[k] = kc[k];
                const float dbias = kc[TAPS];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float xv[TAPS];
#pragma unroll
                    for (int kh = 0; kh < K; ++kh)
#pragma unroll
                        for (int kw = 0; kw < K; ++kw)
                            xv[kh * K + kw] = xc[(r * g.S + kh * g.dil) * g.RS + kw * g.dil];
                    float v = dbias;
#pragma unroll
                    for (int k = 0; k < TAPS; ++k) v = fmaf(tap[k], xv[k], v);
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        acc[mb][r] = mfma_16x16x4(v, pwf[mb], acc[mb][r]);
                }
            }
        }
        if (more) wstore(nxt);
        __builtin_amdgcn_s_waitcnt(0);  // this wave's rows of the next chunk are in LDS
        lds_barrier();                  // ... and every wave's; nobody reads cur any more
    }
    if (!active) return;
    // lane holds pixels wc .. wc + 3 of output channel obase + 16*mb + lane%16
    const int wc = w0 + 16 * wave + 4 * (lane >> 4);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int ol = 16 * mb + (lane & 15);
        if (ol >= ocnt) continue;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int oh = h0 + r;
            if (oh >= d.Ho) continue;
            float *yr = y + ((n * d.O + obase + ol) * d.Ho + oh) * d.Wo;
            if (g.vec && wc + 3 < d.Wo) {
                *reinterpret_cast<floatx4 *>(yr + wc) = acc[mb][r];
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (wc + i < d.Wo) yr[wc + i] = acc[mb][r][i];
            }
        }
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
    note_kernel("conv3d_staged_kernel");
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
        note_kernel("conv3d_mish_tanh_generic_kernel");
        hipLaunchKernelGGL((conv3d_mish_tanh_generic_kernel<4, NB, ACT>), dim3(grid),
                           dim3(64 * kGenWaves), 0, s, x, w, b, y, d, g, tiles, (int)tw);
    } else {
        const int64_t tiles = cdiv(d.O, 16) * d.N * d.OD * d.OH * tw;
        if (hipError_t e = launch_waves(tiles, grid)) return e;
        note_kernel("conv3d_mish_tanh_generic_kernel");
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

template <int K, int P, bool STORE>
hipError_t launch_pool_staged(const float *x, const float *w, const float *conv_b, float *out,
                              const PoolDims &p, hipStream_t s)
{
    constexpr int NBW = P <= 3 ? 2 : 1;
    using G = PoolGeom<K, P, NBW>;
    const Conv3dDims &d = p.conv;
    const int64_t tw = cdiv(p.PW, G::TWP), th = cdiv(p.PH, 4);
    const int64_t tiles = tw * th * p.PD * d.N * cdiv(d.O, 16);
    if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const float inv_count = (float)(1.0 / ((double)p.PD * (double)p.PH * (double)p.PW));
    auto kern = conv3d_pool_staged_kernel<K, P, NBW, STORE>;
    const size_t lds = 4 * (size_t)G::LDS;
    hipError_t e = hipFuncSetAttribute((const void *)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    note_kernel("conv3d_pool_staged_kernel");
    hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(G::NT), lds, s, x, w, conv_b, out, p,
                       tiles, (int)tw, (int)th, inv_count);
    return hipGetLastError();
}

template <int K, bool STORE>
hipError_t launch_pool_staged_p(const float *x, const float *w, const float *conv_b, float *out,
                                const PoolDims &p, int pool, hipStream_t s)
{
    if (pool == 2) return launch_pool_staged<K, 2, STORE>(x, w, conv_b, out, p, s);
    if (pool == 3) return launch_pool_staged<K, 3, STORE>(x, w, conv_b, out, p, s);
    return launch_pool_staged<K, 4, STORE>(x, w, conv_b, out, p, s);
}

template <bool STORE>
hipError_t launch_pool_generic(const float *x, const float *w, const float *conv_b, float *out,
                               const PoolDims &p, const GenConv &g, int pool, hipStream_t s)
{
    // staged kernel: four input channels of one image within 32-bit byte offsets
    const Conv3dDims &d = p.conv;
    if (pool >= 2 && pool <= 4 && g.stride == 1 && d.pad == 0 &&
        16 * d.D * d.H * d.W <= kBufRange) {
        if (g.k == 1) return launch_pool_staged_p<1, STORE>(x, w, conv_b, out, p, pool, s);
        if (g.k == 3) return launch_pool_staged_p<3, STORE>(x, w, conv_b, out, p, pool, s);
        if (g.k == 5) return launch_pool_staged_p<5, STORE>(x, w, conv_b, out, p, pool, s);
    }
    constexpr int MB = 1, NB = 2;
    if (pool < 1 || pool > 16 * NB || pool > kGenericMaxPool) return hipErrorInvalidValue;
    const int twp = 16 * NB / pool;
    const int64_t tw = cdiv(p.PW, twp);
    const int64_t tiles = cdiv(d.O, 16 * MB) * d.N * p.PD * p.PH * tw;
    unsigned grid;
    if (hipError_t e = launch_waves(tiles, grid)) return e;
    const float inv_count = (float)(1.0 / ((double)p.PD * (double)p.PH * (double)p.PW));
    note_kernel("conv3d_pool_sum_generic_kernel");
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

namespace {

template <int MB, int R, int K, class GEO>
hipError_t launch_dwsep_staged_g(const float *x, const float *dw_w, const float *dw_b,
                                 const float *pw_w, const float *pw_b, float *y,
                                 const DwsepDims &d, const GEO &geo, size_t lds, hipStream_t s)
{
    auto kern = dwsep_staged_kernel<MB, R, K, GEO>;
    hipError_t e = hipFuncSetAttribute((const void *)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const int64_t tw = cdiv(d.Wo, 64), th = cdiv(d.Ho, R);
    const int64_t tiles = tw * th * d.N * cdiv(d.O, 16 * MB);
    if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    note_kernel("dwsep_staged_kernel");
    hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(256), lds, s, x, dw_w, dw_b, pw_w, pw_b,
                       y, d, geo, tiles, (int)tw, (int)th);
    return hipGetLastError();
}

template <int MB, int R, int K, int S, int D>
hipError_t launch_dwsep_fixed(const float *x, const float *dw_w, const float *dw_b,
                              const float *pw_w, const float *pw_b, float *y, const DwsepDims &d,
                              const DwStagedGeom &sg, hipStream_t s)
{
    using FG = DwFixedGeom<R, K, S, D>;
    FG fg;
    fg.vec = sg.vec;
    fg.vin = sg.vin;
    const size_t lds = 4 * (2 * (size_t)dws_buffer_floats<MB>(FG::XS) + 16 * MB);
    return launch_dwsep_staged_g<MB, R, K, FG>(x, dw_w, dw_b, pw_w, pw_b, y, d, fg, lds, s);
}

template <int MB, int R>
hipError_t launch_dwsep_staged(const float *x, const float *dw_w, const float *dw_b,
                               const float *pw_w, const float *pw_b, float *y,
                               const DwsepDims &d, const DwStagedGeom &sg, size_t lds,
                               hipStream_t s)
{
    // the pages' kernel sizes 3/5/7 at stride and dilation 1 or 2: compile-time geometry
#define CONVFUSE_FIXED(KK, SS, DD)                                                               \
    if (sg.K == KK && sg.S == SS && sg.dil == DD)                                                \
        return launch_dwsep_fixed<MB, R, KK, SS, DD>(x, dw_w, dw_b, pw_w, pw_b, y, d, sg, s);
    CONVFUSE_FIXED(3, 1, 2) CONVFUSE_FIXED(3, 2, 1) CONVFUSE_FIXED(3, 2, 2)
    CONVFUSE_FIXED(5, 1, 1) CONVFUSE_FIXED(5, 1, 2) CONVFUSE_FIXED(5, 2, 1) CONVFUSE_FIXED(5, 2, 2)
    CONVFUSE_FIXED(7, 1, 1) CONVFUSE_FIXED(7, 1, 2) CONVFUSE_FIXED(7, 2, 1) CONVFUSE_FIXED(7, 2, 2)
#undef CONVFUSE_FIXED
    switch (sg.K) {
    case 1: return launch_dwsep_staged_g<MB, R, 1>(x, dw_w, dw_b, pw_w, pw_b, y, d, sg, lds, s);
    case 2: return launch_dwsep_staged_g<MB, R, 2>(x, dw_w, dw_b, pw_w, pw_b, y, d, sg, lds, s);
    case 3: return launch_dwsep_staged_g<MB, R, 3>(x, dw_w, dw_b, pw_w, pw_b, y, d, sg, lds, s);
    case 4: return launch_dwsep_staged_g<MB, R, 4>(x, dw_w, dw_b, pw_w, pw_b, y, d, sg, lds, s);
    case 5: return launch_dwsep_staged_g<MB, R, 5>(x, dw_w, dw_b, pw_w, pw_b, y, d, sg, lds, s);
    case 6: return launch_dwsep_staged_g<MB, R, 6>(x, dw_w, dw_b, pw_w, pw_b, y, d, sg, lds, s);
    default: return launch_dwsep_staged_g<MB, R, 7>(x, dw_w, dw_b, pw_w, pw_b, y, d, sg, lds, s);
    }
}

// The staged kernel's run-time geometry; false when it does not apply (kernel above 7, tile
// above the LDS size, or the chunk's input bytes beyond 32-bit offsets).  The LDS size is the
// largest of the run-time and compile-time layouts (they are the same).
template <int MB, int R>
bool dwsep_staged_geom(const DwsepDims &d, const GenConv &g, const float *x, const float *y,
                       DwStagedGeom &sg, size_t &lds)
{
    if (g.k < 1 || g.k > 7 || 4 * kDwsCC * d.H * d.W > kBufRange) return false;
    const int64_t reach = (int64_t)(g.k - 1) * g.dilation;
    const int64_t HR = (int64_t)(R - 1) * g.stride + reach + 1;
    const int64_t COLS = 63LL * g.stride + reach + 1;
    if (COLS + 3 > 64 * kDwsCPL || HR > 4096) return false;
    sg.K = g.k;
    sg.S = g.stride;
    sg.dil = g.dilation;
    sg.HR = (int)HR;
    sg.COLS = (int)COLS;
    sg.RS = round_up((int)COLS + 3, 4);
    sg.CS = halo_channel_stride(sg.HR * sg.RS);
    sg.XS = kDwsCC * sg.CS;
    sg.vec = d.Wo % 4 == 0 && ((uintptr_t)y & 15) == 0;
    // 16-byte row loads: 4-aligned rows and at most 64 quads per staged row
    sg.vin = d.W % 4 == 0 && ((uintptr_t)x & 15) == 0 && COLS + 3 <= 256;
    lds = 4 * (2 * (size_t)dws_buffer_floats<MB>(sg.XS) + 16 * MB);
    return lds <= 160 * 1024;
}

}  // namespace

hipError_t launch_dwsep_conv2d_generic(const float *x, const float *dw_w, const float *dw_b,
                                       const float *pw_w, const float *pw_b, float *y,
                                       const DwsepDims &d, const GenConv &g, hipStream_t s)
{
    // LDS-staged kernel when it applies (64 or 128 output channels per workgroup)
    {
        DwStagedGeom sg;
        size_t lds;
        if (d.O > 64) {
            if (dwsep_staged_geom<8, 2>(d, g, x, y, sg, lds))
                return launch_dwsep_staged<8, 2>(x, dw_w, dw_b, pw_w, pw_b, y, d, sg, lds, s);
        } else if (dwsep_staged_geom<4, 2>(d, g, x, y, sg, lds)) {
            return launch_dwsep_staged<4, 2>(x, dw_w, dw_b, pw_w, pw_b, y, d, sg, lds, s);
        }
    }
    const int64_t tw = cdiv(d.Wo, 16);
    unsigned grid;
    if (d.O > 64) {
        const int64_t tiles = cdiv(d.O, 128) * d.N * d.Ho * tw;
        if (hipError_t e = launch_waves(tiles, grid)) return e;
        note_kernel("dwsep_generic_kernel");
        hipLaunchKernelGGL((dwsep_generic_kernel<8>), dim3(grid), dim3(64 * kGenWaves), 0, s, x,
                           dw_w, dw_b, pw_w, pw_b, y, d, g, tiles, (int)tw);
    } else {
        const int64_t tiles = cdiv(d.O, 16) * d.N * d.Ho * tw;
        if (hipError_t e = launch_waves(tiles, grid)) return e;
        note_kernel("dwsep_generic_kernel");
        hipLaunchKernelGGL((dwsep_generic_kernel<1>), dim3(grid), dim3(64 * kGenWaves), 0, s, x,
                           dw_w, dw_b, pw_w, pw_b, y, d, g, tiles, (int)tw);
    }
    return hipGetLastError();
}

}  // namespace convfuse
