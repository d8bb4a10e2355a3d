// conv3d_igemm.hip -- implicit-GEMM Conv3d (k = 3, stride 1) on gfx950 fp32 matrix cores,
// with two fused epilogues:
//   * Mish then tanh, stored to y           (page "Kimi-K2.6 l2_p47", Conv3d + Mish + Tanh)
//   * /divisor, 2x2x2 max-pool, global mean, reduced to one scalar per batch item with one
//     atomic per workgroup                  (page "Kimi-K2.6 l2_p8", the rewrite of the
//                                            output as a sum of channel means plus sum(bias))
//
// GEMM view (page l2_p47, implicit-GEMM paragraph): output channels x output voxels,
// reduction K = Cin * 27 ordered tap-major, channel-minor.  One k-step of the 16x16x4 MFMA
// consumes four consecutive input channels at one tap, so the voxel-side operand of lane l
// is the LDS halo value of channel (l/16) at voxel column (l%16) shifted by the tap: its LDS
// address is a per-lane base plus a compile-time offset.  The Mish/tanh kernel makes the
// voxels the MFMA rows (each lane ends with 4 consecutive voxels of one channel, stored
// together); the pool kernel makes the channels the rows (each lane ends with one voxel of 4
// channels, and window columns pair up between neighbouring lanes).
//
// Workgroup = WD x WH waves.  Each wave owns a box of output voxels and all 16*MB output
// channels of its channel group.  The input halo of the workgroup's box and the matching
// weights (in A-fragment order, [tap][channel group][lane][MB]) are staged into LDS one
// chunk of CC input channels at a time; the next chunk's global loads are issued into
// registers before the current chunk's MFMAs, so their latency hides behind the math.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "conv3d_tile.hpp"

namespace convfuse {

namespace {

// One chunk of the K loop: 27 taps x CC/4 channel groups.  The NB voxel blocks of the wave
// sit at LDS offsets boff[] from the lane base; acc[mb][nb] accumulates output channels
// 16*mb.. of block nb.  VROWS: the voxels are the MFMA's rows (A operand) and each lane ends
// with 4 consecutive voxels of one output channel; otherwise 4 output channels of one voxel.
// (The lane's operand values are the same either way: only the roles of A and B swap.)
template <int MB, int NB, int CC, int HH, int RS, int CS, bool VROWS = false>
__device__ __forceinline__ void igemm_chunk(const float *__restrict__ xs,
                                            const float *__restrict__ ws, int xlane,
                                            const int (&boff)[NB], floatx4 (&acc)[MB][NB])
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int kd = 0; kd < 3; ++kd)
#pragma unroll
        for (int kh = 0; kh < 3; ++kh)
#pragma unroll
            for (int kw = 0; kw < 3; ++kw)
#pragma unroll
                for (int cg = 0; cg < CC / 4; ++cg) {
                    const int tap = (kd * 3 + kh) * 3 + kw;
                    float a[MB];
                    load_afrag<MB>(ws + ((tap * (CC / 4) + cg) * 64 + lane) * MB, a);
                    const int toff = cg * 4 * CS + (kd * HH + kh) * RS + kw;
                    float bv[NB];
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) bv[nb] = xs[xlane + toff + boff[nb]];
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
                            acc[mb][nb] = VROWS ? mfma_16x16x4(bv[nb], a[mb], acc[mb][nb])
                                                : mfma_16x16x4(a[mb], bv[nb], acc[mb][nb]);
                }
}

// Staging of one chunk for a workgroup whose input box is [id0, id0+HD) x [ih0, ih0+HH) x
// columns [iw0 - pad, iw0 - pad + MAIN + 2), plus its weights.  BUF: the halo is read
// through a buffer resource over the chunk's CC input channels of image n (their byte size
// below 2^31), with 32-bit row offsets and dropped offsets for the padding; otherwise
// through plain loads with a branch per row.
template <int MB, int CC, int HD, int HH, int MAIN, int RS, int CS, int NT, bool VEC, bool BUF>
struct ChunkStage {
    using Halo = std::conditional_t<BUF, BufHaloRows<CC * HD * HH, MAIN, NT, VEC>,
                                    HaloRows<CC * HD * HH, MAIN, NT, VEC>>;
    Halo halo;
    WeightChunk<MB, CC, NT, 27> wts;

    __device__ __forceinline__ void load(const float *__restrict__ x, const float *__restrict__ w,
                                         const Conv3dDims &d, int64_t n, int c0, int o0, int id0,
                                         int ih0, int iw0)
    {
        if constexpr (BUF) {
            const int D = (int)d.D, H = (int)d.H, W = (int)d.W, cn = (int)(d.C - c0);
            auto roff = [&](int row) -> int {
                const int hh = row % HH, t = row / HH;
                const int hd = t % HD, c = t / HD;
                const int id = id0 + hd, ih = ih0 + hh;
                if (c >= cn || (unsigned)id >= (unsigned)D || (unsigned)ih >= (unsigned)H)
                    return -1;
                return 4 * (((c * D + id) * H + ih) * W);
            };
            halo.load(buffer_rsrc(x + (n * d.C + c0) * d.D * d.H * d.W), roff, iw0, d.pad, W);
        } else {
            auto src = [&](int row) -> const float * {
                const int hh = row % HH, t = row / HH;
                const int hd = t % HD, c = t / HD;
                const int ci = c0 + c, id = id0 + hd, ih = ih0 + hh;
                if (ci >= d.C || (unsigned)id >= (unsigned)d.D || (unsigned)ih >= (unsigned)d.H)
                    return nullptr;
                return x + (((n * d.C + ci) * d.D + id) * d.H + ih) * d.W;
            };
            halo.load(src, iw0, d.pad, (int)d.W);
        }
        wts.load(w, d, o0, c0, 27, 0);
    }

    __device__ __forceinline__ void store(float *__restrict__ xs, float *__restrict__ ws,
                                          int pad) const
    {
        auto dst = [&](int row) -> float * {
            const int hh = row % HH, t = row / HH;
            const int hd = t % HD, c = t / HD;
            return xs + c * CS + (hd * HH + hh) * RS;
        };
        halo.store(dst, pad);
        wts.store(ws);
    }
};

// ------------------------------------------------------------------ Mish/tanh epilogue
// Wave (wd, wh) owns output row (od0 + wd, oh0 + wh), columns [ow0, ow0 + 16*NBW).
// ACT: y = tanh(mish(conv + b)); otherwise y = conv + b (the unfused path's conv).
// The voxels are the MFMA rows, so each lane ends with 4 consecutive voxels of one output
// channel, stored with SW-float stores (SW = 2 needs 8-byte aligned output rows, SW = 4
// 16-byte aligned ones).
template <int MB, int NBW, int WD, int WH, int CC, bool VEC, bool BUF, bool ACT, int SW>
__global__ __launch_bounds__(64 * WD * WH, 2) void conv3d_mish_tanh_kernel(
    const float *__restrict__ x, const float *__restrict__ w, const float *__restrict__ b,
    float *__restrict__ y, Conv3dDims d, int64_t tiles, int tiles_w, int tiles_h, int tiles_d)
{
    constexpr int NT = 64 * WD * WH;
    constexpr int MAIN = 16 * NBW;
    constexpr int HD = WD + 2, HH = WH + 2;
    constexpr int RS = MAIN + 8;
    constexpr int CS = halo_channel_stride(HD * HH * RS);
    constexpr int XS = CC * CS;
    constexpr int WSZ = 27 * CC * 16 * MB;
    __shared__ __attribute__((aligned(16))) float lds[XS + WSZ];
    float *xs = lds;
    float *ws = lds + XS;

    // Output-channel group fastest: the groups of one spatial tile are neighbouring tiles, so
    // they run close together on one XCD and the later ones find the tile's input in its L2.
    int64_t t = xcd_tile(blockIdx.x, tiles);
    const int ogs = (int)((d.O + 16 * MB - 1) / (16 * MB));
    const int og = (int)(t % ogs); t /= ogs;
    const int tw = (int)(t % tiles_w); t /= tiles_w;
    const int th = (int)(t % tiles_h); t /= tiles_h;
    const int td = (int)(t % tiles_d); t /= tiles_d;
    const int64_t n = t;

    const int od0 = td * WD, oh0 = th * WH, ow0 = tw * MAIN, o0 = og * 16 * MB;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wd = wave / WH, wh = wave % WH;
    // LDS column of voxel column v at tap kw is v + kw + 4 - pad.
    const int xlane = (lane >> 4) * CS + (wd * HH + wh) * RS + (lane & 15) + 4 - d.pad;
    int boff[NBW];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) boff[nb] = 16 * nb;

    ChunkStage<MB, CC, HD, HH, MAIN, RS, CS, NT, VEC, BUF> stage;
    const int id0 = od0 - d.pad, ih0 = oh0 - d.pad;
    stage.load(x, w, d, n, 0, o0, id0, ih0, ow0);

    const int od = od0 + wd, oh = oh0 + wh;
    if (od < d.OD && oh < d.OH) {
        floatx4 acc[MB][NBW];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
        for (int c0 = 0; c0 < d.C; c0 += CC) {
            __syncthreads();
            stage.store(xs, ws, d.pad);
            __syncthreads();
            if (c0 + CC < d.C) stage.load(x, w, d, n, c0 + CC, o0, id0, ih0, ow0);
            igemm_chunk<MB, NBW, CC, HH, RS, CS, true>(xs, ws, xlane, boff, acc);
        }
        store_conv_row<MB, NBW, ACT, SW>(y, b, d, n, od, oh, ow0, o0, acc);
    } else {
        // This wave's row lies past the output: it only helps stage the shared tiles.
        for (int c0 = 0; c0 < d.C; c0 += CC) {
            __syncthreads();
            stage.store(xs, ws, d.pad);
            __syncthreads();
            if (c0 + CC < d.C) stage.load(x, w, d, n, c0 + CC, o0, id0, ih0, ow0);
        }
    }
}

// ------------------------------------------------------------------ pool/sum epilogue
// Wave (wd, wh) owns pooled windows (pd0 + wd, ph0 + wh, [pw0, pw0 + 8*NBW)).  Its 4*NBW
// voxel blocks are (dd, dh, q): conv voxel (2pd + dd, 2ph + dh, 2pw0 + 16q + j) for lane
// column j, so the max over (dd, dh) is taken inside a lane and the max over the window's
// two columns between lanes j and j^1.
// STORE: instead of the sum, write each window's (max + cb) / divisor to the pooled tensor
// y [N][O][PD][PH][PW] (the divided max: division by a constant is monotone, so this is the
// max of the divided values, rounding included).
template <int MB, int NBW, int WD, int WH, int CC, bool VEC, bool BUF, bool PREFETCH, bool STORE>
__global__ __launch_bounds__(64 * WD * WH, 2) void conv3d_pool_sum_kernel(
    const float *__restrict__ x, const float *__restrict__ w, const float *__restrict__ cb,
    float *__restrict__ out, PoolDims pd_, int64_t tiles, int tiles_w, int tiles_h,
    int tiles_d, float inv_count)
{
    constexpr int NT = 64 * WD * WH;
    constexpr int NB = 4 * NBW;
    constexpr int MAIN = 16 * NBW;
    constexpr int HD = 2 * WD + 2, HH = 2 * WH + 2;
    constexpr int RS = MAIN + 8;
    constexpr int CS = halo_channel_stride(HD * HH * RS);
    constexpr int XS = CC * CS;
    constexpr int WSZ = 27 * CC * 16 * MB;
    __shared__ __attribute__((aligned(16))) float lds[XS + WSZ];
    __shared__ float red[NT / 64];
    float *xs = lds;
    float *ws = lds + XS;
    const Conv3dDims &d = pd_.conv;

    int64_t t = xcd_tile(blockIdx.x, tiles);
    const int tw = (int)(t % tiles_w); t /= tiles_w;
    const int th = (int)(t % tiles_h); t /= tiles_h;
    const int td = (int)(t % tiles_d); t /= tiles_d;
    const int64_t n = t % d.N;
    const int og = (int)(t / d.N);

    const int pd0 = td * WD, ph0 = th * WH, pw0 = tw * 8 * NBW, o0 = og * 16 * MB;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wd = wave / WH, wh = wave % WH;
    const int xlane = (lane >> 4) * CS + (2 * wd * HH + 2 * wh) * RS + (lane & 15) + 4;
    int boff[NB];
#pragma unroll
    for (int dd = 0; dd < 2; ++dd)
#pragma unroll
        for (int dh = 0; dh < 2; ++dh)
#pragma unroll
            for (int q = 0; q < NBW; ++q)
                boff[(dd * 2 + dh) * NBW + q] = (dd * HH + dh) * RS + 16 * q;

    ChunkStage<MB, CC, HD, HH, MAIN, RS, CS, NT, VEC, BUF> stage;
    auto next = [&](int c0) {
        // With PREFETCH the chunk after c0 is loaded into registers while c0 computes;
        // without it each chunk is loaded right before it is stored, and other resident
        // workgroups cover the latency.
        if constexpr (PREFETCH) {
            if (c0 + CC < d.C) stage.load(x, w, d, n, c0 + CC, o0, 2 * pd0, 2 * ph0, 2 * pw0);
        }
    };
    auto put = [&](int c0) {
        if constexpr (!PREFETCH) stage.load(x, w, d, n, c0, o0, 2 * pd0, 2 * ph0, 2 * pw0);
        stage.store(xs, ws, 0);
    };
    if constexpr (PREFETCH) stage.load(x, w, d, n, 0, o0, 2 * pd0, 2 * ph0, 2 * pw0);

    const int pdi = pd0 + wd, phi = ph0 + wh;
    float part = 0.0f;
    if (pdi < pd_.PD && phi < pd_.PH) {
        floatx4 acc[MB][NB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
        for (int c0 = 0; c0 < d.C; c0 += CC) {
            __syncthreads();
            put(c0);
            __syncthreads();
            next(c0);
            igemm_chunk<MB, NB, CC, HH, RS, CS>(xs, ws, xlane, boff, acc);
        }
        // (conv + cb) / divisor is monotone in conv: increasing for a positive divisor, so
        // the window maximum of the divided values is (max conv + cb) / divisor; for a
        // negative divisor it is (min conv + cb) / divisor.  The direction is uniform, so
        // each gets its own code.  The sum path adds the undivided (extreme + cb) and divides
        // the workgroup's total once.
        const int j = lane & 15;
        auto windows = [&](auto use_min) {
            constexpr bool MIN = decltype(use_min)::value;
            auto ext = [](float a, float b) { return MIN ? fminf(a, b) : fmaxf(a, b); };
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int o = o0 + 16 * mb + 4 * (lane >> 4) + r;
                    const float cbv = (cb && o < d.O) ? cb[o] : 0.0f;
#pragma unroll
                    for (int q = 0; q < NBW; ++q) {
                        float m = acc[mb][q][r];
#pragma unroll
                        for (int p = 1; p < 4; ++p) m = ext(m, acc[mb][p * NBW + q][r]);
                        m = ext(m, __shfl_xor(m, 1, 64));
                        const int pw = pw0 + 8 * q + (j >> 1);
                        if (o < d.O && (j & 1) == 0 && pw < pd_.PW) {
                            if constexpr (STORE)
                                out[(((n * d.O + o) * pd_.PD + pdi) * pd_.PH + phi) * pd_.PW + pw] =
                                    (m + cbv) / pd_.divisor;
                            else
                                part += m + cbv;
                        }
                    }
                }
        };
        if (pd_.divisor < 0.0f) windows(std::true_type{});
        else windows(std::false_type{});
    } else {
        for (int c0 = 0; c0 < d.C; c0 += CC) {
            __syncthreads();
            put(c0);
            __syncthreads();
            next(c0);
        }
    }
    if constexpr (STORE) return;  // (no barrier follows: every wave returns here)
    part = wave_sum(part);
    if (lane == 0) red[wave] = part;
    __syncthreads();
    if (threadIdx.x == 0) {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < NT / 64; ++i) s += red[i];
        atomicAdd(out + n, s * inv_count / pd_.divisor);
    }
}

// out[n] = sum_c bias[c]: the constant part of the page-l2_p8 rewrite, written before the
// pooled partial sums are added.
__global__ void pool_sum_init_kernel(const float *__restrict__ bias, float *__restrict__ out,
                                     int64_t N, int64_t O)
{
    const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= N) return;
    float s = 0.0f;
    for (int64_t c = 0; c < O; ++c) s += bias[c];
    out[n] = s;
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline bool vec_ok(const float *x, int64_t W) { return W % 4 == 0 && ((uintptr_t)x & 15) == 0; }

// 32-bit byte offsets over one staged chunk of CC input channels
inline bool buf_ok(const Conv3dDims &d, int CC) { return 4 * CC * d.D * d.H * d.W <= kBufRange; }

template <int MB, int NBW, int WD, int WH, int CC, bool VEC, bool BUF, bool ACT>
void launch_act_kernel(const float *x, const float *w, const float *b, float *y,
                       const Conv3dDims &d, int64_t tiles, int64_t tw, int64_t th, int64_t td,
                       hipStream_t s)
{
    const int sw = conv_store_width(y, d.OW);
    auto go = [&](auto kern) {
        note_kernel("conv3d_mish_tanh_kernel");
        hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(64 * WD * WH), 0, s, x, w, b, y, d,
                           tiles, (int)tw, (int)th, (int)td);
    };
    if (sw == 4) go(conv3d_mish_tanh_kernel<MB, NBW, WD, WH, CC, VEC, BUF, ACT, 4>);
    else if (sw == 2) go(conv3d_mish_tanh_kernel<MB, NBW, WD, WH, CC, VEC, BUF, ACT, 2>);
    else go(conv3d_mish_tanh_kernel<MB, NBW, WD, WH, CC, VEC, BUF, ACT, 1>);
}

template <int MB, int NBW, int WD, int WH, int CC, bool ACT>
hipError_t launch_act(const float *x, const float *w, const float *b, float *y,
                      const Conv3dDims &d, hipStream_t s)
{
    const int64_t tw = cdiv(d.OW, 16 * NBW), th = cdiv(d.OH, WH), td = cdiv(d.OD, WD);
    const int64_t og = cdiv(d.O, 16 * MB);
    const int64_t tiles = tw * th * td * d.N * og;
    if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const bool v = vec_ok(x, d.W), bf = buf_ok(d, CC);
    if (v && bf) launch_act_kernel<MB, NBW, WD, WH, CC, true, true, ACT>(x, w, b, y, d, tiles, tw, th, td, s);
    else if (v) launch_act_kernel<MB, NBW, WD, WH, CC, true, false, ACT>(x, w, b, y, d, tiles, tw, th, td, s);
    else if (bf) launch_act_kernel<MB, NBW, WD, WH, CC, false, true, ACT>(x, w, b, y, d, tiles, tw, th, td, s);
    else launch_act_kernel<MB, NBW, WD, WH, CC, false, false, ACT>(x, w, b, y, d, tiles, tw, th, td, s);
    return hipGetLastError();
}

template <int MB, int NBW, int WD, int WH, int CC, bool VEC, bool BUF, bool STORE>
void launch_pool_kernel(const float *x, const float *w, const float *conv_b, float *out,
                        const PoolDims &p, int64_t tiles, int64_t tw, int64_t th, int64_t td,
                        float inv_count, hipStream_t s)
{
    note_kernel("conv3d_pool_sum_kernel");
    hipLaunchKernelGGL((conv3d_pool_sum_kernel<MB, NBW, WD, WH, CC, VEC, BUF, BUF, STORE>),
                       dim3((unsigned)tiles), dim3(64 * WD * WH), 0, s, x, w, conv_b, out, p,
                       tiles, (int)tw, (int)th, (int)td, inv_count);
}

}  // namespace

namespace {

template <bool ACT>
hipError_t launch_conv3d(const float *x, const float *w, const float *b, float *y,
                         const Conv3dDims &d, hipStream_t s)
{
    // 64 output channels per workgroup from 65 up; 32 from 17 to 64 (measured 1.7 % faster on
    // the 64-channel layer: 4 workgroups fit per CU instead of 3, at the cost of staging the
    // input twice from L2)
    const bool wide = d.OW > 16;
    if (d.O > 64) {
        if (wide) return launch_act<4, 4, 2, 2, 4, ACT>(x, w, b, y, d, s);
        return launch_act<4, 1, 2, 2, 4, ACT>(x, w, b, y, d, s);
    }
    if (d.O > 16) {
        if (wide) return launch_act<2, 4, 2, 2, 4, ACT>(x, w, b, y, d, s);
        return launch_act<2, 1, 2, 2, 4, ACT>(x, w, b, y, d, s);
    }
    if (wide) return launch_act<1, 4, 2, 2, 4, ACT>(x, w, b, y, d, s);
    return launch_act<1, 1, 2, 2, 4, ACT>(x, w, b, y, d, s);
}

}  // namespace

hipError_t launch_conv3d_mish_tanh(const float *x, const float *w, const float *b, float *y,
                                   const Conv3dDims &d, hipStream_t s)
{
    return launch_conv3d<true>(x, w, b, y, d, s);
}

hipError_t launch_conv3d_bias(const float *x, const float *w, const float *b, float *y,
                              const Conv3dDims &d, hipStream_t s)
{
    return launch_conv3d<false>(x, w, b, y, d, s);
}

hipError_t launch_pool_sum_init(const float *bias, float *out, int64_t N, int64_t O,
                                hipStream_t s)
{
    note_kernel("pool_sum_init_kernel");
    hipLaunchKernelGGL(pool_sum_init_kernel, dim3((unsigned)cdiv(N, 256)), dim3(256), 0, s, bias,
                       out, N, O);
    return hipGetLastError();
}

namespace {

template <bool STORE>
hipError_t launch_pool(const float *x, const float *w, const float *conv_b, float *out,
                       const PoolDims &p, hipStream_t s)
{
    constexpr int MB = 1, NBW = 4, WD = 1, WH = 4, CC = 4;
    const Conv3dDims &d = p.conv;
    const int64_t tw = cdiv(p.PW, 8 * NBW), th = cdiv(p.PH, WH), td = cdiv(p.PD, WD);
    const int64_t og = cdiv(d.O, 16 * MB);
    const int64_t tiles = tw * th * td * d.N * og;
    if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const float inv_count = (float)(1.0 / ((double)p.PD * (double)p.PH * (double)p.PW));
    const bool v = vec_ok(x, d.W), bf = buf_ok(d, CC);
    if (v && bf) launch_pool_kernel<MB, NBW, WD, WH, CC, true, true, STORE>(x, w, conv_b, out, p, tiles, tw, th, td, inv_count, s);
    else if (v) launch_pool_kernel<MB, NBW, WD, WH, CC, true, false, STORE>(x, w, conv_b, out, p, tiles, tw, th, td, inv_count, s);
    else if (bf) launch_pool_kernel<MB, NBW, WD, WH, CC, false, true, STORE>(x, w, conv_b, out, p, tiles, tw, th, td, inv_count, s);
    else launch_pool_kernel<MB, NBW, WD, WH, CC, false, false, STORE>(x, w, conv_b, out, p, tiles, tw, th, td, inv_count, s);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_conv3d_pool_sum(const float *x, const float *w, const float *conv_b,
                                  const float *bias, float *out, const PoolDims &p,
                                  hipStream_t s)
{
    const hipError_t e = launch_pool_sum_init(bias, out, p.conv.N, p.conv.O, s);
    if (e != hipSuccess) return e;
    return launch_pool<false>(x, w, conv_b, out, p, s);
}

hipError_t launch_conv3d_div_maxpool(const float *x, const float *w, const float *conv_b,
                                     float *y, const PoolDims &p, hipStream_t s)
{
    return launch_pool<true>(x, w, conv_b, y, p, s);
}

}  // namespace convfuse
