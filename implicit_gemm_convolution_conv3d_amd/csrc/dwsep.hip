// dwsep.hip -- fused depthwise 3x3 + pointwise 1x1 Conv2d on gfx950
// (page "Kimi-K2.6 l1_p86", depthwise-separable Conv2d: the fused definition and the
// implicit-GEMM view of the pointwise step, with the depthwise computed while the GEMM
// operand is formed).
//
// GEMM view: output pixels x output channels, reduced over input channels.  For a 16x16x4
// MFMA k-step, lane l forms the pixel-side operand as the depthwise output of channel
// (4*cg + l/16) at pixel column (l%16): nine reads of the staged input halo and nine FMAs,
// so the depthwise tile never leaves registers.  fp32 vector work does not overlap fp32
// matrix work on this chip, so the inner loop holds no other vector instructions.
//
// Each wave owns R output rows x 16 pixel columns and every output channel of its channel
// group, so the input is read once per channel group.  Workgroups are 4 waves wide (tile 64
// columns) and WH waves tall.  Input channels stream through LDS in chunks of CC (32 when the
// weights leave room, else 16): thread t stages channel (t/16)%CC, column quad t%16 of its
// share of the halo rows (one float4 per row when rows are 16-byte aligned, else four
// dwords); the next chunk is loaded into registers while the current one computes.
//
// Two kernels:
//  * persistent (all pointwise weights and depthwise taps fit in LDS next to one chunk):
//    weights are loaded once per workgroup, in MFMA fragment order; workgroups then loop
//    over tiles, and the first chunk of the next tile streams in while the last chunk of the
//    current one computes.  Barriers order LDS only, and outputs leave through buffer
//    stores with a fixed instruction count per tile, so a tile's stores drain while the
//    next tile computes.
//  * chunked (any size): one tile per workgroup, weights staged with every chunk.
//
// Operand roles: the pointwise weights are the MFMA's A operand and the depthwise outputs
// (pixels) its B operand, so each lane ends with 4 output channels of one pixel and a store
// instruction writes 4 channels x 64 contiguous bytes.  With the roles swapped each lane
// would hold 4 consecutive pixels of one channel and could store float4s, 16 channels x 64
// bytes per instruction; on the 512 x 512 layer that order measured 6-9 % slower in this
// kernel, although a store-only test writes it faster: the difference comes from how the
// stores interleave with the halo loads and the matrix work, not from the raw write rate.
#include "common.hpp"
#include "kernels.hpp"

namespace convfuse {

namespace {

constexpr int kDwCC = 16;  // input channels per chunk of the chunked kernel
constexpr int kDwTW = 64;  // output tile width (4 waves x 16 columns)

// Tile geometry: 4*WH waves, R output rows per wave, tile 64 columns x R*WH rows; CC input
// channels per chunk.  Staging threads: (channel, column quad) pairs fill 16*CC threads; the
// remaining factor RG splits the halo rows.
template <int R, int WH, int CC>
struct DwGeom {
    static constexpr int NWAVE = 4 * WH;
    static constexpr int NT = 64 * NWAVE;
    static constexpr int TH = R * WH;                  // output tile rows
    static constexpr int HR = TH + 2;                  // halo rows
    static_assert(NT % (16 * CC) == 0, "whole (channel, quad) groups");
    static constexpr int RG = NT / (16 * CC);          // row groups
    static_assert(HR % RG == 0, "halo rows split evenly over the row groups");
    static constexpr int RPT = HR / RG;                // halo rows per staging thread
    static constexpr int RS = kDwTW + 8;               // LDS row: 4 + 64 columns + edges
    static constexpr int CS = halo_channel_stride(HR * RS);
    static constexpr int XS = CC * CS;                 // one chunk of halo
    static constexpr int EDGES = 2 * CC * HR;          // edge values per chunk
    static constexpr int PE = (EDGES + NT - 1) / NT;   // edge values per thread
};

// Halo rows of one chunk held in registers between global load and LDS store.
template <int R, int WH, int CC>
struct DwHalo {
    floatx4 xr[DwGeom<R, WH, CC>::RPT];
    float edge[DwGeom<R, WH, CC>::PE];
};

// Load (registers) and store (LDS) of one chunk of the halo of tile (n, h0, w0).  Thread t:
// channel sc = (t/16)%CC, column quad sq = t%16, halo rows rg*RPT .. +RPT-1 (rg = t/(16CC));
// edge value e = t + p*NT (< EDGES) is the column left of w0 or right of w0+63 of channel
// e/(2HR), halo row (e%(2HR))/2.  LDS row layout: column 4 + j holds global column w0 + j.
// BUF: loads through a buffer resource over image n (its byte size below 2^31), with
// dropped offsets for the zero padding, instead of branches around plain loads.
template <int R, int WH, int CC, bool VEC, bool BUF>
struct DwHaloStager {
    using G = DwGeom<R, WH, CC>;
    int sc, sq, rg;
    int ec[G::PE], ehr[G::PE], eoff[G::PE];

    __device__ __forceinline__ void init(int tid, int pad)
    {
        sc = (tid >> 4) % CC;
        sq = tid & 15;
        rg = tid / (16 * CC);
#pragma unroll
        for (int p = 0; p < G::PE; ++p) {
            const int e = tid + p * G::NT;
            ec[p] = e < G::EDGES ? e / (2 * G::HR) : CC;  // CC: no edge value
            const int erem = e % (2 * G::HR);
            ehr[p] = erem >> 1;
            const int ej = erem & 1;
            eoff[p] = ej < pad ? -pad + ej : kDwTW + ej - pad;  // edge column - w0
        }
    }

    __device__ __forceinline__ void load(DwHalo<R, WH, CC> &k, const float *__restrict__ x,
                                         const DwsepDims &d, int64_t n, int h0, int w0,
                                         int c0) const
    {
        const int C = (int)d.C, H = (int)d.H, W = (int)d.W;
        const int64_t plane = (int64_t)H * W;
        const int ih0 = h0 - d.pad;
        const int col = w0 + 4 * sq;
        const int ci = c0 + sc;
        if constexpr (BUF) {
            const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(x + n * C * plane);
            const bool cok = ci < C;
            // (channel clamped so that the unused offsets of absent channels stay in range)
            const int base = 4 * (((cok ? ci : 0) * H + ih0) * W + col);
#pragma unroll
            for (int i = 0; i < G::RPT; ++i) {
                const int hr = rg * G::RPT + i;
                const bool rok = cok && (unsigned)(ih0 + hr) < (unsigned)H;
                if constexpr (VEC) {
                    const int off = rok && col < W ? base + 4 * hr * W : kDropOffset;
                    k.xr[i] = __builtin_bit_cast(
                        floatx4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
                } else if (col + 4 <= W) {
                    // rows only 4-byte aligned: buffer loads need dword alignment only, so a
                    // quad inside the row is still one 16-byte load
                    const int off = rok ? base + 4 * hr * W : kDropOffset;
                    k.xr[i] = __builtin_bit_cast(
                        floatx4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
                } else {
                    // the quad the row end cuts (or one past it): single loads, none beyond W
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int off = rok && col + e < W ? base + 4 * (hr * W + e) : kDropOffset;
                        k.xr[i][e] =
                            __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
                    }
                }
            }
#pragma unroll
            for (int p = 0; p < G::PE; ++p) {
                const int eci = c0 + ec[p], eih = ih0 + ehr[p], ecol = w0 + eoff[p];
                const bool eok = ec[p] < CC && eci < C && (unsigned)eih < (unsigned)H &&
                                 (unsigned)ecol < (unsigned)W;
                const int eoffb =
                    eok ? 4 * (((eci < C ? eci : 0) * H + eih) * W + ecol) : kDropOffset;
                k.edge[p] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, eoffb, 0, 0));
            }
            return;
        }
        const float *p = x + (n * C + ci) * plane + (int64_t)ih0 * W + col;
#pragma unroll
        for (int i = 0; i < G::RPT; ++i) {
            const int hr = rg * G::RPT + i;
            floatx4 v = {0.f, 0.f, 0.f, 0.f};
            if (ci < C && (unsigned)(ih0 + hr) < (unsigned)H) {
                const float *rp = p + (int64_t)hr * W;
                if constexpr (VEC) {
                    if (col < W) v = *reinterpret_cast<const floatx4 *>(rp);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (col + e < W) v[e] = rp[e];
                }
            }
            k.xr[i] = v;
        }
#pragma unroll
        for (int q = 0; q < G::PE; ++q) {
            const int eci = c0 + ec[q], eih = ih0 + ehr[q], ecol = w0 + eoff[q];
            float e = 0.0f;
            if (ec[q] < CC && eci < C && (unsigned)eih < (unsigned)H && (unsigned)ecol < (unsigned)W)
                e = x[((n * C + eci) * H + eih) * (int64_t)W + ecol];
            k.edge[q] = e;
        }
    }

    __device__ __forceinline__ void store(float *xs, const DwHalo<R, WH, CC> &k) const
    {
        float *row = xs + sc * G::CS + rg * G::RPT * G::RS + 4 + 4 * sq;
#pragma unroll
        for (int i = 0; i < G::RPT; ++i) *reinterpret_cast<floatx4 *>(row + i * G::RS) = k.xr[i];
#pragma unroll
        for (int p = 0; p < G::PE; ++p)
            if (ec[p] < CC) xs[ec[p] * G::CS + ehr[p] * G::RS + 4 + eoff[p]] = k.edge[p];
    }
};

// One chunk of the K loop, reading LDS array `lds` at per-lane float offsets: xoff, the
// chunk's halo (channel lane/16 of k-step 0 at the lane's pixel column, tap (0, 0)); poff,
// the chunk's fragment-order pointwise weights (lds[poff + cg*64*MB + mb] is the operand of
// k-step cg, output block mb); doff, the depthwise taps [c][12] (9 taps, bias at 9) of the
// chunk's channel lane/16 (channel 4*cg + lane/16 at doff + 48*cg).  The offsets are opaque
// to the optimiser, so each read is one base register plus an immediate offset: the weights
// lie beyond the 16-bit immediate range from the start of LDS, and folding the region start
// into every read costs a vector add per read.
// DW = false: pointwise only (the unfused path's second pass); the operand is the staged
// input itself, x at the centre tap of the K = 3, pad 1 halo.
template <int MB, int R, int RS, int CS, int CC, bool DW = true>
__device__ __forceinline__ void dw_chunk(const float *lds, int xoff, int poff, int doff,
                                         floatx4 (&acc)[MB][R])
{
    asm volatile("" : "+v"(poff), "+v"(doff));
#pragma unroll
    for (int cg = 0; cg < CC / 4; ++cg) {
        const floatx4 k0 = *reinterpret_cast<const floatx4 *>(lds + doff + 48 * cg);
        const floatx4 k1 = *reinterpret_cast<const floatx4 *>(lds + doff + 48 * cg + 4);
        const floatx4 k2 = *reinterpret_cast<const floatx4 *>(lds + doff + 48 * cg + 8);
        const float kw9[9] = {k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3], k2[0]};
        const float dbias = k2[1];
        float pwf[MB];
#pragma unroll
        for (int i = 0; i < MB / 4; ++i) {
            const floatx4 v =
                *reinterpret_cast<const floatx4 *>(lds + poff + cg * 64 * MB + 4 * i);
            pwf[4 * i + 0] = v[0];
            pwf[4 * i + 1] = v[1];
            pwf[4 * i + 2] = v[2];
            pwf[4 * i + 3] = v[3];
        }
        float xv[R + 2][3];
        // one base per k-step; the R + 2 rows x 3 taps are immediate offsets from it
        int xo = xoff + 4 * cg * CS;
        asm volatile("" : "+v"(xo));
#pragma unroll
        for (int hr = 0; hr < R + 2; ++hr)
#pragma unroll
            for (int kw = 0; kw < 3; ++kw) xv[hr][kw] = lds[xo + hr * RS + kw];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float v = xv[r + 1][1];
            if constexpr (DW) {
                v = dbias;
#pragma unroll
                for (int kh = 0; kh < 3; ++kh)
#pragma unroll
                    for (int kw = 0; kw < 3; ++kw) v = fmaf(kw9[kh * 3 + kw], xv[r + kh][kw], v);
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) acc[mb][r] = mfma_16x16x4(pwf[mb], v, acc[mb][r]);
        }
    }
}

// Store one wave's R x 16 outputs of output channels [obase, obase + ocnt): lane holds
// channels 16*mb + 4*(lane/16) + 0..3 of pixel wcol0 + lane%16.
template <int MB, int R>
__device__ __forceinline__ void dw_epilogue(float *__restrict__ y, const DwsepDims &d, int64_t n,
                                            int hbase, int wcol0, int obase, int ocnt,
                                            const floatx4 (&acc)[MB][R])
{
    const int lane = threadIdx.x & 63;
    const int wcol = wcol0 + (lane & 15);
    if (wcol >= d.Wo) return;
    int64_t cstride = (int64_t)d.Ho * d.Wo;
    // Opaque to the optimiser: keeps the per-channel offsets from being hoisted out of the
    // caller's tile loop, where they would pin dozens of scalar registers.
    asm volatile("" : "+s"(cstride));
    float *yp = y + ((n * d.O + obase + 4 * (lane >> 4)) * d.Ho + hbase) * d.Wo + wcol;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int ol = 16 * mb + 4 * (lane >> 4) + r4;
            if (ol < ocnt) {
#pragma unroll
                for (int r = 0; r < R; ++r)
                    if (hbase + r < d.Ho) yp[(int64_t)r * d.Wo] = acc[mb][r][r4];
            }
            yp += r4 == 3 ? 13 * cstride : cstride;
        }
}

// Accumulators start at the pointwise bias.  bs[16*mb + j] is the bias of output channel
// obase + 16*mb + j (0 past the slice or without bias).
template <int MB, int R>
__device__ __forceinline__ void acc_init(floatx4 (&acc)[MB][R], const float *bs)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const floatx4 b = *reinterpret_cast<const floatx4 *>(bs + 16 * mb + 4 * (lane >> 4));
#pragma unroll
        for (int r = 0; r < R; ++r) acc[mb][r] = b;
    }
}

// ----------------------------------------------------------------- persistent kernel
// Store one wave's R x 16 outputs of output channels [obase, obase + ocnt): tb points at
// (n, obase, row h0, column 0); the wave's rows start at h0 + hrow0, its columns at wcol0.
// Byte offsets from tb stay below 2^31 (checked by the host).
template <int MB, int R>
__device__ __forceinline__ void dw_epilogue_buf(float *tb, const DwsepDims &d, int hrow0,
                                                int hleft, int wcol0, int ocnt,
                                                const floatx4 (&acc)[MB][R])
{
    const int lane = threadIdx.x & 63;
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(tb);
    int plane = (int)(d.Ho * d.Wo);  // < 2^25 here
    int wo = (int)d.Wo;
    // Opaque to the optimiser: keeps the per-store offsets and lane masks from being hoisted
    // out of the caller's tile loop, where they would pin dozens of scalar registers.
    asm volatile("" : "+s"(plane), "+s"(wo), "+s"(ocnt));
    // lane holds channels 16*mb + 4*(lane/16) + 0..3 of pixel wcol0 + lane%16
    const int wcol = wcol0 + (lane & 15);
    int vmb = 4 * (4 * (lane >> 4) * plane + hrow0 * wo + wcol);  // channel block mb
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const bool ok = 16 * mb + 4 * (lane >> 4) + r4 < ocnt && r < hleft && wcol < wo;
                const int off = ok ? vmb + 4 * (r4 * plane + r * wo) : kDropOffset;
                // (a vector element is copied out first: bit-casting the element expression
                // itself would reinterpret the vector's first element)
                const float v = acc[mb][r][r4];
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs, off, 0, 0);
            }
        vmb += 64 * plane;
        asm volatile("" : "+v"(vmb));  // one running offset, not MB*4*R folded constants
    }
}

// Fill `total` LDS slots: element e (value(e), typically a global load) goes to
// dst[slot(e)].  B global loads per thread are in flight before the first LDS write.
template <int NT, int B, class V, class S>
__device__ __forceinline__ void lds_fill(float *dst, int total, const V &value, const S &slot)
{
    for (int base = threadIdx.x; base < total; base += B * NT) {
        float v[B];
#pragma unroll
        for (int u = 0; u < B; ++u) {
            const int e = base + u * NT;
            v[u] = e < total ? value(e) : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < B; ++u) {
            const int e = base + u * NT;
            if (e < total) dst[slot(e)] = v[u];
        }
    }
}

// Dynamic LDS: [halo chunk XS][pointwise fragments KS*64*MB][depthwise taps 4*KS*12]
// [pointwise bias 16*MB], KS = (CC/4)*ceil(C/CC) k-steps (whole chunks; zero past C).  Fragment
// order: pwall[(s*64 + lane)*MB + mb] = pw_w[obase + 16*mb + lane%16][4*s + lane/16].
template <int MB, int CC>
constexpr size_t dw_weight_floats(int64_t C)
{
    const int64_t KS = (C + CC - 1) / CC * (CC / 4);
    return (size_t)(KS * 64 * MB + 4 * KS * 12 + 16 * MB);
}

template <int MB, int R, int WH, int CC, bool VEC, bool DW>
__global__ __launch_bounds__(256 * WH, 2 / WH) void dwsep_persistent_kernel(
    const float *__restrict__ x, const float *__restrict__ dw_w, const float *__restrict__ dw_b,
    const float *__restrict__ pw_w, const float *__restrict__ pw_b, float *__restrict__ y,
    DwsepDims d, int obase, int64_t tiles, int tiles_w, int tiles_h)
{
    using G = DwGeom<R, WH, CC>;
    extern __shared__ __attribute__((aligned(16))) float dyn[];
    const int C = (int)d.C;  // small: the weights fit in LDS
    const int KS = (C + CC - 1) / CC * (CC / 4);
    float *xs = dyn;
    float *pwall = dyn + G::XS;
    float *dkall = pwall + KS * 64 * MB;
    float *bs = dkall + 4 * KS * 12;
    const int ocnt = (int)(d.O - obase < 16 * MB ? d.O - obase : 16 * MB);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ww = wave & 3, wh = wave >> 2;

    // Weights, once per workgroup.  Pointwise rows are read along input channels and placed
    // at their fragment slots.
    const int K4 = 4 * KS;
    lds_fill<G::NT, 8>(
        pwall, 16 * MB * K4,
        [&](int e) {
            const int ol = e / K4, c = e - ol * K4;
            return (ol < ocnt && c < C) ? pw_w[(int64_t)(obase + ol) * C + c] : 0.0f;
        },
        [&](int e) {
            const int ol = e / K4, c = e - ol * K4;
            return ((c >> 2) * 64 + (c & 3) * 16 + (ol & 15)) * MB + (ol >> 4);
        });
    lds_fill<G::NT, 4>(
        dkall, K4 * 12,
        [&](int e) {
            const int c = e / 12, k = e - c * 12;
            float v = 0.0f;
            if (DW && c < C) {
                if (k < 9) v = dw_w[(int64_t)c * 9 + k];
                else if (k == 9 && dw_b) v = dw_b[c];
            }
            return v;
        },
        [](int e) { return e; });
    if (tid < 16 * MB) bs[tid] = (pw_b && tid < ocnt) ? pw_b[obase + tid] : 0.0f;

    DwHaloStager<R, WH, CC, VEC, true> hs;
    hs.init(tid, d.pad);
    // lane bases: halo (pixel column 16*ww + j, rows R*wh ..; tap kw reads LDS column
    // 16*ww + j + kw + 4 - pad), pointwise fragments, depthwise taps of channel lane/16
    const float *xl = xs + (lane >> 4) * G::CS + R * wh * G::RS + 16 * ww + (lane & 15) + 4 - d.pad;
    const float *pl = pwall + lane * MB;
    const float *dl = dkall + (lane >> 4) * 12;

    // tile counts are below 2^31 (checked by the host): 32-bit index arithmetic
    auto decode = [&](int64_t tile, int64_t &n, int &h0, int &w0) {
        uint32_t t = (uint32_t)xcd_tile(tile, tiles);
        const uint32_t tw = t % (uint32_t)tiles_w;
        t /= (uint32_t)tiles_w;
        const uint32_t th = t % (uint32_t)tiles_h;
        n = t / (uint32_t)tiles_h;
        h0 = (int)th * G::TH;
        w0 = (int)tw * kDwTW;
    };

    // Per chunk: load the next chunk (after the last one, chunk 0 of the next tile) into
    // registers, compute this one, stage the next one.  After a tile's last chunk the outputs
    // are stored before the staging; that staging is reached on this one path, so its wait
    // covers the prefetched loads and not the stores issued after them.
    int64_t tile = blockIdx.x, n;
    int h0, w0;
    decode(tile, n, h0, w0);
    DwHalo<R, WH, CC> k;
    hs.load(k, x, d, n, h0, w0, 0);
    lds_barrier();  // weights written; no wave reads the halo buffer yet
    hs.store(xs, k);
    lds_barrier();
    floatx4 acc[MB][R];
    for (;;) {
        acc_init<MB, R>(acc, bs);
        const int64_t ntile = tile + gridDim.x;
        int64_t nn = 0;
        int nh0 = 0, nw0 = 0;
        for (int c0 = 0;; c0 += CC) {
            const bool last = c0 + CC >= C;
            int64_t ln = n;
            int lh = h0, lw = w0, lc = c0 + CC;
            if (last) {
                if (ntile < tiles) decode(ntile, nn, nh0, nw0);
                ln = nn;
                lh = nh0;
                lw = nw0;
                lc = 0;
            }
            if (!last || ntile < tiles) hs.load(k, x, d, ln, lh, lw, lc);
            dw_chunk<MB, R, G::RS, G::CS, CC, DW>(
                dyn, (int)(xl - dyn), (int)(pl - dyn) + (c0 / 4) * 64 * MB,
                (int)(dl - dyn) + c0 * 12, acc);
            if (last) break;
            lds_barrier();
            hs.store(xs, k);
            lds_barrier();
        }
        float *tb = y + ((n * d.O + obase) * d.Ho + h0) * d.Wo;
        dw_epilogue_buf<MB, R>(tb, d, R * wh, (int)(d.Ho - h0) - R * wh, w0 + 16 * ww,
                                        ocnt, acc);
        if (ntile >= tiles) break;
        tile = ntile;
        n = nn;
        h0 = nh0;
        w0 = nw0;
        lds_barrier();
        hs.store(xs, k);
        lds_barrier();
    }
}

// ----------------------------------------------------------------- split-bf16 kernel
// Opt-in emulation of the fp32 pointwise GEMM on bf16 matrix cores: each fp32 operand v is
// split into hi = bf16(v) (nearest) and lo = bf16(v - hi), and v*w is taken as
// hi_v*hi_w + hi_v*lo_w + lo_v*hi_w with fp32 accumulation (the dropped lo*lo term and the
// split residuals change each product by at most 3 * 2^-16 |v*w|).  The depthwise step stays fp32 on the vector
// ALUs.  One 16x16x32 bf16 k-step covers a 32-channel chunk: lane group g = lane/16 holds
// the channels g + 4i (i = 0..7) of its output channel (A) or pixel (B), so the four groups
// read four different LDS bank groups of the halo.  Same tiles, staging, prefetch and
// epilogue as the persistent fp32 kernel.
// LDS bytes of the split kernel's weights: pointwise hi and lo fragments (KS k-steps of 32
// channels x 64 lanes x MB, 16 bytes each), depthwise taps [32*KS][12], pointwise bias.
template <int MB>
constexpr size_t split_weight_bytes(int64_t C)
{
    const int64_t KS = (C + 31) / 32;
    return (size_t)(2 * KS * 64 * MB * 16 + KS * 32 * 12 * 4 + 16 * MB * 4);
}

template <int MB, int R, int WH, bool VEC>
__global__ __launch_bounds__(256 * WH, 2 / WH) void dwsep_split_kernel(
    const float *__restrict__ x, const float *__restrict__ dw_w, const float *__restrict__ dw_b,
    const float *__restrict__ pw_w, const float *__restrict__ pw_b, float *__restrict__ y,
    DwsepDims d, int obase, int64_t tiles, int tiles_w, int tiles_h)
{
    constexpr int CC = 32;
    using G = DwGeom<R, WH, CC>;
    extern __shared__ __attribute__((aligned(16))) float dyn[];
    const int C = (int)d.C;  // small: the weights fit in LDS
    const int KS = (C + CC - 1) / CC;
    float *xs = dyn;
    bf16x8 *pwh = reinterpret_cast<bf16x8 *>(dyn + G::XS);
    bf16x8 *pwl = pwh + KS * 64 * MB;
    float *dkall = reinterpret_cast<float *>(pwl + KS * 64 * MB);
    float *bs = dkall + KS * 32 * 12;
    const int ocnt = (int)(d.O - obase < 16 * MB ? d.O - obase : 16 * MB);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ww = wave & 3, wh = wave >> 2;

    // Pointwise fragments: entry (s, l, mb) element i = pw[obase + 16mb + l%16][32s + l/16 + 4i]
    for (int e = tid; e < KS * 64 * MB; e += G::NT) {
        const int mb = e % MB, l = (e / MB) & 63, st = e / (64 * MB);
        const int ol = 16 * mb + (l & 15);
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = 32 * st + (l >> 4) + 4 * i;
            v[i] = (ol < ocnt && c < C) ? pw_w[(int64_t)(obase + ol) * C + c] : 0.0f;
        }
        bf16x8 hi, lo;
        split_bf16(v, hi, lo);
        pwh[e] = hi;
        pwl[e] = lo;
    }
    lds_fill<G::NT, 4>(
        dkall, KS * 32 * 12,
        [&](int e) {
            const int c = e / 12, k = e - c * 12;
            float v = 0.0f;
            if (c < C) {
                if (k < 9) v = dw_w[(int64_t)c * 9 + k];
                else if (k == 9 && dw_b) v = dw_b[c];
            }
            return v;
        },
        [](int e) { return e; });
    if (tid < 16 * MB) bs[tid] = (pw_b && tid < ocnt) ? pw_b[obase + tid] : 0.0f;

    DwHaloStager<R, WH, CC, VEC, true> hs;
    hs.init(tid, d.pad);
    const int g = lane >> 4;
    // lane bases: channel g of the chunk (channel g + 4i at + 4i*CS), pixel column
    // 16*ww + lane%16, tap kw at LDS column + kw; depthwise taps of channel g (+ 48i)
    const float *xl = xs + g * G::CS + R * wh * G::RS + 16 * ww + (lane & 15) + 4 - d.pad;
    const float *dl = dkall + g * 12;

    auto decode = [&](int64_t tile, int64_t &n, int &h0, int &w0) {
        uint32_t t = (uint32_t)xcd_tile(tile, tiles);
        const uint32_t tw = t % (uint32_t)tiles_w;
        t /= (uint32_t)tiles_w;
        const uint32_t th = t % (uint32_t)tiles_h;
        n = t / (uint32_t)tiles_h;
        h0 = (int)th * G::TH;
        w0 = (int)tw * kDwTW;
    };

    // One chunk = one k-step: depthwise of the lane's 8 channels for each of its R rows,
    // split, then three bf16 MFMAs per (output block, row).
    // LDS reads as one base register plus immediate offsets (the offsets are opaque to the
    // optimiser; the weights lie beyond the 16-bit immediate range from the start of LDS)
    const int xoff = (int)(xl - dyn);
    auto chunk = [&](int st, floatx4 (&acc)[MB][R]) {
        int doff = (int)(dl - dyn) + 32 * st * 12;
        int pho = (int)(reinterpret_cast<const float *>(pwh + (st * 64 + lane) * MB) - dyn);
        int plo = (int)(reinterpret_cast<const float *>(pwl + (st * 64 + lane) * MB) - dyn);
        asm volatile("" : "+v"(doff), "+v"(pho), "+v"(plo));
        float dw[R][8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            int xo = xoff + 4 * i * G::CS;
            asm volatile("" : "+v"(xo));
            const float *dk = dyn + doff + 48 * i;
            const floatx4 k0 = *reinterpret_cast<const floatx4 *>(dk);
            const floatx4 k1 = *reinterpret_cast<const floatx4 *>(dk + 4);
            const floatx4 k2 = *reinterpret_cast<const floatx4 *>(dk + 8);
            const float kw9[9] = {k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3], k2[0]};
            float xv[R + 2][3];
#pragma unroll
            for (int hr = 0; hr < R + 2; ++hr)
#pragma unroll
                for (int kw = 0; kw < 3; ++kw) xv[hr][kw] = dyn[xo + hr * G::RS + kw];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float v = k2[1];
#pragma unroll
                for (int kh = 0; kh < 3; ++kh)
#pragma unroll
                    for (int kw = 0; kw < 3; ++kw) v = fmaf(kw9[kh * 3 + kw], xv[r + kh][kw], v);
                dw[r][i] = v;
            }
        }
        const bf16x8 *ph = reinterpret_cast<const bf16x8 *>(dyn + pho);
        const bf16x8 *pl = reinterpret_cast<const bf16x8 *>(dyn + plo);
        bf16x8 dhs[R], dls[R];
#pragma unroll
        for (int r = 0; r < R; ++r) split_bf16(dw[r], dhs[r], dls[r]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const bf16x8 wh_ = ph[mb], wl_ = pl[mb];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const bf16x8 dh = dhs[r], dlo = dls[r];
                acc[mb][r] = mfma_16x16x32_bf16(wh_, dlo, acc[mb][r]);
                acc[mb][r] = mfma_16x16x32_bf16(wl_, dh, acc[mb][r]);
                acc[mb][r] = mfma_16x16x32_bf16(wh_, dh, acc[mb][r]);
            }
        }
    };

    int64_t tile = blockIdx.x, n;
    int h0, w0;
    decode(tile, n, h0, w0);
    DwHalo<R, WH, CC> k;
    hs.load(k, x, d, n, h0, w0, 0);
    lds_barrier();  // weights written; no wave reads the halo buffer yet
    hs.store(xs, k);
    lds_barrier();
    floatx4 acc[MB][R];
    for (;;) {
        acc_init<MB, R>(acc, bs);
        const int64_t ntile = tile + gridDim.x;
        int64_t nn = 0;
        int nh0 = 0, nw0 = 0;
        for (int c0 = 0;; c0 += CC) {
            const bool last = c0 + CC >= C;
            int64_t ln = n;
            int lh = h0, lw = w0, lc = c0 + CC;
            if (last) {
                if (ntile < tiles) decode(ntile, nn, nh0, nw0);
                ln = nn;
                lh = nh0;
                lw = nw0;
                lc = 0;
            }
            if (!last || ntile < tiles) hs.load(k, x, d, ln, lh, lw, lc);
            chunk(c0 / CC, acc);
            if (last) break;
            lds_barrier();
            hs.store(xs, k);
            lds_barrier();
        }
        float *tb = y + ((n * d.O + obase) * d.Ho + h0) * d.Wo;
        dw_epilogue_buf<MB, R>(tb, d, R * wh, (int)(d.Ho - h0) - R * wh, w0 + 16 * ww,
                                        ocnt, acc);
        if (ntile >= tiles) break;
        tile = ntile;
        n = nn;
        h0 = nh0;
        w0 = nw0;
        lds_barrier();
        hs.store(xs, k);
        lds_barrier();
    }
}

// ----------------------------------------------------------------- chunked kernel
// One tile per workgroup (4 waves, R rows x 64 columns); pointwise weights (fragment order)
// and depthwise taps of each chunk are staged with the chunk.
template <int MB>
struct DwWeightChunk {
    static constexpr int QUADS = 16 * MB * kDwCC / 4;
    static constexpr int PQ = (QUADS + 255) / 256;
    floatx4 pw[PQ];
    float dw;
};

template <int MB, int R, bool VEC, bool DW>
__global__ __launch_bounds__(256, 2) void dwsep_chunked_kernel(
    const float *__restrict__ x, const float *__restrict__ dw_w, const float *__restrict__ dw_b,
    const float *__restrict__ pw_w, const float *__restrict__ pw_b, float *__restrict__ y,
    DwsepDims d, int obase, int64_t tiles, int tiles_w, int tiles_h)
{
    using G = DwGeom<R, 1, kDwCC>;
    using WC = DwWeightChunk<MB>;
    constexpr int PS = kDwCC * 16 * MB, DS = kDwCC * 12;
    __shared__ __attribute__((aligned(16))) float lds[G::XS + PS + DS + 16 * MB];
    float *xs = lds;
    float *ps = lds + G::XS;
    float *ds = lds + G::XS + PS;
    float *bs = ds + DS;
    const int C = (int)d.C;
    const int ocnt = (int)(d.O - obase < 16 * MB ? d.O - obase : 16 * MB);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    int64_t t = xcd_tile(blockIdx.x, tiles);
    const int tw = (int)(t % tiles_w);
    t /= tiles_w;
    const int th = (int)(t % tiles_h);
    const int64_t n = t / tiles_h;
    const int h0 = th * R, w0 = tw * kDwTW;

    DwHaloStager<R, 1, kDwCC, VEC, false> hs;
    hs.init(tid, d.pad);
    auto wload = [&](WC &wc, int c0) {
#pragma unroll
        for (int p = 0; p < WC::PQ; ++p) {
            const int qd = tid + 256 * p;
            const int ol = qd >> 2, c = c0 + 4 * (qd & 3);
            floatx4 r = {0.f, 0.f, 0.f, 0.f};
            if (qd < WC::QUADS && ol < ocnt) {
                const float *src = pw_w + (int64_t)(obase + ol) * C + c;
                if constexpr (VEC) {
                    if (c < C) r = *reinterpret_cast<const floatx4 *>(src);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (c + i < C) r[i] = src[i];
                }
            }
            wc.pw[p] = r;
        }
        const int dc = c0 + tid / 12, dk = tid % 12;
        float v = 0.0f;
        if (DW && tid < DS && dc < C) {
            if (dk < 9) v = dw_w[(int64_t)dc * 9 + dk];
            else if (dk == 9 && dw_b) v = dw_b[dc];
        }
        wc.dw = v;
    };
    auto wstore = [&](const WC &wc) {
#pragma unroll
        for (int p = 0; p < WC::PQ; ++p) {
            const int qd = tid + 256 * p;
            if (qd >= WC::QUADS) continue;
            const int ol = qd >> 2, cg = qd & 3;
#pragma unroll
            for (int i = 0; i < 4; ++i) ps[(cg * 64 + i * 16 + (ol & 15)) * MB + (ol >> 4)] = wc.pw[p][i];
        }
        if (tid < DS) ds[tid] = wc.dw;
    };

    const float *xl = xs + (lane >> 4) * G::CS + 16 * wave + (lane & 15) + 4 - d.pad;
    const float *pl = ps + lane * MB;
    const float *dl = ds + (lane >> 4) * 12;
    const bool active = w0 + 16 * wave < d.Wo;

    DwHalo<R, 1, kDwCC> k;
    WC wc;
    hs.load(k, x, d, n, h0, w0, 0);
    wload(wc, 0);
    if (tid < 16 * MB) bs[tid] = (pw_b && tid < ocnt) ? pw_b[obase + tid] : 0.0f;
    if (active) {
        floatx4 acc[MB][R];
        for (int c0 = 0; c0 < C; c0 += kDwCC) {
            lds_barrier();
            hs.store(xs, k);
            wstore(wc);
            lds_barrier();
            if (c0 == 0) acc_init<MB, R>(acc, bs);
            if (c0 + kDwCC < C) {
                hs.load(k, x, d, n, h0, w0, c0 + kDwCC);
                wload(wc, c0 + kDwCC);
            }
            dw_chunk<MB, R, G::RS, G::CS, kDwCC, DW>(lds, (int)(xl - lds), (int)(pl - lds),
                                                              (int)(dl - lds), acc);
        }
        dw_epilogue<MB, R>(y, d, n, h0, w0 + 16 * wave, obase, ocnt, acc);
    } else {
        // This wave's columns lie past the output: it only helps stage the shared tiles.
        for (int c0 = 0; c0 < C; c0 += kDwCC) {
            lds_barrier();
            hs.store(xs, k);
            wstore(wc);
            lds_barrier();
            if (c0 + kDwCC < C) {
                hs.load(k, x, d, n, h0, w0, c0 + kDwCC);
                wload(wc, c0 + kDwCC);
            }
        }
    }
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int cu_count()
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    return cus;
}

constexpr size_t kLdsBytes = 160 * 1024;

template <int MB, int R, int WH, int CC, bool VEC, bool DW>
hipError_t launch_persistent(const float *x, const float *dw_w, const float *dw_b,
                             const float *pw_w, const float *pw_b, float *y, const DwsepDims &d,
                             int obase, size_t lds, int per_cu, hipStream_t s)
{
    using G = DwGeom<R, WH, CC>;
    auto kern = dwsep_persistent_kernel<MB, R, WH, CC, VEC, DW>;
    hipError_t e = hipFuncSetAttribute((const void *)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const int64_t tw = cdiv(d.Wo, kDwTW), th = cdiv(d.Ho, G::TH);
    const int64_t tiles = tw * th * d.N;
    if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    // resident workgroups, a multiple of the XCD count so each stays on one XCD's tiles
    int64_t grid = (int64_t)per_cu * cu_count() / kNumXcd * kNumXcd;
    if (grid < 1) grid = 1;
    if (grid > tiles) grid = tiles;
    note_kernel("dwsep_persistent_kernel");
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(G::NT), lds, s, x, dw_w, dw_b, pw_w, pw_b,
                       y, d, obase, tiles, (int)tw, (int)th);
    return hipGetLastError();
}

template <int MB, int R, bool VEC, bool DW>
hipError_t launch_chunked(const float *x, const float *dw_w, const float *dw_b, const float *pw_w,
                          const float *pw_b, float *y, const DwsepDims &d, int obase,
                          hipStream_t s)
{
    const int64_t tw = cdiv(d.Wo, kDwTW), th = cdiv(d.Ho, R);
    const int64_t tiles = tw * th * d.N;
    if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    note_kernel("dwsep_chunked_kernel");
    hipLaunchKernelGGL((dwsep_chunked_kernel<MB, R, VEC, DW>), dim3((unsigned)tiles),
                       dim3(256), 0, s, x, dw_w, dw_b, pw_w, pw_b, y, d, obase, tiles, (int)tw,
                       (int)th);
    return hipGetLastError();
}

// Pick the kernel for output channels [obase, obase + min(16*MB, O - obase)): the persistent
// kernel with one 8-wave workgroup per CU and 32-channel chunks when its weights and halo fit
// in LDS, else with 16-channel chunks (two 4-wave workgroups per CU, or one 8-wave one), else
// the chunked kernel.
template <int MB, int R, bool VEC, bool DW>
hipError_t launch_slice(const float *x, const float *dw_w, const float *dw_b, const float *pw_w,
                        const float *pw_b, float *y, const DwsepDims &d, int obase, hipStream_t s)
{
    const size_t lds_a = 4 * (dw_weight_floats<MB, 32>(d.C) + (size_t)DwGeom<R, 2, 32>::XS);
    const size_t lds_b = 4 * (dw_weight_floats<MB, 16>(d.C) + (size_t)DwGeom<R, 1, 16>::XS);
    const size_t lds_c = 4 * (dw_weight_floats<MB, 16>(d.C) + (size_t)DwGeom<R, 2, 16>::XS);
    // the persistent kernel addresses one tile's outputs and one input image with 32-bit
    // byte offsets
    const bool small_planes =
        64 * MB * d.Ho * d.Wo <= kBufRange && 4 * d.C * d.H * d.W <= kBufRange;
    if (small_planes && lds_a <= kLdsBytes)
        return launch_persistent<MB, R, 2, 32, VEC, DW>(x, dw_w, dw_b, pw_w, pw_b, y, d,
                                                             obase, lds_a, 1, s);
    if (small_planes && 2 * lds_b <= kLdsBytes)
        return launch_persistent<MB, R, 1, 16, VEC, DW>(x, dw_w, dw_b, pw_w, pw_b, y, d,
                                                             obase, lds_b, 2, s);
    if (small_planes && lds_c <= kLdsBytes)
        return launch_persistent<MB, R, 2, 16, VEC, DW>(x, dw_w, dw_b, pw_w, pw_b, y, d,
                                                             obase, lds_c, 1, s);
    return launch_chunked<MB, 2, VEC, DW>(x, dw_w, dw_b, pw_w, pw_b, y, d, obase, s);
}

template <int MB, int R, bool DW>
hipError_t launch(const float *x, const float *dw_w, const float *dw_b, const float *pw_w,
                  const float *pw_b, float *y, const DwsepDims &d, int obase, hipStream_t s)
{
    // float4 loads need 16-byte aligned input and pointwise rows.
    const bool vin = d.W % 4 == 0 && d.C % 4 == 0 && ((uintptr_t)x & 15) == 0 &&
                     ((uintptr_t)pw_w & 15) == 0;
    if (vin) return launch_slice<MB, R, true, DW>(x, dw_w, dw_b, pw_w, pw_b, y, d, obase, s);
    return launch_slice<MB, R, false, DW>(x, dw_w, dw_b, pw_w, pw_b, y, d, obase, s);
}

}  // namespace

namespace {

template <bool DW>
hipError_t launch_all(const float *x, const float *dw_w, const float *dw_b, const float *pw_w,
                      const float *pw_b, float *y, const DwsepDims &d, hipStream_t s)
{
    // One launch covers up to 192 output channels; wider layers run as several launches over
    // consecutive output-channel slices (each rereads the input).  Up to 128 channels a wave
    // owns 3 output rows (measured faster than 2 or 4 on the 512 x 512 layer: less halo per
    // output row; 4 rows spill registers with 32-channel chunks).
    if (d.O <= 64) return launch<4, 4, DW>(x, dw_w, dw_b, pw_w, pw_b, y, d, 0, s);
    if (d.O <= 128) return launch<8, 3, DW>(x, dw_w, dw_b, pw_w, pw_b, y, d, 0, s);
    for (int64_t o0 = 0; o0 < d.O; o0 += 192) {
        const hipError_t e = launch<12, 2, DW>(x, dw_w, dw_b, pw_w, pw_b, y, d, (int)o0, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_dwsep_conv2d(const float *x, const float *dw_w, const float *dw_b,
                               const float *pw_w, const float *pw_b, float *y,
                               const DwsepDims &d, hipStream_t s)
{
    return launch_all<true>(x, dw_w, dw_b, pw_w, pw_b, y, d, s);
}

namespace {

template <int MB, int R, bool VEC>
hipError_t launch_split_kernel(const float *x, const float *dw_w, const float *dw_b,
                               const float *pw_w, const float *pw_b, float *y, const DwsepDims &d,
                               int obase, size_t lds, hipStream_t s)
{
    using G = DwGeom<R, 2, 32>;
    auto kern = dwsep_split_kernel<MB, R, 2, VEC>;
    hipError_t e = hipFuncSetAttribute((const void *)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const int64_t tw = cdiv(d.Wo, kDwTW), th = cdiv(d.Ho, G::TH);
    const int64_t tiles = tw * th * d.N;
    if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    int64_t grid = (int64_t)cu_count() / kNumXcd * kNumXcd;
    if (grid < 1) grid = 1;
    if (grid > tiles) grid = tiles;
    note_kernel("dwsep_split_kernel");
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(G::NT), lds, s, x, dw_w, dw_b, pw_w, pw_b,
                       y, d, obase, tiles, (int)tw, (int)th);
    return hipGetLastError();
}

// Split-bf16 launch for output channels [obase, obase + 16*MB); false when it does not apply
// (weights + halo above the LDS size, or byte offsets beyond 32 bits).
template <int MB, int R>
bool launch_split_slice(const float *x, const float *dw_w, const float *dw_b, const float *pw_w,
                        const float *pw_b, float *y, const DwsepDims &d, int obase,
                        hipStream_t s, hipError_t &err)
{
    const size_t lds = split_weight_bytes<MB>(d.C) + 4 * (size_t)DwGeom<R, 2, 32>::XS;
    const bool small_planes =
        64 * MB * d.Ho * d.Wo <= kBufRange && 4 * d.C * d.H * d.W <= kBufRange;
    if (!small_planes || lds > kLdsBytes) return false;
    // Every width takes the staging for rows that are only 4-byte aligned (one 16-byte load
    // per quad inside a row, single loads where the row ends).  On 16-byte-aligned rows it
    // issues the same loads as the aligned variant, and its compiled schedule measured 6-7 %
    // faster on a [16,64,512,512] -> 128 layer; the fp32 kernel is the other way round.
    err = launch_split_kernel<MB, R, false>(x, dw_w, dw_b, pw_w, pw_b, y, d, obase, lds, s);
    return true;
}

}  // namespace

hipError_t launch_dwsep_conv2d_split_bf16(const float *x, const float *dw_w, const float *dw_b,
                                          const float *pw_w, const float *pw_b, float *y,
                                          const DwsepDims &d, hipStream_t s)
{
    hipError_t err = hipSuccess;
    bool done;
    if (d.O <= 64) {
        done = launch_split_slice<4, 2>(x, dw_w, dw_b, pw_w, pw_b, y, d, 0, s, err);
    } else if (d.O <= 128) {
        done = launch_split_slice<8, 2>(x, dw_w, dw_b, pw_w, pw_b, y, d, 0, s, err);
    } else {
        done = true;
        for (int64_t o0 = 0; o0 < d.O && done && err == hipSuccess; o0 += 192)
            done = launch_split_slice<12, 2>(x, dw_w, dw_b, pw_w, pw_b, y, d, (int)o0, s, err);
    }
    // Layers the split kernel does not cover run in fp32 (more accurate than asked for).
    if (!done) return launch_all<true>(x, dw_w, dw_b, pw_w, pw_b, y, d, s);
    return err;
}

hipError_t launch_pointwise_conv2d(const float *x, const float *pw_w, const float *pw_b, float *y,
                                   const DwsepDims &d, hipStream_t s)
{
    DwsepDims p = d;
    p.pad = 1;  // centre tap of the 3x3, pad 1 staging geometry: y has the input's H x W
    p.Ho = d.H;
    p.Wo = d.W;
    return launch_all<false>(x, nullptr, nullptr, pw_w, pw_b, y, p, s);
}

}  // namespace convfuse
