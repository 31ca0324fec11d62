// dwconv_wgrad.hip -- weight and bias gradients: the stage-1 kernels
// (tiled NHWC, tiled NCHW, generic) that write per-chunk partial sums, the
// fixed-order stage-2 reduction (optionally with the SGD step) and their
// launcher.
#include "dwconv_device.h"

#include <mutex>

namespace dwconv {

namespace {

// ---------------------------------------------------------------------------
// Weight and bias gradients (LeanMlir "Depthwise": weight-VJP, bias-gradient
// closed form).  Two stages, deterministic (fixed summation order, no
// atomics):
//   stage 1 writes partial sums part[chunk][c][tap], tap = kh*kW + kw for
//           dW and tap = kH*kW for db, each over one chunk of dy positions;
//   stage 2 adds the chunks of every (c, tap) column in a fixed order.
// ---------------------------------------------------------------------------
struct WgradArgs {
    int N, C, mult;         // C: channels of dy (and of dW); x has C / mult
    int H, W, kH, kW, d, pH, pW;
    int OH, OW;             // dy extents
    int nct, nwt, nsp;      // tiled: channel tiles, column tiles, strips
    int strip;              // tiled: row tiles per strip
    int chunks;             // rows of part[]
    int xcd;                // tiled: tile order, 1 = per-XCD ranges (xcd_tile), 2 = band-local
                            // runs (band_tile, NHWC), 0 = in order
};

// Stage 1, any layout, stride, padding and multiplier.  Lanes run along the
// contiguous axis so every load of a wave is one coalesced run: in NHWC
// `cl` consecutive output channels x 256/cl position slots, in NCHW 256
// consecutive positions of one output channel's plane.  A workgroup sums
// one chunk of `ppc` dy positions; the kH*kW taps and the bias column go in
// groups of 8 register accumulators (dy is re-read, from cache, once per
// group), and the slots of a channel are added in LDS in a fixed order.
// Output channel c reads x channel c / mult.
struct WgradGenArgs {
    int N, C, mult;         // C: channels of dy (and of dW); x has C / mult
    int H, W, OH, OW;       // x extents, dy extents
    int kH, kW, d, pH, pW;
    int cl, ncg;            // NHWC: channel lanes (16, 32 or 64), channel groups
    int ppc;                // dy positions per chunk
    int cpi;                // NCHW: chunks per image
};

constexpr int kWgradTapGroup = 8;

template <bool NHWC, int S>
__global__ __launch_bounds__(256) void k_wgrad_gen(const float *__restrict__ x,
                                                   const float *__restrict__ dy,
                                                   float *__restrict__ part, WgradGenArgs a)
{
    __shared__ float red[kWgradTapGroup][256];
    const int tid = threadIdx.x;
    const int KK = a.kH * a.kW;
    const int CI = a.C / a.mult;
    const int per_img = a.OH * a.OW;
    int chunk, c, slot, nslot, p0, p1, n_fixed = 0;
    if (NHWC) {
        const int cg = blockIdx.x % a.ncg;
        chunk = blockIdx.x / a.ncg;
        c = cg * a.cl + tid % a.cl;
        slot = tid / a.cl;
        nslot = 256 / a.cl;
        p0 = chunk * a.ppc;                               // over (n, ho, wo) of all images
        p1 = min(p0 + a.ppc, a.N * per_img);
    } else {
        c = blockIdx.x % a.C;
        chunk = blockIdx.x / a.C;                         // (n, range within the plane)
        n_fixed = chunk / a.cpi;
        slot = tid;
        nslot = 256;
        p0 = (chunk - n_fixed * a.cpi) * a.ppc;           // within image n_fixed
        p1 = min(p0 + a.ppc, per_img);
    }
    const bool cvalid = c < a.C;
    const int ci = c / a.mult;
    for (int tg = 0; tg <= KK; tg += kWgradTapGroup) {
        float acc[kWgradTapGroup];
        int th[kWgradTapGroup], tw[kWgradTapGroup];       // tap offsets; th = -1: bias column
#pragma unroll
        for (int t = 0; t < kWgradTapGroup; ++t) {
            acc[t] = 0.0f;
            const int tap = tg + t;
            th[t] = tap < KK ? (tap / a.kW) * a.d - a.pH : -(1 << 30);
            tw[t] = tap < KK ? (tap % a.kW) * a.d - a.pW : 0;
        }
        if (cvalid) {
            for (int pp = p0 + slot; pp < p1; pp += nslot) {
                int n, rem;
                if (NHWC) {
                    n = pp / per_img;
                    rem = pp - n * per_img;
                } else {
                    n = n_fixed;
                    rem = pp;
                }
                const int ho = rem / a.OW, wo = rem - (rem / a.OW) * a.OW;
                const float g = NHWC ? dy[((n * a.OH + ho) * a.OW + wo) * a.C + c]
                                     : dy[((n * a.C + c) * a.OH + ho) * a.OW + wo];
#pragma unroll
                for (int t = 0; t < kWgradTapGroup; ++t) {
                    const int hi = ho * S + th[t], wi = wo * S + tw[t];
                    if (hi >= 0 && hi < a.H && wi >= 0 && wi < a.W) {
                        const float xv = NHWC ? x[((n * a.H + hi) * a.W + wi) * CI + ci]
                                              : x[((n * CI + ci) * a.H + hi) * a.W + wi];
                        acc[t] = fmaf(xv, g, acc[t]);
                    } else if (tg + t == KK) {
                        acc[t] += g;                      // the bias column
                    }
                }
            }
        }
        // add the slots of each channel in a fixed order
        __syncthreads();
#pragma unroll
        for (int t = 0; t < kWgradTapGroup; ++t)
            red[t][tid] = acc[t];
        __syncthreads();
        if (NHWC) {
            // thread e sums column (tap e / cl, lane e % cl) over the slots
            for (int e = tid; e < kWgradTapGroup * a.cl; e += 256) {
                const int t = e / a.cl, lane = e - t * a.cl;
                const int cc = (blockIdx.x % a.ncg) * a.cl + lane;
                if (tg + t <= KK && cc < a.C) {
                    float sum = 0.0f;
                    for (int sl = 0; sl < nslot; ++sl)
                        sum += red[t][sl * a.cl + lane];
                    part[((long long)chunk * a.C + cc) * (KK + 1) + tg + t] = sum;
                }
            }
        } else {
            // fixed tree over the 256 positions, all 8 taps at once
#pragma unroll
            for (int off = 128; off > 0; off >>= 1) {
                if (tid < off)
#pragma unroll
                    for (int t = 0; t < kWgradTapGroup; ++t)
                        red[t][tid] += red[t][tid + off];
                __syncthreads();
            }
            if (tid < kWgradTapGroup && tg + tid <= KK)
                part[((long long)chunk * a.C + c) * (KK + 1) + tg + tid] = red[tid][0];
        }
    }
}

// Stage 1, NHWC, stride S = 1 or 2: a workgroup (256 threads: CL across
// channels x 256/CL pixel slots of PX dy columns) walks `strip` row tiles of
// one column tile.  Per row tile it stages G input rows (+ column halo) in LDS and
// loads its dy rows straight into registers (each dy element is used by one
// thread only); every thread accumulates x*dy for all kH*kW taps of its
// channels, and at the end the pixel slots are summed through LDS.
// LV: floats per staging load, 4 (C % 4 == 0, 16-byte aligned tensors) or 1
// (any C, one channel per thread).  At stride 2 a tile of TH x TW dy
// positions reads 2*TH - 1 + (KH-1)*D rows and 2*TW - 1 + (KW-1)*D columns
// of x, and dy position (m, j) meets x at (2m + kh*D, 2j + kw*D).  With a
// channel multiplier M the walk runs over dy channels; the x tile is loaded
// with the input channels only and each value is written to LDS M times, once
// per dy channel that reads it.
template <int KH, int KW, int D, int VEC, int CL, int PX, int G, int LV, int S, int M = 1>
__global__ __launch_bounds__(256) void k_wgrad_tiled_nhwc(const float *__restrict__ x,
                                                          const float *__restrict__ dy,
                                                          float *__restrict__ part, WgradArgs a)
{
    static_assert(LV == 4 || (LV == 1 && VEC == 1), "scalar staging: one channel per thread");
    static_assert(S == 1 || S == 2, "stride 1 or 2");
    static_assert(M == 1 || (M == 2 && LV == 4 && S == 1), "multiplier 2: 16-byte staging");
    constexpr int R = (KH - 1) * D + 1, TW = PX * 256 / CL, CG = CL * VEC;
    constexpr int TH = (G - R) / S + 1;     // dy rows per row tile
    static_assert(G >= R && (G - R) % S == 0, "staged rows = S*(TH-1) + R");
    constexpr int TWI = S * (TW - 1) + 1 + (KW - 1) * D, VPC = CG / (M * LV), VPR = TWI * VPC;
    constexpr int VCH = G * VPR, NV = (VCH + 255) / 256, KK = KH * KW, NP = 256 / CL;
    constexpr int XW = S * (PX - 1) + 1 + (KW - 1) * D;
    constexpr int XF = G * TWI * CG;        // staged floats (dy channels)
    // the final per-(channel, tap) sums go through LDS in groups of TG taps
    constexpr int TGF = XF / (256 * VEC);
    constexpr int TG = TGF < 1 ? 1 : (TGF > KK + 1 ? KK + 1 : TGF);
    // For 7x7 windows at stride 1 the staged loads (4 or 16 bytes) go from
    // the buffer straight into LDS, a wave's 64 consecutive loads per
    // instruction (the tile's region rounded up to 64 loads).  That needs the
    // barrier before the loads instead of after them: measured on MI355X it is
    // 4-6% faster (16-byte) and 18-35% faster (4-byte) for 7x7 windows, whose
    // tiles cost the most registers when copied through them, and up to 17%
    // slower for 3x3 and 5x5 ones, which lose more by that barrier.
    constexpr bool DMA = S == 1 && M == 1 && KK >= 49;
    constexpr int XFS = DMA ? (VCH + 63) / 64 * 64 * LV : XF;
    constexpr int LDSF = (XFS > 256 * VEC * TG) ? XFS : 256 * VEC * TG;
    __shared__ float4 lds4[(LDSF + 3) / 4];
    float *lds = reinterpret_cast<float *>(lds4);

    // tiles: channel tile, column tile, strip, image (fastest first)
    int tile = a.xcd == 1   ? xcd_tile(blockIdx.x, gridDim.x)
               : a.xcd == 2 ? band_tile(blockIdx.x, a.nct * a.nwt)
                            : blockIdx.x;
    const int ct = tile % a.nct;
    tile /= a.nct;
    const int chunk = tile;                 // (n, strip, column tile): row of part[]
    const int wt = tile % a.nwt;
    tile /= a.nwt;
    const int sp = tile % a.nsp;
    const int n = tile / a.nsp;
    const int c0 = ct * CG, w0 = wt * TW;
    const int tid = threadIdx.x;
    const int q = tid % CL, p = tid / CL;
    const int cq = c0 + q * VEC;
    const int ow = w0 + p * PX;
    const int cbase = S * w0 - a.pW;
    const int CX = a.C / M;                 // channels of x
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + n * a.H * a.W * CX, a.H * a.W * CX * 4);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(dy + n * a.OH * a.OW * a.C, a.OH * a.OW * a.C * 4);

    float acc[KK + 1][VEC];                 // taps kh*KW + kw, then the bias
#pragma unroll
    for (int t = 0; t <= KK; ++t)
#pragma unroll
        for (int v = 0; v < VEC; ++v)
            acc[t][v] = 0.0f;

    // Staged load e = tid + 256*i is vector cv of staged pixel (g, col):
    // e = (g * TWI + col) * VPC + cv.  VPC is a power of two that divides
    // 256, so cv (hence the x channel) is the same for all of a thread's
    // loads, and (g, col) and the byte offset advance by a fixed step from
    // one load to the next.  A load with g < nrows (<= G) is one of the VCH
    // staged loads.
    static_assert((VPC & (VPC - 1)) == 0 && 256 % VPC == 0, "staging vectors per pixel");
    constexpr int DG = 256 / VPR, DC = (256 % VPR) / VPC;
    const int ch = c0 / M + (tid % VPC) * LV;             // x channel
    const bool chok = ch < CX;
    const int g0 = tid / VPR, col0 = (tid % VPR) / VPC;
    const unsigned pstep = 4u * CX, rstep = pstep * a.W;
    const int wel = __builtin_amdgcn_readfirstlane(tid) & ~63;   // the wave's first element

    const int t0 = sp * a.strip, t1 = min(t0 + a.strip, (a.OH + TH - 1) / TH);
    for (int tt = t0; tt < t1; ++tt) {
        const int h0 = tt * TH;
        const int nrows = S * (min(TH, a.OH - h0) - 1) + R;
        const int rbase = S * h0 - a.pH;
        // this row tile's x rows (+ halo) and, per thread, its dy values
        // (unsigned offsets: positions outside the image may wrap, they are not loaded)
        typedef typename VecT<LV>::type LoadT;
        LoadT stage[DMA ? 1 : NV];
        int g = g0, col = col0;
        if constexpr (DMA) {
            if (tt > t0)
                __syncthreads();          // every thread done with the previous tile
            // recompute the load positions per tile (a few adds each) rather
            // than let the compiler keep all NV of them in registers
            asm volatile("" : "+v"(g), "+v"(col));
        }
        unsigned uoff = (unsigned)(rbase + g) * rstep + (unsigned)(cbase + col) * pstep + 4u * ch;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            if (i > 0) {
                g += DG;
                col += DC;
                uoff += DG * rstep + DC * pstep;
                if (col >= TWI) {
                    col -= TWI;
                    ++g;
                    uoff += rstep - TWI * pstep;
                }
            }
            const int row = rbase + g, gc = cbase + col;
            const bool ok = chok && g < nrows && (unsigned)row < (unsigned)a.H &&
                            (unsigned)gc < (unsigned)a.W;
            const int off = ok ? (int)uoff : kOutOfRange;
            if constexpr (DMA) {
                if ((i + 1) * 256 <= VCH || i * 256 + wel < VCH)   // the wave's run holds staged loads
                    buf_to_lds<4 * LV>(rx, lds + (i * 256 + wel) * LV, off);
            } else if constexpr (LV == 4) {
                stage[i] = buf_f4(rx, off);
            } else {
                stage[i] = buf_f32(rx, off);
            }
        }
        float gv[TH][PX][VEC];
#pragma unroll
        for (int m = 0; m < TH; ++m)
#pragma unroll
            for (int j = 0; j < PX; ++j) {
                const bool ok = h0 + m < a.OH && ow + j < a.OW && cq < a.C;
                buf_vec<VEC>(rg, ok ? (((h0 + m) * a.OW + ow + j) * a.C + cq) * 4 : kOutOfRange,
                             gv[m][j]);
            }
        if (!DMA && tt > t0)
            __syncthreads();              // every thread done with the previous tile
        if constexpr (DMA)
            vm_drain();                   // the barrier does not wait for the LDS loads
#pragma unroll
        for (int i = 0; i < (DMA ? 0 : NV); ++i) {
            const int e = tid + i * 256;
            if ((i + 1) * 256 <= VCH || e < VCH) {
                if constexpr (M == 2) {
                    // x channels ch .. ch+3 feed dy channel slots 2*ch .. 2*ch + 7
                    const float4 v = stage[i];
                    lds4[2 * e] = make_float4(v.x, v.x, v.y, v.y);
                    lds4[2 * e + 1] = make_float4(v.z, v.z, v.w, v.w);
                } else {
                    reinterpret_cast<LoadT *>(lds4)[e] = stage[i];
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < TH; ++m) {
#pragma unroll
            for (int j = 0; j < PX; ++j)
#pragma unroll
                for (int v = 0; v < VEC; ++v)
                    acc[KK][v] += gv[m][j][v];
#pragma unroll
            for (int kh = 0; kh < KH; ++kh) {
                const int u = S * m + kh * D;   // staged row of tap row kh for dy row m
                float xv[XW][VEC];
#pragma unroll
                for (int i = 0; i < XW; ++i) {
                    const float *src = lds + ((u * TWI + S * p * PX + i) * CG + q * VEC);
#pragma unroll
                    for (int v = 0; v < VEC; ++v)
                        xv[i][v] = src[v];
                }
#pragma unroll
                for (int kw = 0; kw < KW; ++kw)
#pragma unroll
                    for (int j = 0; j < PX; ++j)
#pragma unroll
                        for (int v = 0; v < VEC; ++v)
                            acc[kh * KW + kw][v] =
                                fmaf(xv[S * j + kw * D][v], gv[m][j][v], acc[kh * KW + kw][v]);
            }
        }
    }

    // sum the NP pixel slots of every (channel, tap) in a fixed order, TG taps at a time
#pragma unroll
    for (int tb = 0; tb <= KK; tb += TG) {
        __syncthreads();
#pragma unroll
        for (int k = 0; k < TG; ++k)
            if (tb + k <= KK)
#pragma unroll
                for (int v = 0; v < VEC; ++v)
                    lds[(k * 256 + tid) * VEC + v] = acc[tb + k][v];
        __syncthreads();
        for (int e = tid; e < CG * TG; e += 256) {
            const int k = e / CG, cl = e - k * CG;
            const int qq = cl / VEC, v = cl - qq * VEC;
            if (tb + k <= KK) {
                float s = 0.0f;
                for (int pp = 0; pp < NP; ++pp)
                    s += lds[(k * 256 + pp * CL + qq) * VEC + v];
                if (c0 + cl < a.C)
                    part[((long long)chunk * a.C + c0 + cl) * (KK + 1) + tb + k] = s;
            }
        }
    }
}

// Stage 1, NCHW, stride 1 or 2: the NCHW forward's tiling with the roles of
// the operands changed.  A workgroup covers pb dy planes x tx threads per
// plane row (Q adjacent columns each) and walks `strip` row tiles of one
// column tile; per row tile it stages the G x rows (+ column halo) of its
// planes' input planes in LDS and loads its dy values into registers, and
// every thread accumulates x*dy for all kH*kW taps (and dy for the bias) of
// its plane.  At the end every thread parks its sums in LDS and each
// (plane, tap) column is added over the plane's tx threads in thread order.
struct WgradNchwArgs {
    int planes, C, mult;        // dy planes (N * C), dy channels, channel multiplier
    int H, W, OH, OW;           // x extents, dy extents
    int pH, pW, hl, twl;        // pads; staged columns left of a tile, staged floats per row
    int txn, pbn;               // threads per plane row (16..256), planes per workgroup
    int nct, nwt, nsp, strip;   // plane groups, column tiles, strips, row tiles per strip
    int nrt;                    // row tiles per plane
    int xcd;                    // tile order: 1 = per-XCD ranges (xcd_tile), 0 = in order
};

// At stride S = 2 a row tile of TH dy rows reads 2*TH - 1 + (kH-1)*d x rows,
// a thread's Q dy columns meet x columns 2j + kw*d of its window, and the
// staged x row of a tile is 2*tw - 1 + (kW-1)*d columns wide.
template <int KH, int KW, int D, int Q, int G, bool V4, int S>
__global__ __launch_bounds__(256) void k_wgrad_tiled_nchw(const float *__restrict__ x,
                                                          const float *__restrict__ dy,
                                                          float *__restrict__ part,
                                                          WgradNchwArgs a)
{
    typedef NchwGeom<KH, KW, D, Q, G, V4> Gm;
    static_assert(S == 1 || S == 2, "stride 1 or 2");
    constexpr int R = Gm::R, KK = Gm::KK, LV = Gm::LV;
    constexpr int TH = (G - R) / S + 1;                  // dy rows per row tile
    static_assert(G >= R && (G - R) % S == 0, "staged rows = S*(TH-1) + R");
    // per-thread loads for the largest staged tile (x rows of S*Q columns per thread)
    constexpr int NV = nchw_stage_loads(0, G, S * Q, KW, D, V4);
    constexpr int XW = S * (Q - 1) + 1 + (KW - 1) * D;
    extern __shared__ float4 lds4[];
    float *lds = reinterpret_cast<float *>(lds4);

    const int txn = a.txn, pbn = a.pbn;
    const int tw = txn * Q, twl = a.twl, vpr = twl / LV;
    // tiles: strip, column tile, plane group (fastest first)
    int tile = a.xcd ? xcd_tile(blockIdx.x, gridDim.x) : blockIdx.x;
    const int sp = tile % a.nsp;
    tile /= a.nsp;
    const int wt = tile % a.nwt;
    const int pg = tile / a.nwt;
    const int w0 = wt * tw;
    const int tid = threadIdx.x;
    // threads past pbn * txn (when txn does not divide 256) idle along
    const int pli_raw = tid / txn, tx = tid - pli_raw * txn;
    const int pli = min(pli_raw, pbn - 1);             // in-range LDS addresses for idle threads
    const int my_plane = pg * pbn + pli;
    const bool pvalid = pli_raw < pbn && my_plane < a.planes;
    const int oc = w0 + tx * Q;
    const int CI = a.C / a.mult;
    const int cbase = S * w0 - a.hl;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (a.planes / a.C) * CI * a.H * a.W * 4);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(dy, a.planes * a.OH * a.OW * 4);
    const float *rowbase = lds + pli * G * twl + S * tx * Q + (a.hl - a.pW);

    float acc[KK + 1];
#pragma unroll
    for (int t = 0; t <= KK; ++t)
        acc[t] = 0.0f;

    // 16-byte staging (x rows of whole aligned vectors): each thread loads
    // its share of the tile into registers before the barrier that ends the
    // previous tile, so the loads overlap the other waves' last sums, then
    // writes it to LDS.  4-byte staging (any row width) moves 4x as many
    // loads, and there the index arithmetic dominates: those loads go from
    // the buffer straight into LDS, with the indices stepped rather than
    // divided.  Either way staged element e = tid + 256*i of a tile (LV
    // floats) is LDS element e = (pl*G + g)*vpr + cv, for row g of the
    // workgroup's plane pl and vector cv of the row.
    const int nel = pbn * G * vpr;                     // staged elements of a tile
    const int cv0 = tid % vpr, gq0 = tid / vpr;
    const int d_gq = 256 / vpr, d_cv = 256 - d_gq * vpr;
    const int wel = __builtin_amdgcn_readfirstlane(tid) & ~63;   // the wave's first element
    const bool mx = a.mult != 1;

    const int t0 = sp * a.strip, t1 = min(t0 + a.strip, a.nrt);
    for (int tt = t0; tt < t1; ++tt) {
        const int h0 = tt * TH;
        const int nrows = S * (min(TH, a.OH - h0) - 1) + R;
        const int rbase = S * h0 - a.pH;
        float gv[TH][Q];
        if constexpr (V4) {
            float4 sv[NV];
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int e = tid + i * 256;
                const int pl = e / (G * vpr);
                const int rem = e - pl * (G * vpr);
                const int g = rem / vpr;
                const int col = cbase + (rem - g * vpr) * LV;
                const int plane = pg * pbn + pl, row = rbase + g;
                const bool ok = pl < pbn && plane < a.planes && g < nrows && row >= 0 &&
                                row < a.H && col >= 0 && col < a.W;
                // x plane read by dy plane (n, o): (n, o / mult)
                const int xplane = (plane / a.C) * CI + (plane % a.C) / a.mult;
                const int off = ok ? ((xplane * a.H + row) * a.W + col) * 4 : kOutOfRange;
                sv[i] = buf_f4(rx, off);
            }
#pragma unroll
            for (int m = 0; m < TH; ++m)
#pragma unroll
                for (int j = 0; j < Q; ++j) {
                    const bool ok = pvalid && h0 + m < a.OH && oc + j < a.OW;
                    gv[m][j] = buf_f32(rg, ok ? ((my_plane * a.OH + h0 + m) * a.OW + oc + j) * 4
                                              : kOutOfRange);
                }
            if (tt > t0)
                __syncthreads();          // every thread done with the previous tile
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int e = tid + i * 256;
                if (e < nel)
                    lds4[e] = sv[i];
            }
            __syncthreads();
        } else {
            if (tt > t0)
                __syncthreads();          // every thread done with the previous tile
            int s_cv = cv0, s_gq = gq0;
            // recompute the load indices per tile (a few adds each) rather than
            // let the compiler keep all NV of them in registers across the strip
            asm volatile("" : "+v"(s_cv), "+v"(s_gq));
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int pl = s_gq / G, g = s_gq - pl * G;
                const int col = cbase + s_cv;
                s_cv += d_cv;
                s_gq += d_gq;
                if (s_cv >= vpr) {
                    s_cv -= vpr;
                    ++s_gq;
                }
                if (i * 256 + wel < nel) {  // the wave's run of 64 holds staged elements
                    const int plane = pg * pbn + pl, row = rbase + g;
                    const bool ok = pl < pbn && plane < a.planes && g < nrows &&
                                    (unsigned)row < (unsigned)a.H &&
                                    (unsigned)col < (unsigned)a.W;
                    // x plane read by dy plane (n, o): (n, o / mult)
                    const int xplane = mx ? (plane / a.C) * CI + (plane % a.C) / a.mult : plane;
                    const int off = ok ? ((xplane * a.H + row) * a.W + col) * 4 : kOutOfRange;
                    buf_to_lds<4>(rx, lds + i * 256 + wel, off);
                }
            }
#pragma unroll
            for (int m = 0; m < TH; ++m)
#pragma unroll
                for (int j = 0; j < Q; ++j) {
                    const bool ok = pvalid && h0 + m < a.OH && oc + j < a.OW;
                    gv[m][j] = buf_f32(rg, ok ? ((my_plane * a.OH + h0 + m) * a.OW + oc + j) * 4
                                              : kOutOfRange);
                }
            vm_drain();                   // this wave's x rows are in LDS
            __syncthreads();
        }
#pragma unroll
        for (int m = 0; m < TH; ++m) {
#pragma unroll
            for (int j = 0; j < Q; ++j)
                acc[KK] += gv[m][j];
#pragma unroll
            for (int kh = 0; kh < KH; ++kh) {
                float xv[XW];
#pragma unroll
                for (int i = 0; i < XW; ++i)
                    xv[i] = rowbase[(S * m + kh * D) * twl + i];
#pragma unroll
                for (int kw = 0; kw < KW; ++kw)
#pragma unroll
                    for (int j = 0; j < Q; ++j)
                        acc[kh * KW + kw] =
                            fmaf(xv[S * j + kw * D], gv[m][j], acc[kh * KW + kw]);
            }
        }
    }

    // add the tx threads of each plane: every thread parks its KK + 1 sums in
    // LDS, then each (plane, tap) column is added over the plane's threads in
    // thread order (one pass, fixed order)
    constexpr int KP = (KK + 1) | 1;                   // odd row stride: no bank conflicts
    __syncthreads();                                   // every thread done with the tile
#pragma unroll
    for (int t = 0; t <= KK; ++t)
        lds[tid * KP + t] = acc[t];
    __syncthreads();
    const int n_cols = pbn * (KK + 1);
    for (int e = tid; e < n_cols; e += 256) {
        const int pl = e / (KK + 1), t = e - pl * (KK + 1);
        const int plane = pg * pbn + pl;
        if (plane < a.planes) {
            const float *col = lds + pl * txn * KP + t;
            float sum = 0.0f;
            for (int j = 0; j < txn; ++j)
                sum += col[j * KP];
            const int n = plane / a.C, o = plane % a.C;
            const int chunk = (n * a.nwt + wt) * a.nsp + sp;
            part[((long long)chunk * a.C + o) * (KK + 1) + t] = sum;
        }
    }
}

// Stage 2: 256 / S columns of part[] per workgroup and S chunk slices:
// thread t adds column t % (256 / S) over the chunks t / (256 / S) + k*S,
// k = 0, 1, ..., with 8 independent partial sums (8 loads in flight)
// combined in a fixed order, and the S slices are added in LDS in a fixed
// pairwise tree.  The plan takes S = 8 (32-column runs, whole 128-byte
// lines per load) and S = 16 when there are few columns (more workgroups).
// The result depends only on the partial sums, never on timing.
// With w_upd, the LeanMlir page's SGD step is fused in: w_upd -= lr * dW and,
// with b_upd, b_upd -= lr * db (one rounding each: fmaf(-lr, grad, old)).
constexpr int kReduceUnroll = 8;

template <int S>
__global__ __launch_bounds__(256) void k_wgrad_reduce(const float *__restrict__ part,
                                                      float *__restrict__ dw,
                                                      float *__restrict__ db, int chunks,
                                                      int C, int KK, float *__restrict__ w_upd,
                                                      float *__restrict__ b_upd, float lr)
{
    constexpr int CPW = 256 / S;
    __shared__ float red[S][CPW];
    const int cols = C * (KK + 1);
    const int cl = threadIdx.x % CPW, sl = threadIdx.x / CPW;
    const int col = blockIdx.x * CPW + cl;
    const bool valid = col < cols;
    float s[kReduceUnroll];
#pragma unroll
    for (int u = 0; u < kReduceUnroll; ++u)
        s[u] = 0.0f;
    if (valid) {
        int r = sl;
        for (; r + S * (kReduceUnroll - 1) < chunks; r += S * kReduceUnroll) {
            float v[kReduceUnroll];
#pragma unroll
            for (int u = 0; u < kReduceUnroll; ++u)
                v[u] = part[(long long)(r + S * u) * cols + col];
#pragma unroll
            for (int u = 0; u < kReduceUnroll; ++u)
                s[u] += v[u];
        }
#pragma unroll
        for (int u = 0; u < kReduceUnroll - 1; ++u)
            if (r + S * u < chunks)
                s[u] += part[(long long)(r + S * u) * cols + col];
    }
#pragma unroll
    for (int w = kReduceUnroll / 2; w > 0; w >>= 1)
#pragma unroll
        for (int u = 0; u < w; ++u)
            s[u] += s[u + w];
    red[sl][cl] = s[0];
    __syncthreads();
    if (sl == 0 && valid) {
        float v[S];
#pragma unroll
        for (int i = 0; i < S; ++i)
            v[i] = red[i][cl];
#pragma unroll
        for (int w = S / 2; w > 0; w >>= 1)
#pragma unroll
            for (int i = 0; i < w; ++i)
                v[i] += v[i + w];
        const float g = v[0];
        const int c = col / (KK + 1), tap = col - c * (KK + 1);
        if (tap < KK) {
            if (dw)
                dw[c * KK + tap] = g;
            if (w_upd)
                w_upd[c * KK + tap] = fmaf(-lr, g, w_upd[c * KK + tap]);
        } else {
            if (db)
                db[c] = g;
            if (b_upd)
                b_upd[c] = fmaf(-lr, g, b_upd[c]);
        }
    }
}

typedef void (*WgradFn)(const float *, const float *, float *, WgradArgs);

template <int V, int T>
constexpr WgradFn wgrad_fn()
{
    if constexpr (T == 1) {
        constexpr WgradVariant t = kWgradVariants[V];
        return &k_wgrad_tiled_nhwc<t.kH, t.kW, t.d, t.vec, t.cl, t.px, t.g, t.lv, 1, 1>;
    } else if constexpr (T == 2) {
        constexpr WgradVariant t = kWgradS2Variants[V];
        return &k_wgrad_tiled_nhwc<t.kH, t.kW, t.d, t.vec, t.cl, t.px, t.g, t.lv, 2, 1>;
    } else {
        constexpr WgradVariant t = kWgradM2Variants[V];
        return &k_wgrad_tiled_nhwc<t.kH, t.kW, t.d, t.vec, t.cl, t.px, t.g, t.lv, 1, 2>;
    }
}

// T: 1 = stride 1, 2 = stride 2, 3 = channel multiplier 2 (stride 1)
template <int T, int NVAR, int... Vs>
void fill_wgrad(WgradFn (&fn)[NVAR], std::integer_sequence<int, Vs...>)
{
    ((fn[Vs] = wgrad_fn<Vs, T>()), ...);
}

struct WgradTable {
    WgradFn fn[kNumWgradVariants];
    WgradFn fn2[kNumWgradS2Variants];
    WgradFn fnm[kNumWgradM2Variants];
    WgradTable()
    {
        fill_wgrad<1>(fn, std::make_integer_sequence<int, kNumWgradVariants>());
        fill_wgrad<2>(fn2, std::make_integer_sequence<int, kNumWgradS2Variants>());
        fill_wgrad<3>(fnm, std::make_integer_sequence<int, kNumWgradM2Variants>());
    }
};

typedef void (*WgradNchwFn)(const float *, const float *, float *, WgradNchwArgs);

template <int V, int S>
constexpr WgradNchwFn wgrad_nchw_fn()
{
    if constexpr (S == 1) {
        constexpr TiledNchwVariant t = kWgradNchwVariants[V];
        return &k_wgrad_tiled_nchw<t.kH, t.kW, t.d, t.q, t.g, (t.v4 != 0), 1>;
    } else {
        constexpr TiledNchwVariant t = kWgradNchwS2Variants[V];
        return &k_wgrad_tiled_nchw<t.kH, t.kW, t.d, t.q, t.g, (t.v4 != 0), 2>;
    }
}

template <int S, int NVAR, int... Vs>
void fill_wgrad_nchw(WgradNchwFn (&fn)[NVAR], std::integer_sequence<int, Vs...>)
{
    ((fn[Vs] = wgrad_nchw_fn<Vs, S>()), ...);
}

struct WgradNchwTable {
    WgradNchwFn fn[kNumWgradNchwVariants];
    WgradNchwFn fn2[kNumWgradNchwS2Variants];
    WgradNchwTable()
    {
        fill_wgrad_nchw<1>(fn, std::make_integer_sequence<int, kNumWgradNchwVariants>());
        fill_wgrad_nchw<2>(fn2, std::make_integer_sequence<int, kNumWgradNchwS2Variants>());
    }
};

// The allocation-free weight gradient's partial sums live here: one array
// of kScratchBytes per GPU, allocated when the code object is loaded and
// held until the process ends.  Host code never passes `scratch` itself to a
// kernel (on the host the name stands for a host-side shadow): it passes the
// device address scratch_buffer looks up.
__device__ __align__(256) float scratch[kScratchBytes / 4];

constexpr int kMaxScratchDevices = 64;

}  // namespace

int scratch_buffer(void *stream_v, void **ptr)
{
    static std::once_flag once[kMaxScratchDevices];
    static void *addr[kMaxScratchDevices];
    static hipError_t found[kMaxScratchDevices];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices)
        return DWCONV_ERR_SCRATCH;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream_v);
    if (st) {
        int sdev = -1;
        if (hipStreamGetDevice(st, &sdev) != hipSuccess || sdev != dev)
            return DWCONV_ERR_SCRATCH;
    }
    // once per device, with that device current: each GPU holds its own copy
    // of the array at its own address
    std::call_once(once[dev], [dev]() {
        void *a = nullptr;
        found[dev] = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
        addr[dev] = a;
    });
    if (found[dev] != hipSuccess || !addr[dev])
        return DWCONV_ERR_SCRATCH;
    *ptr = addr[dev];
    return DWCONV_OK;
}

int launch_wgrad(const Problem &p, const Plan &pl, const float *x, const float *dy, float *dw,
                 float *db, void *workspace, void *stream_v, float *w_upd, float *b_upd,
                 float lr)
{
    hipStream_t st = reinterpret_cast<hipStream_t>(stream_v);
    float *part = reinterpret_cast<float *>(workspace);
    WgradArgs a;
    a.N = p.N; a.C = p.mult * p.C; a.mult = p.mult;
    a.H = p.H; a.W = p.W; a.kH = p.kH; a.kW = p.kW; a.d = p.dilation;
    a.pH = pl.pH; a.pW = pl.pW; a.OH = pl.OH; a.OW = pl.OW;
    a.nct = pl.nct; a.nwt = pl.nwt; a.nsp = pl.nst; a.strip = pl.strip; a.chunks = (int)pl.chunks;
    a.xcd = pl.xcd;
    int st1;                                  // status of the stage-1 launch
    if (pl.kind == KIND_WGRAD_TILED_NHWC) {
        static const WgradTable table;
        const bool m2 = p.mult == 2;
        if ((p.mult != 1 && !m2) || (m2 && p.stride != 1))
            return DWCONV_ERR_BAD_STRATEGY;
        const int nvar = m2 ? kNumWgradM2Variants
                            : p.stride == 1 ? kNumWgradVariants : kNumWgradS2Variants;
        if (pl.variant < 0 || pl.variant >= nvar)
            return DWCONV_ERR_BAD_STRATEGY;
        st1 = launch_kernel(m2 ? table.fnm[pl.variant]
                               : p.stride == 1 ? table.fn[pl.variant] : table.fn2[pl.variant],
                            dim3((unsigned)pl.grid), dim3(256), 0, st, x, dy, part, a);
    } else if (pl.kind == KIND_WGRAD_TILED_NCHW) {
        static const WgradNchwTable table;
        const int nvar = p.stride == 1 ? kNumWgradNchwVariants : kNumWgradNchwS2Variants;
        if (pl.variant < 0 || pl.variant >= nvar || pl.cl < 16 || pl.cl > 256 ||
            pl.pb != 256 / pl.cl)
            return DWCONV_ERR_BAD_STRATEGY;
        WgradNchwArgs g;
        g.planes = p.N * p.mult * p.C; g.C = p.mult * p.C; g.mult = p.mult;
        g.H = p.H; g.W = p.W; g.OH = pl.OH; g.OW = pl.OW;
        g.pH = pl.pH; g.pW = pl.pW; g.hl = pl.hl; g.twl = pl.twl;
        g.txn = pl.cl;
        g.pbn = pl.pb;
        g.nct = pl.nct; g.nwt = pl.nwt; g.nsp = pl.nst; g.strip = pl.strip; g.nrt = pl.nrt;
        g.xcd = pl.xcd;
        st1 = launch_kernel(p.stride == 1 ? table.fn[pl.variant] : table.fn2[pl.variant],
                            dim3((unsigned)pl.grid), dim3(256), pl.lds_bytes, st, x, dy, part, g);
    } else if (pl.kind == KIND_WGRAD_STREAM_NCHW) {
        st1 = launch_wgrad_stream_nchw(p, pl, x, dy, part, st);
    } else if (pl.kind == KIND_WGRAD_STREAM_NHWC) {
        st1 = launch_wgrad_stream_nhwc(p, pl, x, dy, part, st);
    } else if (pl.kind == KIND_WGRAD_DIRECT) {
        WgradGenArgs g;
        g.N = p.N; g.C = p.mult * p.C; g.mult = p.mult;
        g.H = p.H; g.W = p.W; g.OH = pl.OH; g.OW = pl.OW;
        g.kH = p.kH; g.kW = p.kW; g.d = p.dilation; g.pH = pl.pH; g.pW = pl.pW;
        g.cl = pl.cl; g.ncg = pl.nct; g.ppc = pl.ppc; g.cpi = pl.cpi;
        const dim3 gr((unsigned)pl.grid), b(256);
        const bool nhwc = p.layout == DWCONV_LAYOUT_NHWC;
        auto k = nhwc ? (p.stride == 1 ? &k_wgrad_gen<true, 1> : &k_wgrad_gen<true, 2>)
                      : (p.stride == 1 ? &k_wgrad_gen<false, 1> : &k_wgrad_gen<false, 2>);
        st1 = launch_kernel(k, gr, b, 0, st, x, dy, part, g);
    } else {
        return DWCONV_ERR_BAD_STRATEGY;
    }
    if (st1 != DWCONV_OK)
        return st1;
    const int cols = p.mult * p.C * (p.kH * p.kW + 1);
    if ((pl.red_s != 4 && pl.red_s != 8 && pl.red_s != 16) ||
        pl.grid2 != (cols + 256 / pl.red_s - 1) / (256 / pl.red_s))
        return DWCONV_ERR_BAD_STRATEGY;
    return launch_kernel(pl.red_s == 16  ? &k_wgrad_reduce<16>
                         : pl.red_s == 8 ? &k_wgrad_reduce<8>
                                         : &k_wgrad_reduce<4>,
                         dim3((unsigned)pl.grid2), dim3(256), 0, st, part, dw,
                         db, (int)pl.chunks, p.mult * p.C, p.kH * p.kW, w_upd,
                         w_upd ? b_upd : nullptr, lr);
}

}  // namespace dwconv
