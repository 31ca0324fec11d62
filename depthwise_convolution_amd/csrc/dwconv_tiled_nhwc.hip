// dwconv_tiled_nhwc.hip -- the tiled NHWC kernel (stride 1 or 2; forward,
// input gradient, forward with the epilogue) and its launcher.
#include "dwconv_device.h"

namespace dwconv {

namespace {

// ---------------------------------------------------------------------------
// Tiled NHWC (forward, or input gradient with reversed taps).
//
// One workgroup = 256 threads = CL threads across channels x 256/CL threads
// across columns; each thread owns VEC consecutive channels of PX adjacent
// output columns, so a tile is CL*VEC channels x TW = PX*256/CL columns.
// The workgroup stages G input rows (its TH = G - R + 1 output rows plus the
// (kH-1)*d row halo) of TW + (kW-1)*d columns (column halo) and CL*VEC
// channels into LDS in one pass (with buffer loads that write LDS directly,
// except 4-byte staging at stride 2), together with its channels' weights, then
// walks the rows: each thread reads its kW taps of a row from LDS and adds
// the row into the R rolling accumulators of the output rows it touches;
// after row u, output row u - (R-1) is complete and is stored.  Short-lived
// workgroups with whole-pixel channel tiles keep the HBM traffic a linear
// sweep, which is what streams fastest on MI355X.
// ---------------------------------------------------------------------------
struct TiledArgs {
    int N, C;               // C: channels of the tile walk (the forward's output channels,
                            // the input gradient's dy channels)
    int CR, CW;             // channels of the tensor read / written (C, or C / multiplier)
    int IH, IW, OH, OW;     // extents of the tensor read, and of the grid the tiles cover
    int YH, YW;             // extents of the tensor written (the grid's, except stride-2 fwd)
    int pH, pW;             // top / left zero padding of the tensor read
    int nct, nwt, nst;      // channel tiles, column tiles, row tiles
    int xcd;                // tile order: 1 = per-XCD ranges (xcd_tile), 2 = band-local
                            // runs (band_tile), 0 = in order
    int ntl;                // 1: staged rows that no other tile stages load non-temporally
};

// LV: floats per staging load, 4 (16-byte loads: C % 4 == 0, 16-byte
// aligned tensors) or 1 (any channel count).
template <int KH, int KW, int D, int VEC, int CL, int PX, int G, int LV>
struct TiledGeom {
    static constexpr int R = (KH - 1) * D + 1;      // rows of one window
    static constexpr int TH = G - R + 1;            // output rows per workgroup
    static constexpr int TW = PX * 256 / CL;        // output columns per workgroup
    static constexpr int CG = CL * VEC;             // channels per workgroup
    static constexpr int TWI = TW + (KW - 1) * D;   // input columns staged
    static constexpr int VPC = CG / LV;             // loads per staged pixel
    static constexpr int VPR = TWI * VPC;           // loads per staged row
    static constexpr int VCH = G * VPR;             // loads staged
    static constexpr int NV = (VCH + 255) / 256;    // loads per thread
    static constexpr int XF4 = (VCH * LV + 3) / 4;  // staged tile, in float4
    static constexpr int KK = KH * KW;
    static constexpr int WF = CG * KK;              // weight floats per workgroup
    static_assert(TH >= 1, "a workgroup must produce at least one output row");
    static_assert(256 % CL == 0 && CG % LV == 0 && (LV == 4 || LV == 1), "bad channel tiling");
    static_assert(LV == 4 || VEC == 1, "scalar staging computes one channel per thread");
};

//
// Stride 2 (S == 2) reuses the stride-1 walk (LeanMlir "Depthwise": the
// stride-2 conv is the stride-1 conv kept at every other position, and its
// input-VJP is the stride-1 reversed-kernel conv of the zero-upsampled
// cotangent):
//  * forward: the tiles cover the stride-1 grid 2*Ho-1 x 2*Wo-1 (pads as
//    given), only its even rows are accumulated and only its even positions
//    stored, at y[r/2][c/2];
//  * input gradient: dy is zero-upsampled while it is staged (a staged
//    position takes dy[t/2][v/2] when both are even, else zero), and staged
//    rows that are all zero are skipped.
//
// Channel multiplier M (output channel o reads input channel o/M): the walk
// runs over the forward's output channels (= the input gradient's dy
// channels) either way.
//  * forward: the x tile is loaded with the input channels only and each
//    value is written to LDS M times, once per output channel that reads it;
//  * input gradient: dx channel c sums the M dy channels c*M .. c*M+M-1, so
//    a thread's VEC accumulators are added in groups of M at the store.
template <typename WT, int KH, int KW, int D, int VEC, int CL, int PX, int G, int LV, int MODE,
          int S, int M = 1>
__global__ __launch_bounds__(256) void k_tiled_nhwc(const float *__restrict__ in,
                                                    const void *__restrict__ wv,
                                                    const float *__restrict__ bias,
                                                    float *__restrict__ out, TiledArgs a,
                                                    EpiArgs ep)
{
    constexpr bool IG = MODE == kModeInputGrad, EPI = MODE == kModeFwdEpilogue;
    constexpr bool UPS = S == 2 && IG;        // staged input is the zero-upsampled dy
    constexpr bool DEC = S == 2 && !IG;       // output is the decimated stride-1 grid
    static_assert(S == 1 || S == 2, "stride 1 or 2");
    static_assert(M == 1 || (M == 2 && LV == 4 && VEC % M == 0 && S == 1),
                  "multiplier 2: 16-byte staging, whole groups of M channels per thread");
    constexpr bool XM = M > 1 && !IG;         // x staged with 1/M of the walk's channels
    typedef TiledGeom<KH, KW, D, VEC, CL, PX, G, LV> Gm;
    constexpr int R = Gm::R, TH = Gm::TH, TW = Gm::TW, CG = Gm::CG, TWI = Gm::TWI;
    constexpr int KK = Gm::KK;
    // loads per staged pixel / row / tile, and per thread
    constexpr int VPC = XM ? CG / (M * LV) : Gm::VPC, VPR = TWI * VPC, VCH = G * VPR;
    constexpr int NV = (VCH + 255) / 256;
    constexpr int WF = Gm::WF;
    // The tile goes from the buffer straight into LDS (4- or 16-byte loads),
    // a wave's 64 consecutive staged loads per instruction, so its region is
    // rounded up to 64 loads.  At stride 2 only the 16-byte staging does so
    // (4-byte measured 2-4% slower than the copy through registers, 16-byte
    // mostly 2-8% faster); the multiplier-2 forward, which writes every x
    // value twice, takes the copy too.
    constexpr bool DMA = !XM && (S == 1 || LV == 4);
    constexpr int XF4 = DMA ? (VCH + 63) / 64 * 16 * LV : Gm::XF4;
    __shared__ float4 lds[XF4 + (WF + 3) / 4];
    float *ldsx = reinterpret_cast<float *>(lds);
    float *ldsw = ldsx + XF4 * 4;
    const WT *w = reinterpret_cast<const WT *>(wv);

    // tiles: channel tile, column tile, row tile, image (fastest first)
    int tile = a.xcd == 1   ? xcd_tile(blockIdx.x, gridDim.x)
               : a.xcd == 2 ? band_tile(blockIdx.x, a.nct * a.nwt)
                            : blockIdx.x;
    const int ct = tile % a.nct;
    tile /= a.nct;
    const int wt = tile % a.nwt;
    tile /= a.nwt;
    const int st = tile % a.nst;
    const int n = tile / a.nst;
    const int c0 = ct * CG, w0 = wt * TW, h0 = st * TH;
    const int tid = threadIdx.x;
    const int nrows = min(TH, a.OH - h0) + R - 1;  // staged rows that exist in the strip
    const int rbase = h0 - a.pH, cbase = w0 - a.pW;

    const int q = tid % CL, p = tid / CL;
    const int cq = c0 + q * VEC;
    const bool cvalid = cq < a.C;        // LV == 4: C % 4 == 0, so the whole vector is valid
    const int ow = w0 + p * PX;          // first of this thread's PX output columns

    // 1. Issue every global load up front, the small L2-resident ones first:
    // this workgroup's weights (contiguous in memory) and the thread's bias,
    // then the input tile.  All are buffer loads: weights of channels >= C,
    // a missing bias, and tile elements outside the image read as zero.
    // Loads complete in order, so the weights can be written to LDS while
    // the tile is still in flight (where the tile loads write LDS
    // themselves, a wait for all loads precedes the barrier).
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, a.C * KK * (int)sizeof(WT));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(bias, (!IG && bias) ? a.C * 4 : 0);
    const __amdgpu_buffer_rsrc_t rx =
        make_rsrc(in + n * a.IH * a.IW * a.CR, a.IH * a.IW * a.CR * 4);
    constexpr int NW = (WF + 255) / 256;
    float wst[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i)
        wst[i] = buf_w(rw, c0 * KK + tid + i * 256, (WT *)nullptr);
    // bias and epilogue factors: one 16-byte load per array for 4 channels
    // (C % 4 == 0 with 16-byte staging, so a vector is wholly in or out of range)
    constexpr bool V4F = VEC == 4 && LV == 4;
    float bv[VEC];
    if constexpr (V4F) {
        const float4 b4 = buf_f4(rb, cq * 4);
        bv[0] = b4.x; bv[1] = b4.y; bv[2] = b4.z; bv[3] = b4.w;
    } else {
#pragma unroll
        for (int v = 0; v < VEC; ++v)
            bv[v] = buf_f32(rb, (cq + v) * 4);
    }
    EpiChan ec[VEC];
    if constexpr (EPI && V4F) {
        epi_load4(ep, cq, a.C, ec);
    } else if constexpr (EPI) {
#pragma unroll
        for (int v = 0; v < VEC; ++v)
            ec[v] = epi_load(ep, cq + v, a.C);
    }
    // Staged load e = tid + 256*i is vector cv of staged pixel (g, col):
    // e = (g * TWI + col) * VPC + cv.  VPC is a power of two that divides
    // 256, so cv (hence the channel) is the same for all of a thread's loads,
    // and (g, col) advance by a fixed step from one load to the next.  A load
    // with g < nrows (<= G) is one of the VCH staged loads.
    static_assert((VPC & (VPC - 1)) == 0 && 256 % VPC == 0, "staging vectors per pixel");
    constexpr int DG = 256 / VPR, DC = (256 % VPR) / VPC;
    const int cv = tid % VPC;
    // channel of the tensor read (with XM: an input channel of the tile's c0 / M ..)
    const int ch = (XM ? c0 / M : c0) + cv * LV;
    const bool chok = ch < a.CR;
    int g = tid / VPR, col = (tid % VPR) / VPC;
    // without upsampling the byte offset of (g, col) steps with them
    // (unsigned: positions outside the image may wrap, they are not loaded)
    const unsigned pstep = 4u * a.CR, rstep = pstep * a.IW;
    unsigned uoff = (unsigned)(rbase + g) * rstep + (unsigned)(cbase + col) * pstep + 4u * ch;
    typedef typename VecT<LV>::type LoadT;
    LoadT stage[DMA ? 1 : NV];
    const int wel = __builtin_amdgcn_readfirstlane(tid) & ~63;   // the wave's first element
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
        int off;
        if constexpr (UPS) {
            // upsampled position (row, gc) holds dy[row/2][gc/2] when both are even
            const bool ok = chok && g < nrows && ((row | gc) & 1) == 0 &&
                            (unsigned)row < 2u * (unsigned)a.IH &&
                            (unsigned)gc < 2u * (unsigned)a.IW;
            off = ok ? (((row >> 1) * a.IW + (gc >> 1)) * a.CR + ch) * 4 : kOutOfRange;
        } else {
            const bool ok = chok && g < nrows && (unsigned)row < (unsigned)a.IH &&
                            (unsigned)gc < (unsigned)a.IW;
            off = ok ? (int)uoff : kOutOfRange;
        }
        if constexpr (DMA) {
            if ((i + 1) * 256 <= VCH || i * 256 + wel < VCH) {  // the wave's run holds staged loads
                // a wave whose loads all lie in rows R-1 .. TH-1 (rows the row
                // tiles above and below do not stage; wave-uniform) may load
                // them non-temporally: for tensors too large for the Infinity
                // Cache it streams them past it
                const int e0 = i * 256 + wel;
                if (S == 1 && a.ntl && e0 / VPR >= R - 1 && (e0 + 63) / VPR <= TH - 1)
                    buf_to_lds<4 * LV, true>(rx, ldsx + (i * 256 + wel) * LV, off);
                else
                    buf_to_lds<4 * LV>(rx, ldsx + (i * 256 + wel) * LV, off);
            }
        } else if constexpr (LV == 4) {
            stage[i] = buf_f4(rx, off);
        } else {
            stage[i] = buf_f32(rx, off);
        }
    }
    // 2. weights, then (unless loaded straight into LDS) the tile, into LDS
    // (only a last, partial round of loads needs a bound)
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int e = tid + i * 256;
        if ((i + 1) * 256 <= WF || e < WF)
            ldsw[e] = wst[i];
    }
#pragma unroll
    for (int i = 0; i < (DMA ? 0 : NV); ++i) {
        const int e = tid + i * 256;
        if ((i + 1) * 256 <= VCH || e < VCH) {
            if constexpr (XM) {
                // input channels ch .. ch+3 feed output slots M*ch .. M*ch + 4M - 1
                const float4 v = stage[i];
                lds[2 * e] = make_float4(v.x, v.x, v.y, v.y);
                lds[2 * e + 1] = make_float4(v.z, v.z, v.w, v.w);
            } else {
                reinterpret_cast<LoadT *>(lds)[e] = stage[i];
            }
        }
    }
    if constexpr (DMA)
        vm_drain();                       // the barrier does not wait for the LDS loads
    __syncthreads();

    // per-thread weights (reversed taps for the input gradient)
    float wr[KH][KW][VEC];
    const float *wq = ldsw + q * VEC * KK;
#pragma unroll
    for (int kh = 0; kh < KH; ++kh)
#pragma unroll
        for (int kw = 0; kw < KW; ++kw)
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                const int tap = IG ? (KH - 1 - kh) * KW + (KW - 1 - kw) : kh * KW + kw;
                wr[kh][kw][v] = wq[v * KK + tap];
            }
    if constexpr (EPI) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            epi_finish(ec[v], ep);
            bv[v] = epi_fold_bias(bv[v], ec[v]);
#pragma unroll
            for (int kh = 0; kh < KH; ++kh)
#pragma unroll
                for (int kw = 0; kw < KW; ++kw)
                    wr[kh][kw][v] *= ec[v].inv;
        }
    }
    float acc[R][PX][VEC];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < PX; ++j)
#pragma unroll
            for (int v = 0; v < VEC; ++v)
                acc[r][j][v] = bv[v];

    // 3. walk the staged rows
    constexpr int XW = PX + (KW - 1) * D;  // staged columns one thread reads per row
    float *outp = out + (n * a.YH * a.YW) * a.CW;
    // this thread's first output of the tile's first row (not DEC, not IG with M > 1)
    float *orow = outp + ((h0 * a.OW + ow) * a.CW + cq);
    const int ors = a.OW * a.CW;
    // the walk, with the activation of the fused epilogue as a constant:
    // one copy of the walk per activation, no branch at the stores
    auto walk = [&](auto act_c) __attribute__((always_inline)) {
    constexpr int ACT = decltype(act_c)::value;
#pragma unroll
    for (int u = 0; u < G; ++u) {
        if (u < nrows) {
            // a staged row of the upsampled dy at an odd position is all zero
            if (!(UPS && ((rbase + u) & 1))) {
                float xv[XW][VEC];
#pragma unroll
                for (int i = 0; i < XW; ++i) {
                    const float *src = ldsx + ((u * TWI + p * PX + i) * CG + q * VEC);
#pragma unroll
                    for (int v = 0; v < VEC; ++v)
                        xv[i][v] = src[v];
                }
#pragma unroll
                for (int kh = 0; kh < KH; ++kh) {
                    const int m = u - kh * D;      // output row this tap row feeds
                    if (m >= 0 && m < TH && !(DEC && ((h0 + m) & 1))) {
                        const int slot = m % R;
#pragma unroll
                        for (int kw = 0; kw < KW; ++kw)
#pragma unroll
                            for (int j = 0; j < PX; ++j)
#pragma unroll
                                for (int v = 0; v < VEC; ++v)
                                    acc[slot][j][v] =
                                        fmaf(wr[kh][kw][v], xv[j + kw * D][v], acc[slot][j][v]);
                    }
                }
            }
            const int m = u - (R - 1);             // output row completed by row u
            if (m >= 0) {
                const int r = h0 + m;
#pragma unroll
                for (int j = 0; j < PX; ++j) {
                    if constexpr (EPI)
                        epi_act_c<ACT>(acc[m % R][j]);
                    if constexpr (DEC) {
                        const int c = ow + j;
                        if (cvalid && (r & 1) == 0 && (c & 1) == 0 && (c >> 1) < a.YW)
                            store_vec<VEC>(outp + (((r >> 1) * a.YW + (c >> 1)) * a.CW + cq),
                                           acc[m % R][j]);
                    } else if (IG && M > 1) {
                        // dx channel cq/M + k sums the dy channels (cq/M + k)*M + jj
                        if (cvalid && ow + j < a.OW) {
                            float sum[VEC / M];
#pragma unroll
                            for (int k = 0; k < VEC / M; ++k) {
                                sum[k] = acc[m % R][j][k * M];
#pragma unroll
                                for (int jj = 1; jj < M; ++jj)
                                    sum[k] += acc[m % R][j][k * M + jj];
                            }
                            store_vec<VEC / M>(outp + ((r * a.OW + ow + j) * a.CW + cq / M), sum);
                        }
                    } else if (cvalid && ow + j < a.OW) {
                        store_vec<VEC>(orow + (m * ors + j * a.CW), acc[m % R][j]);
                    }
#pragma unroll
                    for (int v = 0; v < VEC; ++v)
                        acc[m % R][j][v] = bv[v];
                }
            }
        }
    }
    };
    if constexpr (EPI)
        with_act(ep.act, walk);
    else
        walk(std::integral_constant<int, DWCONV_ACT_NONE>());
}

typedef void (*TiledFn)(const float *, const void *, const float *, float *, TiledArgs,
                        EpiArgs);

// Kernel tables of the tiled NHWC kernel: [variant][f16 weights][mode], one
// per variant list: stride 1, stride 2, channel multiplier 2 (stride 1).
constexpr int kTableS1 = 0, kTableS2 = 1, kTableM2 = 2;

template <typename WT, int V, int MODE, int T>
constexpr TiledFn tiled_fn()
{
    if constexpr (T == kTableS1) {
        constexpr TiledVariant t = kTiledVariants[V];
        return &k_tiled_nhwc<WT, t.kH, t.kW, t.d, t.vec, t.cl, t.px, t.g, t.lv, MODE, 1, 1>;
    } else if constexpr (T == kTableS2) {
        constexpr TiledVariant t = kTiledS2Variants[V];
        return &k_tiled_nhwc<WT, t.kH, t.kW, t.d, t.vec, t.cl, t.px, t.g, t.lv, MODE, 2, 1>;
    } else {
        constexpr TiledVariant t = kTiledM2Variants[V];
        return &k_tiled_nhwc<WT, t.kH, t.kW, t.d, t.vec, t.cl, t.px, t.g, t.lv, MODE, 1, 2>;
    }
}

template <int V, int T>
void fill_tiled(TiledFn (&row)[2][3])
{
    row[0][0] = tiled_fn<float, V, kModeFwd, T>();
    row[0][1] = tiled_fn<float, V, kModeInputGrad, T>();
    row[0][2] = tiled_fn<float, V, kModeFwdEpilogue, T>();
    row[1][0] = tiled_fn<half_t, V, kModeFwd, T>();
    row[1][1] = tiled_fn<half_t, V, kModeInputGrad, T>();
    row[1][2] = tiled_fn<half_t, V, kModeFwdEpilogue, T>();
}

template <int T, int NVAR, int... Vs>
void fill_all_tiled(TiledFn (&fn)[NVAR][2][3], std::integer_sequence<int, Vs...>)
{
    (fill_tiled<Vs, T>(fn[Vs]), ...);
}

struct TiledTable {
    TiledFn fn[kNumTiledVariants][2][3];
    TiledFn fn2[kNumTiledS2Variants][2][3];
    TiledFn fnm[kNumTiledM2Variants][2][3];
    TiledTable()
    {
        fill_all_tiled<kTableS1>(fn, std::make_integer_sequence<int, kNumTiledVariants>());
        fill_all_tiled<kTableS2>(fn2, std::make_integer_sequence<int, kNumTiledS2Variants>());
        fill_all_tiled<kTableM2>(fnm, std::make_integer_sequence<int, kNumTiledM2Variants>());
    }
};

}  // namespace

int launch_tiled_nhwc(const Problem &p, const Plan &pl, const float *in, const void *w,
                      const float *b, float *out, hipStream_t st, const EpiArgs &ep)
{
    static const TiledTable table;
    const bool m2 = p.mult == 2;
    if ((p.mult != 1 && !m2) || (m2 && p.stride != 1))
        return DWCONV_ERR_BAD_STRATEGY;
    const int nvar = m2 ? kNumTiledM2Variants
                        : p.stride == 1 ? kNumTiledVariants : kNumTiledS2Variants;
    if (pl.variant < 0 || pl.variant >= nvar)
        return DWCONV_ERR_BAD_STRATEGY;
    const int wt16 = p.wtype == DWCONV_W_F16, mode = mode_of(p, ep);
    TiledFn f = m2 ? table.fnm[pl.variant][wt16][mode]
                   : p.stride == 1 ? table.fn[pl.variant][wt16][mode]
                                   : table.fn2[pl.variant][wt16][mode];
    TiledArgs a;
    a.N = p.N;
    a.C = p.mult * p.C;                                  // output (dy) channels
    a.CR = p.op == DWCONV_OP_FWD ? p.C : p.mult * p.C;   // channels of the tensor read
    a.CW = p.op == DWCONV_OP_FWD ? p.mult * p.C : p.C;   // channels of the tensor written
    a.IH = pl.IH; a.IW = pl.IW; a.OH = pl.OH; a.OW = pl.OW;
    a.YH = pl.YH; a.YW = pl.YW;
    a.pH = pl.pH; a.pW = pl.pW;
    a.nct = pl.nct; a.nwt = pl.nwt; a.nst = pl.nst;
    a.xcd = pl.xcd;
    a.ntl = pl.ntl;
    return launch_kernel(f, dim3((unsigned)pl.grid), dim3(256), 0, st, in, w,
                         p.op == DWCONV_OP_FWD ? b : nullptr, out, a, ep);
}


}  // namespace dwconv
