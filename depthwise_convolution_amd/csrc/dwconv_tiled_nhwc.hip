// dwconv_tiled_nhwc.hip -- the tiled NHWC kernel (stride 1 or 2; forward,
// input gradient, forward with the epilogue) and its launcher.
#include "dwconv_device.h"

namespace dwconv {

namespace {

// ---------------------------------------------------------------------------
// Tiled NHWC (forward, or input gradient with reversed taps).
//
// One workgroup = 256 threads = CL threads across channels x TW = 256/CL
// pixels; each thread owns VEC consecutive channels of one output column.
// The workgroup stages G input rows (its TH = G - R + 1 output rows plus the
// (kH-1)*d row halo) of TW + (kW-1)*d columns (column halo) and CL*VEC
// channels into LDS in one pass, together with its channels' weights, then
// walks the rows: each thread reads its kW taps of a row from LDS and adds
// the row into the R rolling accumulators of the output rows it touches;
// after row u, output row u - (R-1) is complete and is stored.  Short-lived
// workgroups with whole-pixel channel tiles keep the HBM traffic a linear
// sweep, which is what streams fastest on MI355X.
// ---------------------------------------------------------------------------
struct TiledArgs {
    int N, C;
    int IH, IW, OH, OW;     // extents of the tensor read, and of the grid the tiles cover
    int YH, YW;             // extents of the tensor written (the grid's, except stride-2 fwd)
    int pH, pW;             // top / left zero padding of the tensor read
    int nct, nwt, nst;      // channel tiles, column tiles, row tiles
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
template <typename WT, int KH, int KW, int D, int VEC, int CL, int PX, int G, int LV, int MODE,
          int S>
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
    typedef TiledGeom<KH, KW, D, VEC, CL, PX, G, LV> Gm;
    constexpr int R = Gm::R, TH = Gm::TH, TW = Gm::TW, CG = Gm::CG, TWI = Gm::TWI;
    constexpr int VPC = Gm::VPC, VPR = Gm::VPR, VCH = Gm::VCH, NV = Gm::NV, KK = Gm::KK;
    constexpr int WF = Gm::WF, XF4 = Gm::XF4;
    __shared__ float4 lds[XF4 + (WF + 3) / 4];
    float *ldsx = reinterpret_cast<float *>(lds);
    float *ldsw = ldsx + XF4 * 4;
    const WT *w = reinterpret_cast<const WT *>(wv);

    int tile = blockIdx.x;
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
    // the tile is still in flight.
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, a.C * KK * (int)sizeof(WT));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(bias, (!IG && bias) ? a.C * 4 : 0);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(in + n * a.IH * a.IW * a.C, a.IH * a.IW * a.C * 4);
    constexpr int NW = (WF + 255) / 256;
    float wst[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i)
        wst[i] = buf_w(rw, c0 * KK + tid + i * 256, (WT *)nullptr);
    float bv[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v)
        bv[v] = buf_f32(rb, (cq + v) * 4);
    EpiChan ec[VEC];
    if constexpr (EPI) {
#pragma unroll
        for (int v = 0; v < VEC; ++v)
            ec[v] = epi_load(ep, cq + v, a.C);
    }
    typedef typename VecT<LV>::type LoadT;
    LoadT stage[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = tid + i * 256;
        const int g = e / VPR;
        const int rem = e - g * VPR;
        const int col = rem / VPC;
        const int cv = rem - col * VPC;
        const int row = rbase + g, gc = cbase + col, ch = c0 + cv * LV;
        bool ok = e < VCH && g < nrows && row >= 0 && gc >= 0 && ch < a.C;
        int sr = row, sc = gc;                  // position in the tensor read
        if constexpr (UPS) {
            ok = ok && (row & 1) == 0 && (gc & 1) == 0;
            sr = row >> 1;
            sc = gc >> 1;
        }
        ok = ok && sr < a.IH && sc < a.IW;
        const int off = ok ? ((sr * a.IW + sc) * a.C + ch) * 4 : kOutOfRange;
        if constexpr (LV == 4)
            stage[i] = buf_f4(rx, off);
        else
            stage[i] = buf_f32(rx, off);
    }
    // 2. weights, then the tile, into LDS
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int e = tid + i * 256;
        if (e < WF)
            ldsw[e] = wst[i];
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = tid + i * 256;
        if (e < VCH)
            reinterpret_cast<LoadT *>(lds)[e] = stage[i];
    }
    __syncthreads();

    // per-thread weights (reversed taps for the input gradient)
    float wr[KH][KW][VEC];
#pragma unroll
    for (int kh = 0; kh < KH; ++kh)
#pragma unroll
        for (int kw = 0; kw < KW; ++kw)
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                const int tap = IG ? (KH - 1 - kh) * KW + (KW - 1 - kw) : kh * KW + kw;
                wr[kh][kw][v] = ldsw[(q * VEC + v) * KK + tap];
            }
    if constexpr (EPI) {
#pragma unroll
        for (int v = 0; v < VEC; ++v)
            epi_finish(ec[v], ep);
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
    float *outp = out + (n * a.YH * a.YW) * a.C;
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
                        epi_block(acc[m % R][j], ec, ep.act);
                    if constexpr (DEC) {
                        const int c = ow + j;
                        if (cvalid && (r & 1) == 0 && (c & 1) == 0 && (c >> 1) < a.YW)
                            store_vec<VEC>(outp + (((r >> 1) * a.YW + (c >> 1)) * a.C + cq),
                                           acc[m % R][j]);
                    } else if (cvalid && ow + j < a.OW) {
                        store_vec<VEC>(outp + ((r * a.OW + ow + j) * a.C + cq), acc[m % R][j]);
                    }
#pragma unroll
                    for (int v = 0; v < VEC; ++v)
                        acc[m % R][j][v] = bv[v];
                }
            }
        }
    }
}

typedef void (*TiledFn)(const float *, const void *, const float *, float *, TiledArgs,
                        EpiArgs);

// Kernel tables of the tiled NHWC kernel: [variant][f16 weights][mode], one
// per stride (the stride-2 table is built from its own variant list).
template <typename WT, int V, int MODE, int S>
constexpr TiledFn tiled_fn()
{
    if constexpr (S == 1) {
        constexpr TiledVariant t = kTiledVariants[V];
        return &k_tiled_nhwc<WT, t.kH, t.kW, t.d, t.vec, t.cl, t.px, t.g, t.lv, MODE, 1>;
    } else {
        constexpr TiledVariant t = kTiledS2Variants[V];
        return &k_tiled_nhwc<WT, t.kH, t.kW, t.d, t.vec, t.cl, t.px, t.g, t.lv, MODE, 2>;
    }
}

template <int V, int S>
void fill_tiled(TiledFn (&row)[2][3])
{
    row[0][0] = tiled_fn<float, V, kModeFwd, S>();
    row[0][1] = tiled_fn<float, V, kModeInputGrad, S>();
    row[0][2] = tiled_fn<float, V, kModeFwdEpilogue, S>();
    row[1][0] = tiled_fn<half_t, V, kModeFwd, S>();
    row[1][1] = tiled_fn<half_t, V, kModeInputGrad, S>();
    row[1][2] = tiled_fn<half_t, V, kModeFwdEpilogue, S>();
}

template <int S, int NVAR, int... Vs>
void fill_all_tiled(TiledFn (&fn)[NVAR][2][3], std::integer_sequence<int, Vs...>)
{
    (fill_tiled<Vs, S>(fn[Vs]), ...);
}

struct TiledTable {
    TiledFn fn[kNumTiledVariants][2][3];
    TiledFn fn2[kNumTiledS2Variants][2][3];
    TiledTable()
    {
        fill_all_tiled<1>(fn, std::make_integer_sequence<int, kNumTiledVariants>());
        fill_all_tiled<2>(fn2, std::make_integer_sequence<int, kNumTiledS2Variants>());
    }
};


}  // namespace

int launch_tiled_nhwc(const Problem &p, const Plan &pl, const float *in, const void *w,
                      const float *b, float *out, hipStream_t st, const EpiArgs &ep)
{
    static const TiledTable table;
    const int nvar = p.stride == 1 ? kNumTiledVariants : kNumTiledS2Variants;
    if (pl.variant < 0 || pl.variant >= nvar)
        return DWCONV_ERR_BAD_STRATEGY;
    TiledFn f = p.stride == 1 ? table.fn[pl.variant][p.wtype == DWCONV_W_F16][mode_of(p, ep)]
                              : table.fn2[pl.variant][p.wtype == DWCONV_W_F16][mode_of(p, ep)];
    TiledArgs a;
    a.N = p.N; a.C = p.C;
    a.IH = pl.IH; a.IW = pl.IW; a.OH = pl.OH; a.OW = pl.OW;
    a.YH = pl.YH; a.YW = pl.YW;
    a.pH = pl.pH; a.pW = pl.pW;
    a.nct = pl.nct; a.nwt = pl.nwt; a.nst = pl.nst;
    hipLaunchKernelGGL(f, dim3((unsigned)pl.grid), dim3(256), 0, st, in, w,
                       p.op == DWCONV_OP_FWD ? b : nullptr, out, a, ep);
    return DWCONV_OK;
}


}  // namespace dwconv
