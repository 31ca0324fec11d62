// dwconv_tiled_nchw.hip -- the tiled NCHW kernel (stride 1 or 2; forward,
// input gradient, forward with the epilogue) and its launcher.
#include "dwconv_device.h"

namespace dwconv {

namespace {

// ---------------------------------------------------------------------------
// Tiled NCHW (forward, or input gradient with reversed taps).
//
// Channel-outer layout: each (n, c) plane is an image of its own, and the
// weights of a plane are one kernel.  A workgroup of 256 threads covers PB =
// floor(256/TX) planes x TX threads per plane row (TX = clamp(ceil(Wo/Q), 16,
// 256), so narrow planes are packed several to a workgroup; threads past
// PB*TX idle through the walk); each thread owns Q adjacent output columns.
// G input rows of every plane (the TH = G - R + 1 output rows plus the row
// halo) and the column halo are staged in LDS in one pass, then the rows are
// walked with rolling accumulators as in the NHWC kernel.  Loads are buffer loads over the whole tensor: rows
// past the plane or the tensor read as zero, columns outside [0, W) are
// given an out-of-range offset.
// ---------------------------------------------------------------------------
struct TiledNchwArgs {
    int planes, C;          // planes (n, c) of the walk and their channels: the tensor
                            // written in the forward, the tensor read in the input gradient
    int mult;               // forward channel multiplier: walk plane p reads input plane p / mult
    int IH, IW, OH, OW;     // extents of the tensor read, and of the grid the tiles cover
    int YH, YW;             // extents of the tensor written (the grid's, except stride-2 fwd)
    int pH, pW;             // top / left zero padding of the tensor read
    int hl, twl;            // staged columns left of a tile; staged floats per plane row
    int txn, pbn;           // threads per plane row (16..256), planes per workgroup (256 / txn)
    int nct, nwt, nst;      // plane groups, column tiles, row tiles
    int xcd;                // tile order: 1 = per-XCD ranges (xcd_tile), 2 = bands of 8 plane
                            // groups (band_tile), 0 = in order
    int ost8;               // 1: the tensor written is 8-byte aligned (Q-wide vector stores)
};


// Stride 2 (S == 2) as in the NHWC kernel: the forward tiles the stride-1
// grid and keeps its even positions, the input gradient stages dy
// zero-upsampled (4-byte loads only) and skips the all-zero rows.
//
// Input gradient with a channel multiplier M (M > 1, stride 1): dx plane
// n*C + c sums the M dy planes (n*C + c)*M + j, j < M, each with its own
// weights; a workgroup stages the M dy planes of each of its dx planes and
// every thread adds all M of them into its accumulators.
template <typename WT, int KH, int KW, int D, int Q, int G, bool V4, int MODE, int S, int M = 1>
__global__ __launch_bounds__(256) void k_tiled_nchw(const float *__restrict__ in,
                                                    const void *__restrict__ wv,
                                                    const float *__restrict__ bias,
                                                    float *__restrict__ out, TiledNchwArgs a,
                                                    EpiArgs ep)
{
    constexpr bool IG = MODE == kModeInputGrad, EPI = MODE == kModeFwdEpilogue;
    constexpr bool UPS = S == 2 && IG;        // staged input is the zero-upsampled dy
    constexpr bool DEC = S == 2 && !IG;       // output is the decimated stride-1 grid
    static_assert(!(UPS && V4), "upsampled staging uses 4-byte loads");
    static_assert(M == 1 || (IG && S == 1), "a multiplier > 1 here: input gradient, stride 1");
    typedef NchwGeom<KH, KW, D, Q, G, V4> Gm;
    constexpr int R = Gm::R, TH = Gm::TH, KK = Gm::KK, LV = Gm::LV;
    constexpr int NW = (Gm::PBMAX * M * KK + 255) / 256;
    // loads per thread: the whole tile (M planes per walk plane), or with the
    // upsampled dy only its even rows, one dy element per pair of staged
    // columns (the twl/2 pairs of a row: twl is even then)
    constexpr int NV = nchw_stage_loads(UPS ? 1 : 0, M * G, Q, KW, D, V4);
    extern __shared__ float4 lds4[];
    float *lds = reinterpret_cast<float *>(lds4);
    const WT *w = reinterpret_cast<const WT *>(wv);

    const int txn = a.txn, pbn = a.pbn;
    const int tw = txn * Q, twl = a.twl;               // staged floats per plane row
    const int vpr = twl / LV;                          // loads per plane row
    // 4-byte staging without upsampling loads the tile straight into LDS
    // (buffer loads with the LDS flag: a wave writes 64 consecutive staged
    // elements); the weights follow the tile after whole waves of elements
    constexpr bool DMA = !UPS && !V4;
    const int nel = pbn * M * G * vpr;                 // staged elements (LV floats each)
    float *ldsw = lds + (nel + 63) / 64 * 64 * LV;

    // tiles: row tile, column tile, plane group (fastest first), so the row
    // tiles of a plane group, which share halo rows, are consecutive
    // (2: bands of 8 plane groups, one plane group's row tiles per XCD)
    int tile = a.xcd == 1   ? xcd_tile(blockIdx.x, gridDim.x)
               : a.xcd == 2 ? band_tile(blockIdx.x, 8 * a.nst * a.nwt)
                            : blockIdx.x;
    const int st = tile % a.nst;
    tile /= a.nst;
    const int wt = tile % a.nwt;
    const int pg = tile / a.nwt;
    const int w0 = wt * tw, h0 = st * TH;
    const int tid = threadIdx.x;
    const int nrows = min(TH, a.OH - h0) + R - 1;
    const int rbase = h0 - a.pH, cbase = w0 - a.hl;

    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, M * a.C * KK * (int)sizeof(WT));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(bias, (!IG && bias) ? a.C * 4 : 0);
    // with a multiplier (forward only) plane n*C + o reads input plane n*(C/mult) + o/mult,
    // which is (n*C + o) / mult
    // (with M > 1 the input gradient reads M dy planes per walk plane)
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(in, M * (a.planes / a.mult) * a.IH * a.IW * 4);

    // 1. all loads up front: weights of the workgroup's planes, the bias, the tile
    float wst[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int e = tid + i * 256;
        const int pj = e / KK, tap = e - pj * KK;      // pj = pl*M + j
        const int pl = pj / M;
        const int plane = pg * pbn + pl;
        const bool ok = pl < pbn && plane < a.planes;
        // weight row of dy channel (plane % C)*M + j
        const int row = (plane % a.C) * M + (pj - pl * M);
        wst[i] = buf_w(rw, ok ? row * KK + tap : kOutOfRange / 4, (WT *)nullptr);
    }
    // threads past pbn * txn (when txn does not divide 256) idle along
    const int pli_raw = tid / txn, tx = tid - pli_raw * txn;
    const int pli = min(pli_raw, pbn - 1);             // in-range LDS addresses for idle threads
    const int my_plane = pg * pbn + pli;
    const bool pvalid = pli_raw < pbn && my_plane < a.planes;
    float bval = buf_f32(rb, pvalid ? (my_plane % a.C) * 4 : kOutOfRange);
    EpiChan ec{0.0f, 1.0f, 0.0f, 0.0f};
    if constexpr (EPI)
        ec = epi_load(ep, pvalid ? my_plane % a.C : a.C, a.C);
    float sv[NV][LV];
    // upsampled staging: rows g0, g0+2, ... of the tile are the even
    // (upsampled) rows; a pair k of staged columns (2k, 2k+1) holds one dy
    // element at its even column and a zero at the other
    const int g0 = rbase & 1, ge_n = (G - g0 + 1) / 2, hp = twl / 2, c1 = cbase & 1;
    // otherwise load e = tid + i*256 is (pj, g, cv) = (e / (G*vpr), e / vpr % G,
    // e % vpr): the pair (gq = e / vpr, cv) is stepped by 256 per load with no
    // further division
    int s_cv = tid % vpr, s_gq = tid / vpr;
    const int d_gq = 256 / vpr, d_cv = 256 - d_gq * vpr;
    const int wel = __builtin_amdgcn_readfirstlane(tid) & ~63;   // the wave's first element
    // (upsampled staging: e is (pl, ge, k) = (e / (ge_n*hp), e / hp % ge_n,
    // e % hp), stepped the same way; ge_n is one of two compile-time values)
    const int u_k0 = tid % hp, u_gq0 = tid / hp;
    const int u_dgq = 256 / hp, u_dk = 256 - u_dgq * hp;
    constexpr int GEA = (G + 1) / 2, GEB = G / 2;
    int u_k = u_k0, u_gq = u_gq0;
    // Without upsampling, staged element (pj, g, cv) of the tile (pj = pl*M + j)
    // is read from float offset ((xplane*IH + rbase + g)*IW + cbase + cv*LV).
    // When the planes read are consecutive (xplane = xp0 + pj: no forward
    // multiplier) that is obase + gq*IW + pj*(IH - G)*IW + cv*LV with
    // gq = pj*G + g, and gq*IW steps along with gq.  The bounds checks are
    // three unsigned compares against per-workgroup limits.
    const int xp0 = pg * pbn * M;
    const int pjlim = max(0, min(pbn, a.planes - pg * pbn)) * M;     // planes staged
    const int glo = max(0, -rbase), gcnt = max(0, min(nrows, a.IH - rbase) - glo);
    const int obase = (xp0 * a.IH + rbase) * a.IW + cbase;
    const int pjst = (a.IH - G) * a.IW;
    auto stage = [&](auto lin_t) {
        constexpr bool LIN = decltype(lin_t)::value;
        int s_gqw = s_gq * a.IW;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int pj = s_gq / G;                       // pl*M + j
            const int g = s_gq - pj * G;
            const int cf = s_cv * LV, col = cbase + cf;
            const int gw = s_gqw;
            s_cv += d_cv;
            s_gq += d_gq;
            s_gqw += d_gq * a.IW;
            if (s_cv >= vpr) {
                s_cv -= vpr;
                ++s_gq;
                s_gqw += a.IW;
            }
            const bool ok = pj < pjlim && (unsigned)(g - glo) < (unsigned)gcnt &&
                            (unsigned)col < (unsigned)a.IW;
            int src;                                       // float offset in the tensor read
            if constexpr (LIN) {
                // unsigned: a row or plane outside the tensor may wrap; it is not loaded
                src = (int)((unsigned)obase + (unsigned)gw + (unsigned)pj * (unsigned)pjst +
                            (unsigned)cf);
            } else {
                // the forward with a multiplier: plane p reads input plane p / mult
                const int xplane = (pg * pbn + pj) / a.mult;
                src = (xplane * a.IH + rbase + g) * a.IW + col;
            }
            const int off = ok ? src * 4 : kOutOfRange;
            if constexpr (V4) {
                const float4 v = buf_f4(rx, off);
                sv[i][0] = v.x; sv[i][1] = v.y; sv[i][2] = v.z; sv[i][3] = v.w;
            } else if (i * 256 + wel < nel) {   // the wave's run of 64 holds staged elements
                buf_to_lds<4>(rx, lds + i * 256 + wel, off);
            }
        }
    };
    if constexpr (UPS) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int pl = ge_n == GEA ? u_gq / GEA : u_gq / GEB;
            const int ge = u_gq - pl * ge_n, k = u_k;
            u_k += u_dk;
            u_gq += u_dgq;
            if (u_k >= hp) {
                u_k -= hp;
                ++u_gq;
            }
            const int g = g0 + 2 * ge;
            const int plane = pg * pbn + pl, row = rbase + g, col = cbase + 2 * k + c1;
            const int sr = row >> 1, sc = col >> 1;    // position in dy (row, col are even)
            const bool ok = pl < pbn && plane < a.planes && g < nrows && row >= 0 &&
                            col >= 0 && sr < a.IH && sc < a.IW;
            sv[i][0] = buf_f32(rx, ok ? ((plane * a.IH + sr) * a.IW + sc) * 4 : kOutOfRange);
        }
    } else if (M > 1 || a.mult == 1) {
        stage(std::true_type{});
    } else {
        stage(std::false_type{});
    }
    // 2. into LDS
    u_k = u_k0;
    u_gq = u_gq0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int e = tid + i * 256;
        if (e < pbn * M * KK)
            ldsw[e] = wst[i];
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = tid + i * 256;
        if constexpr (UPS) {
            const int pl = ge_n == GEA ? u_gq / GEA : u_gq / GEB;
            const int ge = u_gq - pl * ge_n, k = u_k;
            u_k += u_dk;
            u_gq += u_dgq;
            if (u_k >= hp) {
                u_k -= hp;
                ++u_gq;
            }
            if (e < pbn * ge_n * hp) {
                float2 *dst = reinterpret_cast<float2 *>(lds + (pl * G + g0 + 2 * ge) * twl);
                dst[k] = c1 ? make_float2(0.0f, sv[i][0]) : make_float2(sv[i][0], 0.0f);
            }
        } else if (V4 && e < nel) {
            lds4[e] = make_float4(sv[i][0], sv[i][1], sv[i][2], sv[i][3]);
        }
    }
    if constexpr (DMA)
        vm_drain();                                    // this wave's tile loads are in LDS
    __syncthreads();

    // 3. per-thread weights and rolling accumulators
    float wr[M][KH][KW];
#pragma unroll
    for (int jm = 0; jm < M; ++jm)
#pragma unroll
        for (int kh = 0; kh < KH; ++kh)
#pragma unroll
            for (int kw = 0; kw < KW; ++kw) {
                const int tap = IG ? (KH - 1 - kh) * KW + (KW - 1 - kw) : kh * KW + kw;
                wr[jm][kh][kw] = ldsw[(pli * M + jm) * KK + tap];
            }
    if constexpr (EPI) {
        epi_finish(ec, ep);
        bval = epi_fold_bias(bval, ec);
#pragma unroll
        for (int jm = 0; jm < M; ++jm)
#pragma unroll
            for (int kh = 0; kh < KH; ++kh)
#pragma unroll
                for (int kw = 0; kw < KW; ++kw)
                    wr[jm][kh][kw] *= ec.inv;
    }
    float acc[R][Q];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < Q; ++j)
            acc[r][j] = bval;
    constexpr int XW = Q + (KW - 1) * D;
    const float *rowbase = lds + pli * M * G * twl + tx * Q + (a.hl - a.pW);
    const int oc = w0 + tx * Q;                        // first output column of this thread
    float *outp = out + my_plane * a.YH * a.YW;
    // Q-wide stores need an 8-byte aligned output (Q = 2) and whole vectors
    // per row (OW % Q == 0 keeps every plane and row start on a vector)
    const bool vec_store = !DEC && (Q > 1) && (a.OW % Q == 0) && a.ost8;
    // the walk, with the activation of the fused epilogue as a constant:
    // one copy of the walk per activation, no branch at the stores
    auto walk = [&](auto act_c) __attribute__((always_inline)) {
    constexpr int ACT = decltype(act_c)::value;
#pragma unroll
    for (int u = 0; u < G; ++u) {
        if (u < nrows) {
            // a staged row of the upsampled dy at an odd position is all zero
            if (!(UPS && ((rbase + u) & 1))) {
#pragma unroll
                for (int jm = 0; jm < M; ++jm) {
                    float xv[XW];
#pragma unroll
                    for (int i = 0; i < XW; ++i)
                        xv[i] = rowbase[(jm * G + u) * twl + i];
#pragma unroll
                    for (int kh = 0; kh < KH; ++kh) {
                        const int m = u - kh * D;
                        if (m >= 0 && m < TH && !(DEC && ((h0 + m) & 1))) {
                            const int slot = m % R;
#pragma unroll
                            for (int kw = 0; kw < KW; ++kw)
#pragma unroll
                                for (int j = 0; j < Q; ++j)
                                    acc[slot][j] =
                                        fmaf(wr[jm][kh][kw], xv[j + kw * D], acc[slot][j]);
                        }
                    }
                }
            }
            const int m = u - (R - 1);
            if (m >= 0) {
                if constexpr (EPI)
                    epi_act_c<ACT>(acc[m % R]);
                const int r = h0 + m;
                float *dst = outp + r * a.OW + oc;
                if constexpr (DEC) {
                    if (pvalid && (r & 1) == 0) {
#pragma unroll
                        for (int j = 0; j < Q; ++j) {
                            const int c = oc + j;
                            if ((c & 1) == 0 && (c >> 1) < a.YW)
                                __builtin_nontemporal_store(
                                    acc[m % R][j], outp + (r >> 1) * a.YW + (c >> 1));
                        }
                    }
                } else if (pvalid) {
                    if (vec_store && oc < a.OW) {
                        store_vec<Q>(dst, acc[m % R]);
                    } else {
#pragma unroll
                        for (int j = 0; j < Q; ++j)
                            if (oc + j < a.OW)
                                __builtin_nontemporal_store(acc[m % R][j], dst + j);
                    }
                }
#pragma unroll
                for (int j = 0; j < Q; ++j)
                    acc[m % R][j] = bval;
            }
        }
    }
    };
    if constexpr (EPI)
        with_act(ep.act, walk);
    else
        walk(std::integral_constant<int, DWCONV_ACT_NONE>());
}

typedef void (*TiledNchwFn)(const float *, const void *, const float *, float *, TiledNchwArgs,
                            EpiArgs);

template <typename WT, int V, int MODE, int S>
constexpr TiledNchwFn tiled_nchw_fn()
{
    if constexpr (S == 1) {
        constexpr TiledNchwVariant t = kTiledNchwVariants[V];
        return &k_tiled_nchw<WT, t.kH, t.kW, t.d, t.q, t.g, (t.v4 != 0), MODE, 1>;
    } else {
        constexpr TiledNchwVariant t = kTiledNchwS2Variants[V];
        if constexpr (MODE == kModeInputGrad && t.v4 != 0)
            return nullptr;             // upsampled staging has no 16-byte form
        else
            return &k_tiled_nchw<WT, t.kH, t.kW, t.d, t.q, t.g, (t.v4 != 0), MODE, 2>;
    }
}

template <int V, int S>
void fill_tiled_nchw(TiledNchwFn (&row)[2][3])
{
    row[0][0] = tiled_nchw_fn<float, V, kModeFwd, S>();
    row[0][1] = tiled_nchw_fn<float, V, kModeInputGrad, S>();
    row[0][2] = tiled_nchw_fn<float, V, kModeFwdEpilogue, S>();
    row[1][0] = tiled_nchw_fn<half_t, V, kModeFwd, S>();
    row[1][1] = tiled_nchw_fn<half_t, V, kModeInputGrad, S>();
    row[1][2] = tiled_nchw_fn<half_t, V, kModeFwdEpilogue, S>();
}

template <int S, int NVAR, int... Vs>
void fill_all_tiled_nchw(TiledNchwFn (&fn)[NVAR][2][3], std::integer_sequence<int, Vs...>)
{
    (fill_tiled_nchw<Vs, S>(fn[Vs]), ...);
}

// the input gradient with a channel multiplier of 2 (stride 1): [variant][f16 weights]
template <int... Vs>
void fill_tiled_nchw_m2(TiledNchwFn (&fn)[kNumTiledNchwVariants][2],
                        std::integer_sequence<int, Vs...>)
{
    ((fn[Vs][0] = &k_tiled_nchw<float, kTiledNchwVariants[Vs].kH, kTiledNchwVariants[Vs].kW,
                                kTiledNchwVariants[Vs].d, kTiledNchwVariants[Vs].q,
                                kTiledNchwVariants[Vs].g, (kTiledNchwVariants[Vs].v4 != 0),
                                kModeInputGrad, 1, 2>,
      fn[Vs][1] = &k_tiled_nchw<half_t, kTiledNchwVariants[Vs].kH, kTiledNchwVariants[Vs].kW,
                                kTiledNchwVariants[Vs].d, kTiledNchwVariants[Vs].q,
                                kTiledNchwVariants[Vs].g, (kTiledNchwVariants[Vs].v4 != 0),
                                kModeInputGrad, 1, 2>),
     ...);
}

struct TiledNchwTable {
    TiledNchwFn fn[kNumTiledNchwVariants][2][3];
    TiledNchwFn fn2[kNumTiledNchwS2Variants][2][3];
    TiledNchwFn fnm[kNumTiledNchwVariants][2];
    TiledNchwTable()
    {
        fill_all_tiled_nchw<1>(fn, std::make_integer_sequence<int, kNumTiledNchwVariants>());
        fill_all_tiled_nchw<2>(fn2, std::make_integer_sequence<int, kNumTiledNchwS2Variants>());
        fill_tiled_nchw_m2(fnm, std::make_integer_sequence<int, kNumTiledNchwVariants>());
    }
};

}  // namespace

int launch_tiled_nchw(const Problem &p, const Plan &pl, const float *in, const void *w,
                      const float *b, float *out, hipStream_t st, const EpiArgs &ep)
{
    static const TiledNchwTable table;
    const int nvar = p.stride == 1 ? kNumTiledNchwVariants : kNumTiledNchwS2Variants;
    if (pl.variant < 0 || pl.variant >= nvar || pl.cl < 16 || pl.cl > 256 ||
        pl.pb != 256 / pl.cl)
        return DWCONV_ERR_BAD_STRATEGY;
    // the input gradient with a multiplier: 2 at stride 1 only
    const bool igm = p.op == DWCONV_OP_INPUT_GRAD && p.mult != 1;
    if (igm && (p.mult != 2 || p.stride != 1))
        return DWCONV_ERR_BAD_STRATEGY;
    const int wt16 = p.wtype == DWCONV_W_F16;
    TiledNchwFn f = igm ? table.fnm[pl.variant][wt16]
                        : p.stride == 1 ? table.fn[pl.variant][wt16][mode_of(p, ep)]
                                        : table.fn2[pl.variant][wt16][mode_of(p, ep)];
    if (!f)
        return DWCONV_ERR_BAD_STRATEGY;
    TiledNchwArgs a;
    if (igm) {
        // walk over the dx planes; each reads its 2 dy planes
        a.planes = p.N * p.C; a.C = p.C; a.mult = 1;
    } else {
        a.planes = p.N * p.mult * p.C; a.C = p.mult * p.C; a.mult = p.mult;
    }
    a.IH = pl.IH; a.IW = pl.IW; a.OH = pl.OH; a.OW = pl.OW;
    a.YH = pl.YH; a.YW = pl.YW;
    a.pH = pl.pH; a.pW = pl.pW; a.hl = pl.hl; a.twl = pl.twl;
    a.txn = pl.cl;
    a.pbn = pl.pb;
    a.nct = pl.nct; a.nwt = pl.nwt; a.nst = pl.nst;
    a.xcd = pl.xcd;
    a.ost8 = (reinterpret_cast<std::uintptr_t>(out) & 7u) == 0;
    return launch_kernel(f, dim3((unsigned)pl.grid), dim3(256), pl.lds_bytes, st, in, w,
                         p.op == DWCONV_OP_FWD ? b : nullptr, out, a, ep);
}


}  // namespace dwconv
