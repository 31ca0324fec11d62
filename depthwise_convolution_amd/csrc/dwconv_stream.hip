// dwconv_stream.hip -- the row-streaming NHWC kernel (stride 1; forward,
// input gradient, forward with the epilogue) for windows with many taps, and
// its launcher.
#include "dwconv_device.h"

namespace dwconv {

namespace {

// ---------------------------------------------------------------------------
// Row-streaming NHWC kernel (windows of many taps: the work is the kH*kW
// FMAs per output, so the design goal is a straight run of FMAs).
//
// Every wave is an independent unit: its 64 lanes are CL consecutive
// channels x 64/CL column groups of PX adjacent output columns, of TH output
// rows of one image (CL < 64 for channel counts that would leave much of a
// 64-channel tile empty).  The wave walks
// the TH + kH - 1 input rows its outputs read, top to bottom.  For each row
// every lane loads its channel at the PX + kW - 1 columns it needs straight
// into registers (a wave load reads CL consecutive channels of 64/CL pixels:
// coalesced runs of 4*CL bytes), NB - 1 rows ahead of the row it computes, and
// folds the row into kH rolling accumulators per column (the row's taps for
// each of the kH output rows it touches); after row u, output row
// u - (kH - 1) is complete and is stored.  No LDS tile and no barrier: the
// columns a lane needs are its own loads, the rows stream through registers.
//
// Zero padding costs nothing: each row is read through a buffer descriptor
// that covers exactly that image row (no bytes for a row outside the image),
// and the lane's column offsets are fixed for the whole walk, so a column
// left of the image (a negative offset) or right of it reads zero in
// hardware.  Stores go through a descriptor of the output row the same way,
// so columns and rows past the output and channels past C are dropped.
//
// Dilation D > 1 is split into its D*D phases: output rows D*i + ar and
// columns D*j + ac read only input rows and columns of one phase, D apart,
// so each phase is a dilation-1 correlation on its sub-grid, and a unit
// works on one phase: kH rolling accumulators and PX + kW - 1 staged
// columns, as for D = 1, instead of (kH-1)*D + 1 and PX + (kW-1)*D.
//
// Workgroups of 4 waves share a channel tile, whose weights they stage once
// through LDS (coalesced); each lane then holds its channel's kH*kW taps
// (reversed for the input gradient) in registers.
// ---------------------------------------------------------------------------
struct StreamArgs {
    int C;                  // channels of both tensors (no multiplier)
    int IH, IW, OH, OW;     // extents of the tensor read and the tensor written
    int pH, pW;             // top / left zero padding of the tensor read
    int nct;                // channel tiles of CL
    int ncg, nrt, nph;      // column groups per sub-grid row, row tiles, phases (D*D)
    int upc;                // units per channel tile: N * nrt * nph * ncg
    int xcd;                // workgroup order: 1 = per-XCD ranges (xcd_tile), 0 = in order
    int mblk;               // forward / input gradient: workgroups of the nct CL-wide tiles
    int tcl, tncg, tupc;    // ... and of the tail tile: its channels per lane group (0 =
                            // none), column groups per sub-grid row, units
};

__device__ __forceinline__ int floor_div(int a, int b)
{
    return (a >= 0 ? a : a - b + 1) / b;
}

// One workgroup's work: 4 units (waves) of the channel tile that starts at
// channel c0, with CL channels x 64/CL column groups per wave; `ncg` column
// blocks per sub-grid row, `upc` units in the tile.  `wl` holds at least
// CL * kH * kW floats.  Every thread of the workgroup calls it (a barrier).
template <typename WT, int KH, int KW, int D, int CL, int PX, int TH, int NB, int MODE>
__device__ __forceinline__ void stream_nhwc_tile(const float *__restrict__ in, const WT *w,
                                                 const float *__restrict__ bias,
                                                 float *__restrict__ out, const StreamArgs &a,
                                                 const EpiArgs &ep, float *wl, int c0,
                                                 int unit, int ncg, int upc)
{
    constexpr bool IG = MODE == kModeInputGrad, EPI = MODE == kModeFwdEpilogue;
    constexpr int KK = KH * KW, G = TH + KH - 1, XW = PX + KW - 1;
    // NB rows in registers: the one in use and NB - 1 in flight
    static_assert(NB >= 2, "at least one row in flight");
    constexpr int NWL = (CL * KK + 255) / 256;
    static_assert(CL == 16 || CL == 32 || CL == 64, "channels per lane group");
    const int lane = threadIdx.x & 63;
    const int ch = lane % CL, cs = lane / CL;          // channel in the tile, column group
    // a wave past the last unit only helps stage the weights
    const bool live = unit < upc;
    const int c = c0 + ch;
    const bool cok = c < a.C;

    // 1. the unit: column block (fastest), phase, row tile, image
    int t = live ? unit : 0;
    const int cg = t % ncg;
    t /= ncg;
    const int ph = t % a.nph;
    t /= a.nph;
    const int rt = t % a.nrt;
    const int n = t / a.nrt;
    const int ar = ph / D, ac = ph - (ph / D) * D;
    // output sub-row i (row D*i + ar) with tap kh reads input row
    // D*i + ar + D*kh - pH = D*(i + kh + tr) + br, 0 <= br < D
    const int tr = floor_div(ar - a.pH, D), br = ar - a.pH - D * tr;
    const int tc = floor_div(ac - a.pW, D), bc = ac - a.pW - D * tc;
    const int i0 = rt * TH, j0 = (cg * (64 / CL) + cs) * PX;

    // the lane's byte offsets within a row: staged column k, output column jj
    int vin[XW], vout[PX];
#pragma unroll
    for (int k = 0; k < XW; ++k)
        vin[k] = cok ? (D * (j0 + tc + k) + bc) * (a.C * 4) + c * 4 : kOutOfRange;
#pragma unroll
    for (int jj = 0; jj < PX; ++jj)
        vout[jj] = cok ? (ac + D * (j0 + jj)) * (a.C * 4) + c * 4 : kOutOfRange;
    const int row_bytes_in = a.IW * a.C * 4, row_bytes_out = a.OW * a.C * 4;
    const float *img_in = in + (long long)n * a.IH * a.IW * a.C;
    float *img_out = out + (long long)n * a.OH * a.OW * a.C;

    float xb[NB][XW];
    auto load_row = [&](int g, float (&dst)[XW]) {
        const int ir = D * (i0 + tr + g) + br;
        const bool ok = live && (unsigned)ir < (unsigned)a.IH;
        const __amdgpu_buffer_rsrc_t r =
            make_rsrc(img_in + (ok ? ir : 0) * a.IW * a.C, ok ? row_bytes_in : 0);
#pragma unroll
        for (int k = 0; k < XW; ++k)
            dst[k] = buf_f32(r, vin[k]);
    };
    // the first rows are on their way while the weights are staged
#pragma unroll
    for (int g = 0; g < NB - 1; ++g)
        load_row(g, xb[g]);

    // 2. the channel tile's weights (CL * KK contiguous values; channels
    // past C read as zero) into LDS, then into registers
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, a.C * KK * (int)sizeof(WT));
    float wst[NWL];
#pragma unroll
    for (int i = 0; i < NWL; ++i)
        wst[i] = buf_w(rw, c0 * KK + (int)threadIdx.x + i * 256, (WT *)nullptr);
    float bv = (!IG && bias) ? buf_f32(make_rsrc(bias, a.C * 4), cok ? c * 4 : kOutOfRange)
                             : 0.0f;
    EpiChan ec{0.0f, 1.0f, 0.0f, 0.0f};
    if constexpr (EPI)
        ec = epi_load(ep, cok ? c : a.C, a.C);
#pragma unroll
    for (int i = 0; i < NWL; ++i)
        wl[threadIdx.x + i * 256] = wst[i];
    __syncthreads();
    if (!live)
        return;                                       // a whole wave; no barrier follows
    float wr[KH][KW];
#pragma unroll
    for (int kh = 0; kh < KH; ++kh)
#pragma unroll
        for (int kw = 0; kw < KW; ++kw)
            wr[kh][kw] = wl[ch * KK + (IG ? (KH - 1 - kh) * KW + (KW - 1 - kw) : kh * KW + kw)];
    if constexpr (EPI) {
        epi_finish(ec, ep);
        epi_fold(wr, bv, ec);
    }

    // 3. walk the rows
    float acc[KH][PX];
#pragma unroll
    for (int r = 0; r < KH; ++r)
#pragma unroll
        for (int jj = 0; jj < PX; ++jj)
            acc[r][jj] = bv;
#pragma unroll
    for (int u = 0; u < G; ++u) {
        if (u + NB - 1 < G)
            load_row(u + NB - 1, xb[(u + NB - 1) % NB]);
        const float(&x)[XW] = xb[u % NB];
        // rows outside the image hold zeros: skip their FMAs (uniform branch)
        const int ir = D * (i0 + tr + u) + br;
        if ((unsigned)ir < (unsigned)a.IH) {
#pragma unroll
            for (int kh = 0; kh < KH; ++kh) {
                const int m = u - kh;                 // output row this tap row feeds
                if (m >= 0 && m < TH) {
#pragma unroll
                    for (int kw = 0; kw < KW; ++kw)
#pragma unroll
                        for (int jj = 0; jj < PX; ++jj)
                            acc[m % KH][jj] = fmaf(wr[kh][kw], x[jj + kw], acc[m % KH][jj]);
                }
            }
        }
        const int m = u - (KH - 1);                   // output row completed by row u
        if (m >= 0) {
            float (&v)[PX] = acc[m % KH];
            if constexpr (EPI)
                epi_act_sel(v, ep.act);
            const int oh = ar + D * (i0 + m);
            const bool ok = oh < a.OH;
            const __amdgpu_buffer_rsrc_t ro =
                make_rsrc(img_out + (ok ? oh : 0) * a.OW * a.C, ok ? row_bytes_out : 0);
#pragma unroll
            for (int jj = 0; jj < PX; ++jj)
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v[jj]), ro,
                                                      vout[jj], 0, kStreamStoreAux);
#pragma unroll
            for (int jj = 0; jj < PX; ++jj)
                v[jj] = bv;
        }
    }
}

// Position of workgroup L of the merged order: the tail workgroups (bt of
// them) are spread among the mblk main ones in proportion, segment j being
// main workgroups [j*mblk/bt, (j+1)*mblk/bt) followed by tail workgroup j.
// Returns the main workgroup index, or -1 - j for tail workgroup j.
__device__ __forceinline__ int merged_block(int L, int mblk, int bt)
{
    if (bt == 0)
        return L;
    auto start = [&](int j) { return (int)((long long)j * mblk / bt) + j; };
    int j = (int)((long long)L * bt / (mblk + bt));
    while (j + 1 < bt && start(j + 1) <= L)
        ++j;
    while (j > 0 && start(j) > L)
        --j;
    const int m_end = (int)((long long)(j + 1) * mblk / bt);   // main workgroups before tail j
    return L - j < m_end ? L - j : -1 - j;
}

// The kernel: the main workgroups (mblk of them) run the nct channel tiles of
// CL channels (channel tile fastest, so the tiles of one place run
// together), the others the narrow tail tile of tcl < CL channels (channels
// nct*CL onwards, the last C % CL of them), whose wider column groups need
// fewer units: a few leftover channels take a few lanes of 4x or 2x fewer
// waves instead of a few lanes of a full 64-lane unit per place.  The tail
// workgroups are interleaved with the main ones in proportion, so that an
// XCD's range holds the tail of the images whose main tiles it runs (the
// tail channels share cache lines with the next pixel's first channels).
template <typename WT, int KH, int KW, int D, int CL, int PX, int TH, int NB, int MODE>
__global__ __launch_bounds__(256) void k_stream_nhwc(const float *__restrict__ in,
                                                     const void *__restrict__ wv,
                                                     const float *__restrict__ bias,
                                                     float *__restrict__ out, StreamArgs a,
                                                     EpiArgs ep)
{
    __shared__ float wl[(CL * KH * KW + 255) / 256 * 256];
    const WT *w = reinterpret_cast<const WT *>(wv);
    // the workgroup's place: per-XCD ranges put the row tiles of an image,
    // which share kH - 1 halo rows, on one XCD and so in one L2
    const int L = a.xcd ? xcd_tile(blockIdx.x, gridDim.x) : (int)blockIdx.x;
    const int blk = merged_block(L, a.mblk, (int)gridDim.x - a.mblk);
    const int wave = (int)(threadIdx.x >> 6);
    if (blk >= 0) {
        const int unit = __builtin_amdgcn_readfirstlane((blk / a.nct) * 4 + wave);
        stream_nhwc_tile<WT, KH, KW, D, CL, PX, TH, NB, MODE>(
            in, w, bias, out, a, ep, wl, (blk % a.nct) * CL, unit, a.ncg, a.upc);
        return;
    }
    const int unit = __builtin_amdgcn_readfirstlane((-1 - blk) * 4 + wave);
    if constexpr (CL > 16) {
        if (a.tcl == 16) {
            stream_nhwc_tile<WT, KH, KW, D, 16, PX, TH, NB, MODE>(
                in, w, bias, out, a, ep, wl, a.nct * CL, unit, a.tncg, a.tupc);
            return;
        }
    }
    if constexpr (CL > 32) {
        if (a.tcl == 32)
            stream_nhwc_tile<WT, KH, KW, D, 32, PX, TH, NB, MODE>(
                in, w, bias, out, a, ep, wl, a.nct * CL, unit, a.tncg, a.tupc);
    }
}

// ---------------------------------------------------------------------------
// Row-streaming NCHW kernel: the same walk with lanes along the columns of
// plane rows.  A wave holds PPW planes x LPR lanes per plane row, each lane
// PX adjacent output columns of its plane (narrow planes are packed several
// to a wave; lanes past PPW*LPR idle).  The columns a lane needs overlap its
// neighbours', so each input row is staged once per wave: NL coalesced
// loads of 64 consecutive staged elements (PPW plane rows of LPR*PX +
// kW - 1 columns, columns outside the plane read as zero through an
// out-of-range offset) go into a ring of three row slots in the wave's own
// LDS, and each lane reads its PX + kW - 1 taps from there.  A row is
// loaded into registers several rows ahead (a staged row costs a lane only
// NL registers) and written to one of two LDS slots just before it is read.
// The slots are private to the wave and the wave's LDS operations run in
// order, so no barrier is needed.  A row's
// offset is the wave-uniform soffset of the loads, and a row outside the
// planes reads through a descriptor of no bytes.  A lane's weights are its
// channel's (a wave touches PPW channels: a few cache lines per load).
// Dilation is split into phases as in NHWC: the staged columns are one
// phase's, D apart.
// ---------------------------------------------------------------------------
struct StreamNchwArgs {
    int C, planes;          // channels; planes (n, c) of both tensors
    int IH, IW, OH, OW;     // plane extents of the tensor read and the tensor written
    int pH, pW;             // top / left zero padding of the tensor read
    int lpr, ppw, pitch;    // lanes per plane row, planes per wave, staged columns per plane
    int lpitch;             // LDS floats per staged plane row (pitch rounded up to lpr mod 32)
    int ncb, nrt, nph;      // column blocks (waves across a sub-grid row), row tiles, phase
                            // units (phases / rpu)
    int units;              // waves: plane groups * phase units * row tiles * column blocks
    int rpu;                // weight gradient: row phases a unit walks in turn (1 or D)
};

__device__ __forceinline__ float buf_f32_s(__amdgpu_buffer_rsrc_t r, int off, int soff)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0));
}

template <typename WT, int KH, int KW, int D, int PX, int TH, int NL, int NB, int MODE>
__global__ __launch_bounds__(256) void k_stream_nchw(const float *__restrict__ in,
                                                     const void *__restrict__ wv,
                                                     const float *__restrict__ bias,
                                                     float *__restrict__ out, StreamNchwArgs a,
                                                     EpiArgs ep)
{
    constexpr bool IG = MODE == kModeInputGrad, EPI = MODE == kModeFwdEpilogue;
    constexpr int KK = KH * KW, G = TH + KH - 1, XW = PX + KW - 1;
    // NB rows in registers (NL values per lane each: the one being written to
    // LDS and NB - 1 in flight), two LDS slots used in turn
    static_assert(NB >= 2, "at least one row in flight");
    // a row slot: up to kStreamNchwSlot floats of staged plane rows, then a
    // 64-float area the staging lanes past the last plane write to
    constexpr int SLOT = kStreamNchwSlot + 64;
    __shared__ float ring[4][2][SLOT];
    const WT *w = reinterpret_cast<const WT *>(wv);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int unit = __builtin_amdgcn_readfirstlane((int)blockIdx.x * 4 + wave);
    if (unit >= a.units)
        return;                                       // a whole wave; this kernel has no barrier
    // the unit: column block (fastest), row tile, phase, plane group
    int t = unit;
    const int cb = t % a.ncb;
    t /= a.ncb;
    const int rt = t % a.nrt;
    t /= a.nrt;
    const int ph = t % a.nph;
    const int pg = t / a.nph;
    const int ar = ph / D, ac = ph - (ph / D) * D;
    const int tr = floor_div(ar - a.pH, D), br = ar - a.pH - D * tr;
    const int tc = floor_div(ac - a.pW, D), bc = ac - a.pW - D * tc;
    const int i0 = rt * TH, jb = cb * a.lpr * PX;    // first sub-column of the column block

    // staging: element e = i*64 + lane of a row is column k = e % pitch of
    // plane slot e / pitch, sub-grid column jb + tc + k; it goes to LDS float
    // (e / pitch) * lpitch + k of the row's slot.  With lpitch = lpr (mod 32)
    // the float a lane reads (plane slot ps, column cgl*PX + k) sits at
    // lane + k (mod 32) for PX = 1: the 32 lanes of a half-wave read 32
    // different banks.
    int src[NL], dst[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int e = i * 64 + lane, pse = e / a.pitch, k = e - pse * a.pitch;
        const int plane = pg * a.ppw + pse, col = D * (jb + tc + k) + bc;
        const bool ok = pse < a.ppw && plane < a.planes && (unsigned)col < (unsigned)a.IW;
        src[i] = ok ? (plane * a.IH * a.IW + col) * 4 : kOutOfRange;
        dst[i] = pse < a.ppw ? pse * a.lpitch + k : kStreamNchwSlot + lane;
    }
    const int in_bytes = a.planes * a.IH * a.IW * 4, out_bytes = a.planes * a.OH * a.OW * 4;
    float (*slots)[SLOT] = ring[wave];
    float st[NB][NL];                                 // a staged row between load and LDS write
    auto load_row = [&](int g, float (&dst)[NL]) {
        const int ir = D * (i0 + tr + g) + br;
        const bool ok = (unsigned)ir < (unsigned)a.IH;
        const __amdgpu_buffer_rsrc_t r = make_rsrc(in, ok ? in_bytes : 0);
        const int soff = ok ? ir * a.IW * 4 : 0;
#pragma unroll
        for (int i = 0; i < NL; ++i)
            dst[i] = buf_f32_s(r, src[i], soff);
    };
#pragma unroll
    for (int g = 0; g < NB - 1; ++g)
        load_row(g, st[g]);

    // the lane's plane and columns
    const int ps = lane / a.lpr, cgl = lane - ps * a.lpr;
    const int plane = pg * a.ppw + ps;
    const bool pok = ps < a.ppw && plane < a.planes;
    const int c = pok ? plane % a.C : 0;
    const int rd = min(ps, a.ppw - 1) * a.lpitch + cgl * PX;   // the lane's first staged column
    int vout[PX];
#pragma unroll
    for (int jj = 0; jj < PX; ++jj) {
        const int oc = ac + D * (jb + cgl * PX + jj);
        vout[jj] = pok && oc < a.OW ? (plane * a.OH * a.OW + oc) * 4 : kOutOfRange;
    }
    // weights (reversed taps for the input gradient) and bias of the lane's channel
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, a.C * KK * (int)sizeof(WT));
    // one per-lane base, the tap a constant on top (folded into the loads'
    // immediate offsets; an out-of-range base stays out of range)
    const int wb = pok ? c * KK : kOutOfRange / 4;
    float wr[KH][KW];
#pragma unroll
    for (int kh = 0; kh < KH; ++kh)
#pragma unroll
        for (int kw = 0; kw < KW; ++kw) {
            const int tap = IG ? (KH - 1 - kh) * KW + (KW - 1 - kw) : kh * KW + kw;
            wr[kh][kw] = buf_w(rw, wb + tap, (WT *)nullptr);
        }
    float bv = (!IG && bias) ? buf_f32(make_rsrc(bias, a.C * 4), pok ? c * 4 : kOutOfRange)
                             : 0.0f;
    EpiChan ec{0.0f, 1.0f, 0.0f, 0.0f};
    if constexpr (EPI) {
        ec = epi_load(ep, pok ? c : a.C, a.C);
        epi_finish(ec, ep);
        epi_fold(wr, bv, ec);
    }
    float acc[KH][PX];
#pragma unroll
    for (int r = 0; r < KH; ++r)
#pragma unroll
        for (int jj = 0; jj < PX; ++jj)
            acc[r][jj] = bv;
#pragma unroll
    for (int u = 0; u < G; ++u) {
        // row u into its slot, row u + 2 on its way
#pragma unroll
        for (int i = 0; i < NL; ++i)
            slots[u % 2][dst[i]] = st[u % NB][i];
        if (u + NB - 1 < G)
            load_row(u + NB - 1, st[(u + NB - 1) % NB]);
        // keep the loads NB - 1 rows ahead: the scheduler would otherwise
        // sink them towards their use to save registers
        __builtin_amdgcn_sched_barrier(0);
        float x[XW];
#pragma unroll
        for (int k = 0; k < XW; ++k)
            x[k] = slots[u % 2][rd + k];
        {
#pragma unroll
            for (int kh = 0; kh < KH; ++kh) {
                const int m = u - kh;
                if (m >= 0 && m < TH) {
#pragma unroll
                    for (int kw = 0; kw < KW; ++kw)
#pragma unroll
                        for (int jj = 0; jj < PX; ++jj)
                            acc[m % KH][jj] = fmaf(wr[kh][kw], x[jj + kw], acc[m % KH][jj]);
                }
            }
        }
        const int m = u - (KH - 1);
        if (m >= 0) {
            float (&v)[PX] = acc[m % KH];
            if constexpr (EPI)
                epi_act_sel(v, ep.act);
            const int oh = ar + D * (i0 + m);
            const bool ok = oh < a.OH;
            const __amdgpu_buffer_rsrc_t ro = make_rsrc(out, ok ? out_bytes : 0);
            const int soff = ok ? oh * a.OW * 4 : 0;
#pragma unroll
            for (int jj = 0; jj < PX; ++jj)
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v[jj]), ro,
                                                      vout[jj], soff, kStreamNchwStoreAux);
#pragma unroll
            for (int jj = 0; jj < PX; ++jj)
                v[jj] = bv;
        }
    }
}

// ---------------------------------------------------------------------------
// Plane-per-lane NCHW walk (stride 1): the NHWC walk's lanes on NCHW data.
// A wave takes 16 consecutive planes (n, c) x 4 lane groups, TH output rows
// of one row phase, and a block of 4*PX output columns; lane group cg is
// column phase cg % D and the PX adjacent sub-grid columns (cg / D)*PX ..
// of that phase.  Each lane then runs the NHWC walk: kH rolling accumulators
// per column, PX + kW - 1 staged columns per input row, kH*kW*PX FMAs per
// row.  Waves are independent units (no barrier).
//
// The transposes go through the wave's own LDS.  A plane's row segment is
// a contiguous run in NCHW, so the wave loads each input row of its 16
// planes as consecutive (plane, column) elements over the in-image columns
// of its window only: coalesced runs, loaded NB rows before the row is
// staged.  The row goes to one of three LDS slots (plane p at p*SP, whose
// columns outside the image were zeroed once) two rows before its FMAs, and
// its taps are read into registers one row before them; SP (4 mod 8) puts
// the 64 lanes' taps in 64 different banks.  Completed output rows go the
// other way: each lane writes its PX columns into a row buffer (plane p at
// p*4*PX), and the wave reads it back in (plane, column) order and stores
// contiguous runs.  A wave's LDS operations run in order, so no barrier is
// needed.
//
// Zero padding: rows outside the image are neither staged nor folded in (a
// wave-uniform branch).  Stores of rows past OH, columns past OW and planes
// past the last go through out-of-range offsets and are dropped.
// ---------------------------------------------------------------------------
struct StreamPlanesArgs {
    int C, planes;          // channels; planes (n, c) of both tensors
    int IH, IW, OH, OW;     // plane extents of the tensor read and the tensor written
    int pH, pW;             // top / left zero padding of the tensor read
    int ncb, nrt;           // column blocks of 4*PX output columns, row tiles per phase
    int units;              // waves: plane groups * D row phases * nrt * ncb
    int xcd;                // 1: per-XCD ranges of workgroups (xcd_tile)
};

// True when lane l = 4*ps + cg reading staged column D*k + (cg % D) +
// D*(cg / D)*PX of plane ps (plane pitch SP) hits 64 different banks for
// every tap k.
constexpr bool planes_pitch_ok(int sp, int d, int px, int xw)
{
    for (int k = 0; k < xw; ++k) {
        unsigned long long seen = 0;
        for (int l = 0; l < 64; ++l) {
            const int cg = l % 4, ps = l / 4;
            const int a = ps * sp + cg % d + d * (cg / d) * px + d * k;
            const unsigned long long bit = 1ull << (a % 64);
            if (seen & bit)
                return false;
            seen |= bit;
        }
    }
    return true;
}

template <typename WT, int KH, int KW, int D, int PX, int TH, int NL, int NB, int MODE>
__global__ __launch_bounds__(256) void k_stream_nchw_planes(const float *__restrict__ in,
                                                            const void *__restrict__ wv,
                                                            const float *__restrict__ bias,
                                                            float *__restrict__ out,
                                                            StreamPlanesArgs a, EpiArgs ep)
{
    constexpr bool IG = MODE == kModeInputGrad, EPI = MODE == kModeFwdEpilogue;
    constexpr int KK = KH * KW, G = TH + KH - 1, XW = PX + KW - 1;
    static_assert(4 % D == 0, "the 4 lane groups split into D column phases");
    static_assert(NB >= 2, "at least one row in flight");
    constexpr int BW = 4 * PX;                        // output columns of the block
    constexpr int WS = BW + D * (KW - 1);             // staged columns
    constexpr int SP = (WS + 3) / 8 * 8 + 4;          // LDS floats per staged plane row
    static_assert(planes_pitch_ok(SP, D, PX, XW), "tap reads free of bank conflicts");
    constexpr int SLOT = 16 * SP + 64;                // + where unused staging lanes write
    constexpr int NSLOT = 3;                          // row u read, u + 1 in LDS, u + 2 written
    static_assert(NL >= 1 && 64 * NL <= 16 * WS + 63, "staging loads per lane and row");
    constexpr int OB = 16 * BW;                       // row buffer: plane p at p*BW
    static_assert(OB % 64 == 0, "the row buffer is whole wave loads");
    __shared__ float lds[4][NSLOT * SLOT + OB];
    const WT *w = reinterpret_cast<const WT *>(wv);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int blk = a.xcd ? xcd_tile(blockIdx.x, gridDim.x) : (int)blockIdx.x;
    const int unit = __builtin_amdgcn_readfirstlane(blk * 4 + wave);
    if (unit >= a.units)
        return;                                       // a whole wave; this kernel has no barrier
    float *slots = lds[wave], *obuf = lds[wave] + NSLOT * SLOT;

    // the unit: column block (fastest), row tile, row phase, plane group
    int t = unit;
    const int cb = t % a.ncb;
    t /= a.ncb;
    const int rt = t % a.nrt;
    t /= a.nrt;
    const int ar = t % D;
    const int p0 = (t / D) * 16;                      // first plane
    const int tr = floor_div(ar - a.pH, D), br = ar - a.pH - D * tr;
    const int i0 = rt * TH, oc0 = cb * BW, s0 = oc0 - a.pW;
    // in-image columns of the window: [lo, hi), staged at lo - s0 ..
    const int lo = max(s0, 0), hi = min(s0 + WS, a.IW);
    const int cnt = max(hi - lo, 0), nel = 16 * cnt;
    const int in_bytes = a.planes * a.IH * a.IW * 4, out_bytes = a.planes * a.OH * a.OW * 4;

    // staging: element e = lane + 64*i is in-image column lo + e % cnt of
    // plane e / cnt; it goes to LDS float (e / cnt)*SP + lo - s0 + e % cnt
    // (the plan makes 64*NL >= 16*cnt; elements past that read zero and go
    // to the slot's spare floats)
    int src[NL], dst[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int e = lane + 64 * i, sp = cnt ? e / cnt : 0, col = e - sp * cnt;
        const bool ok = e < nel && p0 + sp < a.planes;
        src[i] = ok ? ((p0 + sp) * a.IH * a.IW + lo + col) * 4 : kOutOfRange;
        dst[i] = e < nel ? sp * SP + lo - s0 + col : 16 * SP + lane;
    }
    float st[NB][NL];
    auto row_ok = [&](int g) {
        return (unsigned)(D * (i0 + tr + g) + br) < (unsigned)a.IH;
    };
    auto load_row = [&](int g, float (&v)[NL]) {
        const int ir = D * (i0 + tr + g) + br;
        const bool ok = (unsigned)ir < (unsigned)a.IH;
        const __amdgpu_buffer_rsrc_t r = make_rsrc(in, ok ? in_bytes : 0);
        const int soff = ok ? ir * a.IW * 4 : 0;
#pragma unroll
        for (int i = 0; i < NL; ++i)
            v[i] = buf_f32_s(r, src[i], soff);
    };
    auto stage_row = [&](int g, const float (&v)[NL]) {
        float *sl = slots + (g % 3) * SLOT;
#pragma unroll
        for (int i = 0; i < NL; ++i)
            sl[dst[i]] = v[i];
    };
#pragma unroll
    for (int g = 0; g < NB && g < G; ++g)
        load_row(g, st[g]);

    // the lane's plane, channel and columns
    const int ps = lane >> 2, cg = lane & 3;
    const int plane = p0 + ps;
    const bool pok = plane < a.planes;
    const int c = pok ? plane % a.C : 0;
    const int ac = cg % D, gq = cg / D;
    const int rb = ps * SP + ac + D * gq * PX;        // staged column of tap 0
    const int ob = ps * BW + ac + D * gq * PX;        // row-buffer float of column 0
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, a.C * KK * (int)sizeof(WT));
    const int wb = pok ? c * KK : kOutOfRange / 4;
    float wr[KH][KW];
#pragma unroll
    for (int kh = 0; kh < KH; ++kh)
#pragma unroll
        for (int kw = 0; kw < KW; ++kw) {
            const int tap = IG ? (KH - 1 - kh) * KW + (KW - 1 - kw) : kh * KW + kw;
            wr[kh][kw] = buf_w(rw, wb + tap, (WT *)nullptr);
        }
    float bv = (!IG && bias) ? buf_f32(make_rsrc(bias, a.C * 4), pok ? c * 4 : kOutOfRange)
                             : 0.0f;
    EpiChan ec{0.0f, 1.0f, 0.0f, 0.0f};
    if constexpr (EPI) {
        ec = epi_load(ep, pok ? c : a.C, a.C);
        epi_finish(ec, ep);
        epi_fold(wr, bv, ec);
    }
    // the lane's share of a row-buffer store: float f = lane + 64*i is
    // column f % BW of plane f / BW
    constexpr int NST = OB / 64;
    int sof[NST];
#pragma unroll
    for (int i = 0; i < NST; ++i) {
        const int f = lane + 64 * i, sp = f / BW, oc = oc0 + f - sp * BW;
        sof[i] = p0 + sp < a.planes && oc < a.OW ? ((p0 + sp) * a.OH * a.OW + oc) * 4
                                                : kOutOfRange;
    }

    // zero the slots once: columns outside the image are never written
    for (int i = lane; i < NSLOT * SLOT; i += 64)
        slots[i] = 0.0f;
    float acc[KH][PX];
#pragma unroll
    for (int r = 0; r < KH; ++r)
#pragma unroll
        for (int jj = 0; jj < PX; ++jj)
            acc[r][jj] = bv;
    // a row's taps are read from LDS one row before its FMAs, so their
    // latency hides behind the FMAs of the row before
    float xr[2][XW];
    auto read_taps = [&](int g, float (&x)[XW]) {
        const float *sl = slots + (g % 3) * SLOT + rb;
#pragma unroll
        for (int k = 0; k < XW; ++k)
            x[k] = sl[D * k];
    };
    // row g's registers are st[g % NB]: row g + NB loads as soon as row g is
    // staged, NB rows before it is staged itself
#pragma unroll
    for (int g = 0; g < 2 && g < G; ++g) {
        if (row_ok(g))
            stage_row(g, st[g % NB]);
        if (g + NB < G)
            load_row(g + NB, st[g % NB]);
    }
    if (row_ok(0))
        read_taps(0, xr[0]);
#pragma unroll
    for (int u = 0; u < G; ++u) {
        // row u + 2 into its slot and row u + 2 + NB into its registers; row
        // u + 1's taps on their way
        if (u + 2 < G && row_ok(u + 2))
            stage_row(u + 2, st[(u + 2) % NB]);
        if (u + 2 + NB < G)
            load_row(u + 2 + NB, st[(u + 2) % NB]);
        if (u + 1 < G && row_ok(u + 1))
            read_taps(u + 1, xr[(u + 1) % 2]);
        __builtin_amdgcn_sched_barrier(0);
        if (row_ok(u)) {
            const float (&x)[XW] = xr[u % 2];
#pragma unroll
            for (int kh = 0; kh < KH; ++kh) {
                const int m = u - kh;
                if (m >= 0 && m < TH) {
#pragma unroll
                    for (int kw = 0; kw < KW; ++kw)
#pragma unroll
                        for (int jj = 0; jj < PX; ++jj)
                            acc[m % KH][jj] = fmaf(wr[kh][kw], x[jj + kw], acc[m % KH][jj]);
                }
            }
        }
        const int m = u - (KH - 1);                   // output row completed by row u
        if (m >= 0) {
            float (&v)[PX] = acc[m % KH];
            if constexpr (EPI)
                epi_act_sel(v, ep.act);
#pragma unroll
            for (int jj = 0; jj < PX; ++jj)
                obuf[ob + D * jj] = v[jj];
#pragma unroll
            for (int jj = 0; jj < PX; ++jj)
                v[jj] = bv;
            const int oh = ar + D * (i0 + m);
            const bool ok = oh < a.OH;
            const __amdgpu_buffer_rsrc_t ro = make_rsrc(out, ok ? out_bytes : 0);
            const int soff = ok ? oh * a.OW * 4 : 0;
#pragma unroll
            for (int i = 0; i < NST; ++i)
                __builtin_amdgcn_raw_buffer_store_b32(
                    __builtin_bit_cast(unsigned, obuf[lane + 64 * i]), ro, sof[i], soff,
                    kStreamNchwStoreAux);
        }
    }
}

// ---------------------------------------------------------------------------
// Row-streaming NHWC weight gradient (stage 1): the NHWC walk's waves (64
// channels, one per lane, x PX output columns x TH output rows of one
// dilation phase) with the roles of the operands changed (LeanMlir
// "Depthwise" weight-VJP: dW[c,kh,kw] is the sum over positions of x at the
// tap times dy, db[c] the sum of dy).  A lane loads its channel's x row (PX
// + kW - 1 columns) and dy row (PX columns) straight into registers, rows
// ahead of use; it keeps the dy rows of the last kH output rows, and each x
// row u meets dy rows u - kh for its kH*kW tap sums (PX FMAs per tap).  The
// workgroup's four waves add their sums in LDS in wave order, and the
// workgroup writes them as one contiguous run of its chunk of the partial
// sums part[chunk][c][tap]; the fixed-order reduction kernel adds the
// chunks.
// ---------------------------------------------------------------------------
// One workgroup's work: 4 units of the channel tile starting at channel c0,
// CL channels x 64/CL column groups per wave (ncg column blocks per
// sub-grid row, upc units), summed into chunk `chunk` of the partial sums;
// `zstep` > 0 (a tail tile) also writes zeros for its channels into chunks
// chunk + zstep, chunk + 2 zstep, ... below nchunks, which hold no units of
// that tile.  Every thread of the workgroup calls it (barriers).
template <int KH, int KW, int D, int PX, int TH, int NB, int CL>
__device__ __forceinline__ void wgrad_stream_nhwc_tile(const float *__restrict__ x,
                                                       const float *__restrict__ dy,
                                                       float *__restrict__ part,
                                                       const StreamArgs &a, float *red, int c0,
                                                       int unit, int ncg, int upc, int chunk,
                                                       int zstep, int nchunks)
{
    constexpr int KK = KH * KW, G = TH + KH - 1, XW = PX + KW - 1, KP = KK + 1;
    constexpr int RG = KH + NB - 1;                   // dy rows in registers
    constexpr int LP = 65;                            // LDS pitch of a sum row
    static_assert(NB >= 2, "at least one row in flight");
    static_assert(CL == 16 || CL == 32 || CL == 64, "channels per lane group");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ch = lane % CL, cs = lane / CL;          // channel in the tile, column group
    // a wave past the last unit adds zeros
    const bool live = unit < upc;
    const int c = c0 + ch;
    const bool cok = c < a.C;
    // the unit: column block (fastest), phase, row tile, image
    int t = live ? unit : 0;
    const int cg = t % ncg;
    t /= ncg;
    const int ph = t % a.nph;
    t /= a.nph;
    const int rt = t % a.nrt;
    const int n = t / a.nrt;
    const int ar = ph / D, ac = ph - (ph / D) * D;
    const int tr = floor_div(ar - a.pH, D), br = ar - a.pH - D * tr;
    const int tc = floor_div(ac - a.pW, D), bc = ac - a.pW - D * tc;
    const int i0 = rt * TH, j0 = (cg * (64 / CL) + cs) * PX;
    int vin[XW], vg[PX];
#pragma unroll
    for (int k = 0; k < XW; ++k)
        vin[k] = cok ? (D * (j0 + tc + k) + bc) * (a.C * 4) + c * 4 : kOutOfRange;
#pragma unroll
    for (int jj = 0; jj < PX; ++jj)
        vg[jj] = cok ? (ac + D * (j0 + jj)) * (a.C * 4) + c * 4 : kOutOfRange;
    const int row_x = a.IW * a.C * 4, row_g = a.OW * a.C * 4;
    const float *img_x = x + (long long)n * a.IH * a.IW * a.C;
    const float *img_g = dy + (long long)n * a.OH * a.OW * a.C;
    float xb[NB][XW], gb[RG][PX];
    auto load_x = [&](int g, float (&d)[XW]) {
        const int ir = D * (i0 + tr + g) + br;
        const bool ok = live && (unsigned)ir < (unsigned)a.IH;
        const __amdgpu_buffer_rsrc_t r =
            make_rsrc(img_x + (ok ? ir : 0) * a.IW * a.C, ok ? row_x : 0);
#pragma unroll
        for (int k = 0; k < XW; ++k)
            d[k] = buf_f32(r, vin[k]);
    };
    auto load_g = [&](int m, float (&d)[PX]) {
        const int oh = ar + D * (i0 + m);
        const bool ok = live && m < TH && oh < a.OH;
        const __amdgpu_buffer_rsrc_t r =
            make_rsrc(img_g + (ok ? oh : 0) * a.OW * a.C, ok ? row_g : 0);
#pragma unroll
        for (int jj = 0; jj < PX; ++jj)
            d[jj] = buf_f32(r, vg[jj]);
    };
#pragma unroll
    for (int g = 0; g < NB - 1; ++g) {
        load_x(g, xb[g]);
        if (g < TH)
            load_g(g, gb[g % RG]);
    }
    float acc[KP];
#pragma unroll
    for (int q = 0; q < KP; ++q)
        acc[q] = 0.0f;
#pragma unroll
    for (int u = 0; u < G; ++u) {
        // x row u + NB - 1 and dy row u + NB - 1 on their way
        if (u + NB - 1 < G) {
            load_x(u + NB - 1, xb[(u + NB - 1) % NB]);
            if (u + NB - 1 < TH)
                load_g(u + NB - 1, gb[(u + NB - 1) % RG]);
        }
        if (u < TH) {
#pragma unroll
            for (int jj = 0; jj < PX; ++jj)
                acc[KK] += gb[u % RG][jj];            // the bias sum
        }
        const int ir = D * (i0 + tr + u) + br;
        if ((unsigned)ir < (unsigned)a.IH) {
            const float(&xv)[XW] = xb[u % NB];
#pragma unroll
            for (int kh = 0; kh < KH; ++kh) {
                const int m = u - kh;                 // dy row this x row meets at tap row kh
                if (m >= 0 && m < TH) {
#pragma unroll
                    for (int jj = 0; jj < PX; ++jj)
#pragma unroll
                        for (int kw = 0; kw < KW; ++kw)
                            acc[kh * KW + kw] =
                                fmaf(xv[jj + kw], gb[m % RG][jj], acc[kh * KW + kw]);
                }
            }
        }
    }
    // waves 1-3 park their sums; wave 0 adds the four in wave order and
    // parks the total in wave 1's rows
    if (wave > 0) {
#pragma unroll
        for (int q = 0; q < KP; ++q)
            red[(wave - 1) * KP * LP + q * LP + lane] = acc[q];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int q = 0; q < KP; ++q)
            red[q * LP + lane] = ((acc[q] + red[q * LP + lane]) + red[KP * LP + q * LP + lane]) +
                                 red[2 * KP * LP + q * LP + lane];
    }
    __syncthreads();
    // the chunk's channels c0 .. c0 + nc - 1 are KP * nc consecutive floats
    // of part; a channel's 64 / CL column groups are added in group order
    const int nc = min(CL, a.C - c0);
    float *dst = part + ((long long)chunk * a.C + c0) * KP;
    for (int e = threadIdx.x; e < nc * KP; e += 256) {
        const int cl = e / KP, q = e - cl * KP;
        float v = red[q * LP + cl];
#pragma unroll
        for (int g = 1; g < 64 / CL; ++g)
            v += red[q * LP + g * CL + cl];
        dst[e] = v;
    }
    if (zstep > 0) {
        for (int z = chunk + zstep; z < nchunks; z += zstep) {
            float *zd = part + ((long long)z * a.C + c0) * KP;
            for (int e = threadIdx.x; e < nc * KP; e += 256)
                zd[e] = 0.0f;
        }
    }
}

// The kernel: main workgroups (the nct 64-channel tiles, chunk = the
// workgroup's unit group) interleaved in proportion with those of the tail
// tile of tcl < 64 channels, as in the forward walk.
template <int KH, int KW, int D, int PX, int TH, int NB>
__global__ __launch_bounds__(256) void k_wgrad_stream_nhwc(const float *__restrict__ x,
                                                           const float *__restrict__ dy,
                                                           float *__restrict__ part,
                                                           StreamArgs a)
{
    __shared__ float red[3 * (KH * KW + 1) * 65];
    const int L = a.xcd ? xcd_tile(blockIdx.x, gridDim.x) : (int)blockIdx.x;
    const int bt = (int)gridDim.x - a.mblk;
    const int blk = merged_block(L, a.mblk, bt);
    const int wave = (int)(threadIdx.x >> 6);
    if (blk >= 0) {
        const int unit = __builtin_amdgcn_readfirstlane((blk / a.nct) * 4 + wave);
        wgrad_stream_nhwc_tile<KH, KW, D, PX, TH, NB, 64>(x, dy, part, a, red, (blk % a.nct) * 64,
                                                          unit, a.ncg, a.upc, blk / a.nct, 0, 0);
        return;
    }
    const int j = -1 - blk;
    const int unit = __builtin_amdgcn_readfirstlane(j * 4 + wave);
    const int tchunks = (a.upc + 3) / 4;              // chunks of a full tile's units
    if (a.tcl == 16)
        wgrad_stream_nhwc_tile<KH, KW, D, PX, TH, NB, 16>(x, dy, part, a, red, a.nct * 64, unit,
                                                          a.tncg, a.tupc, j, bt, tchunks);
    else if (a.tcl == 32)
        wgrad_stream_nhwc_tile<KH, KW, D, PX, TH, NB, 32>(x, dy, part, a, red, a.nct * 64, unit,
                                                          a.tncg, a.tupc, j, bt, tchunks);
}

// ---------------------------------------------------------------------------
// Row-streaming NCHW weight gradient (stage 1): the lanes and the staged x
// rows of the NCHW walk above, with the roles of the operands changed
// (LeanMlir "Depthwise" weight-VJP: dW[c,kh,kw] is the sum over positions
// of x at the tap times dy).  A lane (one column of one plane, of one
// dilation phase) keeps its last kH dy values in registers; each x row u
// read from LDS meets dy rows u - kh, kh < kH, and is added into the lane's
// kH*kW tap sums (and dy into the bias sum).  At the end the LPR lanes of
// each plane are added in lane order through the wave's LDS, and the plane's
// KK + 1 sums are written as a chunk of the partial sums part[chunk][c][tap], chunk = the unit's (image, phase, row tile,
// column block); the fixed-order reduction kernel adds the chunks.
// ---------------------------------------------------------------------------
template <int KH, int KW, int D, int TH, int NL, int NB, int RPU>
__global__ __launch_bounds__(256) void k_wgrad_stream_nchw(const float *__restrict__ x,
                                                           const float *__restrict__ dy,
                                                           float *__restrict__ part,
                                                           StreamNchwArgs a)
{
    constexpr int KK = KH * KW, G = TH + KH - 1, XW = KW;     // one column per lane
    constexpr int RG = KH + NB - 1;                            // dy values in registers
    constexpr int SLOT = kStreamNchwSlot + 64;
    static_assert(NB >= 2, "at least one row in flight");
    __shared__ float ring[4][2][SLOT];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int unit = __builtin_amdgcn_readfirstlane((int)blockIdx.x * 4 + wave);
    if (unit >= a.units)
        return;                                       // a whole wave; this kernel has no barrier
    // the unit: column block, row tile, phase unit pu, plane group.  A phase
    // unit is one phase (rpu = 1) or a column phase whose D row phases the
    // unit walks in turn into the same tap sums (rpu = D: a phase is a set of
    // positions, and the sums run over all of them)
    int t = unit;
    const int cb = t % a.ncb;
    t /= a.ncb;
    const int rt = t % a.nrt;
    t /= a.nrt;
    const int pu = t % a.nph;
    const int pg = t / a.nph;
    static_assert(RPU == 1 || RPU == D, "one row phase or all of them");
    constexpr int rpu = RPU;
    const int ar0 = rpu == 1 ? pu / D : 0, ac = rpu == 1 ? pu - (pu / D) * D : pu;
    const int tc = floor_div(ac - a.pW, D), bc = ac - a.pW - D * tc;
    const int i0 = rt * TH, jb = cb * a.lpr;

    // x staging as in the NCHW walk (element e of a row -> plane slot e / pitch,
    // column e % pitch; LDS at a bank-spreading pitch)
    int src[NL], dst[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int e = i * 64 + lane, pse = e / a.pitch, k = e - pse * a.pitch;
        const int plane = pg * a.ppw + pse, col = D * (jb + tc + k) + bc;
        const bool ok = pse < a.ppw && plane < a.planes && (unsigned)col < (unsigned)a.IW;
        src[i] = ok ? (plane * a.IH * a.IW + col) * 4 : kOutOfRange;
        dst[i] = pse < a.ppw ? pse * a.lpitch + k : kStreamNchwSlot + lane;
    }
    const int x_bytes = a.planes * a.IH * a.IW * 4, dy_bytes = a.planes * a.OH * a.OW * 4;
    float (*slots)[SLOT] = ring[wave];
    // the lane's plane, its dy column (row phases share it)
    const int ps = lane / a.lpr, cgl = lane - ps * a.lpr;
    const int plane = pg * a.ppw + ps;
    const bool pok = ps < a.ppw && plane < a.planes;
    const int rd = min(ps, a.ppw - 1) * a.lpitch + cgl;
    const int oc = ac + D * (jb + cgl);
    const int vg = pok && oc < a.OW ? (plane * a.OH * a.OW + oc) * 4 : kOutOfRange;
    float acc[KK + 1];
#pragma unroll
    for (int q = 0; q <= KK; ++q)
        acc[q] = 0.0f;
#pragma unroll
    for (int ar = ar0; ar < ar0 + rpu; ++ar) {
        const int tr = floor_div(ar - a.pH, D), br = ar - a.pH - D * tr;
        float st[NB][NL];
        auto load_x = [&](int g, float (&d)[NL]) {
            const int ir = D * (i0 + tr + g) + br;
            const bool ok = (unsigned)ir < (unsigned)a.IH;
            const __amdgpu_buffer_rsrc_t r = make_rsrc(x, ok ? x_bytes : 0);
            const int soff = ok ? ir * a.IW * 4 : 0;
#pragma unroll
            for (int i = 0; i < NL; ++i)
                d[i] = buf_f32_s(r, src[i], soff);
        };
        // the lane's dy values of this row phase (row m in gv[m % RG])
        float gv[RG];
        auto load_dy = [&](int m) {
            const int oh = ar + D * (i0 + m);
            const bool ok = m < TH && oh < a.OH;
            const __amdgpu_buffer_rsrc_t r = make_rsrc(dy, ok ? dy_bytes : 0);
            gv[m % RG] = buf_f32_s(r, vg, ok ? oh * a.OW * 4 : 0);
        };
#pragma unroll
        for (int g = 0; g < NB - 1; ++g) {
            load_x(g, st[g]);
            load_dy(g);
        }
#pragma unroll
        for (int u = 0; u < G; ++u) {
#pragma unroll
            for (int i = 0; i < NL; ++i)
                slots[u % 2][dst[i]] = st[u % NB][i];
            if (u + NB - 1 < G) {
                load_x(u + NB - 1, st[(u + NB - 1) % NB]);
                if (u + NB - 1 < TH)
                    load_dy(u + NB - 1);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (u < TH)
                acc[KK] += gv[u % RG];                    // the bias sum
            // rows outside the planes are skipped (here, unlike the forward walk,
            // running their FMAs on the zeros in LDS measured 256 registers)
            const int ir = D * (i0 + tr + u) + br;
            if ((unsigned)ir < (unsigned)a.IH) {
                float xv[XW];
#pragma unroll
                for (int k = 0; k < XW; ++k)
                    xv[k] = slots[u % 2][rd + k];
#pragma unroll
                for (int kh = 0; kh < KH; ++kh) {
                    const int m = u - kh;                 // dy row this x row meets at tap row kh
                    if (m >= 0 && m < TH) {
#pragma unroll
                        for (int kw = 0; kw < KW; ++kw)
                            acc[kh * KW + kw] = fmaf(xv[kw], gv[m % RG], acc[kh * KW + kw]);
                    }
                }
            }
        }
    }
    // add the lpr lanes of each plane through the wave's own ring (no other
    // wave touches it; a wave's LDS operations run in order): in rounds of QB
    // sums, every lane parks its QB sums (sum q at q * 65 + lane), then output
    // o < ppw * QB adds plane o / QB's lpr values of sum o % QB in lane order
    // and is stored into the plane's chunk of the partial sums.  Every lane
    // runs the same read iterations and only the store is predicated: the
    // reads of a round must precede the next round's writes in the wave, and
    // with a read loop that some lanes skip the compiler may issue those
    // lanes' next writes first (each thread alone has no such dependence);
    // the empty asm keeps the compiler from moving LDS accesses across rounds
    constexpr int QB = 9, QP = 65;
    static_assert(QB * QP <= 2 * SLOT, "a round fits the wave's ring");
    float *rr = &ring[wave][0][0];
    const int n_out = a.ppw * QB;
#pragma unroll
    for (int r = 0; r * QB <= KK; ++r) {
#pragma unroll
        for (int qq = 0; qq < QB; ++qq)
            if (r * QB + qq <= KK)
                rr[qq * QP + lane] = acc[r * QB + qq];
        for (int o0 = 0; o0 < n_out; o0 += 64) {
            const int o = o0 + lane;
            const bool live = o < n_out;
            const int ps2 = live ? o / QB : 0, qq = live ? o - ps2 * QB : 0;
            float v = 0.0f;
            for (int l = 0; l < a.lpr; ++l)
                v += rr[qq * QP + ps2 * a.lpr + l];
            const int q = r * QB + qq, plane2 = pg * a.ppw + ps2;
            if (live && q <= KK && plane2 < a.planes) {
                const int n = plane2 / a.C, c = plane2 - n * a.C;
                const int chunk = ((n * a.nph + pu) * a.nrt + rt) * a.ncb + cb;
                part[((long long)chunk * a.C + c) * (KK + 1) + q] = v;
            }
        }
        asm volatile("" ::: "memory");
    }
}

typedef void (*WgradStreamFn)(const float *, const float *, float *, StreamNchwArgs);

template <int V>
void fill_wgrad_stream_row(WgradStreamFn (&row)[2])
{
    constexpr WgradStreamVariant t = kWgradStreamVariants[V];
    row[0] = &k_wgrad_stream_nchw<t.kH, t.kW, t.d, t.th, t.nl, t.nb, 1>;
    row[1] = &k_wgrad_stream_nchw<t.kH, t.kW, t.d, t.th, t.nl, t.nb, t.d>;
}

template <int... Vs>
void fill_wgrad_stream(WgradStreamFn (&fn)[kNumWgradStreamVariants][2],
                       std::integer_sequence<int, Vs...>)
{
    (fill_wgrad_stream_row<Vs>(fn[Vs]), ...);
}

// [variant][0: one row phase per unit, 1: all d row phases per unit]
struct WgradStreamTable {
    WgradStreamFn fn[kNumWgradStreamVariants][2];
    WgradStreamTable()
    {
        fill_wgrad_stream(fn, std::make_integer_sequence<int, kNumWgradStreamVariants>());
    }
};

typedef void (*StreamNchwFn)(const float *, const void *, const float *, float *,
                             StreamNchwArgs, EpiArgs);

template <typename WT, int V, int MODE>
constexpr StreamNchwFn stream_nchw_fn()
{
    constexpr StreamNchwVariant t = kStreamNchwVariants[V];
    return &k_stream_nchw<WT, t.kH, t.kW, t.d, t.px, t.th, t.nl, t.nb, MODE>;
}

template <int V>
void fill_stream_nchw(StreamNchwFn (&row)[2][3])
{
    row[0][0] = stream_nchw_fn<float, V, kModeFwd>();
    row[0][1] = stream_nchw_fn<float, V, kModeInputGrad>();
    row[0][2] = stream_nchw_fn<float, V, kModeFwdEpilogue>();
    row[1][0] = stream_nchw_fn<half_t, V, kModeFwd>();
    row[1][1] = stream_nchw_fn<half_t, V, kModeInputGrad>();
    row[1][2] = stream_nchw_fn<half_t, V, kModeFwdEpilogue>();
}

template <int... Vs>
void fill_all_stream_nchw(StreamNchwFn (&fn)[kNumStreamNchwVariants][2][3],
                          std::integer_sequence<int, Vs...>)
{
    (fill_stream_nchw<Vs>(fn[Vs]), ...);
}

struct StreamNchwTable {
    StreamNchwFn fn[kNumStreamNchwVariants][2][3];
    StreamNchwTable()
    {
        fill_all_stream_nchw(fn, std::make_integer_sequence<int, kNumStreamNchwVariants>());
    }
};

typedef void (*StreamPlanesFn)(const float *, const void *, const float *, float *,
                               StreamPlanesArgs, EpiArgs);

template <typename WT, int V, int MODE>
constexpr StreamPlanesFn stream_planes_fn()
{
    constexpr StreamPlanesVariant t = kStreamPlanesVariants[V];
    return &k_stream_nchw_planes<WT, t.kH, t.kW, t.d, t.px, t.th, t.nl, t.nb, MODE>;
}

template <int V>
void fill_stream_planes(StreamPlanesFn (&row)[2][3])
{
    row[0][0] = stream_planes_fn<float, V, kModeFwd>();
    row[0][1] = stream_planes_fn<float, V, kModeInputGrad>();
    row[0][2] = stream_planes_fn<float, V, kModeFwdEpilogue>();
    row[1][0] = stream_planes_fn<half_t, V, kModeFwd>();
    row[1][1] = stream_planes_fn<half_t, V, kModeInputGrad>();
    row[1][2] = stream_planes_fn<half_t, V, kModeFwdEpilogue>();
}

template <int... Vs>
void fill_all_stream_planes(StreamPlanesFn (&fn)[kNumStreamPlanesVariants][2][3],
                            std::integer_sequence<int, Vs...>)
{
    (fill_stream_planes<Vs>(fn[Vs]), ...);
}

struct StreamPlanesTable {
    StreamPlanesFn fn[kNumStreamPlanesVariants][2][3];
    StreamPlanesTable()
    {
        fill_all_stream_planes(fn,
                               std::make_integer_sequence<int, kNumStreamPlanesVariants>());
    }
};

typedef void (*StreamFn)(const float *, const void *, const float *, float *, StreamArgs,
                         EpiArgs);

template <typename WT, int V, int MODE>
constexpr StreamFn stream_fn()
{
    constexpr StreamVariant t = kStreamVariants[V];
    return &k_stream_nhwc<WT, t.kH, t.kW, t.d, t.cl, t.px, t.th, t.nb, MODE>;
}

template <int V>
void fill_stream(StreamFn (&row)[2][3])
{
    row[0][0] = stream_fn<float, V, kModeFwd>();
    row[0][1] = stream_fn<float, V, kModeInputGrad>();
    row[0][2] = stream_fn<float, V, kModeFwdEpilogue>();
    row[1][0] = stream_fn<half_t, V, kModeFwd>();
    row[1][1] = stream_fn<half_t, V, kModeInputGrad>();
    row[1][2] = stream_fn<half_t, V, kModeFwdEpilogue>();
}

template <int... Vs>
void fill_all_stream(StreamFn (&fn)[kNumStreamVariants][2][3], std::integer_sequence<int, Vs...>)
{
    (fill_stream<Vs>(fn[Vs]), ...);
}

struct StreamTable {
    StreamFn fn[kNumStreamVariants][2][3];
    StreamTable()
    {
        fill_all_stream(fn, std::make_integer_sequence<int, kNumStreamVariants>());
    }
};

typedef void (*WgradStreamNhwcFn)(const float *, const float *, float *, StreamArgs);

template <int V>
constexpr WgradStreamNhwcFn wgrad_stream_nhwc_fn()
{
    constexpr WgradStreamNhwcVariant t = kWgradStreamNhwcVariants[V];
    return &k_wgrad_stream_nhwc<t.kH, t.kW, t.d, t.px, t.th, t.nb>;
}

template <int... Vs>
void fill_wgrad_stream_nhwc(WgradStreamNhwcFn (&fn)[kNumWgradStreamNhwcVariants],
                            std::integer_sequence<int, Vs...>)
{
    ((fn[Vs] = wgrad_stream_nhwc_fn<Vs>()), ...);
}

struct WgradStreamNhwcTable {
    WgradStreamNhwcFn fn[kNumWgradStreamNhwcVariants];
    WgradStreamNhwcTable()
    {
        fill_wgrad_stream_nhwc(fn,
                               std::make_integer_sequence<int, kNumWgradStreamNhwcVariants>());
    }
};

}  // namespace

int launch_stream_nhwc(const Problem &p, const Plan &pl, const float *in, const void *w,
                       const float *b, float *out, hipStream_t st, const EpiArgs &ep)
{
    static const StreamTable table;
    if (p.mult != 1 || p.stride != 1 || pl.variant < 0 || pl.variant >= kNumStreamVariants)
        return DWCONV_ERR_BAD_STRATEGY;
    const StreamVariant &v = kStreamVariants[pl.variant];
    const long long mblk = pl.nct * ((pl.total + 3) / 4);
    if (pl.cl != v.cl || (pl.tail_cl != 0 && pl.tail_cl != 16 && pl.tail_cl != 32) ||
        pl.tail_cl >= v.cl || (pl.tail_cl == 0) != (pl.tail_units == 0) ||
        pl.nct * v.cl + pl.tail_cl < p.C || pl.grid != mblk + (pl.tail_units + 3) / 4)
        return DWCONV_ERR_BAD_STRATEGY;       // the tiles must cover the channels
    StreamFn f = table.fn[pl.variant][p.wtype == DWCONV_W_F16][mode_of(p, ep)];
    StreamArgs a;
    a.C = p.C;
    a.IH = pl.IH; a.IW = pl.IW; a.OH = pl.OH; a.OW = pl.OW;
    a.pH = pl.pH; a.pW = pl.pW;
    a.nct = pl.nct; a.ncg = pl.nwt; a.nrt = pl.nst; a.nph = pl.pb;
    a.upc = (int)pl.total;
    a.xcd = pl.xcd;
    a.mblk = (int)mblk;
    a.tcl = pl.tail_cl; a.tncg = pl.tail_ncg; a.tupc = (int)pl.tail_units;
    return launch_kernel(f, dim3((unsigned)pl.grid), dim3(256), 0, st, in, w,
                         p.op == DWCONV_OP_FWD ? b : nullptr, out, a, ep);
}

int launch_stream_nchw(const Problem &p, const Plan &pl, const float *in, const void *w,
                       const float *b, float *out, hipStream_t st, const EpiArgs &ep)
{
    static const StreamNchwTable table;
    if (p.mult != 1 || p.stride != 1 || pl.variant < 0 || pl.variant >= kNumStreamNchwVariants)
        return DWCONV_ERR_BAD_STRATEGY;
    const StreamNchwVariant &v = kStreamNchwVariants[pl.variant];
    if (pl.pb < 1 || pl.cl < 1 || pl.pb * pl.cl > 64 || pl.pb * pl.hl > 64 * v.nl ||
        pl.pb * pl.twl > kStreamNchwSlot || pl.twl < pl.hl)
        return DWCONV_ERR_BAD_STRATEGY;      // the staged row must fit the wave's slot
    StreamNchwFn f = table.fn[pl.variant][p.wtype == DWCONV_W_F16][mode_of(p, ep)];
    StreamNchwArgs a;
    a.C = p.C;
    a.planes = p.N * p.C;
    a.IH = pl.IH; a.IW = pl.IW; a.OH = pl.OH; a.OW = pl.OW;
    a.pH = pl.pH; a.pW = pl.pW;
    a.lpr = pl.cl; a.ppw = pl.pb; a.pitch = pl.hl; a.lpitch = pl.twl;
    a.ncb = pl.nwt; a.nrt = pl.nst; a.nph = pl.nct;
    a.units = (int)pl.total;
    a.rpu = 1;
    return launch_kernel(f, dim3((unsigned)pl.grid), dim3(256), 0, st, in, w,
                         p.op == DWCONV_OP_FWD ? b : nullptr, out, a, ep);
}

int launch_stream_nchw_planes(const Problem &p, const Plan &pl, const float *in,
                              const void *w, const float *b, float *out, hipStream_t st,
                              const EpiArgs &ep)
{
    static const StreamPlanesTable table;
    if (p.mult != 1 || p.stride != 1 || pl.variant < 0 || pl.variant >= kNumStreamPlanesVariants)
        return DWCONV_ERR_BAD_STRATEGY;
    const StreamPlanesVariant &v = kStreamPlanesVariants[pl.variant];
    const long long planes = (long long)p.N * p.C;
    auto cdiv = [](int x, int y) { return (x + y - 1) / y; };
    // the loads must cover a window's in-image columns for 16 planes
    const int win = 4 * v.px + v.d * (v.kW - 1);
    if (16 * (pl.IW < win ? pl.IW : win) > 64 * v.nl)
        return DWCONV_ERR_BAD_STRATEGY;
    // the workgroups must cover every plane group, row phase, row tile and
    // column block of the tensor written
    if (pl.tw != 4 * v.px || pl.th != v.th || pl.nwt != cdiv(pl.OW, pl.tw) ||
        pl.nst != cdiv(cdiv(pl.OH, v.d), v.th) ||
        pl.total != (planes + 15) / 16 * v.d * pl.nst * pl.nwt || pl.grid != (pl.total + 3) / 4)
        return DWCONV_ERR_BAD_STRATEGY;
    StreamPlanesFn f = table.fn[pl.variant][p.wtype == DWCONV_W_F16][mode_of(p, ep)];
    StreamPlanesArgs a;
    a.C = p.C;
    a.planes = (int)planes;
    a.IH = pl.IH; a.IW = pl.IW; a.OH = pl.OH; a.OW = pl.OW;
    a.pH = pl.pH; a.pW = pl.pW;
    a.ncb = pl.nwt; a.nrt = pl.nst;
    a.units = (int)pl.total;
    a.xcd = pl.xcd;
    return launch_kernel(f, dim3((unsigned)pl.grid), dim3(256), 0, st, in, w,
                         p.op == DWCONV_OP_FWD ? b : nullptr, out, a, ep);
}

int launch_wgrad_stream_nhwc(const Problem &p, const Plan &pl, const float *x, const float *dy,
                             float *part, hipStream_t st)
{
    static const WgradStreamNhwcTable table;
    const long long bt = (pl.tail_units + 3) / 4;
    if (p.mult != 1 || p.stride != 1 || pl.variant < 0 ||
        pl.variant >= kNumWgradStreamNhwcVariants || pl.cl != 64 ||
        pl.chunks != (pl.total + 3) / 4 || pl.grid != pl.nct * pl.chunks + bt ||
        (pl.tail_cl != 0 && pl.tail_cl != 16 && pl.tail_cl != 32) ||
        (pl.tail_cl == 0) != (pl.tail_units == 0) || bt > pl.chunks ||
        pl.nct * 64 + pl.tail_cl < p.C)
        return DWCONV_ERR_BAD_STRATEGY;       // the tiles must cover the channels
    StreamArgs a;
    a.C = p.C;
    a.IH = p.H; a.IW = p.W; a.OH = pl.OH; a.OW = pl.OW;
    a.pH = pl.pH; a.pW = pl.pW;
    a.nct = pl.nct; a.ncg = pl.nwt; a.nrt = pl.nst; a.nph = pl.pb;
    a.upc = (int)pl.total;
    a.xcd = pl.xcd;
    a.mblk = (int)(pl.nct * pl.chunks);
    a.tcl = pl.tail_cl; a.tncg = pl.tail_ncg; a.tupc = (int)pl.tail_units;
    return launch_kernel(table.fn[pl.variant], dim3((unsigned)pl.grid), dim3(256), 0, st, x, dy,
                         part, a);
}

int launch_wgrad_stream_nchw(const Problem &p, const Plan &pl, const float *x, const float *dy,
                             float *part, hipStream_t st)
{
    static const WgradStreamTable table;
    if (p.mult != 1 || p.stride != 1 || pl.variant < 0 || pl.variant >= kNumWgradStreamVariants)
        return DWCONV_ERR_BAD_STRATEGY;
    const WgradStreamVariant &v = kWgradStreamVariants[pl.variant];
    if (pl.pb < 1 || pl.cl < 1 || pl.pb * pl.cl > 64 || pl.pb * pl.hl > 64 * v.nl ||
        pl.pb * pl.twl > kStreamNchwSlot || pl.twl < pl.hl)
        return DWCONV_ERR_BAD_STRATEGY;      // the staged row must fit the wave's slot
    StreamNchwArgs a;
    a.C = p.C;
    a.planes = p.N * p.C;
    a.IH = p.H; a.IW = p.W; a.OH = p.Ho; a.OW = p.Wo;
    a.pH = pl.pH; a.pW = pl.pW;
    a.lpr = pl.cl; a.ppw = pl.pb; a.pitch = pl.hl; a.lpitch = pl.twl;
    a.ncb = pl.nwt; a.nrt = pl.nst; a.nph = pl.nct;
    a.units = (int)pl.total;
    a.rpu = pl.rpu;
    if (a.rpu != 1 && a.rpu != v.d)
        return DWCONV_ERR_BAD_STRATEGY;
    return launch_kernel(table.fn[pl.variant][a.rpu == 1 ? 0 : 1], dim3((unsigned)pl.grid),
                         dim3(256), 0, st, x, dy,
                         part, a);
}

}  // namespace dwconv
