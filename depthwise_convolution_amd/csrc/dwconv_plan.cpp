// dwconv_plan.cpp -- argument validation and kernel selection (host only,
// no HIP runtime calls).
//
// Shape rules (LeanMlir "Depthwise" page, forward equation, read with stride
// s, dilation d and explicit zero padding pt/pb (rows), pl/pr (columns)):
// output row ho reads input rows ho*s + kh*d - pt, and the output keeps the
// window positions that fit, Ho = (H + pt + pb - d*(kH-1) - 1)/s + 1 (same
// for columns).  SAME padding is pt = pb = d*(kH-1)/2 with odd kernels, so
// Ho = ceil(H/s); the page's stride-2 XLA-SAME is pt = d*(kH-1)/2 - 1,
// pb = d*(kH-1)/2 (the odd positions of the stride-1 result).  Selecting the
// tiling from the problem's extents mirrors the cubek-convolution
// "depthwise" module, whose launch space is built from the problem extents
// and a tiling strategy.
#include "dwconv_internal.h"
#include "../../include/dwconv.h"

#include <algorithm>
#include <cstdio>
#include <cstring>

namespace dwconv {

namespace {

constexpr long long kMaxElems = (1LL << 31) - 1;  // 32-bit element indexing
constexpr int kMaxPad = 1 << 16;                   // |pad| bound

int ceil_div(int a, int b) { return (a + b - 1) / b; }

const char *op_tag(const dwconv::Problem &p)
{
    if (p.op == DWCONV_OP_INPUT_GRAD)
        return "ig";
    return p.epi ? "fwd_epi" : "fwd";
}

}  // namespace

Problem same_problem(int op, int wtype, int has_bias, int N, int H, int W, int C, int kH,
                     int kW, int stride, int dilation, int layout)
{
    Problem p;
    std::memset(&p, 0, sizeof p);
    p.op = op; p.wtype = wtype; p.layout = layout; p.has_bias = has_bias;
    p.N = N; p.H = H; p.W = W; p.C = C; p.kH = kH; p.kW = kW;
    p.stride = stride; p.dilation = dilation;
    p.mult = 1;
    p.same = 1;
    // symmetric SAME pads; for even kernels validate_problem rejects the problem
    const long long ph = (long long)dilation * (kH - 1) / 2, pw = (long long)dilation * (kW - 1) / 2;
    p.pt = p.pb = (int)std::min<long long>(std::max<long long>(ph, 0), 1 << 20);
    p.pl = p.pr = (int)std::min<long long>(std::max<long long>(pw, 0), 1 << 20);
    return p;
}

int validate_problem(Problem &p)
{
    if (p.op != DWCONV_OP_FWD && p.op != DWCONV_OP_INPUT_GRAD && p.op != DWCONV_OP_WEIGHT_GRAD)
        return DWCONV_ERR_BAD_OP;
    if (p.N < 1 || p.H < 1 || p.W < 1 || p.C < 1 || p.kH < 1 || p.kW < 1 || p.mult < 1)
        return DWCONV_ERR_BAD_DIM;
    const long long co = (long long)p.C * p.mult;
    const long long in_elems = (long long)p.N * p.H * p.W * p.C;
    if (in_elems > kMaxElems || co * p.kH * p.kW > kMaxElems)
        return DWCONV_ERR_BAD_DIM;
    if (p.stride != 1 && p.stride != 2)
        return DWCONV_ERR_BAD_STRIDE;
    if (p.dilation < 1 || (long long)p.dilation * (std::max(p.kH, p.kW) - 1) >= (1 << 16))
        return DWCONV_ERR_BAD_DILATION;
    if (p.same && (p.kH % 2 == 0 || p.kW % 2 == 0))
        return DWCONV_ERR_EVEN_KERNEL;
    if (p.layout != DWCONV_LAYOUT_NHWC && p.layout != DWCONV_LAYOUT_NCHW)
        return DWCONV_ERR_BAD_LAYOUT;
    if (p.wtype != DWCONV_W_F32 && p.wtype != DWCONV_W_F16)
        return DWCONV_ERR_BAD_WTYPE;
    const int pads[4] = {p.pt, p.pb, p.pl, p.pr};
    for (int i = 0; i < 4; ++i)
        if (pads[i] <= -kMaxPad || pads[i] >= kMaxPad)
            return DWCONV_ERR_BAD_PAD;
    // window positions that fit the padded input (the numerators stay far
    // from overflow: every term is below 2^31 / 4 in magnitude)
    const long long nh = (long long)p.H + p.pt + p.pb - (long long)p.dilation * (p.kH - 1) - 1;
    const long long nw = (long long)p.W + p.pl + p.pr - (long long)p.dilation * (p.kW - 1) - 1;
    if (nh < 0 || nw < 0)
        return DWCONV_ERR_BAD_DIM;
    const long long Ho = nh / p.stride + 1, Wo = nw / p.stride + 1;
    if ((long long)p.N * Ho * Wo * co > kMaxElems)
        return DWCONV_ERR_BAD_DIM;
    p.Ho = (int)Ho;
    p.Wo = (int)Wo;
    return DWCONV_OK;
}

// Effective zero padding and the extents of the tensors read and written,
// per op.  The input gradient runs the reversed-kernel form over dy, which
// is a stride-1 correlation of the zero-upsampled dy with top pad
// d*(kH-1) - pt (and left pad d*(kW-1) - pl).
static void set_extents(const Problem &p, Plan *pl)
{
    if (p.op == DWCONV_OP_INPUT_GRAD) {
        pl->IH = p.Ho; pl->IW = p.Wo; pl->OH = p.H; pl->OW = p.W;
        pl->pH = p.dilation * (p.kH - 1) - p.pt;
        pl->pW = p.dilation * (p.kW - 1) - p.pl;
    } else {
        // forward reads x and writes y; the weight gradient reads x and dy
        pl->IH = p.H; pl->IW = p.W; pl->OH = p.Ho; pl->OW = p.Wo;
        pl->pH = p.pt;
        pl->pW = p.pl;
    }
}

// When the chosen variant's channel tile holds every channel of the problem,
// take a later variant of the same kernel shape and staging width whose tile
// (of at least min_cg channels) the problem still fills to 3/4 with two or
// more tiles: twice the workgroups for a problem that would otherwise give
// each (image, row band, column tile) one.
template <typename V>
static int split_channel_tile(const V *table, int nvar, int best, long long co, int min_cg)
{
    const V &b = table[best];
    if (ceil_div((int)co, b.cl * b.vec) != 1)
        return best;
    for (int i = best + 1; i < nvar; ++i) {
        const V &v = table[i];
        const int cg = v.cl * v.vec, nt = ceil_div((int)co, cg);
        if (v.kH == b.kH && v.kW == b.kW && v.d == b.d && v.lv == b.lv && cg >= min_cg &&
            nt >= 2 && (double)co / (nt * cg) >= 0.75)
            return i;
    }
    return best;
}

static bool plan_tiled_nhwc(const Problem &p, std::uintptr_t ptr_bits, Plan *pl)
{
    if (p.layout != DWCONV_LAYOUT_NHWC)
        return false;
    // a channel multiplier of 2 has its own variants (stride 1, 16-byte staging)
    const bool m2 = p.mult == 2;
    if ((p.mult != 1 && !m2) || (m2 && (p.stride != 1 || p.C % 4 != 0)))
        return false;
    const TiledVariant *table = m2 ? kTiledM2Variants
                                   : p.stride == 1 ? kTiledVariants : kTiledS2Variants;
    const int nvar = m2 ? kNumTiledM2Variants
                        : p.stride == 1 ? kNumTiledVariants : kNumTiledS2Variants;
    const bool v4ok = p.C % 4 == 0 && (ptr_bits & 15u) == 0;   // 16-byte staging loads
    const long long co = (long long)p.mult * p.C;               // channels of the tile walk
    // buffer-load byte offsets are 31-bit: one image and the weights must fit
    if (4LL * pl->IH * pl->IW * co >= (1LL << 31) || 4LL * co * p.kH * p.kW >= (1LL << 31))
        return false;
    // first variant of this kernel shape (table order = preference) whose
    // channel tile the problem fills to at least 3/4; else the one it fills best
    int best = -1;
    double best_fill = -1.0;
    for (int i = 0; i < nvar; ++i) {
        const TiledVariant &v = table[i];
        if (v.kH != p.kH || v.kW != p.kW || v.d != p.dilation || (v.lv == 4 && !v4ok))
            continue;
        const int cg = v.cl * v.vec;
        const double fill = (double)co / (ceil_div((int)co, cg) * cg);
        if (fill >= 0.75) {
            best = i;
            break;
        }
        if (fill > best_fill) {
            best = i;
            best_fill = fill;
        }
    }
    if (best < 0)
        return false;
    // stride 1, no multiplier: 3x3 with 65-128 channels takes two 64-channel
    // tiles (8x112x112x96 on MI355X: 14.4 -> 12.6 us); a 32-channel tile
    // (3 staged rows, for small C) measured 20-40% slower at 48-64 channels
    if (table == kTiledVariants)
        best = split_channel_tile(table, nvar, best, co, 64);
    const TiledVariant &v = table[best];
    const int R = (v.kH - 1) * v.d + 1;
    pl->kind = KIND_TILED_NHWC;
    pl->variant = best;
    pl->vec = v.vec;
    pl->cl = v.cl;
    pl->tw = v.px * 256 / v.cl;
    pl->th = v.g - R + 1;
    // the grid the tiles cover: the output, except at stride 2 forward, where
    // it is the stride-1 grid (2*Ho-1 x 2*Wo-1) whose even positions are kept
    pl->YH = pl->OH;
    pl->YW = pl->OW;
    if (p.stride == 2 && p.op != DWCONV_OP_INPUT_GRAD) {
        pl->OH = 2 * pl->OH - 1;
        pl->OW = 2 * pl->OW - 1;
    }
    pl->nct = ceil_div((int)co, v.cl * v.vec);
    pl->nwt = ceil_div(pl->OW, pl->tw);
    pl->nst = ceil_div(pl->OH, pl->th);
    pl->grid = (long long)p.N * pl->nct * pl->nwt * pl->nst;
    pl->block = 256;
    std::snprintf(pl->name, sizeof pl->name,
                  "tiled_nhwc_s%d_k%dx%d_d%d_v%d_cl%d_px%d_g%d%s%s_%s_%s", p.stride, v.kH, v.kW,
                  v.d, v.vec, v.cl, v.px, v.g, v.lv == 1 ? "_l1" : "", m2 ? "_m2" : "",
                  op_tag(p), p.wtype ? "f16w" : "f32w");
    return true;
}

static bool plan_tiled_nchw(const Problem &p, std::uintptr_t ptr_bits, Plan *pl)
{
    // a channel multiplier runs tiled in the forward (each output plane reads
    // its input plane) and, for 2 at stride 1, in the input gradient (each dx
    // plane sums its 2 dy planes: mig planes staged per walk plane)
    const bool igm = p.op == DWCONV_OP_INPUT_GRAD && p.mult != 1;
    if (p.layout != DWCONV_LAYOUT_NCHW || (igm && (p.mult != 2 || p.stride != 1)))
        return false;
    const int mig = igm ? p.mult : 1;
    // planes of the walk: the forward's output planes, or the input gradient's dx planes
    const long long co = (long long)p.mult * p.C;
    const long long planes = (long long)p.N * (p.op == DWCONV_OP_FWD ? co : p.C);
    // buffer-load byte offsets are 31-bit: the tensor read and the weights must fit
    const long long read_planes = p.op == DWCONV_OP_FWD ? (long long)p.N * p.C : p.N * co;
    if (4LL * read_planes * pl->IH * pl->IW >= (1LL << 31) ||
        4LL * co * p.kH * p.kW >= (1LL << 31))
        return false;
    const TiledNchwVariant *table = p.stride == 1 ? kTiledNchwVariants : kTiledNchwS2Variants;
    const int nvar = p.stride == 1 ? kNumTiledNchwVariants : kNumTiledNchwS2Variants;
    // 16-byte staging loads need whole aligned rows; the stride-2 input
    // gradient stages the zero-upsampled dy element by element
    const bool v4ok = pl->IW % 4 == 0 && (ptr_bits & 15u) == 0 &&
                      !(p.stride == 2 && p.op == DWCONV_OP_INPUT_GRAD);
    int best = -1;
    for (int i = 0; i < nvar; ++i) {
        const TiledNchwVariant &v = table[i];
        if (v.kH == p.kH && v.kW == p.kW && v.d == p.dilation && (v.v4 == 0 || v4ok)) {
            best = i;
            break;
        }
    }
    if (best < 0)
        return false;
    const TiledNchwVariant &v = table[best];
    const int R = (v.kH - 1) * v.d + 1;
    // the grid the tiles cover: the output, except at stride 2 forward, where
    // it is the stride-1 grid (2*Ho-1 x 2*Wo-1) whose even positions are kept
    pl->YH = pl->OH;
    pl->YW = pl->OW;
    if (p.stride == 2 && p.op != DWCONV_OP_INPUT_GRAD) {
        pl->OH = 2 * pl->OH - 1;
        pl->OW = 2 * pl->OW - 1;
    }
    // threads per plane row: ceil(Wo/q), at least 16, at most 256 (wider
    // planes take several column tiles); 256/tx planes share a workgroup
    const int tx = std::max(16, std::min(256, ceil_div(pl->OW, v.q)));
    // staged columns of a plane row: from w0 - hl (hl = the left pad rounded
    // up to whole 16-byte loads) over the tile's tw + d*(kW-1) input columns
    const int lv = v.v4 ? 4 : 1;
    const int hl = v.v4 ? -((-pl->pW) & ~3) : pl->pW;   // ceil to a multiple of 4
    const int span = (hl - pl->pW) + tx * v.q + v.d * (v.kW - 1);
    pl->kind = KIND_TILED_NCHW;
    pl->variant = best;
    pl->vec = 1;
    pl->cl = tx;
    pl->pb = 256 / tx;
    pl->tw = tx * v.q;
    pl->hl = hl;
    pl->twl = (span + lv - 1) / lv * lv;
    const bool ups = p.stride == 2 && p.op == DWCONV_OP_INPUT_GRAD;
    if (ups)
        pl->twl += pl->twl & 1;             // upsampled dy is staged in column pairs
    // the kernel's per-thread load registers must cover the staged tile
    const long long loads = ups ? (long long)pl->pb * ((v.g + 1) / 2) * (pl->twl / 2)
                                : (long long)pl->pb * mig * v.g * (pl->twl / lv);
    if (loads > 256LL * nchw_stage_loads(ups ? 1 : 0, mig * v.g, v.q, v.kW, v.d, v.v4 != 0))
        return false;
    pl->th = v.g - R + 1;
    pl->nct = (int)((planes + pl->pb - 1) / pl->pb);
    pl->nwt = ceil_div(pl->OW, pl->tw);
    pl->nst = ceil_div(pl->OH, pl->th);
    // the staged tile (whole waves of 64 staged elements), then the weights
    const long long tile_el = (long long)mig * pl->pb * v.g * (pl->twl / lv);
    pl->lds_bytes = (int)(4 * ((tile_el + 63) / 64 * 64 * lv + mig * pl->pb * v.kH * v.kW));
    if (pl->lds_bytes > kMaxLdsBytes)
        return false;
    pl->grid = (long long)pl->nct * pl->nwt * pl->nst;
    pl->block = 256;
    char mtag[16] = "";
    if (p.mult != 1)
        std::snprintf(mtag, sizeof mtag, "_m%d", p.mult);
    std::snprintf(pl->name, sizeof pl->name, "tiled_nchw_s%d_k%dx%d_d%d_q%d_g%d_%s_tx%d%s_%s_%s",
                  p.stride, v.kH, v.kW, v.d, v.q, v.g, v.v4 ? "v4" : "v1", tx, mtag, op_tag(p),
                  p.wtype ? "f16w" : "f32w");
    return true;
}

// Tile order of a tiled or NHWC row-streaming plan (kXcdRangeMaxBytes):
// activations are the tensor read and the tensor written, x and y (or dy
// and dx, x and dy).
static int xcd_ranges(const Problem &p)
{
    const long long act =
        4LL * p.N * p.C * ((long long)p.H * p.W + (long long)p.mult * p.Ho * p.Wo);
    return act < kXcdRangeMaxBytes ? 1 : 0;
}

// Channels per lane group of the row-streaming NHWC walks' tail tile (0 =
// none) for 64-channel tiles: the last C % 64 channels, when they fill at
// most half of a tile, run as a tile of 16 or 32 channels per lane group (4
// or 2 column groups, so 4x or 2x fewer waves for them).  Measured at
// 64x30x19xC 7x7 (forward, against full-width tiles only): 16 lanes win
// 3-14% with at most one full tile or C % 4 == 0 (C = 3, 65, 67, 132, 136,
// 144) but lose 3-12% with two or more full tiles and C % 4 != 0 (C =
// 129-139), where 32 lanes win 9-10% (C = 129-139, 147, 150); with three or
// more full tiles and odd C both lose (C = 195, 259: +4.5% with 32 lanes),
// and with dilation 2 (the phase sub-grid is narrower than a 16-lane wave's
// columns) they lose 2-8%.
static int stream_tail_cl(const Problem &p, int d)
{
    const int rem = p.C % 64, full = p.C / 64;
    if (rem == 0 || 2 * rem > 64 || d != 1 || full > 2)
        return 0;
    return (rem <= 16 && (p.C % 4 == 0 || full <= 1)) ? 16 : 32;
}

// Row-streaming NHWC kernel: stride 1, no multiplier, a listed kernel shape.
// Any channel count and 4-byte alignment (4-byte loads and stores).
static bool plan_stream_nhwc(const Problem &p, Plan *pl)
{
    if (p.layout != DWCONV_LAYOUT_NHWC || p.stride != 1 || p.mult != 1 ||
        p.op == DWCONV_OP_WEIGHT_GRAD)
        return false;
    int best = -1;
    for (int i = 0; i < kNumStreamVariants; ++i) {
        const StreamVariant &v = kStreamVariants[i];
        if (v.kH == p.kH && v.kW == p.kW && v.d == p.dilation) {
            best = i;
            break;
        }
    }
    if (best < 0)
        return false;
    const StreamVariant &v = kStreamVariants[best];
    // byte offsets within a row (the lane's columns, up to (kW-1)*d past the
    // row on either side) and row starts within an image are 32-bit
    const long long cb = 4LL * p.C;
    if (cb * (std::max(pl->IW, pl->OW) + 2LL * v.d * v.kW + 8LL * v.px * v.d) >= (1LL << 31) ||
        cb * pl->IH * pl->IW >= (1LL << 31) || cb * pl->OH * pl->OW >= (1LL << 31) ||
        4LL * p.C * p.kH * p.kW >= (1LL << 31))
        return false;
    const int d = v.d;
    const int ohs = ceil_div(pl->OH, d), ows = ceil_div(pl->OW, d);   // phase sub-grid
    pl->kind = KIND_STREAM_NHWC;
    pl->variant = best;
    pl->vec = 1;
    pl->cl = v.cl;
    pl->tw = v.px * (64 / v.cl);                  // output columns of a wave
    pl->th = v.th;
    pl->tail_cl = v.cl == 64 ? stream_tail_cl(p, d) : 0;
    pl->nct = pl->tail_cl ? p.C / v.cl : ceil_div(p.C, v.cl);
    pl->nwt = ceil_div(ows, pl->tw);
    pl->nst = ceil_div(ohs, v.th);
    pl->pb = d * d;                               // phases
    pl->YH = pl->OH;
    pl->YW = pl->OW;
    pl->total = (long long)p.N * pl->nst * pl->pb * pl->nwt;      // wave units per channel tile
    pl->tail_ncg = pl->tail_cl ? ceil_div(ows, v.px * (64 / pl->tail_cl)) : 0;
    pl->tail_units = (long long)p.N * pl->nst * pl->pb * pl->tail_ncg;
    if (pl->total * 4 >= (1LL << 31))
        return false;
    pl->grid = pl->nct * ((pl->total + 3) / 4) + (pl->tail_units + 3) / 4;
    pl->block = 256;
    pl->xcd = xcd_ranges(p);
    char tail[8] = "";
    if (pl->tail_cl)
        std::snprintf(tail, sizeof tail, "t%d_", pl->tail_cl);
    std::snprintf(pl->name, sizeof pl->name, "stream_nhwc_s1_k%dx%d_d%d_cl%d_px%d_th%d_%s%s_%s",
                  v.kH, v.kW, v.d, v.cl, v.px, v.th, tail, op_tag(p), p.wtype ? "f16w" : "f32w");
    return true;
}

// Row-streaming NCHW kernel: stride 1, no multiplier, a listed kernel shape,
// 4-byte alignment.
static bool plan_stream_nchw(const Problem &p, Plan *pl)
{
    if (p.layout != DWCONV_LAYOUT_NCHW || p.stride != 1 || p.mult != 1 ||
        p.op == DWCONV_OP_WEIGHT_GRAD)
        return false;
    int best = -1;
    for (int i = 0; i < kNumStreamNchwVariants; ++i) {
        const StreamNchwVariant &v = kStreamNchwVariants[i];
        if (v.kH == p.kH && v.kW == p.kW && v.d == p.dilation) {
            best = i;
            break;
        }
    }
    if (best < 0)
        return false;
    const StreamNchwVariant &v = kStreamNchwVariants[best];
    const long long planes = (long long)p.N * p.C;
    // byte offsets into the whole tensor are 32-bit (and below the
    // out-of-range offset)
    if (4LL * planes * pl->IH * pl->IW >= (1LL << 31) ||
        4LL * planes * pl->OH * pl->OW >= (1LL << 31) || 4LL * p.C * p.kH * p.kW >= (1LL << 31))
        return false;
    const int d = v.d;
    const int ohs = ceil_div(pl->OH, d), ows = ceil_div(pl->OW, d);   // phase sub-grid
    int lpr = ceil_div(ows, v.px), ncb = 1;
    if (lpr > 64) {
        ncb = ceil_div(lpr, 64);
        lpr = 64;
    }
    // staged columns of a plane row, and their LDS pitch: the next value
    // congruent to lpr mod 32, so the lanes of a half-wave read distinct
    // banks; the planes of a wave must fit its loads and its row slot
    const int pitch = lpr * v.px + v.kW - 1;
    const int lpitch = pitch + ((lpr - pitch) % 32 + 32) % 32;
    const int ppw = std::min(std::min(64 / lpr, 64 * v.nl / pitch), kStreamNchwSlot / lpitch);
    if (ppw < 1)
        return false;
    pl->kind = KIND_STREAM_NCHW;
    pl->variant = best;
    pl->vec = 1;
    pl->cl = lpr;
    pl->pb = ppw;
    pl->hl = pitch;
    pl->twl = lpitch;
    pl->tw = lpr * v.px;
    pl->th = v.th;
    pl->nwt = ncb;
    pl->nst = ceil_div(ohs, v.th);
    pl->nct = d * d;                              // phases
    pl->YH = pl->OH;
    pl->YW = pl->OW;
    pl->total = (planes + ppw - 1) / ppw * pl->nct * pl->nst * ncb;   // wave units
    if (pl->total * 4 >= (1LL << 31))
        return false;
    pl->grid = (pl->total + 3) / 4;
    pl->block = 256;
    std::snprintf(pl->name, sizeof pl->name,
                  "stream_nchw_s1_k%dx%d_d%d_px%d_th%d_nl%d_lpr%d_%s_%s", v.kH, v.kW, v.d, v.px,
                  v.th, v.nl, lpr, op_tag(p), p.wtype ? "f16w" : "f32w");
    return true;
}

// Plane-per-lane NCHW kernel: stride 1, no multiplier, a listed kernel
// shape, 4-byte alignment.
static bool plan_stream_nchw_planes(const Problem &p, Plan *pl)
{
    if (p.layout != DWCONV_LAYOUT_NCHW || p.stride != 1 || p.mult != 1 ||
        p.op == DWCONV_OP_WEIGHT_GRAD)
        return false;
    // the first variant whose loads cover a window's in-image columns for
    // 16 planes (a window spans 4*px + d*(kW-1) columns)
    int best = -1;
    for (int i = 0; i < kNumStreamPlanesVariants; ++i) {
        const StreamPlanesVariant &v = kStreamPlanesVariants[i];
        const int win = std::min(4 * v.px + v.d * (v.kW - 1), pl->IW);
        if (v.kH == p.kH && v.kW == p.kW && v.d == p.dilation && 16 * win <= 64 * v.nl) {
            best = i;
            break;
        }
    }
    if (best < 0)
        return false;
    const StreamPlanesVariant &v = kStreamPlanesVariants[best];
    const long long planes = (long long)p.N * p.C;
    // byte offsets into the whole tensor are 32-bit (and below the
    // out-of-range offset), plane indices too
    if (4LL * (planes + 64) * pl->IH * pl->IW >= (1LL << 31) ||
        4LL * (planes + 64) * pl->OH * pl->OW >= (1LL << 31) ||
        4LL * p.C * p.kH * p.kW >= (1LL << 31))
        return false;
    pl->kind = KIND_STREAM_NCHW_PLANES;
    pl->variant = best;
    pl->vec = 1;
    pl->cl = 16;                                  // planes per wave
    pl->tw = 4 * v.px;                            // output columns of a wave
    pl->th = v.th;
    pl->nct = (int)((planes + 15) / 16);          // plane groups
    pl->nwt = ceil_div(pl->OW, pl->tw);           // column blocks
    pl->nst = ceil_div(ceil_div(pl->OH, v.d), v.th);   // row tiles per row phase
    pl->pb = v.d;                                 // row phases
    pl->YH = pl->OH;
    pl->YW = pl->OW;
    pl->total = (long long)pl->nct * v.d * pl->nst * pl->nwt;   // waves
    if (pl->total * 64 >= (1LL << 31))
        return false;
    pl->grid = (pl->total + 3) / 4;
    pl->block = 256;
    pl->xcd = xcd_ranges(p);
    std::snprintf(pl->name, sizeof pl->name,
                  "stream_nchw_planes_s1_k%dx%d_d%d_px%d_th%d_nl%d_%s_%s", v.kH, v.kW, v.d,
                  v.px, v.th, v.nl, op_tag(p), p.wtype ? "f16w" : "f32w");
    return true;
}

static void plan_direct(const Problem &p, std::uintptr_t ptr_bits, Plan *pl)
{
    // channels of the tensor written: mult*C for the forward, C for the input gradient
    const long long cres = p.op == DWCONV_OP_FWD ? (long long)p.mult * p.C : p.C;
    pl->block = 256;
    pl->variant = -1;
    if (p.layout == DWCONV_LAYOUT_NHWC) {
        pl->kind = KIND_DIRECT_NHWC;
        pl->vec = (p.mult == 1 && p.C % 4 == 0 && (ptr_bits & 15u) == 0) ? 4 : 1;
        pl->total = (long long)p.N * pl->OH * pl->OW * (cres / pl->vec);
    } else {
        pl->kind = KIND_DIRECT_NCHW;
        pl->vec = 1;
        pl->total = (long long)p.N * cres * pl->OH * pl->OW;
    }
    pl->grid = (pl->total + pl->block - 1) / pl->block;
    std::snprintf(pl->name, sizeof pl->name, "direct_%s_s%d_v%d_%s_%s",
                  p.layout == DWCONV_LAYOUT_NHWC ? "nhwc" : "nchw", p.stride, pl->vec,
                  op_tag(p), p.wtype ? "f16w" : "f32w");
}

int make_plan(Problem &p, int strategy, std::uintptr_t ptr_bits, Plan *pl)
{
    if (p.op == DWCONV_OP_WEIGHT_GRAD)
        return make_wgrad_plan(p, strategy, ptr_bits, pl);
    int st = validate_problem(p);
    if (st != DWCONV_OK)
        return st;
    if (strategy != DWCONV_STRATEGY_AUTO && strategy != DWCONV_STRATEGY_DIRECT &&
        strategy != DWCONV_STRATEGY_TILED && strategy != DWCONV_STRATEGY_STREAM &&
        strategy != DWCONV_STRATEGY_STREAM_PLANES)
        return DWCONV_ERR_BAD_STRATEGY;
    std::memset(pl, 0, sizeof *pl);
    set_extents(p, pl);
    if (strategy == DWCONV_STRATEGY_DIRECT) {
        plan_direct(p, ptr_bits, pl);
        return DWCONV_OK;
    }
    if (strategy == DWCONV_STRATEGY_STREAM)
        return (p.layout == DWCONV_LAYOUT_NHWC ? plan_stream_nhwc(p, pl) : plan_stream_nchw(p, pl))
                   ? DWCONV_OK
                   : DWCONV_ERR_BAD_STRATEGY;
    if (strategy == DWCONV_STRATEGY_STREAM_PLANES)
        return plan_stream_nchw_planes(p, pl) ? DWCONV_OK : DWCONV_ERR_BAD_STRATEGY;
    // AUTO: the row-streaming kernels for the windows they have variants
    // for, when the problem gives enough waves (NCHW: one plane per lane
    // first)
    if (strategy == DWCONV_STRATEGY_AUTO) {
        Plan t = *pl;
        if (plan_stream_nchw_planes(p, &t) &&
            t.total >= kStreamPlanesVariants[t.variant].minw) {
            *pl = t;
            return DWCONV_OK;
        }
        t = *pl;
        const bool nhwc = p.layout == DWCONV_LAYOUT_NHWC;
        if (nhwc ? plan_stream_nhwc(p, &t) : plan_stream_nchw(p, &t)) {
            const long long waves = nhwc ? t.nct * t.total + t.tail_units : t.total;
            const int minw = nhwc ? kStreamVariants[t.variant].minw
                                  : kStreamNchwVariants[t.variant].minw;
            if (waves >= minw) {
                *pl = t;
                return DWCONV_OK;
            }
        }
    }
    // Tiled kernels: AUTO takes them when they apply and, for NHWC, when the
    // channel count fills at least half of a channel tile.
    Plan t = *pl;
    bool tiled = (p.layout == DWCONV_LAYOUT_NHWC) ? plan_tiled_nhwc(p, ptr_bits, &t)
                                                  : plan_tiled_nchw(p, ptr_bits, &t);
    if (tiled && strategy == DWCONV_STRATEGY_AUTO && p.layout == DWCONV_LAYOUT_NHWC &&
        p.C < 16)
        tiled = false;
    if (tiled) {
        *pl = t;
        pl->xcd = xcd_ranges(p);
        // tensors larger than the Infinity Cache stream past it: rows only
        // one tile stages load non-temporally there (512x512x256 3x3 NHWC:
        // 92.2 -> 88.5 us); smaller ones keep them (32x56x56x128 5x5 NHWC,
        // whose buffers stay cache-resident between calls: 19.0 -> 25.8 us
        // with them non-temporal)
        pl->ntl = pl->kind == KIND_TILED_NHWC && !pl->xcd;
        // large problems: row bands split over the XCDs (NHWC), or bands of
        // 8 plane groups with one plane group's row tiles per XCD (NCHW)
        if (!pl->xcd && (pl->kind == KIND_TILED_NHWC ? (pl->nct * pl->nwt) % 8 == 0
                                                     : pl->nct % 8 == 0))
            pl->xcd = 2;
        return DWCONV_OK;
    }
    if (strategy == DWCONV_STRATEGY_TILED)
        return DWCONV_ERR_BAD_STRATEGY;
    plan_direct(p, ptr_bits, pl);
    return DWCONV_OK;
}

// ---------------------------------------------------------------------------
// Weight gradient.  Stage 1 writes partial sums [chunk][C][kH*kW + 1] (the
// last column is the bias gradient) to the workspace; stage 2 adds the
// chunks of every column in a fixed order.
// ---------------------------------------------------------------------------
// Row tiles per strip of a tiled weight-gradient plan: `base` workgroups
// cover one strip of every (image, column tile, channel / plane group); the
// strip count is the one nearest kWgradTargetWorkgroups / base (at least 1),
// and the nrt row tiles are split evenly between the strips.  Few, long
// strips keep the partial sums (and their reduction) small; the target keeps
// about two workgroups per compute unit on a large image.
static int wgrad_strip(int nrt, long long base)
{
    long long nsp = (2 * kWgradTargetWorkgroups + base) / (2 * base);   // round to nearest
    nsp = std::max<long long>(1, std::min<long long>(nsp, nrt));
    const long long strip = (nrt + nsp - 1) / nsp;
    return (int)strip;
}

static bool plan_wgrad_tiled(const Problem &p, std::uintptr_t ptr_bits, Plan *pl)
{
    if (p.layout != DWCONV_LAYOUT_NHWC)
        return false;
    // a channel multiplier of 2 has its own variants (stride 1, 16-byte staging)
    const bool m2 = p.mult == 2;
    if ((p.mult != 1 && !m2) || (m2 && (p.stride != 1 || p.C % 4 != 0)))
        return false;
    const long long co = (long long)p.mult * p.C;               // dy channels
    const bool v4ok = p.C % 4 == 0 && (ptr_bits & 15u) == 0;   // 16-byte staging loads
    if (4LL * p.H * p.W * p.C >= (1LL << 31) || 4LL * p.Ho * p.Wo * co >= (1LL << 31))
        return false;
    const WgradVariant *table = m2 ? kWgradM2Variants
                                   : p.stride == 1 ? kWgradVariants : kWgradS2Variants;
    const int nvar = m2 ? kNumWgradM2Variants
                        : p.stride == 1 ? kNumWgradVariants : kNumWgradS2Variants;
    int best = -1;
    double best_fill = -1.0;
    for (int i = 0; i < nvar; ++i) {
        const WgradVariant &v = table[i];
        if (v.kH != p.kH || v.kW != p.kW || v.d != p.dilation || (v.lv == 4 && !v4ok))
            continue;
        const int cg = v.cl * v.vec;
        const double fill = (double)co / (ceil_div((int)co, cg) * cg);
        if (fill >= 0.75) {
            best = i;
            break;
        }
        if (fill > best_fill) {
            best = i;
            best_fill = fill;
        }
    }
    if (best < 0)
        return false;
    // stride 1, no multiplier: 3x3 with 48-64 channels takes two 32-channel
    // tiles (8x112x112x64 on MI355X: 20.0 -> 15.7 us; from two tiles on the
    // wider tile stays faster: 512x512x256 95.5 against 124.4 us)
    if (table == kWgradVariants)
        best = split_channel_tile(table, nvar, best, co, 0);
    const WgradVariant &v = table[best];
    const int R = (v.kH - 1) * v.d + 1;
    pl->kind = KIND_WGRAD_TILED_NHWC;
    pl->variant = best;
    pl->vec = v.vec;
    pl->cl = v.cl;
    pl->tw = v.px * 256 / v.cl;                                  // dy columns per tile
    pl->th = (v.g - R) / p.stride + 1;                           // dy rows per row tile
    pl->nrt = ceil_div(p.Ho, pl->th);                            // row tiles per image
    pl->nct = ceil_div((int)co, v.cl * v.vec);
    pl->nwt = ceil_div(p.Wo, pl->tw);
    pl->strip = wgrad_strip(pl->nrt, (long long)p.N * pl->nct * pl->nwt);
    pl->nst = ceil_div(pl->nrt, pl->strip);                      // strips
    pl->chunks = (long long)p.N * pl->nst * pl->nwt;
    pl->grid = pl->chunks * pl->nct;
    pl->block = 256;
    std::snprintf(pl->name, sizeof pl->name,
                  "wgrad_tiled_nhwc_s%d_k%dx%d_d%d_v%d_cl%d_px%d_g%d%s%s_s%d", p.stride, v.kH,
                  v.kW, v.d, v.vec, v.cl, v.px, v.g, v.lv == 1 ? "_l1" : "", m2 ? "_m2" : "",
                  pl->strip);
    return true;
}

static bool plan_wgrad_tiled_nchw(const Problem &p, std::uintptr_t ptr_bits, Plan *pl)
{
    if (p.layout != DWCONV_LAYOUT_NCHW)
        return false;
    const long long co = (long long)p.mult * p.C, planes = p.N * co;
    if (4LL * p.N * p.C * p.H * p.W >= (1LL << 31) || 4LL * planes * p.Ho * p.Wo >= (1LL << 31))
        return false;
    const TiledNchwVariant *table = p.stride == 1 ? kWgradNchwVariants : kWgradNchwS2Variants;
    const int nvar = p.stride == 1 ? kNumWgradNchwVariants : kNumWgradNchwS2Variants;
    const bool v4ok = p.W % 4 == 0 && (ptr_bits & 15u) == 0;
    int best = -1;
    for (int i = 0; i < nvar; ++i) {
        const TiledNchwVariant &v = table[i];
        if (v.kH == p.kH && v.kW == p.kW && v.d == p.dilation && (v.v4 == 0 || v4ok)) {
            best = i;
            break;
        }
    }
    if (best < 0)
        return false;
    const TiledNchwVariant &v = table[best];
    const int R = (v.kH - 1) * v.d + 1;
    const int tx = std::max(16, std::min(256, ceil_div(p.Wo, v.q)));   // threads per dy row
    const int lv = v.v4 ? 4 : 1;
    const int hl = v.v4 ? -((-pl->pW) & ~3) : pl->pW;
    // staged x columns of a row: the left alignment, then the s*(tw-1) + 1
    // columns the tile's dy columns meet, then the window's d*(kW-1)
    const int span = (hl - pl->pW) + p.stride * (tx * v.q - 1) + 1 + v.d * (v.kW - 1);
    pl->kind = KIND_WGRAD_TILED_NCHW;
    pl->variant = best;
    pl->vec = 1;
    pl->cl = tx;
    pl->pb = 256 / tx;
    pl->tw = tx * v.q;
    pl->hl = hl;
    pl->twl = (span + lv - 1) / lv * lv;
    // the kernel's per-thread load registers must cover the staged x tile
    if ((long long)pl->pb * v.g * (pl->twl / lv) >
        256LL * nchw_stage_loads(0, v.g, p.stride * v.q, v.kW, v.d, v.v4 != 0))
        return false;
    pl->th = (v.g - R) / p.stride + 1;                           // dy rows per row tile
    pl->nct = (int)((planes + pl->pb - 1) / pl->pb);
    pl->nwt = ceil_div(p.Wo, pl->tw);
    pl->nrt = ceil_div(p.Ho, pl->th);                            // row tiles per plane
    pl->strip = wgrad_strip(pl->nrt, (long long)pl->nct * pl->nwt);
    pl->nst = ceil_div(pl->nrt, pl->strip);
    pl->chunks = (long long)p.N * pl->nwt * pl->nst;
    pl->grid = (long long)pl->nct * pl->nwt * pl->nst;
    const int kp = (p.kH * p.kW + 1) | 1;                        // per-thread sums, padded
    // the x tile (4-byte staging loads it into LDS by whole waves of 64)
    const int tile_floats = (pl->pb * v.g * (pl->twl / lv) + 63) / 64 * 64 * lv;
    pl->lds_bytes = 4 * std::max(tile_floats, kp * 256);
    if (pl->lds_bytes > kMaxLdsBytes)
        return false;
    pl->block = 256;
    std::snprintf(pl->name, sizeof pl->name, "wgrad_tiled_nchw_s%d_k%dx%d_d%d_q%d_g%d_%s_tx%d_s%d",
                  p.stride, v.kH, v.kW, v.d, v.q, v.g, v.v4 ? "v4" : "v1", tx, pl->strip);
    return true;
}

// Row-streaming NCHW weight gradient: stride 1, no multiplier, a listed
// kernel shape; the NCHW walk's geometry over dy (the forward's output).
static bool plan_wgrad_stream_nchw(const Problem &p, Plan *pl)
{
    if (p.layout != DWCONV_LAYOUT_NCHW || p.stride != 1 || p.mult != 1)
        return false;
    int best = -1;
    for (int i = 0; i < kNumWgradStreamVariants; ++i) {
        const WgradStreamVariant &v = kWgradStreamVariants[i];
        if (v.kH == p.kH && v.kW == p.kW && v.d == p.dilation) {
            best = i;
            break;
        }
    }
    if (best < 0)
        return false;
    const WgradStreamVariant &v = kWgradStreamVariants[best];
    const long long planes = (long long)p.N * p.C;
    if (4LL * planes * p.H * p.W >= (1LL << 31) || 4LL * planes * p.Ho * p.Wo >= (1LL << 31))
        return false;
    const int d = v.d;
    const int ohs = ceil_div(p.Ho, d), ows = ceil_div(p.Wo, d);
    int lpr = ows, ncb = 1;
    if (lpr > 64) {
        ncb = ceil_div(lpr, 64);
        lpr = 64;
    }
    const int pitch = lpr + v.kW - 1;
    const int lpitch = pitch + ((lpr - pitch) % 32 + 32) % 32;
    const int ppw = std::min(std::min(64 / lpr, 64 * v.nl / pitch), kStreamNchwSlot / lpitch);
    if (ppw < 1)
        return false;
    pl->kind = KIND_WGRAD_STREAM_NCHW;
    pl->variant = best;
    pl->vec = 1;
    pl->cl = lpr;
    pl->pb = ppw;
    pl->hl = pitch;
    pl->twl = lpitch;
    pl->tw = lpr;
    pl->th = v.th;
    pl->nwt = ncb;
    pl->nst = ceil_div(ohs, v.th);
    // a unit walks one phase, or all d row phases of one column phase when
    // one-phase units would exceed 4096 waves (more than the 5 a SIMD holds
    // at once would take two rounds; their per-unit reduction also counts
    // more): 64x30x19x128 7x7 d2, 5464 -> 2732 waves, 24.2 -> 22.4 us
    const long long groups = (planes + ppw - 1) / ppw;
    pl->rpu = (d > 1 && groups * d * d * ceil_div(ohs, v.th) * ncb > kWgradStreamPhaseWaves) ? d : 1;
    pl->nct = d * d / pl->rpu;                    // phase units per plane group
    pl->total = (planes + ppw - 1) / ppw * pl->nct * pl->nst * ncb;
    if (pl->total * 4 >= (1LL << 31))
        return false;
    pl->chunks = (long long)p.N * pl->nct * pl->nst * ncb;
    pl->grid = (pl->total + 3) / 4;
    pl->block = 256;
    std::snprintf(pl->name, sizeof pl->name, "wgrad_stream_nchw_s1_k%dx%d_d%d_th%d_nl%d_lpr%d",
                  v.kH, v.kW, v.d, v.th, v.nl, lpr);
    return true;
}

// Row-streaming NHWC weight gradient: stride 1, no multiplier, a listed
// kernel shape.  One chunk of partial sums per workgroup (four waves).
static bool plan_wgrad_stream_nhwc(const Problem &p, Plan *pl)
{
    if (p.layout != DWCONV_LAYOUT_NHWC || p.stride != 1 || p.mult != 1)
        return false;
    int best = -1;
    for (int i = 0; i < kNumWgradStreamNhwcVariants; ++i) {
        const WgradStreamNhwcVariant &v = kWgradStreamNhwcVariants[i];
        if (v.kH == p.kH && v.kW == p.kW && v.d == p.dilation) {
            best = i;
            break;
        }
    }
    if (best < 0)
        return false;
    const WgradStreamNhwcVariant &v = kWgradStreamNhwcVariants[best];
    // byte offsets within a row (a lane's columns, up to (kW-1)*d past the
    // row on either side) and row starts within an image are 32-bit
    const long long cb = 4LL * p.C;
    if (cb * (std::max(p.W, pl->OW) + 2LL * v.d * v.kW + 8LL * v.px * v.d) >= (1LL << 31) ||
        cb * p.H * p.W >= (1LL << 31) || cb * pl->OH * pl->OW >= (1LL << 31))
        return false;
    const int d = v.d;
    const int ohs = ceil_div(pl->OH, d), ows = ceil_div(pl->OW, d);   // phase sub-grid
    pl->kind = KIND_WGRAD_STREAM_NHWC;
    pl->variant = best;
    pl->vec = 1;
    pl->cl = 64;
    pl->tw = v.px;
    pl->th = v.th;
    // leftover channels as a narrower tail tile, as in the forward walk; its
    // workgroups write their partial sums into the first chunks and zeros
    // into the rest of the tail channels' chunks
    pl->tail_cl = stream_tail_cl(p, d);
    pl->nct = pl->tail_cl ? p.C / 64 : ceil_div(p.C, 64);
    pl->nwt = ceil_div(ows, v.px);
    pl->nst = ceil_div(ohs, v.th);
    pl->pb = d * d;                               // phases
    pl->total = (long long)p.N * pl->nst * pl->pb * pl->nwt;      // wave units per channel tile
    pl->tail_ncg = pl->tail_cl ? ceil_div(ows, v.px * (64 / pl->tail_cl)) : 0;
    pl->tail_units = (long long)p.N * pl->nst * pl->pb * pl->tail_ncg;
    if (pl->total * 4 >= (1LL << 31))
        return false;
    pl->chunks = (pl->total + 3) / 4;             // one per workgroup of a channel tile
    pl->grid = pl->nct * pl->chunks + (pl->tail_units + 3) / 4;
    pl->block = 256;
    pl->xcd = xcd_ranges(p);
    char tail[8] = "";
    if (pl->tail_cl)
        std::snprintf(tail, sizeof tail, "_t%d", pl->tail_cl);
    std::snprintf(pl->name, sizeof pl->name, "wgrad_stream_nhwc_s1_k%dx%d_d%d_px%d_th%d%s", v.kH,
                  v.kW, v.d, v.px, v.th, tail);
    return true;
}

static void plan_wgrad_direct(const Problem &p, Plan *pl)
{
    // any layout / stride / padding / multiplier: the generic kernel, with
    // lanes along the contiguous axis and chunks sized for >= ~2048 workgroups
    const long long co = (long long)p.mult * p.C;
    const long long per_img = (long long)pl->OH * pl->OW;
    const long long target_wg = 2048;
    pl->kind = KIND_WGRAD_DIRECT;
    pl->variant = -1;
    pl->block = 256;
    if (p.layout == DWCONV_LAYOUT_NHWC) {
        int cl = 16;
        double best = -1.0;
        for (int c : {64, 32, 16}) {                      // widest lane run that fills >= 3/4
            const double fill = (double)co / ((co + c - 1) / c * c);
            if (fill >= 0.75) {
                cl = c;
                break;
            }
            if (fill > best) {
                best = fill;
                cl = c;
            }
        }
        const long long ncg = (co + cl - 1) / cl, slots = 256 / cl;
        const long long total = p.N * per_img;
        const long long ppt = std::min<long long>(32, std::max<long long>(2, total * ncg / (slots * target_wg)));
        const long long ppc = slots * ppt;
        pl->cl = cl;
        pl->nct = (int)ncg;
        pl->ppc = (int)ppc;
        pl->chunks = (total + ppc - 1) / ppc;
        pl->grid = pl->chunks * ncg;
    } else {
        const long long ppt = std::min<long long>(16, std::max<long long>(2, p.N * per_img * co / (256 * target_wg)));
        const long long ppc = 256 * ppt;
        const long long cpi = (per_img + ppc - 1) / ppc;
        pl->cl = 256;
        pl->nct = 1;
        pl->ppc = (int)ppc;
        pl->cpi = (int)cpi;
        pl->chunks = p.N * cpi;
        pl->grid = pl->chunks * co;
    }
    std::snprintf(pl->name, sizeof pl->name, "wgrad_direct_%s_s%d_cl%d_ppc%d",
                  p.layout == DWCONV_LAYOUT_NHWC ? "nhwc" : "nchw", p.stride, pl->cl, pl->ppc);
}

int make_wgrad_plan(Problem &p, int strategy, std::uintptr_t ptr_bits, Plan *pl)
{
    int st = validate_problem(p);
    if (st != DWCONV_OK)
        return st;
    if (strategy != DWCONV_STRATEGY_AUTO && strategy != DWCONV_STRATEGY_DIRECT &&
        strategy != DWCONV_STRATEGY_TILED && strategy != DWCONV_STRATEGY_STREAM)
        return DWCONV_ERR_BAD_STRATEGY;
    std::memset(pl, 0, sizeof *pl);
    set_extents(p, pl);
    bool tiled = false;
    if (strategy == DWCONV_STRATEGY_STREAM || strategy == DWCONV_STRATEGY_AUTO) {
        Plan t = *pl;
        const bool nhwc = p.layout == DWCONV_LAYOUT_NHWC;
        if (nhwc ? plan_wgrad_stream_nhwc(p, &t) : plan_wgrad_stream_nchw(p, &t)) {
            const long long waves = nhwc ? t.nct * t.total + t.tail_units : t.total;
            const int minw = nhwc ? kWgradStreamNhwcVariants[t.variant].minw
                                  : kWgradStreamVariants[t.variant].minw;
            if (strategy == DWCONV_STRATEGY_STREAM || waves >= minw) {
                *pl = t;
                tiled = true;
            }
        }
        if (!tiled && strategy == DWCONV_STRATEGY_STREAM)
            return DWCONV_ERR_BAD_STRATEGY;
    }
    if (!tiled && strategy != DWCONV_STRATEGY_DIRECT) {
        Plan t = *pl;
        tiled = p.layout == DWCONV_LAYOUT_NHWC ? plan_wgrad_tiled(p, ptr_bits, &t)
                                               : plan_wgrad_tiled_nchw(p, ptr_bits, &t);
        if (tiled) {
            *pl = t;
            pl->xcd = xcd_ranges(p);
            if (!pl->xcd && pl->kind == KIND_WGRAD_TILED_NHWC && (pl->nct * pl->nwt) % 8 == 0)
                pl->xcd = 2;
        } else if (strategy == DWCONV_STRATEGY_TILED)
            return DWCONV_ERR_BAD_STRATEGY;
    }
    if (!tiled)
        plan_wgrad_direct(p, pl);
    const long long cols = (long long)p.mult * p.C * (p.kH * p.kW + 1);
    if (pl->chunks * cols >= (1LL << 31))
        return DWCONV_ERR_BAD_DIM;
    pl->workspace = 4 * pl->chunks * cols;
    // the reduction: 8 chunk slices of 32 columns per workgroup (128-byte
    // runs), 16 slices of 16 columns when there are few columns
    pl->red_s = cols <= kReduceFewColumns ? 16 : 8;
    pl->grid2 = (cols + 256 / pl->red_s - 1) / (256 / pl->red_s);
    return DWCONV_OK;
}

}  // namespace dwconv
