// dwconv_plan.cpp -- argument validation and kernel selection (host only,
// no HIP runtime calls).
//
// Shape rules (LeanMlir "Depthwise" page, forward equation, read with stride
// s and dilation d): pH = d*(kH-1)/2, pW = d*(kW-1)/2 with odd kernels (SAME
// padding), Ho = ceil(H/s), Wo = ceil(W/s).  Selecting the tiling from the
// problem's extents mirrors the cubek-convolution "depthwise" module, whose
// launch space is built from the problem extents and a tiling strategy.
#include "dwconv_internal.h"
#include "../../include/dwconv.h"

#include <algorithm>
#include <cstdio>
#include <cstring>

namespace dwconv {

namespace {

constexpr long long kMaxElems = (1LL << 31) - 1;  // 32-bit element indexing
constexpr int kNumCUs = 256;                       // MI355X compute units

int ceil_div(int a, int b) { return (a + b - 1) / b; }

constexpr bool kHaveTiledNchw = false;

}  // namespace

int validate_problem(const Problem &p)
{
    if (p.op != DWCONV_OP_FWD && p.op != DWCONV_OP_INPUT_GRAD)
        return DWCONV_ERR_BAD_OP;
    if (p.N < 1 || p.H < 1 || p.W < 1 || p.C < 1 || p.kH < 1 || p.kW < 1)
        return DWCONV_ERR_BAD_DIM;
    const long long in_elems = (long long)p.N * p.H * p.W * p.C;
    if (in_elems > kMaxElems || (long long)p.C * p.kH * p.kW > kMaxElems)
        return DWCONV_ERR_BAD_DIM;
    if (p.stride != 1 && p.stride != 2)
        return DWCONV_ERR_BAD_STRIDE;
    if (p.dilation < 1 || (long long)p.dilation * (std::max(p.kH, p.kW) - 1) >= (1 << 16))
        return DWCONV_ERR_BAD_DILATION;
    if (p.kH % 2 == 0 || p.kW % 2 == 0)
        return DWCONV_ERR_EVEN_KERNEL;
    if (p.layout != DWCONV_LAYOUT_NHWC && p.layout != DWCONV_LAYOUT_NCHW)
        return DWCONV_ERR_BAD_LAYOUT;
    if (p.wtype != DWCONV_W_F32 && p.wtype != DWCONV_W_F16)
        return DWCONV_ERR_BAD_WTYPE;
    return DWCONV_OK;
}

static int find_tiled_shape(const Problem &p)
{
    for (int i = 0; i < kNumTiledShapes; ++i)
        if (kTiledShapes[i].kH == p.kH && kTiledShapes[i].kW == p.kW &&
            kTiledShapes[i].d == p.dilation)
            return i;
    return -1;
}

// Strip height: aim for about eight workgroups per compute unit, keeping a
// strip at least one window height tall when the image allows it.
static int pick_strip_rows(int H, long long tiles_per_strip_row, int R)
{
    const long long target = 8LL * kNumCUs;
    long long strips = (target + tiles_per_strip_row - 1) / tiles_per_strip_row;
    if (strips < 1)
        strips = 1;
    int th = (int)std::max<long long>(1, (H + strips - 1) / strips);
    th = std::max(th, std::min(H, R));
    return std::min(th, 64);
}

static bool plan_tiled_nhwc(const Problem &p, std::uintptr_t ptr_bits, Plan *pl)
{
    const int s = find_tiled_shape(p);
    if (s < 0 || p.stride != 1 || p.layout != DWCONV_LAYOUT_NHWC)
        return false;
    if (p.C % 4 != 0 || (ptr_bits & 15u) != 0)
        return false;
    const TiledShape &ts = kTiledShapes[s];
    const int R = (ts.kH - 1) * ts.d + 1;
    pl->kind = KIND_TILED_NHWC;
    pl->shape = s;
    pl->vec = ts.vec;
    pl->cl = (p.C / ts.vec <= 8) ? 8 : 16;
    pl->tw = 256 / pl->cl;
    const int cg = pl->cl * ts.vec;
    pl->nct = ceil_div(p.C, cg);
    pl->nwt = ceil_div(p.W, pl->tw);
    pl->th = pick_strip_rows(p.H, (long long)p.N * pl->nct * pl->nwt, R);
    pl->nst = ceil_div(p.H, pl->th);
    pl->grid = (long long)p.N * pl->nst * pl->nwt * pl->nct;
    pl->block = 256;
    std::snprintf(pl->name, sizeof pl->name, "tiled_nhwc_s1_k%dx%d_d%d_v%d_cl%d_%s_%s",
                  ts.kH, ts.kW, ts.d, ts.vec, pl->cl, p.op ? "ig" : "fwd",
                  p.wtype ? "f16w" : "f32w");
    return true;
}

static bool plan_tiled_nchw(const Problem &p, std::uintptr_t ptr_bits, Plan *pl)
{
    if (!kHaveTiledNchw)
        return false;
    const int s = find_tiled_shape(p);
    if (s < 0 || p.stride != 1 || p.layout != DWCONV_LAYOUT_NCHW)
        return false;
    if (p.W % kNchwQ != 0 || (ptr_bits & 15u) != 0)
        return false;
    const TiledShape &ts = kTiledShapes[s];
    const int R = (ts.kH - 1) * ts.d + 1;
    pl->kind = KIND_TILED_NCHW;
    pl->shape = s;
    pl->vec = 1;
    pl->cl = 0;
    pl->tw = 256 * kNchwQ;  // one workgroup spans up to 1024 output columns
    pl->nct = p.N * p.C;    // planes
    pl->nwt = ceil_div(p.W, pl->tw);
    pl->th = pick_strip_rows(p.H, (long long)pl->nct * pl->nwt, R);
    pl->nst = ceil_div(p.H, pl->th);
    pl->grid = (long long)pl->nct * pl->nwt * pl->nst;
    pl->block = 256;
    std::snprintf(pl->name, sizeof pl->name, "tiled_nchw_s1_k%dx%d_d%d_%s_%s",
                  ts.kH, ts.kW, ts.d, p.op ? "ig" : "fwd", p.wtype ? "f16w" : "f32w");
    return true;
}

static void plan_direct(const Problem &p, std::uintptr_t ptr_bits, Plan *pl)
{
    pl->block = 256;
    pl->shape = -1;
    if (p.layout == DWCONV_LAYOUT_NHWC) {
        pl->kind = KIND_DIRECT_NHWC;
        pl->vec = (p.C % 4 == 0 && (ptr_bits & 15u) == 0) ? 4 : 1;
        pl->total = (long long)p.N * pl->OH * pl->OW * (p.C / pl->vec);
    } else {
        pl->kind = KIND_DIRECT_NCHW;
        pl->vec = 1;
        pl->total = (long long)p.N * p.C * pl->OH * pl->OW;
    }
    pl->grid = (pl->total + pl->block - 1) / pl->block;
    std::snprintf(pl->name, sizeof pl->name, "direct_%s_s%d_v%d_%s_%s",
                  p.layout == DWCONV_LAYOUT_NHWC ? "nhwc" : "nchw", p.stride, pl->vec,
                  p.op ? "ig" : "fwd", p.wtype ? "f16w" : "f32w");
}

int make_plan(const Problem &p, int strategy, std::uintptr_t ptr_bits, Plan *pl)
{
    int st = validate_problem(p);
    if (st != DWCONV_OK)
        return st;
    if (strategy != DWCONV_STRATEGY_AUTO && strategy != DWCONV_STRATEGY_DIRECT &&
        strategy != DWCONV_STRATEGY_TILED)
        return DWCONV_ERR_BAD_STRATEGY;
    std::memset(pl, 0, sizeof *pl);
    const int Ho = ceil_div(p.H, p.stride), Wo = ceil_div(p.W, p.stride);
    pl->pH = p.dilation * (p.kH - 1) / 2;
    pl->pW = p.dilation * (p.kW - 1) / 2;
    if (p.op == DWCONV_OP_FWD) {
        pl->IH = p.H; pl->IW = p.W; pl->OH = Ho; pl->OW = Wo;
    } else {
        pl->IH = Ho; pl->IW = Wo; pl->OH = p.H; pl->OW = p.W;
    }
    if (strategy == DWCONV_STRATEGY_DIRECT) {
        plan_direct(p, ptr_bits, pl);
        return DWCONV_OK;
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
        return DWCONV_OK;
    }
    if (strategy == DWCONV_STRATEGY_TILED)
        return DWCONV_ERR_BAD_STRATEGY;
    plan_direct(p, ptr_bits, pl);
    return DWCONV_OK;
}

}  // namespace dwconv
