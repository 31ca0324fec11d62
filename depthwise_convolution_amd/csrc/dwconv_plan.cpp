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

int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace

int validate_problem(const Problem &p)
{
    if (p.op != DWCONV_OP_FWD && p.op != DWCONV_OP_INPUT_GRAD && p.op != DWCONV_OP_WEIGHT_GRAD)
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

static bool plan_tiled_nhwc(const Problem &p, std::uintptr_t ptr_bits, Plan *pl)
{
    if (p.stride != 1 || p.layout != DWCONV_LAYOUT_NHWC)
        return false;
    if (p.C % 4 != 0 || (ptr_bits & 15u) != 0)
        return false;
    // buffer-load byte offsets are 31-bit: one image and the weights must fit
    if (4LL * p.H * p.W * p.C >= (1LL << 31) || 4LL * p.C * p.kH * p.kW >= (1LL << 31))
        return false;
    // first variant of this kernel shape (table order = preference) whose
    // channel tile the problem fills to at least 3/4; else the one it fills best
    int best = -1;
    double best_fill = -1.0;
    for (int i = 0; i < kNumTiledVariants; ++i) {
        const TiledVariant &v = kTiledVariants[i];
        if (v.kH != p.kH || v.kW != p.kW || v.d != p.dilation)
            continue;
        const int cg = v.cl * v.vec;
        const double fill = (double)p.C / (ceil_div(p.C, cg) * cg);
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
    const TiledVariant &v = kTiledVariants[best];
    const int R = (v.kH - 1) * v.d + 1;
    pl->kind = KIND_TILED_NHWC;
    pl->variant = best;
    pl->vec = v.vec;
    pl->cl = v.cl;
    pl->tw = v.px * 256 / v.cl;
    pl->th = v.g - R + 1;
    pl->nct = ceil_div(p.C, v.cl * v.vec);
    pl->nwt = ceil_div(p.W, pl->tw);
    pl->nst = ceil_div(p.H, pl->th);
    pl->grid = (long long)p.N * pl->nct * pl->nwt * pl->nst;
    pl->block = 256;
    std::snprintf(pl->name, sizeof pl->name, "tiled_nhwc_s1_k%dx%d_d%d_v%d_cl%d_px%d_g%d_%s_%s",
                  v.kH, v.kW, v.d, v.vec, v.cl, v.px, v.g, p.op ? "ig" : "fwd",
                  p.wtype ? "f16w" : "f32w");
    return true;
}

static bool plan_tiled_nchw(const Problem &p, std::uintptr_t ptr_bits, Plan *pl)
{
    if (p.stride != 1 || p.layout != DWCONV_LAYOUT_NCHW)
        return false;
    // buffer-load byte offsets are 31-bit: the whole tensor and the weights must fit
    if (4LL * p.N * p.C * p.H * p.W >= (1LL << 31) || 4LL * p.C * p.kH * p.kW >= (1LL << 31))
        return false;
    const bool v4ok = p.W % 4 == 0 && (ptr_bits & 15u) == 0;
    int best = -1;
    for (int i = 0; i < kNumTiledNchwVariants; ++i) {
        const TiledNchwVariant &v = kTiledNchwVariants[i];
        if (v.kH == p.kH && v.kW == p.kW && v.d == p.dilation && (v.v4 == 0 || v4ok)) {
            best = i;
            break;
        }
    }
    if (best < 0)
        return false;
    const TiledNchwVariant &v = kTiledNchwVariants[best];
    const int R = (v.kH - 1) * v.d + 1;
    int tx = 16;                                 // threads per plane row: pow2 >= W/q, >= 16
    while (tx < 256 && tx * v.q < p.W)
        tx *= 2;
    const int pW = v.d * (v.kW - 1) / 2;
    const int halo = v.v4 ? (pW + 3) / 4 * 4 : pW;
    pl->kind = KIND_TILED_NCHW;
    pl->variant = best;
    pl->vec = 1;
    pl->cl = tx;
    pl->pb = 256 / tx;
    pl->tw = tx * v.q;
    pl->th = v.g - R + 1;
    pl->nct = ceil_div(p.N * p.C, pl->pb);
    pl->nwt = ceil_div(p.W, pl->tw);
    pl->nst = ceil_div(p.H, pl->th);
    pl->lds_bytes = 4 * (pl->pb * v.g * (pl->tw + 2 * halo) + pl->pb * v.kH * v.kW);
    pl->grid = (long long)pl->nct * pl->nwt * pl->nst;
    pl->block = 256;
    std::snprintf(pl->name, sizeof pl->name, "tiled_nchw_s1_k%dx%d_d%d_q%d_g%d_%s_tx%d_%s_%s",
                  v.kH, v.kW, v.d, v.q, v.g, v.v4 ? "v4" : "v1", tx, p.op ? "ig" : "fwd",
                  p.wtype ? "f16w" : "f32w");
    return true;
}

static void plan_direct(const Problem &p, std::uintptr_t ptr_bits, Plan *pl)
{
    pl->block = 256;
    pl->variant = -1;
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
    if (p.op == DWCONV_OP_WEIGHT_GRAD)
        return make_wgrad_plan(p, strategy, ptr_bits, pl);
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

// ---------------------------------------------------------------------------
// Weight gradient.  Stage 1 writes partial sums [chunk][C][kH*kW + 1] (the
// last column is the bias gradient) to the workspace; stage 2 adds the
// chunks of every column in a fixed order.
// ---------------------------------------------------------------------------
static bool plan_wgrad_tiled(const Problem &p, std::uintptr_t ptr_bits, Plan *pl)
{
    if (p.stride != 1 || p.layout != DWCONV_LAYOUT_NHWC || p.C % 4 != 0 || (ptr_bits & 15u))
        return false;
    if (4LL * p.H * p.W * p.C >= (1LL << 31))
        return false;
    int best = -1;
    double best_fill = -1.0;
    for (int i = 0; i < kNumWgradVariants; ++i) {
        const WgradVariant &v = kWgradVariants[i];
        if (v.kH != p.kH || v.kW != p.kW || v.d != p.dilation)
            continue;
        const int cg = v.cl * v.vec;
        const double fill = (double)p.C / (ceil_div(p.C, cg) * cg);
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
    const WgradVariant &v = kWgradVariants[best];
    const int R = (v.kH - 1) * v.d + 1;
    pl->kind = KIND_WGRAD_TILED_NHWC;
    pl->variant = best;
    pl->vec = v.vec;
    pl->cl = v.cl;
    pl->tw = v.px * 256 / v.cl;
    pl->th = v.g - R + 1;
    pl->strip = v.strip;
    pl->nct = ceil_div(p.C, v.cl * v.vec);
    pl->nwt = ceil_div(p.W, pl->tw);
    pl->nst = ceil_div(ceil_div(p.H, pl->th), v.strip);   // strips
    pl->chunks = (long long)p.N * pl->nst * pl->nwt;
    pl->grid = pl->chunks * pl->nct;
    pl->block = 256;
    std::snprintf(pl->name, sizeof pl->name, "wgrad_tiled_nhwc_s1_k%dx%d_d%d_v%d_cl%d_px%d_g%d_s%d",
                  v.kH, v.kW, v.d, v.vec, v.cl, v.px, v.g, v.strip);
    return true;
}

static void plan_wgrad_direct(const Problem &p, Plan *pl)
{
    const long long positions = (long long)p.N * pl->OH * pl->OW;   // dy positions
    pl->kind = KIND_WGRAD_DIRECT;
    pl->variant = -1;
    pl->chunks = (positions + kWgradChunk - 1) / kWgradChunk;
    pl->grid = pl->chunks * p.C;
    pl->block = 256;
    std::snprintf(pl->name, sizeof pl->name, "wgrad_direct_%s_s%d",
                  p.layout == DWCONV_LAYOUT_NHWC ? "nhwc" : "nchw", p.stride);
}

int make_wgrad_plan(const Problem &p, int strategy, std::uintptr_t ptr_bits, Plan *pl)
{
    int st = validate_problem(p);
    if (st != DWCONV_OK)
        return st;
    if (strategy != DWCONV_STRATEGY_AUTO && strategy != DWCONV_STRATEGY_DIRECT &&
        strategy != DWCONV_STRATEGY_TILED)
        return DWCONV_ERR_BAD_STRATEGY;
    std::memset(pl, 0, sizeof *pl);
    pl->pH = p.dilation * (p.kH - 1) / 2;
    pl->pW = p.dilation * (p.kW - 1) / 2;
    pl->IH = p.H; pl->IW = p.W;
    pl->OH = ceil_div(p.H, p.stride); pl->OW = ceil_div(p.W, p.stride);
    bool tiled = false;
    if (strategy != DWCONV_STRATEGY_DIRECT) {
        Plan t = *pl;
        tiled = plan_wgrad_tiled(p, ptr_bits, &t);
        if (tiled)
            *pl = t;
        else if (strategy == DWCONV_STRATEGY_TILED)
            return DWCONV_ERR_BAD_STRATEGY;
    }
    if (!tiled)
        plan_wgrad_direct(p, pl);
    const long long cols = (long long)p.C * (p.kH * p.kW + 1);
    if (pl->chunks * cols >= (1LL << 31))
        return DWCONV_ERR_BAD_DIM;
    pl->workspace = 4 * pl->chunks * cols;
    pl->grid2 = (cols + 15) / 16;
    return DWCONV_OK;
}

}  // namespace dwconv
