// dwconv_api.cpp -- the extern "C" entry points of libdwconv (include/dwconv.h).
//
// Order of work in every entry point: validate the arguments (pointers,
// alignment, overlap, dimensions, enums) without touching the GPU, make the
// plan, then enqueue one kernel.  Rejecting an unsupported configuration up
// front follows the pages' lesson that a late failure (a verifier error deep
// in a compiler pipeline, Reactant.jl issue #331) is worse than an early
// ValueError (ExecuTorch's MLX conv-transpose weight path).
#include "../../include/dwconv.h"
#include "dwconv_internal.h"

#include <cmath>
#include <cstdint>
#include <cstring>

using dwconv::Plan;
using dwconv::Problem;

namespace {

struct Range {
    std::uintptr_t lo, hi;  // [lo, hi)
};

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

Range range_of(const void *p, long long bytes)
{
    const std::uintptr_t lo = reinterpret_cast<std::uintptr_t>(p);
    return Range{lo, lo + static_cast<std::uintptr_t>(bytes)};
}

int check_pointers(const Problem &p, const float *in, const void *w, const float *b,
                   const float *out)
{
    if (!in || !w || !out)
        return DWCONV_ERR_NULL_PTR;
    const std::uintptr_t f32_bits = reinterpret_cast<std::uintptr_t>(in) |
                                    reinterpret_cast<std::uintptr_t>(out) |
                                    reinterpret_cast<std::uintptr_t>(b);
    if ((f32_bits & 3u) != 0)
        return DWCONV_ERR_MISALIGNED;
    const std::uintptr_t wbits = reinterpret_cast<std::uintptr_t>(w);
    if ((p.wtype == DWCONV_W_F32 && (wbits & 3u)) || (wbits & 1u))
        return DWCONV_ERR_MISALIGNED;
    const long long co = (long long)p.mult * p.C;
    const long long big = 4LL * p.N * p.H * p.W * p.C, small = 4LL * p.N * p.Ho * p.Wo * co;
    const long long in_bytes = p.op == DWCONV_OP_FWD ? big : small;
    const long long out_bytes = p.op == DWCONV_OP_FWD ? small : big;
    const long long w_bytes = co * p.kH * p.kW * (p.wtype == DWCONV_W_F16 ? 2 : 4);
    const Range o = range_of(out, out_bytes);
    if (overlap(o, range_of(in, in_bytes)) || overlap(o, range_of(w, w_bytes)))
        return DWCONV_ERR_ALIAS;
    if (b && overlap(o, range_of(b, 4LL * co)))
        return DWCONV_ERR_ALIAS;
    return DWCONV_OK;
}

int run(Problem p, const float *in, const void *w, const float *b, float *out, int strategy,
        void *stream, const dwconv::Epilogue *epi = nullptr)
{
    if (p.op != DWCONV_OP_FWD && p.op != DWCONV_OP_INPUT_GRAD)
        return DWCONV_ERR_BAD_OP;
    int st = dwconv::validate_problem(p);
    if (st != DWCONV_OK)
        return st;
    if (p.op == DWCONV_OP_INPUT_GRAD && b)
        return DWCONV_ERR_BAD_OP;
    st = check_pointers(p, in, w, b, out);
    if (st != DWCONV_OK)
        return st;
    Plan pl;
    // the kernels' vector loads and stores (16-byte staging, 4-channel bias
    // and BatchNorm loads, vector stores) are chosen only when every float
    // array they touch is 16-byte aligned
    std::uintptr_t bits = reinterpret_cast<std::uintptr_t>(in) |
                          reinterpret_cast<std::uintptr_t>(out) |
                          reinterpret_cast<std::uintptr_t>(b);
    if (epi && epi->gamma)
        bits |= reinterpret_cast<std::uintptr_t>(epi->gamma) |
                reinterpret_cast<std::uintptr_t>(epi->beta) |
                reinterpret_cast<std::uintptr_t>(epi->mean) |
                reinterpret_cast<std::uintptr_t>(epi->var);
    st = dwconv::make_plan(p, strategy, bits, &pl);
    if (st != DWCONV_OK)
        return st;
    return dwconv::launch_plan(p, pl, in, w, b, out, stream, epi);
}

// Problem with explicit pads (host array top, bottom, left, right) and a
// channel multiplier.  Returns DWCONV_ERR_NULL_PTR for a NULL pads array.
int general_problem(int op, int wtype, int has_bias, int N, int H, int W, int C, int mult,
                    int kH, int kW, int stride, int dilation, const int *pads, int layout,
                    Problem *p)
{
    if (!pads)
        return DWCONV_ERR_NULL_PTR;
    *p = dwconv::same_problem(op, wtype, has_bias, N, H, W, C, kH, kW, stride, dilation,
                              layout);
    p->same = 0;
    p->mult = mult;
    p->pt = pads[0]; p->pb = pads[1]; p->pl = pads[2]; p->pr = pads[3];
    return DWCONV_OK;
}

int describe(Problem p, int strategy, char *name, int name_len, long long *grid, int *block,
             std::uintptr_t addr_bits = 0)
{
    if ((p.op == DWCONV_OP_INPUT_GRAD || p.op == DWCONV_OP_WEIGHT_GRAD) && p.has_bias)
        return DWCONV_ERR_BAD_OP;
    Plan pl;
    const int st = dwconv::make_plan(p, strategy, addr_bits, &pl);
    if (st != DWCONV_OK)
        return st;
    if (name && name_len > 0) {
        std::strncpy(name, pl.name, (size_t)name_len - 1);
        name[name_len - 1] = '\0';
    }
    if (grid)
        *grid = pl.grid;
    if (block)
        *block = pl.block;
    return DWCONV_OK;
}

int wgrad_workspace(Problem p, int strategy, long long *bytes)
{
    if (!bytes)
        return DWCONV_ERR_NULL_PTR;
    // The plan depends on pointer alignment, which is not known here: report
    // the larger of the aligned plan and the fallback plan.
    Plan a, u;
    int st = dwconv::make_plan(p, strategy, 0, &a);
    if (st != DWCONV_OK)
        return st;
    const long long need_a = a.workspace;
    long long need_u = 0;
    if (dwconv::make_plan(p, strategy, 4, &u) == DWCONV_OK)
        need_u = u.workspace;
    *bytes = need_a > need_u ? need_a : need_u;
    return DWCONV_OK;
}

int wgrad(Problem p, const float *x, const float *dy, float *dw, float *db, void *workspace,
          long long workspace_bytes, int strategy, void *stream, float *w_upd = nullptr,
          float *b_upd = nullptr, float lr = 0.0f)
{
    int st = dwconv::validate_problem(p);
    if (st != DWCONV_OK)
        return st;
    if (!x || !dy || (!dw && !w_upd))
        return DWCONV_ERR_NULL_PTR;
    const std::uintptr_t bits = reinterpret_cast<std::uintptr_t>(x) |
                                reinterpret_cast<std::uintptr_t>(dy) |
                                reinterpret_cast<std::uintptr_t>(dw) |
                                reinterpret_cast<std::uintptr_t>(db) |
                                reinterpret_cast<std::uintptr_t>(w_upd) |
                                reinterpret_cast<std::uintptr_t>(b_upd);
    if ((bits & 3u) != 0)
        return DWCONV_ERR_MISALIGNED;
    Plan pl;
    st = dwconv::make_plan(p, strategy,
                           reinterpret_cast<std::uintptr_t>(x) |
                               reinterpret_cast<std::uintptr_t>(dy), &pl);
    if (st != DWCONV_OK)
        return st;
    if (!workspace || (reinterpret_cast<std::uintptr_t>(workspace) & 15u) != 0 ||
        workspace_bytes < pl.workspace)
        return DWCONV_ERR_WORKSPACE;
    const long long co = (long long)p.mult * p.C;
    const Range rx = range_of(x, 4LL * p.N * p.H * p.W * p.C);
    const Range rg = range_of(dy, 4LL * p.N * p.Ho * p.Wo * co);
    const Range none{0, 0};
    const long long wbytes = 4LL * co * p.kH * p.kW;
    // everything the call writes: gradients, workspace, updated weights / bias
    const Range outs[5] = {dw ? range_of(dw, wbytes) : none, range_of(workspace, pl.workspace),
                           db ? range_of(db, 4LL * co) : none,
                           w_upd ? range_of(w_upd, wbytes) : none,
                           (w_upd && b_upd) ? range_of(b_upd, 4LL * co) : none};
    for (int i = 0; i < 5; ++i) {
        if (outs[i].hi == outs[i].lo)
            continue;
        if (overlap(outs[i], rx) || overlap(outs[i], rg))
            return DWCONV_ERR_ALIAS;
        for (int j = i + 1; j < 5; ++j)
            if (outs[j].hi != outs[j].lo && overlap(outs[i], outs[j]))
                return DWCONV_ERR_ALIAS;
    }
    return dwconv::launch_wgrad(p, pl, x, dy, dw, db, workspace, stream, w_upd, b_upd, lr);
}

}  // namespace

extern "C" {

int dwconv2d_fwd(const float *x, const void *w, int wtype, const float *b, float *y,
                 int N, int H, int W, int C, int kH, int kW,
                 int stride, int dilation, int layout, void *stream)
{
    const Problem p = dwconv::same_problem(DWCONV_OP_FWD, wtype, b != nullptr, N, H, W, C, kH,
                                           kW, stride, dilation, layout);
    return run(p, x, w, b, y, DWCONV_STRATEGY_AUTO, stream);
}

int dwconv2d_input_grad(const float *dy, const void *w, int wtype, float *dx,
                        int N, int H, int W, int C, int kH, int kW,
                        int stride, int dilation, int layout, void *stream)
{
    const Problem p = dwconv::same_problem(DWCONV_OP_INPUT_GRAD, wtype, 0, N, H, W, C, kH, kW,
                                           stride, dilation, layout);
    return run(p, dy, w, nullptr, dx, DWCONV_STRATEGY_AUTO, stream);
}

int dwconv2d_launch(int op, const float *in, const void *w, int wtype, const float *b,
                    float *out, int N, int H, int W, int C, int kH, int kW,
                    int stride, int dilation, int layout, int strategy, void *stream)
{
    const Problem p = dwconv::same_problem(op, wtype, b != nullptr, N, H, W, C, kH, kW, stride,
                                           dilation, layout);
    return run(p, in, w, b, out, strategy, stream);
}

int dwconv2d_describe(int op, int wtype, int has_bias, int N, int H, int W, int C,
                      int kH, int kW, int stride, int dilation, int layout, int strategy,
                      char *name, int name_len, long long *grid, int *block)
{
    const Problem p = dwconv::same_problem(op, wtype, has_bias, N, H, W, C, kH, kW, stride,
                                           dilation, layout);
    return describe(p, strategy, name, name_len, grid, block);
}

int dwconv2d_weight_grad_workspace_size(int N, int H, int W, int C, int kH, int kW,
                                        int stride, int dilation, int layout, int strategy,
                                        long long *bytes)
{
    const Problem p = dwconv::same_problem(DWCONV_OP_WEIGHT_GRAD, DWCONV_W_F32, 0, N, H, W, C,
                                           kH, kW, stride, dilation, layout);
    return wgrad_workspace(p, strategy, bytes);
}

int dwconv2d_weight_grad(const float *x, const float *dy, float *dw, float *db,
                         void *workspace, long long workspace_bytes,
                         int N, int H, int W, int C, int kH, int kW,
                         int stride, int dilation, int layout, int strategy, void *stream)
{
    const Problem p = dwconv::same_problem(DWCONV_OP_WEIGHT_GRAD, DWCONV_W_F32, 0, N, H, W, C,
                                           kH, kW, stride, dilation, layout);
    return wgrad(p, x, dy, dw, db, workspace, workspace_bytes, strategy, stream);
}

int dwconv2d_same_pads(int mode, int H, int W, int kH, int kW, int stride, int dilation,
                       int *pads)
{
    if (!pads)
        return DWCONV_ERR_NULL_PTR;
    if (H < 1 || W < 1 || kH < 1 || kW < 1)
        return DWCONV_ERR_BAD_DIM;
    if (stride != 1 && stride != 2)
        return DWCONV_ERR_BAD_STRIDE;
    if (dilation < 1 || (long long)dilation * ((kH > kW ? kH : kW) - 1) >= (1 << 16))
        return DWCONV_ERR_BAD_DILATION;
    if (kH % 2 == 0 || kW % 2 == 0)
        return DWCONV_ERR_EVEN_KERNEL;
    if (mode != DWCONV_PAD_SAME && mode != DWCONV_PAD_XLA_SAME)
        return DWCONV_ERR_BAD_PAD;
    const int ph = dilation * (kH - 1) / 2, pw = dilation * (kW - 1) / 2;
    // XLA-SAME at stride 2 keeps the odd positions of the stride-1 result:
    // one pad less before, and floor(n/2) outputs
    const int shift = (mode == DWCONV_PAD_XLA_SAME && stride == 2) ? 1 : 0;
    pads[0] = ph - shift; pads[1] = ph;
    pads[2] = pw - shift; pads[3] = pw;
    return DWCONV_OK;
}

int dwconv2d_out_extents(int H, int W, int kH, int kW, int stride, int dilation,
                         const int *pads, int *Ho, int *Wo)
{
    Problem p;
    int st = general_problem(DWCONV_OP_FWD, DWCONV_W_F32, 0, 1, H, W, 1, 1, kH, kW, stride,
                             dilation, pads, DWCONV_LAYOUT_NHWC, &p);
    if (st != DWCONV_OK)
        return st;
    st = dwconv::validate_problem(p);
    if (st != DWCONV_OK)
        return st;
    if (Ho)
        *Ho = p.Ho;
    if (Wo)
        *Wo = p.Wo;
    return DWCONV_OK;
}

int dwconv2d_launch_ex(int op, const float *in, const void *w, int wtype, const float *b,
                       float *out, int N, int H, int W, int C, int mult, int kH, int kW,
                       int stride, int dilation, const int *pads, int layout, int strategy,
                       void *stream)
{
    Problem p;
    const int st = general_problem(op, wtype, b != nullptr, N, H, W, C, mult, kH, kW, stride,
                                   dilation, pads, layout, &p);
    if (st != DWCONV_OK)
        return st;
    return run(p, in, w, b, out, strategy, stream);
}

int dwconv2d_describe_ex(int op, int wtype, int has_bias, int N, int H, int W, int C, int mult,
                         int kH, int kW, int stride, int dilation, const int *pads, int layout,
                         int strategy, char *name, int name_len, long long *grid, int *block)
{
    Problem p;
    const int st = general_problem(op, wtype, has_bias, N, H, W, C, mult, kH, kW, stride,
                                   dilation, pads, layout, &p);
    if (st != DWCONV_OK)
        return st;
    return describe(p, strategy, name, name_len, grid, block);
}

int dwconv2d_describe_addr_ex(int op, int wtype, int has_bias, int N, int H, int W, int C,
                              int mult, int kH, int kW, int stride, int dilation, const int *pads,
                              int layout, int strategy, unsigned long long addr_bits, char *name,
                              int name_len, long long *grid, int *block)
{
    Problem p;
    const int st = general_problem(op, wtype, has_bias, N, H, W, C, mult, kH, kW, stride,
                                   dilation, pads, layout, &p);
    if (st != DWCONV_OK)
        return st;
    return describe(p, strategy, name, name_len, grid, block,
                    static_cast<std::uintptr_t>(addr_bits));
}

int dwconv2d_weight_grad_workspace_size_ex(int N, int H, int W, int C, int mult, int kH, int kW,
                                           int stride, int dilation, const int *pads,
                                           int layout, int strategy, long long *bytes)
{
    Problem p;
    const int st = general_problem(DWCONV_OP_WEIGHT_GRAD, DWCONV_W_F32, 0, N, H, W, C, mult, kH,
                                   kW, stride, dilation, pads, layout, &p);
    if (st != DWCONV_OK)
        return st;
    return wgrad_workspace(p, strategy, bytes);
}

int dwconv2d_fwd_bn_act_ex(const float *x, const void *w, int wtype, const float *b,
                           const float *gamma, const float *beta, const float *mean,
                           const float *var, float eps, int act, float *y,
                           int N, int H, int W, int C, int mult, int kH, int kW, int stride,
                           int dilation, const int *pads, int layout, int strategy, void *stream)
{
    Problem p;
    int st = general_problem(DWCONV_OP_FWD, wtype, b != nullptr, N, H, W, C, mult, kH, kW, stride,
                             dilation, pads, layout, &p);
    if (st != DWCONV_OK)
        return st;
    p.epi = 1;
    if (act < DWCONV_ACT_NONE || act > DWCONV_ACT_SILU)
        return DWCONV_ERR_BAD_EPILOGUE;
    const int nbn = (gamma != nullptr) + (beta != nullptr) + (mean != nullptr) + (var != nullptr);
    if (nbn != 0 && nbn != 4)
        return DWCONV_ERR_BAD_EPILOGUE;
    if (nbn == 4 && !(std::isfinite(eps) && eps >= 0.0f))
        return DWCONV_ERR_BAD_EPILOGUE;
    const float *bn[4] = {gamma, beta, mean, var};
    if (nbn == 4) {
        st = dwconv::validate_problem(p);   // Ho, Wo for the overlap checks
        if (st != DWCONV_OK)
            return st;
        const Range ry = range_of(y, 4LL * p.N * p.Ho * p.Wo * p.mult * p.C);
        for (int i = 0; i < 4; ++i) {
            if (reinterpret_cast<std::uintptr_t>(bn[i]) & 3u)
                return DWCONV_ERR_MISALIGNED;
            if (y && overlap(ry, range_of(bn[i], 4LL * p.mult * p.C)))
                return DWCONV_ERR_ALIAS;
        }
    }
    const dwconv::Epilogue epi{gamma, beta, mean, var, eps, act};
    return run(p, x, w, b, y, strategy, stream, &epi);
}

int dwconv2d_weight_grad_sgd_ex(const float *x, const float *dy, float *w, float *b, float lr,
                                float *dw, float *db, void *workspace, long long workspace_bytes,
                                int N, int H, int W, int C, int mult, int kH, int kW, int stride,
                                int dilation, const int *pads, int layout, int strategy,
                                void *stream)
{
    Problem p;
    const int st = general_problem(DWCONV_OP_WEIGHT_GRAD, DWCONV_W_F32, 0, N, H, W, C, mult, kH,
                                   kW, stride, dilation, pads, layout, &p);
    if (st != DWCONV_OK)
        return st;
    if (!w)
        return DWCONV_ERR_NULL_PTR;
    if (!std::isfinite(lr))
        return DWCONV_ERR_BAD_EPILOGUE;
    return wgrad(p, x, dy, dw, db, workspace, workspace_bytes, strategy, stream, w, b, lr);
}

int dwconv2d_weight_grad_ex(const float *x, const float *dy, float *dw, float *db,
                            void *workspace, long long workspace_bytes,
                            int N, int H, int W, int C, int mult, int kH, int kW,
                            int stride, int dilation, const int *pads, int layout, int strategy,
                            void *stream)
{
    Problem p;
    const int st = general_problem(DWCONV_OP_WEIGHT_GRAD, DWCONV_W_F32, 0, N, H, W, C, mult, kH,
                                   kW, stride, dilation, pads, layout, &p);
    if (st != DWCONV_OK)
        return st;
    return wgrad(p, x, dy, dw, db, workspace, workspace_bytes, strategy, stream);
}

int dwconv2d_weight_grad_noalloc_ex(const float *x, const float *dy, float *dw, float *db,
                                    int N, int H, int W, int C, int mult, int kH, int kW,
                                    int stride, int dilation, const int *pads, int layout,
                                    int strategy, void *stream)
{
    static_assert(DWCONV_SCRATCH_BYTES == dwconv::kScratchBytes, "one scratch size");
    Problem p;
    int st = general_problem(DWCONV_OP_WEIGHT_GRAD, DWCONV_W_F32, 0, N, H, W, C, mult, kH, kW,
                             stride, dilation, pads, layout, &p);
    if (st != DWCONV_OK)
        return st;
    st = dwconv::validate_problem(p);
    if (st != DWCONV_OK)
        return st;
    if (!x || !dy || !dw)
        return DWCONV_ERR_NULL_PTR;
    // the plan the launch below makes (same pointers, same choice)
    Plan pl;
    st = dwconv::make_plan(p, strategy,
                           reinterpret_cast<std::uintptr_t>(x) |
                               reinterpret_cast<std::uintptr_t>(dy), &pl);
    if (st != DWCONV_OK)
        return st;
    if (pl.workspace > dwconv::kScratchBytes)
        return DWCONV_ERR_SCRATCH;
    void *scr = nullptr;
    st = dwconv::scratch_buffer(stream, &scr);
    if (st != DWCONV_OK)
        return st;
    return wgrad(p, x, dy, dw, db, scr, dwconv::kScratchBytes, strategy, stream);
}

const char *dwconv2d_strerror(int status)
{
    switch (status) {
    case DWCONV_OK: return "ok";
    case DWCONV_ERR_NULL_PTR: return "null tensor pointer";
    case DWCONV_ERR_BAD_DIM: return "bad dimension (< 1, no output position, or a tensor of 2^31 or more elements)";
    case DWCONV_ERR_BAD_STRIDE: return "stride must be 1 or 2";
    case DWCONV_ERR_BAD_DILATION: return "dilation must be >= 1 and d*(k-1) < 65536";
    case DWCONV_ERR_EVEN_KERNEL: return "kernel extents must be odd (SAME padding)";
    case DWCONV_ERR_BAD_LAYOUT: return "unknown layout";
    case DWCONV_ERR_BAD_WTYPE: return "unknown weight type";
    case DWCONV_ERR_ALIAS: return "output overlaps an input";
    case DWCONV_ERR_MISALIGNED: return "misaligned tensor pointer";
    case DWCONV_ERR_LAUNCH: return "kernel launch failed";
    case DWCONV_ERR_BAD_OP: return "unknown op, or a bias given to the input gradient";
    case DWCONV_ERR_BAD_STRATEGY: return "unknown strategy, or it does not apply to this problem";
    case DWCONV_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case DWCONV_ERR_BAD_PAD: return "pad out of range (|pad| >= 65536) or unknown padding mode";
    case DWCONV_ERR_BAD_EPILOGUE:
        return "bad epilogue: unknown activation, partial BatchNorm, bad eps or learning rate";
    case DWCONV_ERR_SCRATCH:
        return "allocation-free weight gradient: needs more than the library's 16 MiB scratch "
               "array, or the stream is not on the current device";
    default: return "unknown status";
    }
}

int dwconv2d_version(void) { return 200; }

}  // extern "C"
