// dwconv_direct.hip -- direct kernels: one thread per output (NCHW) or per
// channel vector (NHWC), taps read from global memory through the caches.
// They run every valid problem the tiled kernels do not: any kernel shape
// (even ones with explicit pads), stride 1 or 2, any pads, channel
// multipliers, misaligned pointers.
#include "dwconv_device.h"

namespace dwconv {

namespace {

struct DirectArgs {
    int N, CI, CO, mult;  // channels of the tensor read / written; channel multiplier
    int kH, kW, d, pH, pW;
    int IH, IW, OH, OW;   // extents of the tensor read and the tensor written
    int total;            // threads that do work
};

// ---------------------------------------------------------------------------
// Direct kernels.  A thread computes V consecutive channels r of one output
// position of the tensor written.
// Forward:  out[oh,ow,r] = b[r] + sum_taps in[oh*S + kh*d - pH, ow*S + kw*d - pW, r/mult]
//                                           * W[r,kh,kw]
// Input grad: th = oh + kh*d - pH on the zero-upsampled dy grid; a tap
//   contributes when th >= 0 is a multiple of S and th/S is a row of dy,
//   reading dy[th/S] with the reversed tap W[o, kH-1-kh, kW-1-kw], for each of
//   the mult output channels o = r*mult + j that read input channel r.
// V > 1 only with mult == 1 (consecutive channels of both tensors).
// ---------------------------------------------------------------------------
template <typename WT, int V, bool IG, int S>
__global__ __launch_bounds__(256) void k_direct_nhwc(const float *__restrict__ in,
                                                     const WT *__restrict__ w,
                                                     const float *__restrict__ bias,
                                                     float *__restrict__ out, DirectArgs a,
                                                     EpiArgs ep)
{
    const unsigned gt = blockIdx.x * 256u + threadIdx.x;
    if (gt >= (unsigned)a.total)
        return;
    int t = (int)gt;
    const int CV = a.CO / V;
    const int cv = t % CV;
    t /= CV;
    const int ow = t % a.OW;
    t /= a.OW;
    const int oh = t % a.OH;
    const int n = t / a.OH;
    const int r0 = cv * V;
    const int kk = a.kH * a.kW;
    const int nrep = IG ? a.mult : 1;

    float acc[V];
#pragma unroll
    for (int v = 0; v < V; ++v)
        acc[v] = (!IG && bias) ? bias[r0 + v] : 0.0f;

    for (int j = 0; j < nrep; ++j) {
        const int sc = IG ? r0 * a.mult + j : r0 / a.mult;   // channel of the tensor read
        const int wc = IG ? sc : r0;                          // filter
        for (int kh = 0; kh < a.kH; ++kh) {
            int ih;
            if (!IG) {
                ih = oh * S + kh * a.d - a.pH;
                if (ih < 0 || ih >= a.IH)
                    continue;
            } else {
                const int th = oh + kh * a.d - a.pH;
                if (th < 0 || (S == 2 && (th & 1)))
                    continue;
                ih = th / S;
                if (ih >= a.IH)
                    continue;
            }
            for (int kw = 0; kw < a.kW; ++kw) {
                int iw;
                if (!IG) {
                    iw = ow * S + kw * a.d - a.pW;
                    if (iw < 0 || iw >= a.IW)
                        continue;
                } else {
                    const int tw = ow + kw * a.d - a.pW;
                    if (tw < 0 || (S == 2 && (tw & 1)))
                        continue;
                    iw = tw / S;
                    if (iw >= a.IW)
                        continue;
                }
                float xv[V];
                load_vec<V>(in + ((n * a.IH + ih) * a.IW + iw) * a.CI + sc, xv);
                const int tap = IG ? (a.kH - 1 - kh) * a.kW + (a.kW - 1 - kw) : kh * a.kW + kw;
#pragma unroll
                for (int v = 0; v < V; ++v)
                    acc[v] = fmaf(widen(w[(wc + v) * kk + tap]), xv[v], acc[v]);
            }
        }
    }
    if (!IG && ep.on) {
#pragma unroll
        for (int v = 0; v < V; ++v)
            acc[v] = apply_epi(acc[v], epi_chan(ep, r0 + v, a.CO), ep.act);
    }
    store_vec<V>(out + ((n * a.OH + oh) * a.OW + ow) * a.CO + r0, acc);
}

// Direct NCHW: thread = (n, r, oh, ow), consecutive threads along ow.
template <typename WT, bool IG, int S>
__global__ __launch_bounds__(256) void k_direct_nchw(const float *__restrict__ in,
                                                     const WT *__restrict__ w,
                                                     const float *__restrict__ bias,
                                                     float *__restrict__ out, DirectArgs a,
                                                     EpiArgs ep)
{
    const unsigned gt = blockIdx.x * 256u + threadIdx.x;
    if (gt >= (unsigned)a.total)
        return;
    int t = (int)gt;
    const int ow = t % a.OW;
    t /= a.OW;
    const int oh = t % a.OH;
    t /= a.OH;
    const int r = t % a.CO;
    const int n = t / a.CO;
    const int kk = a.kH * a.kW;
    const int nrep = IG ? a.mult : 1;
    float acc = (!IG && bias) ? bias[r] : 0.0f;
    for (int j = 0; j < nrep; ++j) {
        const int sc = IG ? r * a.mult + j : r / a.mult;
        const float *plane = in + (n * a.CI + sc) * (a.IH * a.IW);
        const WT *wc = w + (IG ? sc : r) * kk;
        for (int kh = 0; kh < a.kH; ++kh) {
            int ih;
            if (!IG) {
                ih = oh * S + kh * a.d - a.pH;
                if (ih < 0 || ih >= a.IH)
                    continue;
            } else {
                const int th = oh + kh * a.d - a.pH;
                if (th < 0 || (S == 2 && (th & 1)))
                    continue;
                ih = th / S;
                if (ih >= a.IH)
                    continue;
            }
            for (int kw = 0; kw < a.kW; ++kw) {
                int iw;
                if (!IG) {
                    iw = ow * S + kw * a.d - a.pW;
                    if (iw < 0 || iw >= a.IW)
                        continue;
                } else {
                    const int tw = ow + kw * a.d - a.pW;
                    if (tw < 0 || (S == 2 && (tw & 1)))
                        continue;
                    iw = tw / S;
                    if (iw >= a.IW)
                        continue;
                }
                const int tap = IG ? (a.kH - 1 - kh) * a.kW + (a.kW - 1 - kw) : kh * a.kW + kw;
                acc = fmaf(widen(wc[tap]), plane[ih * a.IW + iw], acc);
            }
        }
    }
    if (!IG && ep.on)
        acc = apply_epi(acc, epi_chan(ep, r, a.CO), ep.act);
    __builtin_nontemporal_store(acc, out + ((n * a.CO + r) * a.OH + oh) * a.OW + ow);
}

DirectArgs direct_args(const Problem &p, const Plan &pl)
{
    DirectArgs a;
    a.N = p.N; a.mult = p.mult;
    a.CI = p.op == DWCONV_OP_FWD ? p.C : p.mult * p.C;   // channels of the tensor read
    a.CO = p.op == DWCONV_OP_FWD ? p.mult * p.C : p.C;   // channels of the tensor written
    a.kH = p.kH; a.kW = p.kW; a.d = p.dilation;
    a.pH = pl.pH; a.pW = pl.pW;
    a.IH = pl.IH; a.IW = pl.IW; a.OH = pl.OH; a.OW = pl.OW;
    a.total = (int)pl.total;
    return a;
}

template <typename WT>
int launch_direct_t(const Problem &p, const Plan &pl, const float *in, const void *wv,
                   const float *b, float *out, hipStream_t st, const EpiArgs &ep)
{
    const DirectArgs a = direct_args(p, pl);
    const WT *w = reinterpret_cast<const WT *>(wv);
    const dim3 grid((unsigned)pl.grid), block(256);
    const bool ig = p.op == DWCONV_OP_INPUT_GRAD;
    const int s = p.stride;
#define DW_DIRECT_NHWC(V, IGV, SV) \
    return launch_kernel(&k_direct_nhwc<WT, V, IGV, SV>, grid, block, 0, st, in, w, b, out, a, ep)
#define DW_DIRECT_NCHW(IGV, SV) \
    return launch_kernel(&k_direct_nchw<WT, IGV, SV>, grid, block, 0, st, in, w, b, out, a, ep)
    if (pl.kind == KIND_DIRECT_NHWC) {
        if (pl.vec == 4) {
            if (!ig) { if (s == 1) DW_DIRECT_NHWC(4, false, 1); else DW_DIRECT_NHWC(4, false, 2); }
            else     { if (s == 1) DW_DIRECT_NHWC(4, true, 1);  else DW_DIRECT_NHWC(4, true, 2); }
        } else {
            if (!ig) { if (s == 1) DW_DIRECT_NHWC(1, false, 1); else DW_DIRECT_NHWC(1, false, 2); }
            else     { if (s == 1) DW_DIRECT_NHWC(1, true, 1);  else DW_DIRECT_NHWC(1, true, 2); }
        }
    } else {
        if (!ig) { if (s == 1) DW_DIRECT_NCHW(false, 1); else DW_DIRECT_NCHW(false, 2); }
        else     { if (s == 1) DW_DIRECT_NCHW(true, 1);  else DW_DIRECT_NCHW(true, 2); }
    }
#undef DW_DIRECT_NHWC
#undef DW_DIRECT_NCHW
}

}  // namespace

int launch_direct(const Problem &p, const Plan &pl, const float *in, const void *w,
                  const float *b, float *out, hipStream_t st, const EpiArgs &ep)
{
    if (p.wtype == DWCONV_W_F16)
        return launch_direct_t<half_t>(p, pl, in, w, b, out, st, ep);
    return launch_direct_t<float>(p, pl, in, w, b, out, st, ep);
}

}  // namespace dwconv
