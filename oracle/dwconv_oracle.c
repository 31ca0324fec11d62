/*
 * dwconv_oracle.c -- plain CPU oracle for depthwise 2-D convolution.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke
 * check of the entry module and the bench's CPU-baseline leg may load this
 * library.  It shares no source, header, table or helper with the HIP path
 * and includes no HIP header.  Every routine is the plain definition written
 * out as loops, accumulating in double precision, one output at a time, with
 * no blocking, fusion or reordering.
 *
 * Sources (web pages; each function cites the passage it follows):
 *   [Lean]  LeanMlir, Proofs/Architectures/Depthwise (lean.brettkoonce.com):
 *           the forward equation (SAME, stride 1), the "regular conv minus the
 *           channel sum" comparison, the closed-form input gradient (direct
 *           sum over output positions, and the reversed-kernel form), the
 *           stride-2 definition (stride-1 SAME then keep even positions) and
 *           its input-VJP (zero-upsample the cotangent, then reversed-kernel
 *           stride-1 depthwise), the bias-gradient closed form.
 *   [ggml]  llama.cpp PR #21565 "metal : add CONV_2D_DW": f32 and f16 kernel
 *           weights with f32 input/output; the CPU backend bug of reading
 *           f16 weights as raw float bytes.
 *
 * Readings where the pages leave a step open (stated once here):
 *   - padding is SAME with p = dilation*(k-1)/2 per axis, k odd;
 *   - stride s and dilation d enter as x[h*s + kh*d - p] (the general form of
 *     the Lean forward equation), so stride 2 keeps the EVEN positions of the
 *     stride-1 result;
 *   - the operation is cross-correlation (no kernel flip) as in the Lean
 *     forward equation;
 *   - taps whose input position falls outside the image are skipped (the
 *     zero padding contributes nothing);
 *   - output extents are Ho = ceil(H/s), Wo = ceil(W/s).
 *
 * Layouts: layout 0 = NHWC (channel innermost, the ggml page's CWHN),
 *          layout 1 = NCHW (channel outer, the ggml page's WHCN).
 * Weights: always [C][kH][kW] contiguous; wtype 0 = IEEE binary32,
 *          wtype 1 = IEEE binary16 (decoded here from its bit pattern).
 *
 * Besides each value the routines can return S, the sum of the absolute
 * values of the products that entered it; callers use it to size the
 * rounding bound 1e-5*S + 1e-6 that a float32 implementation must meet.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (see oracle/build.py).  The same
 * source built with -DDWO_ACC_T=float (oracle/build.py, build_timing) is the
 * CPU timing baseline: the forward and the input gradient then form each
 * product and accumulate in single precision, as a float32 implementation
 * would; every other line is the same.  The parity build accumulates in
 * double.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

#ifndef DWO_ACC_T
#define DWO_ACC_T double
#endif
/* accumulation type of dwo_fwd and dwo_input_grad (double for parity) */
typedef DWO_ACC_T acc_t;

/* ------------------------------------------------------------------ */
/* IEEE 754 binary16 -> double, from the format's definition:           */
/* 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.             */
/*   e == 0      : subnormal, value = f * 2^-24                          */
/*   e == 31     : infinity (f == 0) or NaN                              */
/*   otherwise   : value = (1024 + f) * 2^(e - 25)                       */
/* The ggml page records a CPU backend that read f16 weights as raw     */
/* float bytes; widening by value, as here, is the fix it describes.    */
/* ------------------------------------------------------------------ */
double dwo_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* Weight tap W[c][kh][kw] as a double. */
static double wtap(const void *w, int wtype, int kH, int kW, int c, int kh, int kw)
{
    size_t i = ((size_t)c * kH + kh) * kW + kw;
    if (wtype == 1)
        return dwo_half_to_double(((const uint16_t *)w)[i]);
    return (double)((const float *)w)[i];
}

/* Element offset of logical (n, c, h, w) in a tensor of extents (N, C, H, W). */
static size_t at(int layout, int C, int H, int W, int n, int c, int h, int w)
{
    if (layout == 0)
        return (((size_t)n * H + h) * W + w) * C + c;
    return (((size_t)n * C + c) * H + h) * W + w;
}

static int out_extent(int in, int s) { return (in + s - 1) / s; }

/* ------------------------------------------------------------------ */
/* Forward.  [Lean] forward equation                                    */
/*   y[c,h,w] = sum_{kh,kw} x[c, h+kh-p, w+kw-p] * W[c,kh,kw] + b[c]     */
/* with stride s and dilation d: input position (ho*s + kh*d - pH,      */
/* wo*s + kw*d - pW).  No sum over channels: channel c of y reads only  */
/* channel c of x and filter c.  b may be NULL (no bias).               */
/* y and S (nullable) have extents (N, C, Ho, Wo) in `layout`.           */
/* ------------------------------------------------------------------ */
int dwo_fwd(const float *x, const void *w, int wtype, const float *b,
            double *y, double *S,
            int N, int H, int W, int C, int kH, int kW,
            int s, int d, int layout, int nthreads)
{
    const int pH = d * (kH - 1) / 2, pW = d * (kW - 1) / 2;
    const int Ho = out_extent(H, s), Wo = out_extent(W, s);
    long nc;
#pragma omp parallel for schedule(dynamic) num_threads(nthreads > 0 ? nthreads : 1)
    for (nc = 0; nc < (long)N * C; ++nc) {
        const int n = (int)(nc / C), c = (int)(nc % C);
        for (int ho = 0; ho < Ho; ++ho)
            for (int wo = 0; wo < Wo; ++wo) {
                acc_t acc = b ? (acc_t)b[c] : 0, sabs = 0;
                for (int kh = 0; kh < kH; ++kh) {
                    const int hi = ho * s + kh * d - pH;
                    if (hi < 0 || hi >= H)
                        continue;
                    for (int kw = 0; kw < kW; ++kw) {
                        const int wi = wo * s + kw * d - pW;
                        if (wi < 0 || wi >= W)
                            continue;
                        const acc_t t = (acc_t)x[at(layout, C, H, W, n, c, hi, wi)] *
                                        (acc_t)wtap(w, wtype, kH, kW, c, kh, kw);
                        acc += t;
                        sabs += fabs(t);
                    }
                }
                const size_t o = at(layout, C, Ho, Wo, n, c, ho, wo);
                y[o] = acc;
                if (S)
                    S[o] = sabs;
            }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Input gradient, reversed-kernel form.  [Lean] reversed-kernel        */
/* formula for the stride-1 input VJP                                   */
/*   dx[c,h,w] = sum_{kh,kw} W[c,kH-1-kh,kW-1-kw] * dy[c,h+kh-p,w+kw-p]  */
/* and, for stride s, [Lean] stride-2 input VJP: zero-upsample the      */
/* cotangent onto the positions the forward kept (multiples of s on the */
/* H x W grid), then run the reversed-kernel stride-1 depthwise on that */
/* grid.  The upsampled value at grid position (t_h, t_w) is            */
/* dy[t_h/s, t_w/s] when both are multiples of s, else zero; with       */
/* dilation the tap offset is kh*d.  dy has extents (N,C,Ho,Wo), dx has */
/* (N,C,H,W).                                                           */
/* ------------------------------------------------------------------ */
int dwo_input_grad(const float *dy, const void *w, int wtype,
                   double *dx, double *S,
                   int N, int H, int W, int C, int kH, int kW,
                   int s, int d, int layout, int nthreads)
{
    const int pH = d * (kH - 1) / 2, pW = d * (kW - 1) / 2;
    const int Ho = out_extent(H, s), Wo = out_extent(W, s);
    long nc;
#pragma omp parallel for schedule(dynamic) num_threads(nthreads > 0 ? nthreads : 1)
    for (nc = 0; nc < (long)N * C; ++nc) {
        const int n = (int)(nc / C), c = (int)(nc % C);
        for (int h = 0; h < H; ++h)
            for (int x_w = 0; x_w < W; ++x_w) {
                acc_t acc = 0, sabs = 0;
                for (int kh = 0; kh < kH; ++kh) {
                    const int th = h + kh * d - pH;        /* row on the upsampled grid */
                    if (th < 0 || th >= H || th % s != 0)  /* padding, or an inserted zero */
                        continue;
                    for (int kw = 0; kw < kW; ++kw) {
                        const int tw = x_w + kw * d - pW;
                        if (tw < 0 || tw >= W || tw % s != 0)
                            continue;
                        const acc_t t = (acc_t)wtap(w, wtype, kH, kW, c, kH - 1 - kh, kW - 1 - kw) *
                                        (acc_t)dy[at(layout, C, Ho, Wo, n, c, th / s, tw / s)];
                        acc += t;
                        sabs += fabs(t);
                    }
                }
                const size_t o = at(layout, C, H, W, n, c, h, x_w);
                dx[o] = acc;
                if (S)
                    S[o] = sabs;
            }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Input gradient, direct form.  [Lean] closed-form input gradient as a */
/* sum over output positions (ho, wo) with reconstructed kernel offsets */
/* kh_nat = hi + pH - ho, kw_nat = wi + pW - wo, contributing only when */
/* the offset lies in [0,kH) x [0,kW); with stride s and dilation d the */
/* reconstructed offset satisfies kh_nat*d = hi + pH - ho*s.  Brute     */
/* force over every output position: O(H*W*Ho*Wo) per channel, for     */
/* small inputs only.  Written independently of dwo_input_grad so that  */
/* agreement between the two is a check of both.                        */
/* ------------------------------------------------------------------ */
int dwo_input_grad_direct(const float *dy, const void *w, int wtype, double *dx,
                          int N, int H, int W, int C, int kH, int kW,
                          int s, int d, int layout)
{
    const int pH = d * (kH - 1) / 2, pW = d * (kW - 1) / 2;
    const int Ho = out_extent(H, s), Wo = out_extent(W, s);
    for (int n = 0; n < N; ++n)
        for (int c = 0; c < C; ++c)
            for (int hi = 0; hi < H; ++hi)
                for (int wi = 0; wi < W; ++wi) {
                    double acc = 0.0;
                    for (int ho = 0; ho < Ho; ++ho) {
                        const int eh = hi + pH - ho * s;      /* = kh_nat * d */
                        if (eh < 0 || eh % d != 0 || eh / d >= kH)
                            continue;
                        for (int wo = 0; wo < Wo; ++wo) {
                            const int ew = wi + pW - wo * s;
                            if (ew < 0 || ew % d != 0 || ew / d >= kW)
                                continue;
                            acc += wtap(w, wtype, kH, kW, c, eh / d, ew / d) *
                                   (double)dy[at(layout, C, Ho, Wo, n, c, ho, wo)];
                        }
                    }
                    dx[at(layout, C, H, W, n, c, hi, wi)] = acc;
                }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Regular (dense) convolution.  [Lean] comparison with regular conv2d: */
/*   y[o,h,w] = sum_{c,kh,kw} x[c, ...] * Wd[o,c,kh,kw] + b[o]           */
/* depthwise is the same minus the sum over c.  Wd is [Co][C][kH][kW]   */
/* float32; same padding, stride and dilation reading as dwo_fwd.  Used */
/* with a Wd that is zero off the diagonal o == c to check that the     */
/* depthwise routine mixes no channels.  O(C*Co) per pixel: small only. */
/* ------------------------------------------------------------------ */
int dwo_dense_conv(const float *x, const float *wd, const float *b, double *y,
                   int N, int H, int W, int C, int Co, int kH, int kW,
                   int s, int d, int layout)
{
    const int pH = d * (kH - 1) / 2, pW = d * (kW - 1) / 2;
    const int Ho = out_extent(H, s), Wo = out_extent(W, s);
    for (int n = 0; n < N; ++n)
        for (int o = 0; o < Co; ++o)
            for (int ho = 0; ho < Ho; ++ho)
                for (int wo = 0; wo < Wo; ++wo) {
                    double acc = b ? (double)b[o] : 0.0;
                    for (int c = 0; c < C; ++c)
                        for (int kh = 0; kh < kH; ++kh) {
                            const int hi = ho * s + kh * d - pH;
                            if (hi < 0 || hi >= H)
                                continue;
                            for (int kw = 0; kw < kW; ++kw) {
                                const int wi = wo * s + kw * d - pW;
                                if (wi < 0 || wi >= W)
                                    continue;
                                acc += (double)x[at(layout, C, H, W, n, c, hi, wi)] *
                                       (double)wd[(((size_t)o * C + c) * kH + kh) * kW + kw];
                            }
                        }
                    y[at(layout, Co, Ho, Wo, n, o, ho, wo)] = acc;
                }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Weight gradient.  [Lean] depthwise weight-VJP: the forward is affine */
/* in W, the output (c, ho, wo) being b[c] + sum_{kh,kw} W[c,kh,kw] *   */
/* (padded x term); its transpose is                                    */
/*   dW[c,kh,kw] = sum_{n,ho,wo} x[n,c,ho*s+kh*d-pH, wo*s+kw*d-pW] *     */
/*                 dy[n,c,ho,wo]                                        */
/* over in-range input positions (the stride-2 weight-VJP is the same   */
/* sum at the kept positions).  dW is [C][kH][kW] double.               */
/* ------------------------------------------------------------------ */
int dwo_weight_grad(const float *x, const float *dy, double *dw, double *S,
                    int N, int H, int W, int C, int kH, int kW,
                    int s, int d, int layout, int nthreads)
{
    const int pH = d * (kH - 1) / 2, pW = d * (kW - 1) / 2;
    const int Ho = out_extent(H, s), Wo = out_extent(W, s);
    long t;
#pragma omp parallel for schedule(dynamic) num_threads(nthreads > 0 ? nthreads : 1)
    for (t = 0; t < (long)C * kH * kW; ++t) {
        const int c = (int)(t / ((long)kH * kW));
        const int kh = (int)((t / kW) % kH), kw = (int)(t % kW);
        double acc = 0.0, sabs = 0.0;
        for (int n = 0; n < N; ++n)
            for (int ho = 0; ho < Ho; ++ho) {
                const int hi = ho * s + kh * d - pH;
                if (hi < 0 || hi >= H)
                    continue;
                for (int wo = 0; wo < Wo; ++wo) {
                    const int wi = wo * s + kw * d - pW;
                    if (wi < 0 || wi >= W)
                        continue;
                    const double p = (double)x[at(layout, C, H, W, n, c, hi, wi)] *
                                     (double)dy[at(layout, C, Ho, Wo, n, c, ho, wo)];
                    acc += p;
                    sabs += fabs(p);
                }
            }
        dw[t] = acc;
        if (S)
            S[t] = sabs;
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Bias gradient.  [Lean] closed form db[c] = sum_{h,w} dy[c,h,w],      */
/* summed over the batch as well.                                       */
/* ------------------------------------------------------------------ */
int dwo_bias_grad(const float *dy, double *db, double *S,
                  int N, int Ho, int Wo, int C, int layout)
{
    for (int c = 0; c < C; ++c) {
        double acc = 0.0, sabs = 0.0;
        for (int n = 0; n < N; ++n)
            for (int h = 0; h < Ho; ++h)
                for (int w = 0; w < Wo; ++w) {
                    const double v = (double)dy[at(layout, C, Ho, Wo, n, c, h, w)];
                    acc += v;
                    sabs += fabs(v);
                }
        db[c] = acc;
        if (S)
            S[c] = sabs;
    }
    return 0;
}

/* ================================================================== */
/* General form: explicit per-side padding and a channel multiplier.    */
/*                                                                      */
/* [Lean] stride-2 XLA-SAME: the stride-1 SAME result kept at the ODD   */
/* positions, with a backward that zero-upsamples the cotangent onto    */
/* those same odd positions.  Keeping phase-1 positions equals reading  */
/* input row ho*s + kh*d - pt with a top pad pt one smaller than the    */
/* symmetric p, so both SAME variants are instances of one forward with */
/* explicit pads (pt, pb, pl, pr); the output extents are the number of */
/* window positions that fit: Ho = (H + pt + pb - d*(kH-1) - 1)/s + 1.  */
/* [Reactant issue 331] grouped conv with groups = C_in and             */
/* C_out = m*C_in (the "4 => 8, groups = 4" layer): output channel o    */
/* reads input channel o/m only, with its own filter W[o] and bias b[o].*/
/* m = 1 is the plain depthwise operator.                               */
/* Here H, W, C are the INPUT extents and channels; y / dy have         */
/* (N, m*C, Ho, Wo); W is [m*C][kH][kW]; b is [m*C] or NULL.            */
/* ================================================================== */

/* Forward.  [Lean] forward equation, with stride s, dilation d, top and */
/* left pads pt, pl, and input channel o/m for output channel o:        */
/*   y[n,o,ho,wo] = b[o] + sum_{kh,kw} x[n, o/m, ho*s+kh*d-pt,          */
/*                                       wo*s+kw*d-pl] * W[o,kh,kw]     */
/* over in-range input positions.                                        */
int dwo_fwd_general(const float *x, const void *w, int wtype, const float *b,
                    double *y, double *S,
                    int N, int H, int W, int C, int m, int kH, int kW,
                    int s, int d, int pt, int pl, int Ho, int Wo,
                    int layout, int nthreads)
{
    const int Co = m * C;
    long no;
#pragma omp parallel for schedule(dynamic) num_threads(nthreads > 0 ? nthreads : 1)
    for (no = 0; no < (long)N * Co; ++no) {
        const int n = (int)(no / Co), o = (int)(no % Co), c = o / m;
        for (int ho = 0; ho < Ho; ++ho)
            for (int wo = 0; wo < Wo; ++wo) {
                double acc = b ? (double)b[o] : 0.0, sabs = 0.0;
                for (int kh = 0; kh < kH; ++kh) {
                    const int hi = ho * s + kh * d - pt;
                    if (hi < 0 || hi >= H)
                        continue;
                    for (int kw = 0; kw < kW; ++kw) {
                        const int wi = wo * s + kw * d - pl;
                        if (wi < 0 || wi >= W)
                            continue;
                        const double t = (double)x[at(layout, C, H, W, n, c, hi, wi)] *
                                         wtap(w, wtype, kH, kW, o, kh, kw);
                        acc += t;
                        sabs += fabs(t);
                    }
                }
                const size_t q = at(layout, Co, Ho, Wo, n, o, ho, wo);
                y[q] = acc;
                if (S)
                    S[q] = sabs;
            }
    }
    return 0;
}

/* Input gradient: the transpose of dwo_fwd_general.  [Lean] closed-form */
/* input gradient, reconstructed-offset form: input position (h, w)     */
/* receives dy[ho,wo]*W[kh,kw] exactly when ho*s + kh*d - pt = h and    */
/* wo*s + kw*d - pl = w.  Enumerated by tap: ho = (h + pt - kh*d)/s     */
/* must be a whole number in [0, Ho) (otherwise the upsampled cotangent */
/* holds an inserted zero or padding there), likewise wo.  Input        */
/* channel c collects the m output channels c*m .. c*m+m-1 that read it.*/
int dwo_input_grad_general(const float *dy, const void *w, int wtype,
                           double *dx, double *S,
                           int N, int H, int W, int C, int m, int kH, int kW,
                           int s, int d, int pt, int pl, int Ho, int Wo,
                           int layout, int nthreads)
{
    const int Co = m * C;
    long nc;
#pragma omp parallel for schedule(dynamic) num_threads(nthreads > 0 ? nthreads : 1)
    for (nc = 0; nc < (long)N * C; ++nc) {
        const int n = (int)(nc / C), c = (int)(nc % C);
        for (int h = 0; h < H; ++h)
            for (int x_w = 0; x_w < W; ++x_w) {
                double acc = 0.0, sabs = 0.0;
                for (int j = 0; j < m; ++j) {
                    const int o = c * m + j;
                    for (int kh = 0; kh < kH; ++kh) {
                        const int eh = h + pt - kh * d;          /* = ho * s */
                        if (eh < 0 || eh % s != 0 || eh / s >= Ho)
                            continue;
                        for (int kw = 0; kw < kW; ++kw) {
                            const int ew = x_w + pl - kw * d;
                            if (ew < 0 || ew % s != 0 || ew / s >= Wo)
                                continue;
                            const double t = wtap(w, wtype, kH, kW, o, kh, kw) *
                                (double)dy[at(layout, Co, Ho, Wo, n, o, eh / s, ew / s)];
                            acc += t;
                            sabs += fabs(t);
                        }
                    }
                }
                const size_t q = at(layout, C, H, W, n, c, h, x_w);
                dx[q] = acc;
                if (S)
                    S[q] = sabs;
            }
    }
    return 0;
}

/* Weight gradient of dwo_fwd_general.  [Lean] depthwise weight-VJP,    */
/* with the general index map:                                           */
/*   dW[o,kh,kw] = sum_{n,ho,wo} x[n, o/m, ho*s+kh*d-pt, wo*s+kw*d-pl] * */
/*                 dy[n,o,ho,wo]   over in-range input positions.        */
/* The bias gradient is dwo_bias_grad on dy (m*C channels).              */
int dwo_weight_grad_general(const float *x, const float *dy, double *dw, double *S,
                            int N, int H, int W, int C, int m, int kH, int kW,
                            int s, int d, int pt, int pl, int Ho, int Wo,
                            int layout, int nthreads)
{
    const int Co = m * C;
    long t;
#pragma omp parallel for schedule(dynamic) num_threads(nthreads > 0 ? nthreads : 1)
    for (t = 0; t < (long)Co * kH * kW; ++t) {
        const int o = (int)(t / ((long)kH * kW)), c = o / m;
        const int kh = (int)((t / kW) % kH), kw = (int)(t % kW);
        double acc = 0.0, sabs = 0.0;
        for (int n = 0; n < N; ++n)
            for (int ho = 0; ho < Ho; ++ho) {
                const int hi = ho * s + kh * d - pt;
                if (hi < 0 || hi >= H)
                    continue;
                for (int wo = 0; wo < Wo; ++wo) {
                    const int wi = wo * s + kw * d - pl;
                    if (wi < 0 || wi >= W)
                        continue;
                    const double p = (double)x[at(layout, C, H, W, n, c, hi, wi)] *
                                     (double)dy[at(layout, Co, Ho, Wo, n, o, ho, wo)];
                    acc += p;
                    sabs += fabs(p);
                }
            }
        dw[t] = acc;
        if (S)
            S[t] = sabs;
    }
    return 0;
}

/* Version tag so a stale build is detectable. */
int dwo_version(void) { return 2; }
