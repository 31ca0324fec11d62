// dwconv_kernels.hip -- gfx950 kernels of depthwise 2-D convolution and the
// launchers that run a plan.
//
// What is computed (LeanMlir "Depthwise" page): the forward equation
//   y[c,h,w] = b[c] + sum_{kh,kw} x[c, h*s + kh*d - pH, w*s + kw*d - pW] * W[c,kh,kw]
// (one filter per channel, no channel sum, zero padding; with a channel
// multiplier m output channel o reads input channel o/m), its input gradient
// in the reversed-kernel form with stride 2 handled as the zero-upsampled
// cotangent (only upsampled positions that are multiples of s carry a
// value), and its weight and bias gradients.
//
// Design (gfx950, 64-wide waves, HBM-bound): the channel axis is a batch
// axis, so there is no contraction for the matrix cores; each output is a
// kH*kW-tap dot product done with fp32 FMAs (cubek-convolution "depthwise"
// module: the contraction is over window taps only, channels innermost so
// consecutive lanes read consecutive channels, and the pass is
// bandwidth-bound).  Weights are widened to fp32 once per thread (f16 by
// value, never by reinterpreting bytes: the ggml PR's CPU-backend bug).
//
//  * direct kernels: one thread per output (NCHW) or per channel vector
//    (NHWC); taps read from global memory through the caches.  They cover
//    every valid problem (stride 2, any pads, multipliers, even kernels).
//  * tiled NHWC / NCHW kernels (stride 1): a short-lived workgroup stages the
//    input rows its output rows need (tile plus (k-1)*d halo, zero outside
//    the image, via raw buffer loads) and its weights in LDS in one load
//    phase, then walks the rows: each thread reads its kW horizontal taps per
//    staged row from LDS and folds the row into R = (kH-1)*d + 1 rolling
//    accumulators, so every input element is fetched from HBM about once and
//    reused for all kH*kW taps.  Compile-time modes: forward, input gradient
//    (reversed taps, no bias), forward with the BatchNorm / activation
//    epilogue.
//  * weight gradient: per-chunk partial sums (tiled NHWC, tiled NCHW or the
//    generic coalesced kernel), then a fixed-order reduction that can also
//    apply the SGD step.
//  * every output store is non-temporal: outputs are write-once streams.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <utility>

#include "dwconv_internal.h"
#include "../../include/dwconv.h"

namespace dwconv {

namespace {

typedef _Float16 half_t;

__device__ __forceinline__ float widen(float v) { return v; }
__device__ __forceinline__ float widen(half_t v) { return (float)v; }

template <int V> struct VecT;
template <> struct VecT<1> { typedef float type; };
template <> struct VecT<2> { typedef float2 type; };
template <> struct VecT<4> { typedef float4 type; };

template <int V>
__device__ __forceinline__ void load_vec(const float *p, float (&v)[V])
{
    typedef typename VecT<V>::type T;
    const T t = *reinterpret_cast<const T *>(p);
    const float *f = reinterpret_cast<const float *>(&t);
#pragma unroll
    for (int i = 0; i < V; ++i)
        v[i] = f[i];
}

// Outputs are written once and never re-read by the kernel: store them
// non-temporally so they stream to HBM instead of displacing the input rows
// (and their halos) that neighbouring workgroups still read from L2.
typedef float f4_ext __attribute__((ext_vector_type(4)));
typedef float f2_ext __attribute__((ext_vector_type(2)));

template <int V>
__device__ __forceinline__ void store_vec(float *p, const float (&v)[V])
{
    if constexpr (V == 4) {
        const f4_ext t = {v[0], v[1], v[2], v[3]};
        __builtin_nontemporal_store(t, reinterpret_cast<f4_ext *>(p));
    } else if constexpr (V == 2) {
        const f2_ext t = {v[0], v[1]};
        __builtin_nontemporal_store(t, reinterpret_cast<f2_ext *>(p));
    } else {
        __builtin_nontemporal_store(v[0], p);
    }
}

// Raw buffer loads (gfx9 family buffer descriptors, stride 0): an offset at
// or beyond the descriptor's byte count reads as zero in hardware, which
// gives zero padding and tail handling without branches around the loads.
constexpr int kBufWord3 = 0x00020000;
constexpr int kOutOfRange = 0x7ffffff0;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, kBufWord3);
}

typedef unsigned int u4_ext __attribute__((ext_vector_type(4)));

// Note: the 128-bit result must be reinterpreted as a whole vector; taking
// its 32-bit lanes apart one by one has been seen to shrink the load to a
// single dword on this compiler, leaving the other lanes undefined.
__device__ __forceinline__ float4 buf_f4(__amdgpu_buffer_rsrc_t r, int off)
{
    const u4_ext t = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    const f4_ext f = __builtin_bit_cast(f4_ext, t);
    return make_float4(f.x, f.y, f.z, f.w);
}

__device__ __forceinline__ float buf_f32(__amdgpu_buffer_rsrc_t r, int off)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

typedef unsigned int u2_ext __attribute__((ext_vector_type(2)));

// V consecutive floats (V = 1, 2 or 4) with one buffer load of matching width.
template <int V>
__device__ __forceinline__ void buf_vec(__amdgpu_buffer_rsrc_t r, int off, float (&out)[V])
{
    if constexpr (V == 4) {
        const float4 t = buf_f4(r, off);
        out[0] = t.x; out[1] = t.y; out[2] = t.z; out[3] = t.w;
    } else if constexpr (V == 2) {
        const u2_ext t = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
        const f2_ext f = __builtin_bit_cast(f2_ext, t);
        out[0] = f.x; out[1] = f.y;
    } else {
        out[0] = buf_f32(r, off);
    }
}

// One weight element, widened to fp32 (f16 by value).
__device__ __forceinline__ float buf_w(__amdgpu_buffer_rsrc_t r, int idx, float *)
{
    return buf_f32(r, idx * 4);
}
__device__ __forceinline__ float buf_w(__amdgpu_buffer_rsrc_t r, int idx, half_t *)
{
    return (float)__builtin_bit_cast(half_t, __builtin_amdgcn_raw_buffer_load_b16(r, idx * 2, 0, 0));
}

// ---------------------------------------------------------------------------
// Forward epilogue: inference-form BatchNorm and an activation, applied per
// output channel before the store (the LeanMlir page's fused depthwise +
// BatchNorm codegen; textbook layer definitions):
//   t = (z - mean) * gamma / sqrt(var + eps) + beta,   y = act(t)
// with z the convolution result (bias included).  Without BatchNorm
// (gamma == NULL) the affine step is the identity.
// ---------------------------------------------------------------------------
struct EpiArgs {
    const float *gamma, *beta, *mean, *var;   // all NULL: no BatchNorm
    float eps;
    int act;                                  // DWCONV_ACT_*
    int on;                                   // direct kernels: apply the epilogue
};

// Per-channel affine factors: y_pre = fmaf(z - mu, inv, be).  epi_load
// issues the loads (inv holds gamma, var the variance until epi_finish).
struct EpiChan {
    float mu, inv, be, var;
};

__device__ __forceinline__ float apply_act(float t, int act)
{
    if (act == DWCONV_ACT_RELU)
        return fmaxf(t, 0.0f);
    if (act == DWCONV_ACT_RELU6)
        return fminf(fmaxf(t, 0.0f), 6.0f);
    if (act == DWCONV_ACT_SILU)
        return __fdividef(t, 1.0f + __expf(-t));
    return t;
}

// Factors of channel c (c < channels) read through buffer descriptors.
__device__ __forceinline__ EpiChan epi_load(const EpiArgs &ep, int c, int channels)
{
    EpiChan e{0.0f, 1.0f, 0.0f, 0.0f};
    if (ep.gamma) {
        const int bytes = channels * 4;
        const int off = c < channels ? c * 4 : kOutOfRange;
        e.inv = buf_f32(make_rsrc(ep.gamma, bytes), off);
        e.var = buf_f32(make_rsrc(ep.var, bytes), off);
        e.mu = buf_f32(make_rsrc(ep.mean, bytes), off);
        e.be = buf_f32(make_rsrc(ep.beta, bytes), off);
    }
    return e;
}

__device__ __forceinline__ void epi_finish(EpiChan &e, const EpiArgs &ep)
{
    if (ep.gamma)
        e.inv = e.inv / sqrtf(e.var + ep.eps);
}

__device__ __forceinline__ EpiChan epi_chan(const EpiArgs &ep, int c, int channels)
{
    EpiChan e = epi_load(ep, c, channels);
    epi_finish(e, ep);
    return e;
}

__device__ __forceinline__ float apply_epi(float z, EpiChan e, int act)
{
    return apply_act(fmaf(z - e.mu, e.inv, e.be), act);
}

// The epilogue over a block of N values (value i of channel factors e[i % NE]),
// with one branch on the activation for the whole block.  SiLU uses the
// hardware exponential and reciprocal (a few ulp, far inside the tolerance
// its tests derive).
template <int N, int NE>
__device__ __forceinline__ void epi_block(float (&v)[N], const EpiChan (&e)[NE], int act)
{
#pragma unroll
    for (int i = 0; i < N; ++i)
        v[i] = fmaf(v[i] - e[i % NE].mu, e[i % NE].inv, e[i % NE].be);
    if (act == DWCONV_ACT_RELU) {
#pragma unroll
        for (int i = 0; i < N; ++i)
            v[i] = fmaxf(v[i], 0.0f);
    } else if (act == DWCONV_ACT_RELU6) {
#pragma unroll
        for (int i = 0; i < N; ++i)
            v[i] = fminf(fmaxf(v[i], 0.0f), 6.0f);
    } else if (act == DWCONV_ACT_SILU) {
#pragma unroll
        for (int i = 0; i < N; ++i)
            v[i] = __fdividef(v[i], 1.0f + __expf(-v[i]));
    }
}

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

// ---------------------------------------------------------------------------
// Tiled NHWC, stride 1 (forward, or input gradient with reversed taps).
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

// ---------------------------------------------------------------------------
// Tiled NCHW, stride 1 (forward, or input gradient with reversed taps).
//
// Channel-outer layout: each (n, c) plane is an image of its own, and the
// weights of a plane are one kernel.  A workgroup of 256 threads covers PB
// planes x TX threads per plane row (TX = 256/PB, a power of two >= W/Q so
// narrow planes are packed several to a workgroup); each thread owns Q
// adjacent output columns.  G input rows of every plane (the TH = G - R + 1
// output rows plus the row halo) and HALO columns on each side are staged
// in LDS in one pass, then the rows are walked with rolling accumulators as
// in the NHWC kernel.  Loads are buffer loads over the whole tensor: rows
// past the plane or the tensor read as zero, columns outside [0, W) are
// given an out-of-range offset.
// ---------------------------------------------------------------------------
struct TiledNchwArgs {
    int planes, C;
    int IH, IW, OH, OW;     // extents of the tensor read, and of the grid the tiles cover
    int YH, YW;             // extents of the tensor written (the grid's, except stride-2 fwd)
    int pH, pW;             // top / left zero padding of the tensor read
    int hl, twl;            // staged columns left of a tile; staged floats per plane row
    int txn, pbn;           // threads per plane row (16..256), planes per workgroup (256 / txn)
    int nct, nwt, nst;      // plane groups, column tiles, row tiles
};

template <int KH, int KW, int D, int Q, int G, bool V4>
struct NchwGeom {
    static constexpr int R = (KH - 1) * D + 1;
    static constexpr int TH = G - R + 1;
    static constexpr int KK = KH * KW;
    static constexpr int LV = V4 ? 4 : 1;                      // floats per load
    // staged columns beyond a tile's own: the window's d*(kW-1), plus up to
    // 3 columns of alignment with 16-byte loads
    static constexpr int EXTRA = V4 ? (D * (KW - 1) + 3 + 3) / 4 * 4 : D * (KW - 1);
    static constexpr int PBMAX = 16;                           // TX >= 16
    // per-thread loads for the largest staged tile: G rows x (256*Q + PBMAX*EXTRA) floats
    static constexpr int NV = (G * (256 * Q + PBMAX * EXTRA) / LV + 255) / 256;
    static constexpr int NW = (PBMAX * KK + 255) / 256;
    static_assert(TH >= 1, "a workgroup must produce at least one output row");
};

// Stride 2 (S == 2) as in the NHWC kernel: the forward tiles the stride-1
// grid and keeps its even positions, the input gradient stages dy
// zero-upsampled (4-byte loads only) and skips the all-zero rows.
template <typename WT, int KH, int KW, int D, int Q, int G, bool V4, int MODE, int S>
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
    typedef NchwGeom<KH, KW, D, Q, G, V4> Gm;
    constexpr int R = Gm::R, TH = Gm::TH, KK = Gm::KK, LV = Gm::LV;
    constexpr int NW = Gm::NW;
    // loads per thread: the whole tile, or with the upsampled dy only its
    // even rows, one dy element per pair of staged columns (the twl/2 pairs
    // of a row: twl is even then)
    constexpr int NV = UPS ? ((G + 1) / 2 * ((256 * Q + Gm::PBMAX * Gm::EXTRA) / 2 + Gm::PBMAX) +
                              255) / 256
                           : Gm::NV;
    extern __shared__ float4 lds4[];
    float *lds = reinterpret_cast<float *>(lds4);
    const WT *w = reinterpret_cast<const WT *>(wv);

    const int txn = a.txn, pbn = a.pbn;
    const int tw = txn * Q, twl = a.twl;               // staged floats per plane row
    const int vpr = twl / LV;                          // loads per plane row
    float *ldsw = lds + pbn * G * twl;

    int tile = blockIdx.x;
    const int pg = tile % a.nct;
    tile /= a.nct;
    const int wt = tile % a.nwt;
    const int st = tile / a.nwt;
    const int w0 = wt * tw, h0 = st * TH;
    const int tid = threadIdx.x;
    const int nrows = min(TH, a.OH - h0) + R - 1;
    const int rbase = h0 - a.pH, cbase = w0 - a.hl;

    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, a.C * KK * (int)sizeof(WT));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(bias, (!IG && bias) ? a.C * 4 : 0);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(in, a.planes * a.IH * a.IW * 4);

    // 1. all loads up front: weights of the workgroup's planes, the bias, the tile
    float wst[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int e = tid + i * 256;
        const int pl = e / KK, tap = e - pl * KK;
        const int plane = pg * pbn + pl;
        const bool ok = pl < pbn && plane < a.planes;
        wst[i] = buf_w(rw, ok ? (plane % a.C) * KK + tap : kOutOfRange / 4, (WT *)nullptr);
    }
    // threads past pbn * txn (when txn does not divide 256) idle along
    const int pli_raw = tid / txn, tx = tid - pli_raw * txn;
    const int pli = min(pli_raw, pbn - 1);             // in-range LDS addresses for idle threads
    const int my_plane = pg * pbn + pli;
    const bool pvalid = pli_raw < pbn && my_plane < a.planes;
    const float bval = buf_f32(rb, pvalid ? (my_plane % a.C) * 4 : kOutOfRange);
    EpiChan ec{0.0f, 1.0f, 0.0f, 0.0f};
    if constexpr (EPI)
        ec = epi_load(ep, pvalid ? my_plane % a.C : a.C, a.C);
    float sv[NV][LV];
    // upsampled staging: rows g0, g0+2, ... of the tile are the even
    // (upsampled) rows; a pair k of staged columns (2k, 2k+1) holds one dy
    // element at its even column and a zero at the other
    const int g0 = rbase & 1, ge_n = (G - g0 + 1) / 2, hp = twl / 2, c1 = cbase & 1;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = tid + i * 256;
        if constexpr (UPS) {
            const int pl = e / (ge_n * hp);
            const int rem = e - pl * (ge_n * hp);
            const int ge = rem / hp, k = rem - ge * hp;
            const int g = g0 + 2 * ge;
            const int plane = pg * pbn + pl, row = rbase + g, col = cbase + 2 * k + c1;
            const int sr = row >> 1, sc = col >> 1;    // position in dy (row, col are even)
            const bool ok = pl < pbn && plane < a.planes && g < nrows && row >= 0 &&
                            col >= 0 && sr < a.IH && sc < a.IW;
            sv[i][0] = buf_f32(rx, ok ? ((plane * a.IH + sr) * a.IW + sc) * 4 : kOutOfRange);
        } else {
            const int pl = e / (G * vpr);
            const int rem = e - pl * (G * vpr);
            const int g = rem / vpr;
            const int col = cbase + (rem - g * vpr) * LV;
            const int plane = pg * pbn + pl, row = rbase + g;
            const bool ok = pl < pbn && plane < a.planes && g < nrows && row >= 0 &&
                            row < a.IH && col >= 0 && col < a.IW;
            const int off = ok ? ((plane * a.IH + row) * a.IW + col) * 4 : kOutOfRange;
            if constexpr (V4) {
                const float4 v = buf_f4(rx, off);
                sv[i][0] = v.x; sv[i][1] = v.y; sv[i][2] = v.z; sv[i][3] = v.w;
            } else {
                sv[i][0] = buf_f32(rx, off);
            }
        }
    }
    // 2. into LDS
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int e = tid + i * 256;
        if (e < pbn * KK)
            ldsw[e] = wst[i];
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = tid + i * 256;
        if constexpr (UPS) {
            if (e < pbn * ge_n * hp) {
                const int pl = e / (ge_n * hp);
                const int rem = e - pl * (ge_n * hp);
                const int ge = rem / hp, k = rem - ge * hp;
                float2 *dst = reinterpret_cast<float2 *>(lds + (pl * G + g0 + 2 * ge) * twl);
                dst[k] = c1 ? make_float2(0.0f, sv[i][0]) : make_float2(sv[i][0], 0.0f);
            }
        } else if (e < pbn * G * vpr) {
            if constexpr (V4)
                lds4[e] = make_float4(sv[i][0], sv[i][1], sv[i][2], sv[i][3]);
            else
                lds[e] = sv[i][0];
        }
    }
    __syncthreads();

    // 3. per-thread weights and rolling accumulators
    float wr[KH][KW];
#pragma unroll
    for (int kh = 0; kh < KH; ++kh)
#pragma unroll
        for (int kw = 0; kw < KW; ++kw) {
            const int tap = IG ? (KH - 1 - kh) * KW + (KW - 1 - kw) : kh * KW + kw;
            wr[kh][kw] = ldsw[pli * KK + tap];
        }
    if constexpr (EPI)
        epi_finish(ec, ep);
    float acc[R][Q];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < Q; ++j)
            acc[r][j] = bval;
    constexpr int XW = Q + (KW - 1) * D;
    const float *rowbase = lds + pli * G * twl + tx * Q + (a.hl - a.pW);
    const int oc = w0 + tx * Q;                        // first output column of this thread
    float *outp = out + my_plane * a.YH * a.YW;
    const bool vec_store = !DEC && (Q > 1) && (a.OW % Q == 0);
#pragma unroll
    for (int u = 0; u < G; ++u) {
        if (u < nrows) {
            // a staged row of the upsampled dy at an odd position is all zero
            if (!(UPS && ((rbase + u) & 1))) {
                float xv[XW];
#pragma unroll
                for (int i = 0; i < XW; ++i)
                    xv[i] = rowbase[u * twl + i];
#pragma unroll
                for (int kh = 0; kh < KH; ++kh) {
                    const int m = u - kh * D;
                    if (m >= 0 && m < TH && !(DEC && ((h0 + m) & 1))) {
                        const int slot = m % R;
#pragma unroll
                        for (int kw = 0; kw < KW; ++kw)
#pragma unroll
                            for (int j = 0; j < Q; ++j)
                                acc[slot][j] = fmaf(wr[kh][kw], xv[j + kw * D], acc[slot][j]);
                    }
                }
            }
            const int m = u - (R - 1);
            if (m >= 0) {
                if constexpr (EPI) {
                    const EpiChan e1[1] = {ec};
                    epi_block(acc[m % R], e1, ep.act);
                }
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
}

// ---------------------------------------------------------------------------
// Weight and bias gradients (LeanMlir "Depthwise": weight-VJP, bias-gradient
// closed form).  Two stages, deterministic (fixed summation order, no
// atomics):
//   stage 1 writes partial sums part[chunk][c][tap], tap = kh*kW + kw for
//           dW and tap = kH*kW for db, each over one chunk of dy positions;
//   stage 2 adds the chunks of every (c, tap) column in a fixed order.
// ---------------------------------------------------------------------------
struct WgradArgs {
    int N, C, mult;         // C: channels of dy (and of dW); x has C / mult
    int H, W, kH, kW, d, pH, pW;
    int OH, OW;             // dy extents
    int nct, nwt, nsp;      // tiled: channel tiles, column tiles, strips
    int strip;              // tiled: row tiles per strip
    int chunks;             // rows of part[]
};

// Stage 1, any layout, stride, padding and multiplier.  Lanes run along the
// contiguous axis so every load of a wave is one coalesced run: in NHWC
// `cl` consecutive output channels x 256/cl position slots, in NCHW 256
// consecutive positions of one output channel's plane.  A workgroup sums
// one chunk of `ppc` dy positions; the kH*kW taps and the bias column go in
// groups of 8 register accumulators (dy is re-read, from cache, once per
// group), and the slots of a channel are added in LDS in a fixed order.
// Output channel c reads x channel c / mult.
struct WgradGenArgs {
    int N, C, mult;         // C: channels of dy (and of dW); x has C / mult
    int H, W, OH, OW;       // x extents, dy extents
    int kH, kW, d, pH, pW;
    int cl, ncg;            // NHWC: channel lanes (16, 32 or 64), channel groups
    int ppc;                // dy positions per chunk
    int cpi;                // NCHW: chunks per image
};

constexpr int kWgradTapGroup = 8;

template <bool NHWC, int S>
__global__ __launch_bounds__(256) void k_wgrad_gen(const float *__restrict__ x,
                                                   const float *__restrict__ dy,
                                                   float *__restrict__ part, WgradGenArgs a)
{
    __shared__ float red[kWgradTapGroup][256];
    const int tid = threadIdx.x;
    const int KK = a.kH * a.kW;
    const int CI = a.C / a.mult;
    const int per_img = a.OH * a.OW;
    int chunk, c, slot, nslot, p0, p1, n_fixed = 0;
    if (NHWC) {
        const int cg = blockIdx.x % a.ncg;
        chunk = blockIdx.x / a.ncg;
        c = cg * a.cl + tid % a.cl;
        slot = tid / a.cl;
        nslot = 256 / a.cl;
        p0 = chunk * a.ppc;                               // over (n, ho, wo) of all images
        p1 = min(p0 + a.ppc, a.N * per_img);
    } else {
        c = blockIdx.x % a.C;
        chunk = blockIdx.x / a.C;                         // (n, range within the plane)
        n_fixed = chunk / a.cpi;
        slot = tid;
        nslot = 256;
        p0 = (chunk - n_fixed * a.cpi) * a.ppc;           // within image n_fixed
        p1 = min(p0 + a.ppc, per_img);
    }
    const bool cvalid = c < a.C;
    const int ci = c / a.mult;
    for (int tg = 0; tg <= KK; tg += kWgradTapGroup) {
        float acc[kWgradTapGroup];
        int th[kWgradTapGroup], tw[kWgradTapGroup];       // tap offsets; th = -1: bias column
#pragma unroll
        for (int t = 0; t < kWgradTapGroup; ++t) {
            acc[t] = 0.0f;
            const int tap = tg + t;
            th[t] = tap < KK ? (tap / a.kW) * a.d - a.pH : -(1 << 30);
            tw[t] = tap < KK ? (tap % a.kW) * a.d - a.pW : 0;
        }
        if (cvalid) {
            for (int pp = p0 + slot; pp < p1; pp += nslot) {
                int n, rem;
                if (NHWC) {
                    n = pp / per_img;
                    rem = pp - n * per_img;
                } else {
                    n = n_fixed;
                    rem = pp;
                }
                const int ho = rem / a.OW, wo = rem - (rem / a.OW) * a.OW;
                const float g = NHWC ? dy[((n * a.OH + ho) * a.OW + wo) * a.C + c]
                                     : dy[((n * a.C + c) * a.OH + ho) * a.OW + wo];
#pragma unroll
                for (int t = 0; t < kWgradTapGroup; ++t) {
                    const int hi = ho * S + th[t], wi = wo * S + tw[t];
                    if (hi >= 0 && hi < a.H && wi >= 0 && wi < a.W) {
                        const float xv = NHWC ? x[((n * a.H + hi) * a.W + wi) * CI + ci]
                                              : x[((n * CI + ci) * a.H + hi) * a.W + wi];
                        acc[t] = fmaf(xv, g, acc[t]);
                    } else if (tg + t == KK) {
                        acc[t] += g;                      // the bias column
                    }
                }
            }
        }
        // add the slots of each channel in a fixed order
        __syncthreads();
#pragma unroll
        for (int t = 0; t < kWgradTapGroup; ++t)
            red[t][tid] = acc[t];
        __syncthreads();
        if (NHWC) {
            // thread e sums column (tap e / cl, lane e % cl) over the slots
            for (int e = tid; e < kWgradTapGroup * a.cl; e += 256) {
                const int t = e / a.cl, lane = e - t * a.cl;
                const int cc = (blockIdx.x % a.ncg) * a.cl + lane;
                if (tg + t <= KK && cc < a.C) {
                    float sum = 0.0f;
                    for (int sl = 0; sl < nslot; ++sl)
                        sum += red[t][sl * a.cl + lane];
                    part[((long long)chunk * a.C + cc) * (KK + 1) + tg + t] = sum;
                }
            }
        } else {
            // fixed tree over the 256 positions, all 8 taps at once
#pragma unroll
            for (int off = 128; off > 0; off >>= 1) {
                if (tid < off)
#pragma unroll
                    for (int t = 0; t < kWgradTapGroup; ++t)
                        red[t][tid] += red[t][tid + off];
                __syncthreads();
            }
            if (tid < kWgradTapGroup && tg + tid <= KK)
                part[((long long)chunk * a.C + c) * (KK + 1) + tg + tid] = red[tid][0];
        }
    }
}

// Stage 1, NHWC, stride S = 1 or 2: a workgroup (256 threads: CL across
// channels x 256/CL pixel slots of PX dy columns) walks `strip` row tiles of
// one column tile.  Per row tile it stages G input rows (+ column halo) in LDS and
// loads its dy rows straight into registers (each dy element is used by one
// thread only); every thread accumulates x*dy for all kH*kW taps of its
// channels, and at the end the pixel slots are summed through LDS.
// LV: floats per staging load, 4 (C % 4 == 0, 16-byte aligned tensors) or 1
// (any C, one channel per thread).  At stride 2 a tile of TH x TW dy
// positions reads 2*TH - 1 + (KH-1)*D rows and 2*TW - 1 + (KW-1)*D columns
// of x, and dy position (m, j) meets x at (2m + kh*D, 2j + kw*D).
template <int KH, int KW, int D, int VEC, int CL, int PX, int G, int LV, int S>
__global__ __launch_bounds__(256) void k_wgrad_tiled_nhwc(const float *__restrict__ x,
                                                          const float *__restrict__ dy,
                                                          float *__restrict__ part, WgradArgs a)
{
    static_assert(LV == 4 || (LV == 1 && VEC == 1), "scalar staging: one channel per thread");
    static_assert(S == 1 || S == 2, "stride 1 or 2");
    constexpr int R = (KH - 1) * D + 1, TW = PX * 256 / CL, CG = CL * VEC;
    constexpr int TH = (G - R) / S + 1;     // dy rows per row tile
    static_assert(G >= R && (G - R) % S == 0, "staged rows = S*(TH-1) + R");
    constexpr int TWI = S * (TW - 1) + 1 + (KW - 1) * D, VPC = CG / LV, VPR = TWI * VPC;
    constexpr int VCH = G * VPR, NV = (VCH + 255) / 256, KK = KH * KW, NP = 256 / CL;
    constexpr int XW = S * (PX - 1) + 1 + (KW - 1) * D;
    constexpr int XF = VCH * LV;            // staged floats
    // the final per-(channel, tap) sums go through LDS in groups of TG taps
    constexpr int TGF = XF / (256 * VEC);
    constexpr int TG = TGF < 1 ? 1 : (TGF > KK + 1 ? KK + 1 : TGF);
    constexpr int LDSF = (XF > 256 * VEC * TG) ? XF : 256 * VEC * TG;
    __shared__ float4 lds4[(LDSF + 3) / 4];
    float *lds = reinterpret_cast<float *>(lds4);

    int tile = blockIdx.x;
    const int ct = tile % a.nct;
    tile /= a.nct;
    const int chunk = tile;                 // (n, strip, column tile): row of part[]
    const int wt = tile % a.nwt;
    tile /= a.nwt;
    const int sp = tile % a.nsp;
    const int n = tile / a.nsp;
    const int c0 = ct * CG, w0 = wt * TW;
    const int tid = threadIdx.x;
    const int q = tid % CL, p = tid / CL;
    const int cq = c0 + q * VEC;
    const int ow = w0 + p * PX;
    const int cbase = S * w0 - a.pW;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + n * a.H * a.W * a.C, a.H * a.W * a.C * 4);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(dy + n * a.OH * a.OW * a.C, a.OH * a.OW * a.C * 4);

    float acc[KK + 1][VEC];                 // taps kh*KW + kw, then the bias
#pragma unroll
    for (int t = 0; t <= KK; ++t)
#pragma unroll
        for (int v = 0; v < VEC; ++v)
            acc[t][v] = 0.0f;

    const int t0 = sp * a.strip, t1 = min(t0 + a.strip, (a.OH + TH - 1) / TH);
    for (int tt = t0; tt < t1; ++tt) {
        const int h0 = tt * TH;
        const int nrows = S * (min(TH, a.OH - h0) - 1) + R;
        const int rbase = S * h0 - a.pH;
        // this row tile's x rows (+ halo) and, per thread, its dy values
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
            const bool ok = e < VCH && g < nrows && row >= 0 && row < a.H && gc >= 0 &&
                            gc < a.W && ch < a.C;
            const int off = ok ? ((row * a.W + gc) * a.C + ch) * 4 : kOutOfRange;
            if constexpr (LV == 4)
                stage[i] = buf_f4(rx, off);
            else
                stage[i] = buf_f32(rx, off);
        }
        float gv[TH][PX][VEC];
#pragma unroll
        for (int m = 0; m < TH; ++m)
#pragma unroll
            for (int j = 0; j < PX; ++j) {
                const bool ok = h0 + m < a.OH && ow + j < a.OW && cq < a.C;
                buf_vec<VEC>(rg, ok ? (((h0 + m) * a.OW + ow + j) * a.C + cq) * 4 : kOutOfRange,
                             gv[m][j]);
            }
        if (tt > t0)
            __syncthreads();              // every thread done with the previous tile
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int e = tid + i * 256;
            if (e < VCH)
                reinterpret_cast<LoadT *>(lds4)[e] = stage[i];
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < TH; ++m) {
#pragma unroll
            for (int j = 0; j < PX; ++j)
#pragma unroll
                for (int v = 0; v < VEC; ++v)
                    acc[KK][v] += gv[m][j][v];
#pragma unroll
            for (int kh = 0; kh < KH; ++kh) {
                const int u = S * m + kh * D;   // staged row of tap row kh for dy row m
                float xv[XW][VEC];
#pragma unroll
                for (int i = 0; i < XW; ++i) {
                    const float *src = lds + ((u * TWI + S * p * PX + i) * CG + q * VEC);
#pragma unroll
                    for (int v = 0; v < VEC; ++v)
                        xv[i][v] = src[v];
                }
#pragma unroll
                for (int kw = 0; kw < KW; ++kw)
#pragma unroll
                    for (int j = 0; j < PX; ++j)
#pragma unroll
                        for (int v = 0; v < VEC; ++v)
                            acc[kh * KW + kw][v] =
                                fmaf(xv[S * j + kw * D][v], gv[m][j][v], acc[kh * KW + kw][v]);
            }
        }
    }

    // sum the NP pixel slots of every (channel, tap) in a fixed order, TG taps at a time
#pragma unroll
    for (int tb = 0; tb <= KK; tb += TG) {
        __syncthreads();
#pragma unroll
        for (int k = 0; k < TG; ++k)
            if (tb + k <= KK)
#pragma unroll
                for (int v = 0; v < VEC; ++v)
                    lds[(k * 256 + tid) * VEC + v] = acc[tb + k][v];
        __syncthreads();
        for (int e = tid; e < CG * TG; e += 256) {
            const int k = e / CG, cl = e - k * CG;
            const int qq = cl / VEC, v = cl - qq * VEC;
            if (tb + k <= KK) {
                float s = 0.0f;
                for (int pp = 0; pp < NP; ++pp)
                    s += lds[(k * 256 + pp * CL + qq) * VEC + v];
                if (c0 + cl < a.C)
                    part[((long long)chunk * a.C + c0 + cl) * (KK + 1) + tb + k] = s;
            }
        }
    }
}

// Stage 1, NCHW stride 1: the NCHW forward's tiling with the roles of the
// operands changed.  A workgroup covers pb dy planes x tx threads per plane
// row (Q adjacent columns each) and walks `strip` row tiles of one column
// tile; per row tile it stages the G x rows (+ column halo) of its planes'
// input planes in LDS and loads its dy values into registers, and every
// thread accumulates x*dy for all kH*kW taps (and dy for the bias) of its
// plane.  The tx threads of each plane are then added with a fixed tree in
// LDS, TG taps at a time.
struct WgradNchwArgs {
    int planes, C, mult;        // dy planes (N * C), dy channels, channel multiplier
    int H, W, OH, OW;           // x extents, dy extents
    int pH, pW, hl, twl;        // pads; staged columns left of a tile, staged floats per row
    int txn, pbn;               // threads per plane row (16..256), planes per workgroup
    int nct, nwt, nsp, strip;   // plane groups, column tiles, strips, row tiles per strip
    int nrt;                    // row tiles per plane
};

// At stride S = 2 a row tile of TH dy rows reads 2*TH - 1 + (kH-1)*d x rows,
// a thread's Q dy columns meet x columns 2j + kw*d of its window, and the
// staged x row of a tile is 2*tw - 1 + (kW-1)*d columns wide.
template <int KH, int KW, int D, int Q, int G, bool V4, int S>
__global__ __launch_bounds__(256) void k_wgrad_tiled_nchw(const float *__restrict__ x,
                                                          const float *__restrict__ dy,
                                                          float *__restrict__ part,
                                                          WgradNchwArgs a)
{
    typedef NchwGeom<KH, KW, D, Q, G, V4> Gm;
    static_assert(S == 1 || S == 2, "stride 1 or 2");
    constexpr int R = Gm::R, KK = Gm::KK, LV = Gm::LV;
    constexpr int TH = (G - R) / S + 1;                  // dy rows per row tile
    static_assert(G >= R && (G - R) % S == 0, "staged rows = S*(TH-1) + R");
    // per-thread loads for the largest staged tile: G rows x (256*S*Q + 16*EXTRA) floats
    constexpr int NV = (G * (256 * S * Q + Gm::PBMAX * Gm::EXTRA) / LV + 255) / 256;
    constexpr int XW = S * (Q - 1) + 1 + (KW - 1) * D;
    extern __shared__ float4 lds4[];
    float *lds = reinterpret_cast<float *>(lds4);

    const int txn = a.txn, pbn = a.pbn;
    const int tw = txn * Q, twl = a.twl, vpr = twl / LV;
    int tile = blockIdx.x;
    const int pg = tile % a.nct;
    tile /= a.nct;
    const int wt = tile % a.nwt;
    const int sp = tile / a.nwt;
    const int w0 = wt * tw;
    const int tid = threadIdx.x;
    // threads past pbn * txn (when txn does not divide 256) idle along
    const int pli_raw = tid / txn, tx = tid - pli_raw * txn;
    const int pli = min(pli_raw, pbn - 1);             // in-range LDS addresses for idle threads
    const int my_plane = pg * pbn + pli;
    const bool pvalid = pli_raw < pbn && my_plane < a.planes;
    const int oc = w0 + tx * Q;
    const int CI = a.C / a.mult;
    const int cbase = S * w0 - a.hl;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (a.planes / a.C) * CI * a.H * a.W * 4);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(dy, a.planes * a.OH * a.OW * 4);
    const float *rowbase = lds + pli * G * twl + S * tx * Q + (a.hl - a.pW);

    float acc[KK + 1];
#pragma unroll
    for (int t = 0; t <= KK; ++t)
        acc[t] = 0.0f;

    const int t0 = sp * a.strip, t1 = min(t0 + a.strip, a.nrt);
    for (int tt = t0; tt < t1; ++tt) {
        const int h0 = tt * TH;
        const int nrows = S * (min(TH, a.OH - h0) - 1) + R;
        const int rbase = S * h0 - a.pH;
        float sv[NV][LV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int e = tid + i * 256;
            const int pl = e / (G * vpr);
            const int rem = e - pl * (G * vpr);
            const int g = rem / vpr;
            const int col = cbase + (rem - g * vpr) * LV;
            const int plane = pg * pbn + pl, row = rbase + g;
            const bool ok = pl < pbn && plane < a.planes && g < nrows && row >= 0 && row < a.H &&
                            col >= 0 && col < a.W;
            // x plane read by dy plane (n, o): (n, o / mult)
            const int xplane = (plane / a.C) * CI + (plane % a.C) / a.mult;
            const int off = ok ? ((xplane * a.H + row) * a.W + col) * 4 : kOutOfRange;
            if constexpr (V4) {
                const float4 v = buf_f4(rx, off);
                sv[i][0] = v.x; sv[i][1] = v.y; sv[i][2] = v.z; sv[i][3] = v.w;
            } else {
                sv[i][0] = buf_f32(rx, off);
            }
        }
        float gv[TH][Q];
#pragma unroll
        for (int m = 0; m < TH; ++m)
#pragma unroll
            for (int j = 0; j < Q; ++j) {
                const bool ok = pvalid && h0 + m < a.OH && oc + j < a.OW;
                gv[m][j] = buf_f32(rg, ok ? ((my_plane * a.OH + h0 + m) * a.OW + oc + j) * 4
                                          : kOutOfRange);
            }
        if (tt > t0)
            __syncthreads();              // every thread done with the previous tile
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int e = tid + i * 256;
            if (e < pbn * G * vpr) {
                if constexpr (V4)
                    lds4[e] = make_float4(sv[i][0], sv[i][1], sv[i][2], sv[i][3]);
                else
                    lds[e] = sv[i][0];
            }
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < TH; ++m) {
#pragma unroll
            for (int j = 0; j < Q; ++j)
                acc[KK] += gv[m][j];
#pragma unroll
            for (int kh = 0; kh < KH; ++kh) {
                float xv[XW];
#pragma unroll
                for (int i = 0; i < XW; ++i)
                    xv[i] = rowbase[(S * m + kh * D) * twl + i];
#pragma unroll
                for (int kw = 0; kw < KW; ++kw)
#pragma unroll
                    for (int j = 0; j < Q; ++j)
                        acc[kh * KW + kw] =
                            fmaf(xv[S * j + kw * D], gv[m][j], acc[kh * KW + kw]);
            }
        }
    }

    // add the tx threads of each plane: every thread parks its KK + 1 sums in
    // LDS, then each (plane, tap) column is added over the plane's threads in
    // thread order (one pass, fixed order)
    constexpr int KP = (KK + 1) | 1;                   // odd row stride: no bank conflicts
    __syncthreads();                                   // every thread done with the tile
#pragma unroll
    for (int t = 0; t <= KK; ++t)
        lds[tid * KP + t] = acc[t];
    __syncthreads();
    const int n_cols = pbn * (KK + 1);
    for (int e = tid; e < n_cols; e += 256) {
        const int pl = e / (KK + 1), t = e - pl * (KK + 1);
        const int plane = pg * pbn + pl;
        if (plane < a.planes) {
            const float *col = lds + pl * txn * KP + t;
            float sum = 0.0f;
            for (int j = 0; j < txn; ++j)
                sum += col[j * KP];
            const int n = plane / a.C, o = plane % a.C;
            const int chunk = (n * a.nwt + wt) * a.nsp + sp;
            part[((long long)chunk * a.C + o) * (KK + 1) + t] = sum;
        }
    }
}

// Stage 2: 64 columns of part[] per workgroup, one per lane, so every wave
// load is one coalesced run; wave w adds the chunks w, w+4, w+8, ... with 8
// independent partial sums (8 loads in flight), combined in a fixed order,
// and the 4 waves are added in a fixed order in LDS.  The result depends
// only on the partial sums, never on timing.
// With w_upd, the LeanMlir page's SGD step is fused in: w_upd -= lr * dW and,
// with b_upd, b_upd -= lr * db (one rounding each: fmaf(-lr, grad, old)).
constexpr int kReduceUnroll = 8;

__global__ __launch_bounds__(256) void k_wgrad_reduce(const float *__restrict__ part,
                                                      float *__restrict__ dw,
                                                      float *__restrict__ db, int chunks,
                                                      int C, int KK, float *__restrict__ w_upd,
                                                      float *__restrict__ b_upd, float lr)
{
    __shared__ float red[4][64];
    const int cols = C * (KK + 1);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int col = blockIdx.x * 64 + lane;
    const bool valid = col < cols;
    float s[kReduceUnroll];
#pragma unroll
    for (int u = 0; u < kReduceUnroll; ++u)
        s[u] = 0.0f;
    if (valid) {
        int r = wv;
        for (; r + 4 * (kReduceUnroll - 1) < chunks; r += 4 * kReduceUnroll) {
            float v[kReduceUnroll];
#pragma unroll
            for (int u = 0; u < kReduceUnroll; ++u)
                v[u] = part[(long long)(r + 4 * u) * cols + col];
#pragma unroll
            for (int u = 0; u < kReduceUnroll; ++u)
                s[u] += v[u];
        }
#pragma unroll
        for (int u = 0; u < kReduceUnroll - 1; ++u)
            if (r + 4 * u < chunks)
                s[u] += part[(long long)(r + 4 * u) * cols + col];
    }
#pragma unroll
    for (int w = kReduceUnroll / 2; w > 0; w >>= 1)
#pragma unroll
        for (int u = 0; u < w; ++u)
            s[u] += s[u + w];
    red[wv][lane] = s[0];
    __syncthreads();
    if (wv == 0 && valid) {
        const float g = (red[0][lane] + red[1][lane]) + (red[2][lane] + red[3][lane]);
        const int c = col / (KK + 1), tap = col - c * (KK + 1);
        if (tap < KK) {
            if (dw)
                dw[c * KK + tap] = g;
            if (w_upd)
                w_upd[c * KK + tap] = fmaf(-lr, g, w_upd[c * KK + tap]);
        } else {
            if (db)
                db[c] = g;
            if (b_upd)
                b_upd[c] = fmaf(-lr, g, b_upd[c]);
        }
    }
}

// ---------------------------------------------------------------------------
// Launch helpers
// ---------------------------------------------------------------------------
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
void launch_direct(const Problem &p, const Plan &pl, const float *in, const void *wv,
                   const float *b, float *out, hipStream_t st, const EpiArgs &ep)
{
    const DirectArgs a = direct_args(p, pl);
    const WT *w = reinterpret_cast<const WT *>(wv);
    const dim3 grid((unsigned)pl.grid), block(256);
    const bool ig = p.op == DWCONV_OP_INPUT_GRAD;
    const int s = p.stride;
#define DW_DIRECT_NHWC(V, IGV, SV) \
    hipLaunchKernelGGL((k_direct_nhwc<WT, V, IGV, SV>), grid, block, 0, st, in, w, b, out, a, ep)
#define DW_DIRECT_NCHW(IGV, SV) \
    hipLaunchKernelGGL((k_direct_nchw<WT, IGV, SV>), grid, block, 0, st, in, w, b, out, a, ep)
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

int mode_of(const Problem &p, const EpiArgs &ep)
{
    if (p.op == DWCONV_OP_INPUT_GRAD)
        return kModeInputGrad;
    return ep.on ? kModeFwdEpilogue : kModeFwd;
}

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

struct TiledNchwTable {
    TiledNchwFn fn[kNumTiledNchwVariants][2][3];
    TiledNchwFn fn2[kNumTiledNchwS2Variants][2][3];
    TiledNchwTable()
    {
        fill_all_tiled_nchw<1>(fn, std::make_integer_sequence<int, kNumTiledNchwVariants>());
        fill_all_tiled_nchw<2>(fn2, std::make_integer_sequence<int, kNumTiledNchwS2Variants>());
    }
};

int launch_tiled_nchw(const Problem &p, const Plan &pl, const float *in, const void *w,
                      const float *b, float *out, hipStream_t st, const EpiArgs &ep)
{
    static const TiledNchwTable table;
    const int nvar = p.stride == 1 ? kNumTiledNchwVariants : kNumTiledNchwS2Variants;
    if (pl.variant < 0 || pl.variant >= nvar || pl.cl < 16 || pl.cl > 256 ||
        pl.pb != 256 / pl.cl)
        return DWCONV_ERR_BAD_STRATEGY;
    TiledNchwFn f = p.stride == 1
                        ? table.fn[pl.variant][p.wtype == DWCONV_W_F16][mode_of(p, ep)]
                        : table.fn2[pl.variant][p.wtype == DWCONV_W_F16][mode_of(p, ep)];
    if (!f)
        return DWCONV_ERR_BAD_STRATEGY;
    TiledNchwArgs a;
    a.planes = p.N * p.C; a.C = p.C;
    a.IH = pl.IH; a.IW = pl.IW; a.OH = pl.OH; a.OW = pl.OW;
    a.YH = pl.YH; a.YW = pl.YW;
    a.pH = pl.pH; a.pW = pl.pW; a.hl = pl.hl; a.twl = pl.twl;
    a.txn = pl.cl;
    a.pbn = pl.pb;
    a.nct = pl.nct; a.nwt = pl.nwt; a.nst = pl.nst;
    hipLaunchKernelGGL(f, dim3((unsigned)pl.grid), dim3(256), pl.lds_bytes, st, in, w,
                       p.op == DWCONV_OP_FWD ? b : nullptr, out, a, ep);
    return DWCONV_OK;
}

typedef void (*WgradFn)(const float *, const float *, float *, WgradArgs);

template <int V, int S>
constexpr WgradFn wgrad_fn()
{
    if constexpr (S == 1) {
        constexpr WgradVariant t = kWgradVariants[V];
        return &k_wgrad_tiled_nhwc<t.kH, t.kW, t.d, t.vec, t.cl, t.px, t.g, t.lv, 1>;
    } else {
        constexpr WgradVariant t = kWgradS2Variants[V];
        return &k_wgrad_tiled_nhwc<t.kH, t.kW, t.d, t.vec, t.cl, t.px, t.g, t.lv, 2>;
    }
}

template <int S, int NVAR, int... Vs>
void fill_wgrad(WgradFn (&fn)[NVAR], std::integer_sequence<int, Vs...>)
{
    ((fn[Vs] = wgrad_fn<Vs, S>()), ...);
}

struct WgradTable {
    WgradFn fn[kNumWgradVariants];
    WgradFn fn2[kNumWgradS2Variants];
    WgradTable()
    {
        fill_wgrad<1>(fn, std::make_integer_sequence<int, kNumWgradVariants>());
        fill_wgrad<2>(fn2, std::make_integer_sequence<int, kNumWgradS2Variants>());
    }
};

}  // namespace

typedef void (*WgradNchwFn)(const float *, const float *, float *, WgradNchwArgs);

template <int V, int S>
constexpr WgradNchwFn wgrad_nchw_fn()
{
    if constexpr (S == 1) {
        constexpr TiledNchwVariant t = kTiledNchwVariants[V];
        return &k_wgrad_tiled_nchw<t.kH, t.kW, t.d, t.q, t.g, (t.v4 != 0), 1>;
    } else {
        constexpr TiledNchwVariant t = kWgradNchwS2Variants[V];
        return &k_wgrad_tiled_nchw<t.kH, t.kW, t.d, t.q, t.g, (t.v4 != 0), 2>;
    }
}

template <int S, int NVAR, int... Vs>
void fill_wgrad_nchw(WgradNchwFn (&fn)[NVAR], std::integer_sequence<int, Vs...>)
{
    ((fn[Vs] = wgrad_nchw_fn<Vs, S>()), ...);
}

struct WgradNchwTable {
    WgradNchwFn fn[kNumTiledNchwVariants];
    WgradNchwFn fn2[kNumWgradNchwS2Variants];
    WgradNchwTable()
    {
        fill_wgrad_nchw<1>(fn, std::make_integer_sequence<int, kNumTiledNchwVariants>());
        fill_wgrad_nchw<2>(fn2, std::make_integer_sequence<int, kNumWgradNchwS2Variants>());
    }
};

// Run a validated plan on `stream`.  Returns a DWCONV_ status.
int launch_plan(const Problem &p, const Plan &pl, const float *in, const void *w,
                const float *b, float *out, void *stream_v, const Epilogue *epi)
{
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_v);
    const float *bb = p.op == DWCONV_OP_FWD ? b : nullptr;
    EpiArgs ep{nullptr, nullptr, nullptr, nullptr, 0.0f, DWCONV_ACT_NONE, 0};
    if (epi && p.op == DWCONV_OP_FWD) {
        ep.gamma = epi->gamma; ep.beta = epi->beta; ep.mean = epi->mean; ep.var = epi->var;
        ep.eps = epi->eps;
        ep.act = epi->act;
        ep.on = 1;
    }
    int st = DWCONV_OK;
    switch (pl.kind) {
    case KIND_DIRECT_NHWC:
    case KIND_DIRECT_NCHW:
        if (p.wtype == DWCONV_W_F16)
            launch_direct<half_t>(p, pl, in, w, bb, out, stream, ep);
        else
            launch_direct<float>(p, pl, in, w, bb, out, stream, ep);
        break;
    case KIND_TILED_NHWC:
        st = launch_tiled_nhwc(p, pl, in, w, bb, out, stream, ep);
        break;
    case KIND_TILED_NCHW:
        st = launch_tiled_nchw(p, pl, in, w, bb, out, stream, ep);
        break;
    default:
        return DWCONV_ERR_BAD_STRATEGY;
    }
    if (st != DWCONV_OK)
        return st;
    return hipGetLastError() == hipSuccess ? DWCONV_OK : DWCONV_ERR_LAUNCH;
}

int launch_wgrad(const Problem &p, const Plan &pl, const float *x, const float *dy, float *dw,
                 float *db, void *workspace, void *stream_v, float *w_upd, float *b_upd,
                 float lr)
{
    hipStream_t st = reinterpret_cast<hipStream_t>(stream_v);
    float *part = reinterpret_cast<float *>(workspace);
    WgradArgs a;
    a.N = p.N; a.C = p.mult * p.C; a.mult = p.mult;
    a.H = p.H; a.W = p.W; a.kH = p.kH; a.kW = p.kW; a.d = p.dilation;
    a.pH = pl.pH; a.pW = pl.pW; a.OH = pl.OH; a.OW = pl.OW;
    a.nct = pl.nct; a.nwt = pl.nwt; a.nsp = pl.nst; a.strip = pl.strip; a.chunks = (int)pl.chunks;
    if (pl.kind == KIND_WGRAD_TILED_NHWC) {
        static const WgradTable table;
        const int nvar = p.stride == 1 ? kNumWgradVariants : kNumWgradS2Variants;
        if (pl.variant < 0 || pl.variant >= nvar)
            return DWCONV_ERR_BAD_STRATEGY;
        hipLaunchKernelGGL(p.stride == 1 ? table.fn[pl.variant] : table.fn2[pl.variant],
                           dim3((unsigned)pl.grid), dim3(256), 0, st, x, dy, part, a);
    } else if (pl.kind == KIND_WGRAD_TILED_NCHW) {
        static const WgradNchwTable table;
        const int nvar = p.stride == 1 ? kNumTiledNchwVariants : kNumWgradNchwS2Variants;
        if (pl.variant < 0 || pl.variant >= nvar || pl.cl < 16 || pl.cl > 256 ||
            pl.pb != 256 / pl.cl)
            return DWCONV_ERR_BAD_STRATEGY;
        WgradNchwArgs g;
        g.planes = p.N * p.mult * p.C; g.C = p.mult * p.C; g.mult = p.mult;
        g.H = p.H; g.W = p.W; g.OH = pl.OH; g.OW = pl.OW;
        g.pH = pl.pH; g.pW = pl.pW; g.hl = pl.hl; g.twl = pl.twl;
        g.txn = pl.cl;
        g.pbn = pl.pb;
        g.nct = pl.nct; g.nwt = pl.nwt; g.nsp = pl.nst; g.strip = pl.strip; g.nrt = pl.nrt;
        hipLaunchKernelGGL(p.stride == 1 ? table.fn[pl.variant] : table.fn2[pl.variant],
                           dim3((unsigned)pl.grid), dim3(256), pl.lds_bytes, st, x, dy, part, g);
    } else if (pl.kind == KIND_WGRAD_DIRECT) {
        WgradGenArgs g;
        g.N = p.N; g.C = p.mult * p.C; g.mult = p.mult;
        g.H = p.H; g.W = p.W; g.OH = pl.OH; g.OW = pl.OW;
        g.kH = p.kH; g.kW = p.kW; g.d = p.dilation; g.pH = pl.pH; g.pW = pl.pW;
        g.cl = pl.cl; g.ncg = pl.nct; g.ppc = pl.ppc; g.cpi = pl.cpi;
        const dim3 gr((unsigned)pl.grid), b(256);
        const bool nhwc = p.layout == DWCONV_LAYOUT_NHWC;
        if (nhwc && p.stride == 1)
            hipLaunchKernelGGL((k_wgrad_gen<true, 1>), gr, b, 0, st, x, dy, part, g);
        else if (nhwc)
            hipLaunchKernelGGL((k_wgrad_gen<true, 2>), gr, b, 0, st, x, dy, part, g);
        else if (p.stride == 1)
            hipLaunchKernelGGL((k_wgrad_gen<false, 1>), gr, b, 0, st, x, dy, part, g);
        else
            hipLaunchKernelGGL((k_wgrad_gen<false, 2>), gr, b, 0, st, x, dy, part, g);
    } else {
        return DWCONV_ERR_BAD_STRATEGY;
    }
    hipLaunchKernelGGL(k_wgrad_reduce, dim3((unsigned)pl.grid2), dim3(256), 0, st, part, dw, db,
                       (int)pl.chunks, p.mult * p.C, p.kH * p.kW, w_upd,
                       w_upd ? b_upd : nullptr, lr);
    return hipGetLastError() == hipSuccess ? DWCONV_OK : DWCONV_ERR_LAUNCH;
}

}  // namespace dwconv
