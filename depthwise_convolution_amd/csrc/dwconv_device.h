// dwconv_device.h -- what the gfx950 kernel files of the library share.
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
// One translation unit per kernel family:
//  * dwconv_direct.hip: one thread per output (NCHW) or per channel vector
//    (NHWC); taps read from global memory through the caches.  They cover
//    every valid problem (any kernel, pads, multipliers).
//  * dwconv_tiled_nhwc.hip / dwconv_tiled_nchw.hip (stride 1 or 2): a
//    short-lived workgroup stages the input rows its output rows need (tile
//    plus (k-1)*d halo, zero outside the image, via raw buffer loads) and
//    its weights in LDS in one load phase, then walks the rows: each thread
//    reads its kW horizontal taps per staged row from LDS and folds the row
//    into R = (kH-1)*d + 1 rolling accumulators, so every input element is
//    fetched from HBM about once and reused for all kH*kW taps.
//    Compile-time modes: forward, input gradient (reversed taps, no bias),
//    forward with the BatchNorm / activation epilogue.
//  * dwconv_wgrad.hip: weight gradient, per-chunk partial sums (tiled NHWC,
//    tiled NCHW or a generic coalesced kernel), then a fixed-order reduction
//    that can also apply the SGD step.
//  * dwconv_launch.hip: runs a plan (the dispatch over the families).
// Every output store is non-temporal: outputs are write-once streams.
//
// This header: fp16 weight widening, vector loads and non-temporal stores,
// raw buffer loads (a read outside the buffer returns zero in hardware),
// the forward epilogue (BatchNorm + activation), the NCHW tile geometry and
// the launchers of the kernel families.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <tuple>
#include <type_traits>
#include <utility>

#include "dwconv_internal.h"
#include "../../include/dwconv.h"

namespace dwconv {

// Arguments of the forward epilogue (a kernel argument; `on` = 0: none).
struct EpiArgs {
    const float *gamma, *beta, *mean, *var;   // all NULL: no BatchNorm
    float eps;
    int act;                                  // DWCONV_ACT_*
    int on;                                   // direct kernels: apply the epilogue
};

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

// Workgroup -> tile order.  MI355X hands the workgroups of a launch to its
// 8 XCDs in turn (workgroup b runs on XCD b % 8), and each XCD has an L2 of
// its own.  The tiled kernels number their tiles so that tiles sharing halo
// rows or columns are close in the numbering (in NCHW the row tiles of a
// plane group are consecutive).  For problems up to a few hundred MiB the
// plan has workgroup b take tile xcd_tile(b): XCD k then runs one
// contiguous range of tiles, in order, so a halo that a tile shares with its
// neighbours is read from HBM once into that XCD's L2.  Larger problems take
// tile b: all XCDs sweep the tensor front to back together, which streams
// from HBM faster than eight separate ranges.
// A bijection of [0, nb): XCD k < nb % 8 takes nb / 8 + 1 tiles, the others
// nb / 8.
__device__ __forceinline__ int xcd_tile(int b, int nb)
{
    const int per = nb >> 3, extra = nb & 7, k = b & 7;
    return k * per + min(k, extra) + (b >> 3);
}

// Band-local order (large NHWC problems): the tiles of a row band (the
// channel and column tiles of one row tile, `band` of them, a multiple of
// 8) are split into 8 runs of consecutive tiles, run k going to XCD k, so
// most column neighbours share an L2 while all XCDs still sweep the tensor
// band by band.  A bijection of [0, nb) when band divides nb.
__device__ __forceinline__ int band_tile(int b, int band)
{
    const int run = band >> 3, k = b >> 3;
    return (k / run) * band + (b & 7) * run + k % run;
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

// Raw buffer load straight into LDS (the LDS flag of gfx950's buffer loads):
// lane k of the wave writes its BYTES (4 or 16) to lds + k*BYTES, where
// `lds` is the same in every lane; an offset outside the buffer writes
// zeros.  The data reaches LDS asynchronously: drain the wave's vector
// memory counter (vm_drain) before the barrier that hands the tile to the
// other waves.  NT: the non-temporal cache policy (for data no other
// workgroup reads).
template <int BYTES, bool NT = false>
__device__ __forceinline__ void buf_to_lds(__amdgpu_buffer_rsrc_t r, float *lds, int off)
{
    static_assert(BYTES == 4 || BYTES == 16, "4- or 16-byte loads");
    auto *dst = (__attribute__((address_space(3))) void *)lds;
    constexpr int aux = NT ? 2 : 0;
    if constexpr (BYTES == 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 4, off, 0, 0, aux);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, off, 0, 0, aux);
}

__device__ __forceinline__ void vm_drain() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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

// Factors of the 4 channels c .. c+3 with one 16-byte load per array (c a
// multiple of 4, channels % 4 == 0: the vector is wholly in or out of range).
__device__ __forceinline__ void epi_load4(const EpiArgs &ep, int c, int channels,
                                          EpiChan (&e)[4])
{
    float4 g = make_float4(1.0f, 1.0f, 1.0f, 1.0f), va = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float4 mu = va, be = va;
    if (ep.gamma) {
        const int bytes = channels * 4;
        const int off = c < channels ? c * 4 : kOutOfRange;
        g = buf_f4(make_rsrc(ep.gamma, bytes), off);
        va = buf_f4(make_rsrc(ep.var, bytes), off);
        mu = buf_f4(make_rsrc(ep.mean, bytes), off);
        be = buf_f4(make_rsrc(ep.beta, bytes), off);
    }
    e[0] = EpiChan{mu.x, g.x, be.x, va.x};
    e[1] = EpiChan{mu.y, g.y, be.y, va.y};
    e[2] = EpiChan{mu.z, g.z, be.z, va.z};
    e[3] = EpiChan{mu.w, g.w, be.w, va.w};
}

__device__ __forceinline__ void epi_finish(EpiChan &e, const EpiArgs &ep)
{
    if (ep.gamma)
        e.inv = e.inv / sqrtf(e.var + ep.eps);
}

// The tiled and row-streaming kernels fold the affine step into the
// channel's weights and bias once per thread: act(inv*(sum w*x + b - mu) +
// be) = act(sum (w*inv)*x + ((b - mu)*inv + be)), the same quantity in
// another rounding order, so that each output pays for the activation only.
__device__ __forceinline__ float epi_fold_bias(float b, const EpiChan &e)
{
    return fmaf(b - e.mu, e.inv, e.be);
}

// The fold for a thread of one channel: its taps and its bias.
template <int KH, int KW>
__device__ __forceinline__ void epi_fold(float (&wr)[KH][KW], float &bv, const EpiChan &e)
{
    bv = epi_fold_bias(bv, e);
#pragma unroll
    for (int kh = 0; kh < KH; ++kh)
#pragma unroll
        for (int kw = 0; kw < KW; ++kw)
            wr[kh][kw] *= e.inv;
}

// The activation alone (after the fold), fixed at compile time.  SiLU uses
// the hardware exponential and the compiler's fast division (a few ulp, far
// inside the tolerance its tests derive).
template <int ACT, int N>
__device__ __forceinline__ void epi_act_c(float (&v)[N])
{
#pragma unroll
    for (int i = 0; i < N; ++i) {
        if constexpr (ACT == DWCONV_ACT_RELU)
            v[i] = fmaxf(v[i], 0.0f);
        else if constexpr (ACT == DWCONV_ACT_RELU6)
            v[i] = fminf(fmaxf(v[i], 0.0f), 6.0f);
        else if constexpr (ACT == DWCONV_ACT_SILU)
            v[i] = __fdividef(v[i], 1.0f + __expf(-v[i]));
    }
}

// Calls f(std::integral_constant<int, act>) for the run-time activation, so
// that a kernel holds one copy of its walk per activation instead of a
// branch at every store.
template <typename F>
__device__ __forceinline__ void with_act(int act, F &&f)
{
    if (act == DWCONV_ACT_RELU)
        f(std::integral_constant<int, DWCONV_ACT_RELU>());
    else if (act == DWCONV_ACT_RELU6)
        f(std::integral_constant<int, DWCONV_ACT_RELU6>());
    else if (act == DWCONV_ACT_SILU)
        f(std::integral_constant<int, DWCONV_ACT_SILU>());
    else
        f(std::integral_constant<int, DWCONV_ACT_NONE>());
}

// The activation alone (after the fold): ReLU and ReLU6 by selects, one
// branch for SiLU (same results as epi_act_c, NaN included): the
// row-streaming walks, whose fully unrolled walks are too long to hold one
// copy per activation.
template <int N>
__device__ __forceinline__ void epi_act_sel(float (&v)[N], int act)
{
    const bool clamp = act == DWCONV_ACT_RELU || act == DWCONV_ACT_RELU6;
    const float hi = act == DWCONV_ACT_RELU6 ? 6.0f : __builtin_inff();
#pragma unroll
    for (int i = 0; i < N; ++i)
        v[i] = clamp ? fminf(fmaxf(v[i], 0.0f), hi) : v[i];
    if (act == DWCONV_ACT_SILU) {
#pragma unroll
        for (int i = 0; i < N; ++i)
            v[i] = __fdividef(v[i], 1.0f + __expf(-v[i]));
    }
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

template <int KH, int KW, int D, int Q, int G, bool V4>
struct NchwGeom {
    static constexpr int R = (KH - 1) * D + 1;
    static constexpr int TH = G - R + 1;
    static constexpr int KK = KH * KW;
    static constexpr int LV = V4 ? 4 : 1;                      // floats per load
    static constexpr int PBMAX = 16;                           // TX >= 16
    // per-thread loads for the largest staged tile (every staged float)
    static constexpr int NV = nchw_stage_loads(0, G, Q, KW, D, V4);
    static constexpr int NW = (PBMAX * KK + 255) / 256;
    static_assert(TH >= 1, "a workgroup must produce at least one output row");
};

inline int mode_of(const Problem &p, const EpiArgs &ep)
{
    if (p.op == DWCONV_OP_INPUT_GRAD)
        return kModeInputGrad;
    return ep.on ? kModeFwdEpilogue : kModeFwd;
}

}  // namespace

// Enqueue kernel k with its own launch status (hipLaunchKernel's return
// value, not the thread's last-error slot, which other code may have left
// set).  Arguments are converted to the kernel's parameter types.
template <typename... P, typename... A>
int launch_kernel(void (*k)(P...), dim3 grid, dim3 block, size_t lds_bytes, hipStream_t st,
                  A &&...args)
{
    static_assert(sizeof...(P) == sizeof...(A), "one argument per kernel parameter");
    std::tuple<P...> params(std::forward<A>(args)...);
    return std::apply(
        [&](auto &...q) {
            void *argv[] = {static_cast<void *>(&q)...};
            return hipLaunchKernel(reinterpret_cast<const void *>(k), grid, block, argv,
                                   lds_bytes, st) == hipSuccess
                       ? DWCONV_OK
                       : DWCONV_ERR_LAUNCH;
        },
        params);
}

// Launchers of the kernel families (one translation unit each): each
// enqueues its kernels on `st` and returns a DWCONV_ status.
int launch_direct(const Problem &p, const Plan &pl, const float *in, const void *w,
                  const float *b, float *out, hipStream_t st, const EpiArgs &ep);
int launch_tiled_nhwc(const Problem &p, const Plan &pl, const float *in, const void *w,
                      const float *b, float *out, hipStream_t st, const EpiArgs &ep);
int launch_tiled_nchw(const Problem &p, const Plan &pl, const float *in, const void *w,
                      const float *b, float *out, hipStream_t st, const EpiArgs &ep);
int launch_stream_nhwc(const Problem &p, const Plan &pl, const float *in, const void *w,
                       const float *b, float *out, hipStream_t st, const EpiArgs &ep);
int launch_stream_nchw(const Problem &p, const Plan &pl, const float *in, const void *w,
                       const float *b, float *out, hipStream_t st, const EpiArgs &ep);
int launch_stream_nchw_planes(const Problem &p, const Plan &pl, const float *in,
                              const void *w, const float *b, float *out, hipStream_t st,
                              const EpiArgs &ep);
int launch_wgrad_stream_nchw(const Problem &p, const Plan &pl, const float *x, const float *dy,
                             float *part, hipStream_t st);
int launch_wgrad_stream_nhwc(const Problem &p, const Plan &pl, const float *x, const float *dy,
                             float *part, hipStream_t st);

}  // namespace dwconv
