// dwconv_internal.h -- problem description, launch plan and the planner /
// launcher interface shared by the host translation units of libdwconv.
//
// The planner (dwconv_plan.cpp) is plain C++ with no HIP runtime call, so the
// validation and kernel selection it does can run on a host without a GPU.
// The launchers (dwconv_launch.hip, dwconv_wgrad.hip) turn a plan into kernel
// launches.
#pragma once

#include <cstdint>

namespace dwconv {

// One depthwise problem, as the C ABI receives it (see include/dwconv.h).
// C counts INPUT channels; the output has mult*C channels, output channel o
// reading input channel o / mult (mult = 1: plain depthwise).  Zero padding
// is explicit per side (pt, pb, pl, pr; negative values crop); the SAME entry
// points fill in the symmetric pads d*(k-1)/2 and set `same`.
struct Problem {
    int op;        // DWCONV_OP_FWD, DWCONV_OP_INPUT_GRAD or DWCONV_OP_WEIGHT_GRAD
    int wtype;     // DWCONV_W_F32 / DWCONV_W_F16
    int layout;    // DWCONV_LAYOUT_NHWC / DWCONV_LAYOUT_NCHW
    int has_bias;
    int N, H, W, C, kH, kW, stride, dilation;
    int mult;             // channel multiplier (output channels per input channel)
    int pt, pb, pl, pr;   // zero padding: top, bottom, left, right
    int same;             // 1: symmetric SAME entry point (odd kernels required)
    int epi;              // 1: forward with the BatchNorm / activation epilogue
    int Ho, Wo;           // output extents, set by validate_problem
};

// Forward epilogue: inference-form BatchNorm (gamma, beta, mean, var of the
// output channels; all NULL for none) and an activation DWCONV_ACT_*.
struct Epilogue {
    const float *gamma, *beta, *mean, *var;
    float eps;
    int act;
};

// Compile-time modes of the tiled kernels.
constexpr int kModeFwd = 0, kModeInputGrad = 1, kModeFwdEpilogue = 2;

// Problem with symmetric SAME padding and no channel multiplier.
Problem same_problem(int op, int wtype, int has_bias, int N, int H, int W, int C, int kH,
                     int kW, int stride, int dilation, int layout);

enum Kind {
    KIND_DIRECT_NHWC = 1,  // one thread per (n, row, col, channel vector); taps from global
    KIND_DIRECT_NCHW = 2,  // one thread per (n, channel, row, col); taps from global
    KIND_TILED_NHWC = 3,   // stride 1 or 2: LDS row chunks with halo, rolling row accumulators
    KIND_TILED_NCHW = 4,   // stride 1 or 2: LDS tiles of one or more planes, rolling row accumulators
    KIND_WGRAD_DIRECT = 5, // weight gradient, any layout/stride: lanes along the contiguous axis
    KIND_WGRAD_TILED_NHWC = 6, // weight gradient, NHWC stride 1 or 2: LDS x tiles, strips of row tiles
    KIND_WGRAD_TILED_NCHW = 7, // weight gradient, NCHW stride 1 or 2: LDS x plane rows, dy in registers
    KIND_STREAM_NHWC = 8,  // stride 1, many taps: rows streamed through registers, phases of D
    KIND_STREAM_NCHW = 9,  // the same with lanes along plane columns, rows staged per wave
    KIND_WGRAD_STREAM_NCHW = 10, // weight gradient, NCHW stride 1: the NCHW row walk, tap sums per lane
    KIND_WGRAD_STREAM_NHWC = 11, // weight gradient, NHWC stride 1: the NHWC row walk, tap sums per lane
    KIND_STREAM_NCHW_PLANES = 12, // NCHW stride 1, many taps: the NHWC walk with one plane per lane,
                                  // rows and output rows transposed through LDS
};

// Compile-time variants of the tiled NHWC kernel.  A tiled plan exists only
// for a (kH, kW, dilation) listed here; everything else runs the direct
// kernels.  `vec`: channels per thread; `cl`: threads across channels; `px`:
// adjacent output pixels per thread (a workgroup of 256 threads covers
// cl*vec channels of px*256/cl pixels); `g`: input rows staged per
// workgroup, which yields g - (kH-1)*d output rows; `lv`: floats per staging
// load (4: needs C % 4 == 0 and 16-byte aligned tensors; 1: any C).
//
// For each kernel shape the variants are listed in order of preference: the
// order of their measured throughput on MI355X for channel counts that fill
// their channel tile.  The planner takes the first one whose channel tile
// the problem fills to at least 3/4.
struct TiledVariant { int kH, kW, d, vec, cl, px, g, lv; };
// (The 32-channel 3x3 tile takes 2 output rows of 4 staged rows and 2
// channels per thread: 1x112x112x32 forward 3.42 -> 3.08 us and input
// gradient 3.38 -> 3.06 us against 1 output row and 4 channels per thread;
// taller tiles (6-10 staged rows, fewer and longer workgroups) were slower,
// 3.4-4.5 us.)
constexpr TiledVariant kTiledVariants[] = {
    {3, 3, 1, 4, 32, 1, 8, 4},   {3, 3, 1, 4, 16, 1, 6, 4},   {3, 3, 1, 2, 16, 1, 4, 4},
    {5, 5, 1, 1, 32, 1, 12, 4},
    {7, 7, 1, 1, 32, 1, 16, 4},
    {7, 7, 2, 2, 16, 1, 20, 4},
    {1, 15, 1, 4, 32, 1, 2, 4},  {1, 15, 1, 4, 16, 1, 2, 4},
    {1, 31, 1, 2, 32, 1, 2, 4},
    // 1x1 (a per-channel scale and bias): no halo, so its HBM traffic is the
    // tensors themselves, which calibrates the traffic counters of the
    // kernels above (the same 16-byte loads straight into LDS)
    {1, 1, 1, 4, 32, 1, 8, 4},
    // scalar staging (lv = 1): any channel count, e.g. a prime one
    {3, 3, 1, 1, 32, 2, 8, 1},   {5, 5, 1, 1, 32, 1, 12, 1},
    {7, 7, 1, 1, 32, 1, 14, 1},  {7, 7, 2, 1, 32, 1, 28, 1},
    {1, 15, 1, 1, 32, 1, 2, 1},  {1, 31, 1, 1, 32, 1, 2, 1},
};
constexpr int kNumTiledVariants = sizeof(kTiledVariants) / sizeof(kTiledVariants[0]);

// Variants of the tiled NHWC kernel at stride 2 (same fields; the tile
// covers the stride-1 grid, so g >= kH*d + 1 leaves at least two rows, one
// of them even).
constexpr TiledVariant kTiledS2Variants[] = {
    {3, 3, 1, 4, 8, 2, 6, 4},   {3, 3, 1, 1, 32, 1, 6, 1},
    {5, 5, 1, 4, 8, 1, 8, 4},   {5, 5, 1, 1, 32, 1, 8, 1},
};
constexpr int kNumTiledS2Variants = sizeof(kTiledS2Variants) / sizeof(kTiledS2Variants[0]);

// Variants of the tiled NHWC kernel with a channel multiplier of 2 (stride
// 1; cl*vec counts output channels; 16-byte staging, vec a multiple of 2).
constexpr TiledVariant kTiledM2Variants[] = {
    {3, 3, 1, 4, 32, 2, 8, 4},  {3, 3, 1, 4, 16, 1, 6, 4},  {3, 3, 1, 4, 8, 1, 3, 4},
    {5, 5, 1, 4, 8, 1, 10, 4},
};
constexpr int kNumTiledM2Variants = sizeof(kTiledM2Variants) / sizeof(kTiledM2Variants[0]);

// Variants of the row-streaming NHWC kernel (stride 1, no multiplier, any
// channel count and alignment): a wave computes `cl` channels x 64/cl column
// groups of `px` adjacent output columns x `th` output rows of one dilation
// phase (the sub-grid of rows and columns D apart), with `nb` input rows in
// registers.  The AUTO strategy takes a variant when the problem gives at
// least `minw` waves (smaller problems finish sooner on the tiled kernels'
// short-lived workgroups).
// Measured on MI355X (amortised launches, 64x30x19x128 7x7): forward 15.1 ->
// 9.9 us against the tiled kernel, dilation 2 26.4 -> 9.6 us; 5 rows per
// wave beat 4, 6 and 10 (d = 1) and 8 beat 5 and 15 (d = 2); 32- and
// 16-channel lane groups measured 2-40% slower than 64 (a prime channel
// count included: its 64-channel tiles start mid cache line, and narrower
// groups touch more lines per load); 4 rows in registers 1-3% slower than 3.
// At 1x30x19x128 the tiled kernel is faster (7x7: 4.8 against 5.7 us).  For
// 5x5 and 3x3 windows (HBM-bound) the tiled kernel stays faster
// (32x56x56x128 5x5: 20.2 against 21.5 us).
struct StreamVariant { int kH, kW, d, cl, px, th, nb, minw; };
constexpr StreamVariant kStreamVariants[] = {
    {7, 7, 1, 64, 5, 5, 3, 1024}, {7, 7, 2, 64, 5, 8, 3, 1024},
};
constexpr int kNumStreamVariants = sizeof(kStreamVariants) / sizeof(kStreamVariants[0]);

// Variants of the row-streaming NCHW kernel (stride 1, no multiplier): each
// lane computes `px` adjacent output columns of one plane for `th` output
// rows of one dilation phase; a wave stages each input row in `nl` loads of
// 64 elements (its planes' rows with the column halo) and keeps `nb` rows in
// registers, so lanes per plane row and planes per wave follow from the
// plane width at plan time; `minw` as for NHWC.
// Measured (64x30x19x128): 7x7 forward 19.5 -> 17.5 us, dilation 2 27.2 ->
// 23.7 us (1x30x19x128 d = 2: 10.9 -> 7.1 us; d = 1 stays tiled there: 7.1
// against 10.1 us).  Lanes reading their own columns from global memory
// (no LDS row) measured 29-45 us: 5x the L1 requests per FMA of NHWC.
struct StreamNchwVariant { int kH, kW, d, px, th, nl, nb, minw; };
constexpr StreamNchwVariant kStreamNchwVariants[] = {
    {7, 7, 1, 1, 30, 2, 6, 1024}, {7, 7, 2, 1, 15, 2, 6, 64},
};
constexpr int kNumStreamNchwVariants = sizeof(kStreamNchwVariants) / sizeof(kStreamNchwVariants[0]);

// Variants of the plane-per-lane NCHW kernel (stride 1, no multiplier): a
// wave takes 16 planes x 4 lane groups of `px` columns (4*px output columns)
// and `th` output rows of one row phase; it stages a row's in-image columns
// with `nl` loads per lane (so planes at most 4*nl columns wide, or the
// staged window if narrower, take the variant), `nb` rows ahead; AUTO takes
// the first variant that fits from `minw` waves (kNever: never).
// Measured on MI355X (64x30x19x128 7x7, rocprof medians, forward), against
// the lane-along-columns kernel: dilation 2 14.5 against 16.2 us; dilation 1
// 14.8 against 14.3 us, so AUTO keeps the other kernel there.  3 or 4 rows
// ahead instead of 2, and 6 rows per unit instead of 5, measured the same.
constexpr int kNever = 1 << 30;
struct StreamPlanesVariant { int kH, kW, d, px, th, nl, nb, minw; };
constexpr StreamPlanesVariant kStreamPlanesVariants[] = {
    {7, 7, 1, 5, 5, 5, 2, kNever}, {7, 7, 1, 5, 5, 7, 2, kNever},
    {7, 7, 2, 5, 5, 5, 2, 1024}, {7, 7, 2, 5, 5, 8, 2, 1024},
};
constexpr int kNumStreamPlanesVariants =
    sizeof(kStreamPlanesVariants) / sizeof(kStreamPlanesVariants[0]);

// LDS floats of one staged row slot of the row-streaming NCHW kernel (the
// planes of a wave, each at a bank-spreading pitch).
constexpr int kStreamNchwSlot = 256;

// Variants of the row-streaming NCHW weight gradient (stride 1, no
// multiplier): the NCHW walk's lanes and staging (one column per lane), dy
// rows per unit `th`, `nl` loads per staged x row, `nb` rows in flight;
// AUTO takes it from `minw` waves.  Measured (both stages, 64x30x19x128):
// 7x7 31.3 -> 25.6 us against the tiled kernel, 7x7 d2 53.3 -> 38.4 us
// (1x30x19x128 d2: 16.3 -> 13.2 us; d1 stays tiled there, 13.6 against
// 16.0 us); half the rows per unit measured 12-40% slower.  4 rows in
// flight instead of 6 (stage 1, same-box A/B): d1 17.4 -> 16.9 us, d2 19.8
// -> 19.1 us (3 or 5: d2 19.2, 19.5 us).
struct WgradStreamVariant { int kH, kW, d, th, nl, nb, minw; };
// Waves above which a unit of the row-streaming NCHW weight gradient walks
// all row phases of its column phase (dilation > 1).
constexpr long long kWgradStreamPhaseWaves = 4096;
constexpr WgradStreamVariant kWgradStreamVariants[] = {
    {7, 7, 1, 30, 2, 4, 1024}, {7, 7, 2, 15, 2, 4, 64},
};
constexpr int kNumWgradStreamVariants =
    sizeof(kWgradStreamVariants) / sizeof(kWgradStreamVariants[0]);

// Variants of the row-streaming NHWC weight gradient (stride 1, no
// multiplier): the NHWC walk's waves (64 channels x `px` columns x `th` dy
// rows of one phase), `nb` x rows in flight; AUTO takes it from `minw`
// waves.
struct WgradStreamNhwcVariant { int kH, kW, d, px, th, nb, minw; };
constexpr WgradStreamNhwcVariant kWgradStreamNhwcVariants[] = {
    {7, 7, 1, 5, 5, 3, 1024}, {7, 7, 2, 5, 8, 3, 1024},
};
constexpr int kNumWgradStreamNhwcVariants =
    sizeof(kWgradStreamNhwcVariants) / sizeof(kWgradStreamNhwcVariants[0]);

// Cache policy of the row-streaming kernels' stores (gfx950 buffer-store
// cache-policy bits: 2 = non-temporal, 0 = write-back).  NHWC: a store
// covers whole 256-byte pixels of 64 channels, written once, non-temporal.
// NCHW: a store writes one row (OW floats) of each plane of the wave, and
// the row before and after, stored later, share its first and last cache
// lines; write-back lets L2 merge those partial lines before they go to HBM.
constexpr int kStreamStoreAux = 2;
constexpr int kStreamNchwStoreAux = 0;

// Compile-time variants of the tiled NHWC weight-gradient kernel: workgroup
// geometry as for the forward (vec, cl, px, g, lv).  A workgroup walks a strip of
// row tiles of g - (kH-1)*d rows (its partial sums cover them all); the
// planner sizes the strips for about kWgradTargetWorkgroups workgroups.
struct WgradVariant { int kH, kW, d, vec, cl, px, g, lv; };
constexpr WgradVariant kWgradVariants[] = {
    {3, 3, 1, 2, 32, 1, 6, 4},  {3, 3, 1, 4, 8, 1, 6, 4},
    {5, 5, 1, 2, 16, 1, 11, 4},
    {7, 7, 1, 1, 32, 1, 14, 4},
    {7, 7, 2, 1, 32, 1, 22, 4},
    // 1xK: one-row tiles 24 columns wide (64 channels x 6 columns per
    // thread): the column halo of a tile is kW - 1 columns, so narrow tiles
    // stage mostly halo (8 columns: 38 staged for 8 used at 1x31) and split
    // one-row images into several chunks.  64x1x24x256 1x31, both stages:
    // 16.4 -> 8.75 us against 8-column, two-row tiles; 64x1x24x128 1x15
    // 8.9 -> 6.2 us; 1x1x24x256 1x31 7.5 -> 6.6 us.
    {1, 15, 1, 1, 64, 6, 1, 4},
    {1, 31, 1, 1, 64, 6, 1, 4},
    // 4-byte staging (lv = 1): any channel count
    {3, 3, 1, 1, 32, 1, 10, 1}, {5, 5, 1, 1, 32, 1, 12, 1},
    {7, 7, 1, 1, 32, 1, 16, 1}, {7, 7, 2, 1, 32, 1, 22, 1},
    {1, 15, 1, 1, 32, 1, 2, 1}, {1, 31, 1, 1, 32, 1, 2, 1},
};
constexpr long long kWgradTargetWorkgroups = 512;

// LDS a plan may ask for: all of a gfx950 workgroup's 160 KiB (dynamic LDS
// above 64 KiB launches without raising a per-kernel limit on this target;
// the 7x7 dilation-2 input gradient with a multiplier of 2 takes 98 KiB).
constexpr int kMaxLdsBytes = 160 * 1024;

// Tile order of the tiled kernels.  Below this many bytes of activations
// (the tensor an op reads plus the one it writes, or x plus dy for the
// weight gradient) each XCD takes a contiguous range of tiles, so the halos
// neighbouring tiles share stay in one L2; from it on, all XCDs sweep the
// tiles in order together, which streams a large tensor from HBM faster.
// Measured on MI355X (NHWC and NCHW, all three ops): the per-XCD ranges are
// 3-15% faster up to 374 MiB, equal at 512 MiB and 5% slower at 1 GiB.  From
// it the NHWC kernels keep the band-by-band sweep but split each row band
// (a strip, for the weight gradient) into 8 runs, one per XCD, when the
// band's tile count is a multiple of 8: 1.5% faster on the 512x512x256
// forward / input gradient, 4% on its weight gradient.  The NCHW forward /
// input gradient takes bands of 8 plane groups, one plane group's row tiles
// per XCD in order (the plane-group count a multiple of 8): 2-3% faster.
constexpr long long kXcdRangeMaxBytes = 448LL << 20;

// Weight-gradient reduction: up to this many columns (channels x (taps + 1))
// the reduction kernel spreads each column's chunks over 16 slices (16
// columns per workgroup), above it over 8 (32 columns, whole 128-byte runs
// per load).  Measured against 4 slices of 64 columns (the earlier shape):
// 64x30x19x128 7x7 NHWC (384 chunks) 21.6 -> 19.6 us, 7x7 d2 NCHW 38.2 ->
// 36.9 us, 64x1x24x256 1x31 NHWC 17.2 -> 16.4 us, 1x224x224x32 3x3 s2 NHWC
// (320 columns, 266 chunks) 9.7 -> 7.8 us with 16 slices; within 3% on the
// rest of the workloads.
constexpr int kReduceFewColumns = 512;
constexpr int kNumWgradVariants = sizeof(kWgradVariants) / sizeof(kWgradVariants[0]);

// Variants of the tiled NHWC weight gradient at stride 2 (g = staged x rows
// = 2*(dy rows) - 1 + (kH-1)*d).
constexpr WgradVariant kWgradS2Variants[] = {
    {3, 3, 1, 4, 8, 1, 7, 4},
    {5, 5, 1, 4, 8, 1, 7, 4},
    {3, 3, 1, 1, 32, 1, 7, 1},  {5, 5, 1, 1, 32, 1, 7, 1},
};
constexpr int kNumWgradS2Variants = sizeof(kWgradS2Variants) / sizeof(kWgradS2Variants[0]);

// Variants of the tiled NHWC weight gradient with a channel multiplier of 2
// (stride 1; cl*vec counts dy channels; 16-byte staging).
constexpr WgradVariant kWgradM2Variants[] = {
    {3, 3, 1, 4, 16, 1, 6, 4},  {3, 3, 1, 4, 8, 1, 6, 4},
    {5, 5, 1, 4, 16, 1, 8, 4},
};
constexpr int kNumWgradM2Variants = sizeof(kWgradM2Variants) / sizeof(kWgradM2Variants[0]);


// Compile-time variants of the tiled NCHW kernel (same preference rule).
// A workgroup of 256 threads covers pb planes (channels) x tx threads per
// plane row, tx = 256/pb chosen at plan time from W; each thread owns `q`
// adjacent output columns; `g` input rows are staged per workgroup; `v4`
// selects 16-byte loads (needs W % 4 == 0).
struct TiledNchwVariant { int kH, kW, d, q, g, v4; };
constexpr TiledNchwVariant kTiledNchwVariants[] = {
    {3, 3, 1, 2, 8, 1},   {3, 3, 1, 2, 8, 0},
    {5, 5, 1, 2, 12, 1},  {5, 5, 1, 2, 12, 0},
    {7, 7, 1, 1, 16, 1},  {7, 7, 1, 1, 16, 0},
    {7, 7, 2, 1, 27, 1},  {7, 7, 2, 1, 27, 0},
    {1, 15, 1, 2, 2, 1},  {1, 15, 1, 2, 2, 0},
    {1, 31, 1, 2, 2, 1},  {1, 31, 1, 2, 2, 0},
};
constexpr int kNumTiledNchwVariants = sizeof(kTiledNchwVariants) / sizeof(kTiledNchwVariants[0]);

// Variants of the tiled NCHW weight gradient at stride 1 (measured apart
// from the forward's: 5x5 with one column per thread, 7x7 with fewer staged
// rows per tile).
constexpr TiledNchwVariant kWgradNchwVariants[] = {
    {3, 3, 1, 2, 8, 1},   {3, 3, 1, 2, 8, 0},
    {5, 5, 1, 1, 12, 1},  {5, 5, 1, 1, 12, 0},
    {7, 7, 1, 1, 12, 1},  {7, 7, 1, 1, 21, 0},
    {7, 7, 2, 1, 17, 1},  {7, 7, 2, 1, 23, 0},
    {1, 15, 1, 2, 2, 1},  {1, 15, 1, 2, 2, 0},
    {1, 31, 1, 2, 2, 1},  {1, 31, 1, 2, 2, 0},
};
constexpr int kNumWgradNchwVariants = sizeof(kWgradNchwVariants) / sizeof(kWgradNchwVariants[0]);

// Per-thread staging loads of the tiled NCHW kernels (a compile-time bound
// each kernel sizes its load registers with, and the planner checks its tile
// against).  A workgroup stages g rows of pb planes, twl floats each, with
// tx >= 16 threads per row, so pb <= 16; a row holds the tile's cols_per_thr
// * tx columns plus at most `extra` more (the window's d*(kW-1) and, with
// 16-byte loads, up to 3 alignment columns on each side).
//   kind 0: every staged float, 4 or 1 per load (forward, input gradient at
//           stride 1, weight gradient; cols_per_thr = s*q for the weight
//           gradient's x rows at stride s);
//   kind 1: the stride-2 input gradient's upsampled dy, one load per pair
//           of staged columns of the even rows only.
constexpr int nchw_extra_cols(int kW, int d, bool v4)
{
    return v4 ? (d * (kW - 1) + 3 + 3) / 4 * 4 : d * (kW - 1);
}
constexpr int nchw_stage_loads(int kind, int g, int cols_per_thr, int kW, int d, bool v4)
{
    return kind == 0 ? (g * (256 * cols_per_thr + 16 * nchw_extra_cols(kW, d, v4)) / (v4 ? 4 : 1) +
                        255) / 256
                     : ((g + 1) / 2 * ((256 * cols_per_thr + 16 * nchw_extra_cols(kW, d, false)) / 2 +
                                       16) + 255) / 256;
}

// Variants of the tiled NCHW kernel at stride 2 (the tile covers the
// stride-1 grid; the input gradient stages with 4-byte loads, v4 = 0).
constexpr TiledNchwVariant kTiledNchwS2Variants[] = {
    {3, 3, 1, 2, 8, 1}, {3, 3, 1, 2, 8, 0},
    {5, 5, 1, 2, 12, 1}, {5, 5, 1, 2, 12, 0},
};
constexpr int kNumTiledNchwS2Variants =
    sizeof(kTiledNchwS2Variants) / sizeof(kTiledNchwS2Variants[0]);

// Variants of the tiled NCHW weight gradient at stride 2 (g = staged x rows
// = 2*(dy rows) - 1 + (kH-1)*d).
constexpr TiledNchwVariant kWgradNchwS2Variants[] = {
    {3, 3, 1, 2, 7, 1}, {3, 3, 1, 2, 7, 0},
    {5, 5, 1, 2, 9, 1}, {5, 5, 1, 2, 9, 0},
};
constexpr int kNumWgradNchwS2Variants =
    sizeof(kWgradNchwS2Variants) / sizeof(kWgradNchwS2Variants[0]);

struct Plan {
    int kind;
    int vec;            // NHWC: channels per thread (4 or 1)
    int variant;        // tiled: index into the kernel's variant table
    int cl;             // tiled NHWC: threads across channels; tiled NCHW: threads per
                        // plane row; generic weight gradient (NHWC): channel lanes
    int tw;             // tiled: output columns per tile
    int th;             // tiled: output rows per workgroup (one row tile)
    int nct, nwt, nst;  // tiled: channel tiles (NHWC) or plane groups (NCHW), column tiles,
                        // row tiles (weight gradient: strips of row tiles)
    int pb;             // tiled NCHW: planes per workgroup (256 / cl)
    int xcd;            // tiled: 1 = each XCD takes a contiguous range of tiles, 2 = band-local
                        // runs (NHWC) or plane-group bands (NCHW forward / input gradient),
                        // 0 = in order
    int rpu;            // row-streaming NCHW weight gradient: row phases a unit walks (1 or d)
    int ntl;            // tiled: 1 = a tile's rows that no other tile stages load
                        // non-temporally (activations too large for the Infinity Cache)
    int lds_bytes;      // tiled NCHW: dynamic LDS per workgroup
    int hl, twl;        // tiled NCHW: staged columns left of a tile, staged floats per row
    int nrt;            // weight gradient, tiled: row tiles per image / plane
    int strip;          // weight gradient, tiled: row tiles per strip (per workgroup)
    int ppc, cpi;       // weight gradient, generic: dy positions per chunk; NCHW chunks per image
    long long chunks;   // weight gradient: partial sums per weight (rows of the workspace)
    long long workspace;// weight gradient: workspace bytes
    long long grid2;    // weight gradient: workgroups of the reduction kernel
    int red_s;          // weight gradient: chunk slices per reduction workgroup (4 or 16)
    int tail_cl;        // row-streaming NHWC: channels per lane group of the tail tile (0 =
                        // none; nct then counts every channel tile)
    int tail_ncg;       // row-streaming NHWC: column groups per sub-grid row of the tail tile
    long long tail_units;// row-streaming NHWC: units (waves) of the tail tile
    int pH, pW;
    int IH, IW, OH, OW; // extents of the tensor read (in) and written (out) by this op
                        // (tiled NHWC stride-2 forward: OH, OW = the stride-1 grid it tiles)
    int YH, YW;         // tiled: extents of the tensor written
    long long total;    // direct: number of threads doing work
    long long grid;     // workgroups
    int block;          // threads per workgroup
    char name[96];
};

// Validate dimensions, pads and enums (not pointers) and set p.Ho, p.Wo.
// Returns a DWCONV_ status.
int validate_problem(Problem &p);

// Choose the kernel and its launch geometry.  `ptr_bits` is the bitwise OR
// of the tensor pointers' addresses (0 when unknown); vector widths are only
// chosen when it shows 16-byte alignment.  Returns a DWCONV_ status.
int make_plan(Problem &p, int strategy, std::uintptr_t ptr_bits, Plan *out);

// Plan the weight gradient (op DWCONV_OP_WEIGHT_GRAD).  Returns a status.
int make_wgrad_plan(Problem &p, int strategy, std::uintptr_t ptr_bits, Plan *out);

// Enqueue the two kernels of a weight-gradient plan.
// Weight and bias gradients of a plan made by make_wgrad_plan.  dw and db
// (either may be NULL) receive the gradients; when w_upd is not NULL the
// fused SGD step w_upd -= lr * dW (and b_upd -= lr * db when b_upd is not
// NULL) is applied in the same reduction.
int launch_wgrad(const Problem &p, const Plan &pl, const float *x, const float *dy, float *dw,
                 float *db, void *workspace, void *stream, float *w_upd = nullptr,
                 float *b_upd = nullptr, float lr = 0.0f);

// Scratch array held by the library on every GPU it runs on, for the
// allocation-free weight gradient (its partial sums): bytes per device.
constexpr long long kScratchBytes = 16LL << 20;

// Device address of this library's scratch array on the device that
// `stream` (a hipStream_t; NULL: the current device's) belongs to, which
// must be the current device.  Looked up once per device.  Returns
// DWCONV_OK, or DWCONV_ERR_SCRATCH when the stream is on another device or
// the runtime cannot locate the array.
int scratch_buffer(void *stream, void **ptr);

// Enqueue the kernel of a plan made by make_plan on `stream` (a hipStream_t);
// `epi` (forward only, may be NULL) is the fused epilogue.
// Returns DWCONV_OK, or DWCONV_ERR_LAUNCH if the runtime reports an error.
int launch_plan(const Problem &p, const Plan &pl, const float *in, const void *w,
                const float *b, float *out, void *stream, const Epilogue *epi = nullptr);

}  // namespace dwconv
