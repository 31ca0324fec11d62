/*
 * dwconv.h -- C ABI of the MI355X (gfx950) depthwise 2-D convolution library
 * (libdwconv.so).  Plain pointers and sizes only.
 *
 * The operation (LeanMlir "Depthwise" page, forward equation, with stride s
 * and dilation d, and the ggml CONV_2D_DW op of llama.cpp PR #21565 for the
 * layouts and weight types):
 *
 *   y[n,c,ho,wo] = b[c] + sum_{kh<kH, kw<kW} x[n, c, ho*s + kh*d - pH,
 *                                               wo*s + kw*d - pW] * W[c,kh,kw]
 *
 * one filter per channel and no sum over channels; positions outside the
 * image contribute nothing (SAME zero padding), pH = d*(kH-1)/2,
 * pW = d*(kW-1)/2, Ho = ceil(H/s), Wo = ceil(W/s).  Stride 2 keeps the even
 * positions of the stride-1 result (LeanMlir "Depthwise", stride-2 SAME).
 *
 * Its input gradient (LeanMlir "Depthwise", reversed-kernel formula and the
 * stride-2 input-VJP: zero-upsample dy onto the even positions, then the
 * reversed-kernel stride-1 depthwise):
 *
 *   dx[n,c,h,w] = sum_{kh,kw} W[c, kH-1-kh, kW-1-kw] * u[n, c, h + kh*d - pH,
 *                                                        w + kw*d - pW]
 *   u[n,c,t,v]  = dy[n, c, t/s, v/s] if t and v are multiples of s, else 0.
 *
 * Shapes.  H and W are always the forward INPUT extents: x and dx are
 * [N,H,W,C] (NHWC) or [N,C,H,W] (NCHW); y and dy are [N,Ho,Wo,C] or
 * [N,C,Ho,Wo] in the same layout.  W (the weights) is [C][kH][kW] contiguous
 * in both layouts, float32 or IEEE binary16; b is [C] float32 or NULL.
 * Every tensor is dense in its layout (no strides).
 *
 * Ownership and execution.  All tensor pointers are DEVICE pointers owned by
 * the caller.  The library allocates no memory and keeps no state between
 * calls (its kernel tables are filled once, on first use, under the C++
 * static-initialisation guard), so calls may be made from any host thread.  Work is enqueued asynchronously on `stream` (a hipStream_t;
 * NULL means the default stream); a return of DWCONV_OK means "validated and
 * enqueued".  The output (y or dx) is fully overwritten, never accumulated
 * into.  Inputs and outputs must not overlap (no in-place operation).
 *
 * Errors.  Every argument is validated before anything is enqueued; a
 * negative status means nothing was launched and the output is untouched.
 */
#ifndef DWCONV_H
#define DWCONV_H

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
#define DWCONV_OK                0
#define DWCONV_ERR_NULL_PTR     -1  /* input, weights or output pointer is NULL      */
#define DWCONV_ERR_BAD_DIM      -2  /* N,H,W,C,kH,kW < 1, or a tensor has >= 2^31 elements */
#define DWCONV_ERR_BAD_STRIDE   -3  /* stride not 1 or 2                             */
#define DWCONV_ERR_BAD_DILATION -4  /* dilation < 1, or d*(k-1) >= 2^16              */
#define DWCONV_ERR_EVEN_KERNEL  -5  /* kH or kW even: SAME padding needs an odd kernel */
#define DWCONV_ERR_BAD_LAYOUT   -6  /* layout not NHWC or NCHW                       */
#define DWCONV_ERR_BAD_WTYPE    -7  /* weight type not F32 or F16                    */
#define DWCONV_ERR_ALIAS        -8  /* output bytes overlap an input's bytes         */
#define DWCONV_ERR_MISALIGNED   -9  /* float pointer not 4-byte or half not 2-byte aligned */
#define DWCONV_ERR_LAUNCH      -10  /* the HIP runtime reported an error at launch   */
#define DWCONV_ERR_BAD_OP      -11  /* op not FWD or INPUT_GRAD                      */
#define DWCONV_ERR_BAD_STRATEGY -12 /* strategy unknown, or not applicable to the problem */
#define DWCONV_ERR_WORKSPACE   -13  /* workspace NULL, misaligned or smaller than required */
#define DWCONV_ERR_BAD_PAD     -14  /* a pad with |pad| >= 2^16, or an unknown padding mode */
#define DWCONV_ERR_BAD_EPILOGUE -15 /* unknown activation, BatchNorm pointers not all given
                                       or all NULL, eps negative or not finite, or a
                                       learning rate that is not finite               */
#define DWCONV_ERR_SCRATCH     -16  /* allocation-free weight gradient: the problem needs more
                                       than the library's scratch array holds, or the stream
                                       is not on the current device                   */

/* ---- enumerations (passed as int) -------------------------------------- */
#define DWCONV_LAYOUT_NHWC 0   /* channel innermost (the ggml page's CWHN)    */
#define DWCONV_LAYOUT_NCHW 1   /* channel outer     (the ggml page's WHCN)    */

#define DWCONV_W_F32 0         /* weights are float32                         */
#define DWCONV_W_F16 1         /* weights are IEEE binary16, widened exactly  */

#define DWCONV_OP_FWD        0 /* y  = dwconv(x; W, b)                        */
#define DWCONV_OP_INPUT_GRAD 1 /* dx = dwconv_input_grad(dy; W)               */
#define DWCONV_OP_WEIGHT_GRAD 2 /* dW, db = dwconv_weight_grad(x, dy): an op code of the
                                   describe calls; run by the weight-gradient entry points */

/* Padding modes of dwconv2d_same_pads. */
#define DWCONV_PAD_SAME     0  /* symmetric: d*(k-1)/2 on every side (odd kernels)   */
#define DWCONV_PAD_XLA_SAME 1  /* LeanMlir "Depthwise" stride-2 XLA-SAME: the stride-1
                                  SAME result kept at the ODD positions               */

/* Activations of the fused forward epilogue. */
#define DWCONV_ACT_NONE  0     /* y = t                                       */
#define DWCONV_ACT_RELU  1     /* y = max(t, 0)                               */
#define DWCONV_ACT_RELU6 2     /* y = min(max(t, 0), 6)   (MobileNetV2)       */
#define DWCONV_ACT_SILU  3     /* y = t / (1 + exp(-t))   (EfficientNet)      */

/* Which tiling to run a problem under (cubek-convolution "depthwise" module:
 * a strategy enum selects the tiling, one launch function runs it). */
#define DWCONV_STRATEGY_AUTO   0 /* pick the fastest applicable kernel          */
#define DWCONV_STRATEGY_DIRECT 1 /* one thread per output vector, taps from global memory;
                                    applies to every valid problem               */
#define DWCONV_STRATEGY_TILED  2 /* LDS-staged input rows with halo, register-blocked
                                    output rows; applies where a tiled kernel exists
                                    for the (layout, stride, kernel, dilation)    */
#define DWCONV_STRATEGY_STREAM 3 /* each wave walks its rows with the input streamed
                                    through registers (NHWC: lanes along 64 channels;
                                    NCHW: lanes along plane columns, each row staged
                                    once per wave), dilation split into its phases;
                                    applies at stride 1 without a multiplier to the
                                    forward and input gradient (both layouts) and the
                                    NCHW weight gradient, for the kernel shapes it has
                                    variants for (7x7, dilation 1 or 2)            */
#define DWCONV_STRATEGY_STREAM_PLANES 4 /* NCHW only: the NHWC row walk with one plane
                                    per lane group (16 planes x 4 column groups per
                                    wave), input rows and output rows transposed
                                    through the wave's LDS; stride 1
                                    without a multiplier, forward and input gradient,
                                    for the kernel shapes it has variants for (7x7,
                                    dilation 1 or 2)                              */

/*
 * Forward.  x: input [N,H,W,C] / [N,C,H,W] float32.  w: [C][kH][kW] of type
 * wtype.  b: [C] float32 or NULL (no bias).  y: output [N,Ho,Wo,C] /
 * [N,C,Ho,Wo] float32.  stride in {1,2}; dilation >= 1; kH, kW odd.
 */
int dwconv2d_fwd(const float *x, const void *w, int wtype, const float *b, float *y,
                 int N, int H, int W, int C, int kH, int kW,
                 int stride, int dilation, int layout, void *stream);

/*
 * Input gradient.  dy: [N,Ho,Wo,C] / [N,C,Ho,Wo] float32.  w as for the
 * forward.  dx: output [N,H,W,C] / [N,C,H,W] float32.  H, W are the forward
 * input extents.  No bias term.
 */
int dwconv2d_input_grad(const float *dy, const void *w, int wtype, float *dx,
                        int N, int H, int W, int C, int kH, int kW,
                        int stride, int dilation, int layout, void *stream);

/*
 * Either operation under an explicit strategy (DWCONV_STRATEGY_*).  `in` is
 * x (forward) or dy (input gradient); `out` is y or dx; b must be NULL for
 * the input gradient.  Same shapes, ownership and errors as above; an
 * explicit strategy that does not apply returns DWCONV_ERR_BAD_STRATEGY.
 */
int dwconv2d_launch(int op, const float *in, const void *w, int wtype, const float *b,
                    float *out, int N, int H, int W, int C, int kH, int kW,
                    int stride, int dilation, int layout, int strategy, void *stream);

/*
 * Describe, without launching anything or touching the GPU, the kernel a
 * dwconv2d_launch call with these arguments would run: writes a
 * NUL-terminated kernel name (at most name_len bytes, truncated) into `name`
 * and the grid and block sizes into grid[0], block[0] when those are not
 * NULL.  Validates dimensions, stride, dilation, kernel size, layout, wtype,
 * op and strategy as the launch would; pointer checks are skipped.
 */
int dwconv2d_describe(int op, int wtype, int has_bias, int N, int H, int W, int C,
                      int kH, int kW, int stride, int dilation, int layout, int strategy,
                      char *name, int name_len, long long *grid, int *block);

/*
 * Weight and bias gradients (LeanMlir "Depthwise": the weight-VJP -- the
 * forward is affine in W -- and the bias-gradient closed form):
 *
 *   dW[c,kh,kw] = sum_{n,ho,wo} x[n, c, ho*s + kh*d - pH, wo*s + kw*d - pW] * dy[n,c,ho,wo]
 *   db[c]       = sum_{n,ho,wo} dy[n,c,ho,wo]
 *
 * over in-range input positions.  x: [N,H,W,C] / [N,C,H,W] float32; dy:
 * [N,Ho,Wo,C] / [N,C,Ho,Wo] float32; dw: [C][kH][kW] float32 output; db: [C]
 * float32 output or NULL.  Both outputs are overwritten.  The sums are
 * deterministic (fixed order, no atomics): per-tile partial sums go to
 * `workspace`, a caller-owned device buffer of at least the size that
 * dwconv2d_weight_grad_workspace_size reports for the same arguments
 * (16-byte aligned; its contents on entry do not matter), and a second
 * kernel adds them up.  strategy: DWCONV_STRATEGY_AUTO / DIRECT / TILED /
 * STREAM as for dwconv2d_launch.  Errors as above, plus DWCONV_ERR_WORKSPACE when the
 * workspace is NULL, misaligned or too small.
 */
int dwconv2d_weight_grad_workspace_size(int N, int H, int W, int C, int kH, int kW,
                                        int stride, int dilation, int layout, int strategy,
                                        long long *bytes);

int dwconv2d_weight_grad(const float *x, const float *dy, float *dw, float *db,
                         void *workspace, long long workspace_bytes,
                         int N, int H, int W, int C, int kH, int kW,
                         int stride, int dilation, int layout, int strategy, void *stream);

/* ---- general form: explicit padding and a channel multiplier -----------
 *
 * The operation with explicit zero padding pads = {top, bottom, left, right}
 * (a host array of 4 ints; negative values crop) and a channel multiplier
 * mult >= 1 (grouped convolution with groups = C input channels and
 * mult*C output channels, the "4 => 8, groups = 4" layer of Reactant.jl
 * issue 331; output channel o reads input channel o / mult):
 *
 *   y[n,o,ho,wo] = b[o] + sum_{kh,kw} x[n, o/mult, ho*s + kh*d - top,
 *                                          wo*s + kw*d - left] * W[o,kh,kw]
 *
 * over in-range input positions; the output keeps every window position
 * that fits the padded input:
 *
 *   Ho = (H + top + bottom - d*(kH-1) - 1) / s + 1   (floor; must be >= 1)
 *   Wo = (W + left + right - d*(kW-1) - 1) / s + 1
 *
 * The input gradient is its transpose (each input position collects
 * W[o,kh,kw] * dy[n,o,ho,wo] over the mult output channels o reading it and
 * the (ho, kh) with ho*s + kh*d - top = h, likewise for columns): the
 * zero-upsampled dy placed on the positions the forward kept, run through
 * the reversed-kernel correlation.  The weight and bias gradients are
 *
 *   dW[o,kh,kw] = sum_{n,ho,wo} x[n, o/mult, ho*s+kh*d-top, wo*s+kw*d-left] * dy[n,o,ho,wo]
 *   db[o]       = sum_{n,ho,wo} dy[n,o,ho,wo]
 *
 * Kernel extents may be even here (the pads are explicit).  Shapes: x, dx
 * [N,H,W,C] / [N,C,H,W]; y, dy [N,Ho,Wo,mult*C] / [N,mult*C,Ho,Wo]; W
 * [mult*C][kH][kW] (the same bytes as a transposed convolution's
 * [C_in][C_out/groups][kH][kW] weight for dy -> dx, ExecuTorch MLX
 * conv-transpose weight page); b [mult*C] or NULL.  Ownership, execution
 * and errors as for the SAME entry points, plus DWCONV_ERR_NULL_PTR for a
 * NULL pads array and DWCONV_ERR_BAD_PAD.  With pads from
 * dwconv2d_same_pads(DWCONV_PAD_SAME, ...) and mult = 1 every call below is
 * the SAME entry point of the same name.
 */

/* Pads of a padding mode (DWCONV_PAD_SAME or DWCONV_PAD_XLA_SAME) for odd
 * kernels: writes {top, bottom, left, right} to pads[0..3].  SAME gives
 * d*(k-1)/2 everywhere; XLA_SAME at stride 2 gives top = d*(kH-1)/2 - 1,
 * bottom = d*(kH-1)/2 (same for columns), so that Ho = floor(H/2) and
 * output row ho is the stride-1 SAME row 2*ho + 1 (at stride 1 it equals
 * SAME).  On even extents with kernels of two or more taps these are XLA's
 * own SAME pads.  Host only. */
int dwconv2d_same_pads(int mode, int H, int W, int kH, int kW, int stride, int dilation,
                       int *pads);

/* Output extents Ho, Wo (either may be NULL) of a padded problem; validates
 * as the launch would.  Host only. */
int dwconv2d_out_extents(int H, int W, int kH, int kW, int stride, int dilation,
                         const int *pads, int *Ho, int *Wo);

/* dwconv2d_launch with explicit pads and a channel multiplier.  C is the
 * number of INPUT channels (x, dx); y, dy, W and b have mult*C. */
int dwconv2d_launch_ex(int op, const float *in, const void *w, int wtype, const float *b,
                       float *out, int N, int H, int W, int C, int mult, int kH, int kW,
                       int stride, int dilation, const int *pads, int layout, int strategy,
                       void *stream);

/* dwconv2d_describe with explicit pads and a channel multiplier (op may be
 * DWCONV_OP_WEIGHT_GRAD). */
int dwconv2d_describe_ex(int op, int wtype, int has_bias, int N, int H, int W, int C, int mult,
                         int kH, int kW, int stride, int dilation, const int *pads, int layout,
                         int strategy, char *name, int name_len, long long *grid, int *block);

/* dwconv2d_describe_ex for tensors at given addresses: addr_bits is the
 * bitwise OR of the addresses the launch would pass (in, out and b for the
 * forward and input gradient, plus the BatchNorm arrays of the fused
 * forward; x and dy for the weight gradient).  The kernels use 16-byte
 * loads and stores only when every one of those addresses is a multiple of
 * 16; with addr_bits = 0 this is dwconv2d_describe_ex.  Host only; lets a
 * caller see which kernel a tensor view at an offset gets. */
int dwconv2d_describe_addr_ex(int op, int wtype, int has_bias, int N, int H, int W, int C,
                              int mult, int kH, int kW, int stride, int dilation, const int *pads,
                              int layout, int strategy, unsigned long long addr_bits, char *name,
                              int name_len, long long *grid, int *block);

/* Weight and bias gradients with explicit pads and a channel multiplier:
 * dw is [mult*C][kH][kW], db [mult*C] or NULL; workspace as for
 * dwconv2d_weight_grad, sized by dwconv2d_weight_grad_workspace_size_ex. */
int dwconv2d_weight_grad_workspace_size_ex(int N, int H, int W, int C, int mult, int kH, int kW,
                                           int stride, int dilation, const int *pads,
                                           int layout, int strategy, long long *bytes);

int dwconv2d_weight_grad_ex(const float *x, const float *dy, float *dw, float *db,
                            void *workspace, long long workspace_bytes,
                            int N, int H, int W, int C, int mult, int kH, int kW,
                            int stride, int dilation, const int *pads, int layout, int strategy,
                            void *stream);

/* Allocation-free weight and bias gradients, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight training or
 * serving loops, harnesses that forbid hipMalloc): dwconv2d_weight_grad_ex
 * without the workspace arguments.  The per-tile partial sums go to a
 * scratch array the library holds on each GPU (DWCONV_SCRATCH_BYTES = 16 MiB
 * per device, allocated when the library's code is loaded on that device and
 * kept until the process ends); nothing here calls hipMalloc, hipFree or an
 * allocating library routine.  The stream must belong to the current device.
 * A problem whose partial sums need more than the array holds (the
 * workspace size dwconv2d_weight_grad_workspace_size_ex reports for the same
 * arguments, up to the 16 MiB) returns DWCONV_ERR_SCRATCH before anything
 * is enqueued.  Every call on one GPU shares that GPU's array, which keeps
 * the last call's contents (every partial sum is written before it is read,
 * so nothing needs clearing): calls that may overlap on one GPU -- on
 * different streams, or from different host threads -- race and must be
 * serialised by the caller.  Results equal those of dwconv2d_weight_grad_ex
 * with the same arguments, bit for bit (same kernels, same order). */
#define DWCONV_SCRATCH_BYTES (16LL << 20)

int dwconv2d_weight_grad_noalloc_ex(const float *x, const float *dy, float *dw, float *db,
                                    int N, int H, int W, int C, int mult, int kH, int kW,
                                    int stride, int dilation, const int *pads, int layout,
                                    int strategy, void *stream);

/* ---- fused epilogues ----------------------------------------------------
 *
 * Forward with inference-form BatchNorm and an activation fused into the
 * store (the LeanMlir page's fused depthwise + BatchNorm codegen; the
 * activations of the networks it names), per output channel o:
 *
 *   z = conv(x; W, b)  (as dwconv2d_launch_ex),
 *   t = (z - mean[o]) * gamma[o] / sqrt(var[o] + eps) + beta[o],   y = act(t)
 *
 * gamma, beta, mean, var: [mult*C] float32 device arrays, all four given or
 * all NULL (then t = z); eps >= 0; act: DWCONV_ACT_*.  One pass: y is
 * written once, already normalised and activated.  Errors as for
 * dwconv2d_launch_ex, plus DWCONV_ERR_BAD_EPILOGUE (unknown act, some but
 * not all BatchNorm arrays, eps negative or not finite) and
 * DWCONV_ERR_ALIAS when y overlaps a BatchNorm array.
 */
int dwconv2d_fwd_bn_act_ex(const float *x, const void *w, int wtype, const float *b,
                           const float *gamma, const float *beta, const float *mean,
                           const float *var, float eps, int act, float *y,
                           int N, int H, int W, int C, int mult, int kH, int kW, int stride,
                           int dilation, const int *pads, int layout, int strategy, void *stream);

/*
 * Weight and bias gradients with the SGD step fused into their reduction
 * (LeanMlir "Depthwise": the weight and bias SGD steps W - lr*dW and
 * b - lr*db, at stride 1, stride 2 and XLA-SAME alike):
 *
 *   w[o,kh,kw] <- w[o,kh,kw] - lr * dW[o,kh,kw],   b[o] <- b[o] - lr * db[o]
 *
 * each rounded once (fused multiply-add).  w: [mult*C][kH][kW] float32,
 * updated in place; b: [mult*C] float32 updated in place, or NULL; dw, db:
 * optional outputs of the gradients themselves (NULL to skip).  lr must be
 * finite.  Workspace and other arguments as for dwconv2d_weight_grad_ex;
 * every array written must not overlap x, dy or another array written.
 */
int dwconv2d_weight_grad_sgd_ex(const float *x, const float *dy, float *w, float *b, float lr,
                                float *dw, float *db, void *workspace, long long workspace_bytes,
                                int N, int H, int W, int C, int mult, int kH, int kW, int stride,
                                int dilation, const int *pads, int layout, int strategy,
                                void *stream);

/* Static text for a status code ("unknown status" for unknown codes). */
const char *dwconv2d_strerror(int status);

/* Library version: major*10000 + minor*100 + patch. */
int dwconv2d_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DWCONV_H */
