// dwconv_launch.hip -- runs a validated forward / input-gradient plan: the
// dispatch over the kernel families and the launch status.
#include "dwconv_device.h"

namespace dwconv {

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
    switch (pl.kind) {
    case KIND_DIRECT_NHWC:
    case KIND_DIRECT_NCHW:
        return launch_direct(p, pl, in, w, bb, out, stream, ep);
    case KIND_TILED_NHWC:
        return launch_tiled_nhwc(p, pl, in, w, bb, out, stream, ep);
    case KIND_TILED_NCHW:
        return launch_tiled_nchw(p, pl, in, w, bb, out, stream, ep);
    case KIND_STREAM_NHWC:
        return launch_stream_nhwc(p, pl, in, w, bb, out, stream, ep);
    case KIND_STREAM_NCHW:
        return launch_stream_nchw(p, pl, in, w, bb, out, stream, ep);
    case KIND_STREAM_NCHW_PLANES:
        return launch_stream_nchw_planes(p, pl, in, w, bb, out, stream, ep);
    default:
        return DWCONV_ERR_BAD_STRATEGY;
    }
}

}  // namespace dwconv
