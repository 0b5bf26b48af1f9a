// mq_api.cpp -- C ABI of the library: host-side validation and kernel dispatch.
//
// Every call validates its arguments on the host, then enqueues kernels on the caller's stream.
// Nothing here allocates, synchronizes or reads device memory.
#include "../../include/mq.h"
#include "mq_kernels.hpp"
#include "mq_wgrad_sum.hpp"

#include <stdint.h>
#include <stdlib.h>

namespace {

bool fmt_ok(int32_t f) { return f == MQ_NVFP4 || f == MQ_NVFP6; }

// Squares of a tensor of positive dimensions, in 64-bit arithmetic (every factor is below 2^31,
// so the product of the four fits unless the tensor has 2^62 squares or more: callers compare
// it with limits far below that, and saturate the first two factors' product first).
int64_t squares(int32_t o0, int32_t o1, int32_t r, int32_t s)
{
    const int64_t planes = (int64_t)o0 * o1, tiles = (((int64_t)r + 3) / 4) * (((int64_t)s + 3) / 4);
    const int64_t cap = (int64_t)1 << 62;
    return planes > cap / tiles ? cap : planes * tiles;
}

// The kernels read codes with 16-byte loads and scales with aligned 4-byte loads (which may
// cover up to 3 bytes past the last scale, always inside the same aligned word).
bool qtensor_ok(const mq_qtensor *q)
{
    return q && q->o0 > 0 && q->o1 > 0 && q->r > 0 && q->s > 0 && fmt_ok(q->fmt) &&
           q->role >= MQ_ROLE_ACT && q->role <= MQ_ROLE_GRAD && q->codes && q->scales &&
           q->tscale && ((uintptr_t)q->codes & 15u) == 0 && ((uintptr_t)q->scales & 3u) == 0 &&
           ((uintptr_t)q->tscale & 3u) == 0;
}

// Geometry of a convolution, or false if it is not a valid convolution.
bool conv_geom(const mq_conv *p, mq::ConvGeom *g)
{
    if (!p) return false;
    if (p->N < 1 || p->Cin < 1 || p->H < 1 || p->W < 1 || p->Cout < 1 || p->Kh < 1 ||
        p->Kw < 1 || p->stride_h < 1 || p->stride_w < 1 || p->pad_h < 0 || p->pad_w < 0)
        return false;
    // padded extents in 64 bits (every field is below 2^31)
    const int64_t hp = (int64_t)p->H + 2 * (int64_t)p->pad_h, wp = (int64_t)p->W + 2 * (int64_t)p->pad_w;
    if (hp < p->Kh || wp < p->Kw) return false;
    g->N = p->N; g->Cin = p->Cin; g->H = p->H; g->W = p->W; g->Cout = p->Cout;
    g->Kh = p->Kh; g->Kw = p->Kw; g->sh = p->stride_h; g->sw = p->stride_w;
    g->ph = p->pad_h; g->pw = p->pad_w;
    const int64_t ho = (hp - p->Kh) / p->stride_h + 1, wo = (wp - p->Kw) / p->stride_w + 1;
    if (ho > INT32_MAX || wo > INT32_MAX) return false;
    g->Ho = (int)ho;
    g->Wo = (int)wo;
    g->N4 = (int)(((int64_t)p->N + 3) / 4);
    g->Cin4 = (int)(((int64_t)p->Cin + 3) / 4);
    g->Cout4 = (int)(((int64_t)p->Cout + 3) / 4);
    return true;
}

// a * b * c for non-negative factors below 2^31, saturated at 2^62 (no overflow)
int64_t mul3_sat(int64_t a, int64_t b, int64_t c)
{
    const int64_t cap = (int64_t)1 << 62, ab = a * b; // below 2^62
    return (c != 0 && ab > cap / c) ? cap : ab * c;
}

// Limits of the implemented kernels: 32-bit index arithmetic inside the GEMM kernels.
bool conv_supported(const mq::ConvGeom &g)
{
    const int64_t lim = (int64_t)1 << 30;
    if (mul3_sat(g.H, g.W, g.N4) >= lim / 4 || mul3_sat(g.Ho, g.Wo, g.N4) >= lim / 4) return false;
    if (mul3_sat(g.Kh, g.Kw, g.Cin4 > g.Cout4 ? g.Cin4 : g.Cout4) >= lim / 4) return false;
    return true;
}

bool dims_are(const mq_qtensor *q, int32_t a, int32_t b, int32_t c, int32_t d, int32_t role)
{
    return q->o0 == a && q->o1 == b && q->r == c && q->s == d && q->role == role;
}

mq::QOperand operand(const mq_qtensor *q) { return {q->codes, q->scales, q->tscale}; }

mq_status launch_status(hipError_t e) { return e == hipSuccess ? MQ_OK : MQ_ERR_LAUNCH; }

// Optional amax workspace of a relayout: null, or at least MQ_QUANTIZE_WS_BYTES, 4-byte aligned.
mq_status amax_ws_check(const uint32_t *ws, size_t bytes)
{
    if (!ws) return MQ_OK;
    if (bytes < MQ_QUANTIZE_WS_BYTES) return MQ_ERR_WORKSPACE;
    return (reinterpret_cast<uintptr_t>(ws) & 3u) ? MQ_ERR_ARG : MQ_OK;
}

} // namespace

namespace mq {

// Host-side validation of mq_conv_backward's arguments (everything but the workspace).
mq_status backward_check(const mq_conv *p, const mq_qtensor *w, const mq_qtensor *gy,
                         const mq_qtensor *x, const float *gw, const float *gx)
{
    ConvGeom g;
    if (!conv_geom(p, &g) || !qtensor_ok(w) || !qtensor_ok(gy) || !qtensor_ok(x) || !gw || !gx)
        return MQ_ERR_ARG;
    if (!dims_are(w, p->Kh, p->Kw, p->Cout, p->Cin, MQ_ROLE_WEIGHT) ||
        !dims_are(gy, g.Ho, g.Wo, p->Cout, p->N, MQ_ROLE_GRAD) ||
        !dims_are(x, p->H, p->W, p->Cin, p->N, MQ_ROLE_ACT) || w->fmt != gy->fmt ||
        x->fmt != gy->fmt)
        return MQ_ERR_SHAPE;
    if (!conv_supported(g)) return MQ_ERR_UNSUPPORTED;
    return MQ_OK;
}

} // namespace mq

extern "C" {

const char *mq_status_str(mq_status st)
{
    switch (st) {
    case MQ_OK: return "MQ_OK";
    case MQ_ERR_ARG: return "MQ_ERR_ARG: invalid argument";
    case MQ_ERR_SHAPE: return "MQ_ERR_SHAPE: tensor shapes or formats do not match";
    case MQ_ERR_UNSUPPORTED: return "MQ_ERR_UNSUPPORTED: outside the implemented set";
    case MQ_ERR_WORKSPACE: return "MQ_ERR_WORKSPACE: workspace missing or too small";
    case MQ_ERR_LAUNCH: return "MQ_ERR_LAUNCH: kernel launch failed";
    }
    return "unknown mq_status";
}

size_t mq_codes_bytes(int32_t o0, int32_t o1, int32_t r, int32_t s, int32_t fmt)
{
    if (o0 < 1 || o1 < 1 || r < 1 || s < 1 || !fmt_ok(fmt)) return 0;
    return (size_t)squares(o0, o1, r, s) * (fmt == MQ_NVFP4 ? 8u : 12u);
}

size_t mq_scales_bytes(int32_t o0, int32_t o1, int32_t r, int32_t s)
{
    if (o0 < 1 || o1 < 1 || r < 1 || s < 1) return 0;
    return (size_t)squares(o0, o1, r, s);
}

mq_status mq_relayout_cbf(const float *src, float *dst, int32_t N, int32_t C, int32_t H,
                          int32_t W, int32_t inverse, uint32_t *amax_ws, size_t amax_ws_bytes,
                          hipStream_t stream)
{
    if (!src || !dst || N < 1 || C < 1 || H < 1 || W < 1 || (inverse != 0 && inverse != 1))
        return MQ_ERR_ARG;
    if (C > 65535) return MQ_ERR_UNSUPPORTED;
    const mq_status ws = amax_ws_check(amax_ws, amax_ws_bytes);
    if (ws != MQ_OK) return ws;
    return launch_status(mq::launch_relayout_cbf(src, dst, N, C, H, W, inverse, amax_ws, stream));
}

mq_status mq_relayout_weight(const float *src, float *dst, int32_t Cout, int32_t Cin,
                             int32_t Kh, int32_t Kw, int32_t inverse, uint32_t *amax_ws,
                             size_t amax_ws_bytes, hipStream_t stream)
{
    if (!src || !dst || Cout < 1 || Cin < 1 || Kh < 1 || Kw < 1 ||
        (inverse != 0 && inverse != 1))
        return MQ_ERR_ARG;
    const mq_status ws = amax_ws_check(amax_ws, amax_ws_bytes);
    if (ws != MQ_OK) return ws;
    return launch_status(mq::launch_relayout_weight(src, dst, Cout, Cin, Kh, Kw, inverse, amax_ws,
                                                    stream));
}

mq_status mq_quantize(const float *src, const mq_qtensor *dst, int32_t rnd, uint64_t seed,
                      uint32_t *amax_ws, size_t amax_ws_bytes, uint32_t flags, hipStream_t stream)
{
    if (!src || !qtensor_ok(dst) || (rnd != MQ_RNE && rnd != MQ_SR)) return MQ_ERR_ARG;
    if (flags & ~(uint32_t)MQ_QUANTIZE_AMAX_READY) return MQ_ERR_ARG;
    if (!amax_ws || amax_ws_bytes < MQ_QUANTIZE_WS_BYTES) return MQ_ERR_WORKSPACE;
    if (squares(dst->o0, dst->o1, dst->r, dst->s) >= ((int64_t)1 << 31)) return MQ_ERR_UNSUPPORTED;
    if ((reinterpret_cast<uintptr_t>(amax_ws) & 3u) != 0) return MQ_ERR_ARG;
    return launch_status(mq::launch_quantize(src, (int64_t)dst->o0 * dst->o1, dst->r, dst->s,
                                             dst->fmt, rnd, seed, dst->codes, dst->scales,
                                             dst->tscale, amax_ws,
                                             (flags & MQ_QUANTIZE_AMAX_READY) != 0, stream));
}

mq_status mq_quantize_nchw(const float *src, const mq_qtensor *dst, int32_t rnd, uint64_t seed,
                           uint32_t *amax_ws, size_t amax_ws_bytes, uint32_t flags,
                           hipStream_t stream)
{
    if (!src || !qtensor_ok(dst) || (rnd != MQ_RNE && rnd != MQ_SR)) return MQ_ERR_ARG;
    if (flags & ~(uint32_t)MQ_QUANTIZE_AMAX_READY) return MQ_ERR_ARG;
    if (dst->role == MQ_ROLE_WEIGHT) return MQ_ERR_SHAPE;
    if (!amax_ws || amax_ws_bytes < MQ_QUANTIZE_WS_BYTES) return MQ_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(amax_ws) & 3u) != 0) return MQ_ERR_ARG;
    // zero-padded source (4*ceil(N/4) x 4*ceil(C/4) planes) below 2^31 bytes
    // zero-padded source: 16 floats per square
    if (squares(dst->o0, dst->o1, dst->r, dst->s) >= ((int64_t)1 << 31) / 64) return MQ_ERR_UNSUPPORTED;
    return launch_status(mq::launch_quantize_nchw(src, dst->s, dst->r, dst->o0, dst->o1, dst->fmt,
                                                  rnd, seed, dst->codes, dst->scales, dst->tscale,
                                                  amax_ws, (flags & MQ_QUANTIZE_AMAX_READY) != 0,
                                                  stream));
}

mq_status mq_quantize_batch(const mq_quant_job *jobs, int32_t njobs, hipStream_t stream)
{
    if (!jobs || njobs < 1) return MQ_ERR_ARG;
    if (njobs > MQ_QUANTIZE_BATCH_MAX) return MQ_ERR_UNSUPPORTED;
    mq::QuantJobDesc d[MQ_QUANTIZE_BATCH_MAX];
    for (int i = 0; i < njobs; ++i) {
        const mq_quant_job &j = jobs[i];
        const mq_qtensor *q = &j.dst;
        if (!j.src || !qtensor_ok(q) || (j.rnd != MQ_RNE && j.rnd != MQ_SR)) return MQ_ERR_ARG;
        if (j.layout != MQ_SRC_DENSE && j.layout != MQ_SRC_NCHW && j.layout != MQ_SRC_OIHW)
            return MQ_ERR_ARG;
        if (j.flags & ~(uint32_t)MQ_QUANTIZE_AMAX_READY) return MQ_ERR_ARG;
        if (!j.amax_ws || j.amax_ws_bytes < MQ_QUANTIZE_WS_BYTES) return MQ_ERR_WORKSPACE;
        if ((reinterpret_cast<uintptr_t>(j.amax_ws) & 3u) != 0) return MQ_ERR_ARG;
        for (int k = 0; k < i; ++k)
            if (jobs[k].amax_ws == j.amax_ws) return MQ_ERR_ARG; // one workspace per tensor
        if (q->fmt != jobs[0].dst.fmt) return MQ_ERR_SHAPE;
        if ((j.layout == MQ_SRC_NCHW && q->role == MQ_ROLE_WEIGHT) ||
            (j.layout == MQ_SRC_OIHW && q->role != MQ_ROLE_WEIGHT))
            return MQ_ERR_SHAPE;
        if (squares(q->o0, q->o1, q->r, q->s) >= ((int64_t)1 << 31)) return MQ_ERR_UNSUPPORTED;
        if (j.layout == MQ_SRC_NCHW) {
            if (squares(q->o0, q->o1, q->r, q->s) >= ((int64_t)1 << 31) / 64) return MQ_ERR_UNSUPPORTED;
        }
        d[i].src = j.src;
        d[i].layout = j.layout == MQ_SRC_NCHW ? 1 : (j.layout == MQ_SRC_OIHW ? 2 : 0);
        d[i].o0 = q->o0; d[i].o1 = q->o1; d[i].r = q->r; d[i].s = q->s;
        d[i].rnd = j.rnd; d[i].seed = j.seed;
        d[i].codes = q->codes; d[i].scales = q->scales; d[i].tscale = q->tscale;
        d[i].amax_ws = j.amax_ws;
        d[i].amax_ready = (j.flags & MQ_QUANTIZE_AMAX_READY) != 0;
    }
    return launch_status(mq::launch_quantize_batch(d, njobs, jobs[0].dst.fmt, stream));
}

mq_status mq_quantize_weight(const float *w, const mq_qtensor *dst, int32_t rnd, uint64_t seed,
                             uint32_t *amax_ws, size_t amax_ws_bytes, hipStream_t stream)
{
    if (!w || !qtensor_ok(dst) || (rnd != MQ_RNE && rnd != MQ_SR)) return MQ_ERR_ARG;
    if (dst->role != MQ_ROLE_WEIGHT) return MQ_ERR_SHAPE;
    if (!amax_ws || amax_ws_bytes < MQ_QUANTIZE_WS_BYTES) return MQ_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(amax_ws) & 3u) != 0) return MQ_ERR_ARG;
    if (squares(dst->o0, dst->o1, dst->r, dst->s) >= ((int64_t)1 << 31)) return MQ_ERR_UNSUPPORTED;
    return launch_status(mq::launch_quantize_weight(w, dst->r, dst->s, dst->o0, dst->o1, dst->fmt,
                                                    rnd, seed, dst->codes, dst->scales,
                                                    dst->tscale, amax_ws, stream));
}

mq_status mq_conv_fwd(const mq_conv *p, const mq_qtensor *x, const mq_qtensor *w, float *y,
                      hipStream_t stream)
{
    mq::ConvGeom g;
    if (!conv_geom(p, &g) || !qtensor_ok(x) || !qtensor_ok(w) || !y) return MQ_ERR_ARG;
    if (!dims_are(x, p->H, p->W, p->Cin, p->N, MQ_ROLE_ACT) ||
        !dims_are(w, p->Kh, p->Kw, p->Cout, p->Cin, MQ_ROLE_WEIGHT) || x->fmt != w->fmt)
        return MQ_ERR_SHAPE;
    if (!conv_supported(g)) return MQ_ERR_UNSUPPORTED;
    if (mq::spatial_supported(g))
        return launch_status(
            mq::launch_conv_fwd_spatial(g, x->fmt, operand(x), operand(w), y, stream));
    return launch_status(mq::launch_conv_fwd(g, x->fmt, operand(x), operand(w), y, stream));
}

size_t mq_wgrad_workspace_bytes(const mq_conv *p)
{
    mq::ConvGeom g;
    if (!conv_geom(p, &g)) return 0;
    return mq::wgrad_fast_supported(g) ? mq::wgrad_fast_workspace_bytes(g)
                                        : mq::wgrad_workspace_bytes(g);
}

mq_status mq_conv_wgrad(const mq_conv *p, const mq_qtensor *gy, const mq_qtensor *x, float *gw,
                        void *ws, size_t ws_bytes, hipStream_t stream)
{
    mq::ConvGeom g;
    if (!conv_geom(p, &g) || !qtensor_ok(gy) || !qtensor_ok(x) || !gw) return MQ_ERR_ARG;
    if (!dims_are(gy, g.Ho, g.Wo, p->Cout, p->N, MQ_ROLE_GRAD) ||
        !dims_are(x, p->H, p->W, p->Cin, p->N, MQ_ROLE_ACT) || gy->fmt != x->fmt)
        return MQ_ERR_SHAPE;
    if (!conv_supported(g)) return MQ_ERR_UNSUPPORTED;
    if (mq::wgrad_fast_supported(g)) {
        if (!ws || ws_bytes < mq::wgrad_fast_workspace_bytes(g)) return MQ_ERR_WORKSPACE;
        return launch_status(mq::launch_conv_wgrad_fast(g, x->fmt, operand(gy), operand(x), gw,
                                                        ws, ws_bytes, stream));
    }
    if (!ws || ws_bytes < mq::wgrad_workspace_bytes(g)) return MQ_ERR_WORKSPACE;
    return launch_status(mq::launch_conv_wgrad(g, x->fmt, operand(gy), operand(x), gw, ws,
                                               ws_bytes, stream));
}

mq_status mq_conv_dgrad(const mq_conv *p, const mq_qtensor *w, const mq_qtensor *gy, float *gx,
                        hipStream_t stream)
{
    mq::ConvGeom g;
    if (!conv_geom(p, &g) || !qtensor_ok(w) || !qtensor_ok(gy) || !gx) return MQ_ERR_ARG;
    if (!dims_are(w, p->Kh, p->Kw, p->Cout, p->Cin, MQ_ROLE_WEIGHT) ||
        !dims_are(gy, g.Ho, g.Wo, p->Cout, p->N, MQ_ROLE_GRAD) || w->fmt != gy->fmt)
        return MQ_ERR_SHAPE;
    if (!conv_supported(g)) return MQ_ERR_UNSUPPORTED;
    if (mq::spatial_supported(g))
        return launch_status(
            mq::launch_conv_dgrad_spatial(g, w->fmt, operand(w), operand(gy), gx, stream));
    return launch_status(mq::launch_conv_dgrad(g, w->fmt, operand(w), operand(gy), gx, stream));
}

mq_status mq_conv_backward(const mq_conv *p, const mq_qtensor *w, const mq_qtensor *gy,
                           const mq_qtensor *x, float *gw, float *gx, void *ws, size_t ws_bytes,
                           hipStream_t stream)
{
    const mq_status chk = mq::backward_check(p, w, gy, x, gw, gx);
    if (chk != MQ_OK) return chk;
    mq::ConvGeom g;
    conv_geom(p, &g);
    if (mq::wgrad_fast_supported(g) && mq::spatial_supported(g)) {
        if (!ws || ws_bytes < mq::wgrad_fast_workspace_bytes(g)) return MQ_ERR_WORKSPACE;
        mq::WgradSum sum;
        const hipError_t e = mq::launch_conv_wgrad_partials(g, x->fmt, operand(gy), operand(x),
                                                            gw, ws, ws_bytes, stream, &sum);
        if (e != hipSuccess) return launch_status(e);
        return launch_status(mq::launch_conv_dgrad_spatial(g, w->fmt, operand(w), operand(gy),
                                                           gx, stream, &sum));
    }
    const mq_status st = mq_conv_wgrad(p, gy, x, gw, ws, ws_bytes, stream);
    if (st != MQ_OK) return st;
    return mq_conv_dgrad(p, w, gy, gx, stream);
}

mq_status mq_conv_fwd_amax(const mq_conv *p, const mq_qtensor *x, const mq_qtensor *w, float *y,
                           uint32_t *amax_ws, size_t amax_ws_bytes, hipStream_t stream)
{
    if (!amax_ws) return MQ_ERR_WORKSPACE;
    const mq_status wst = amax_ws_check(amax_ws, amax_ws_bytes);
    if (wst != MQ_OK) return wst;
    mq::ConvGeom g;
    if (!conv_geom(p, &g) || !qtensor_ok(x) || !qtensor_ok(w) || !y) return MQ_ERR_ARG;
    if (!dims_are(x, p->H, p->W, p->Cin, p->N, MQ_ROLE_ACT) ||
        !dims_are(w, p->Kh, p->Kw, p->Cout, p->Cin, MQ_ROLE_WEIGHT) || x->fmt != w->fmt)
        return MQ_ERR_SHAPE;
    if (!conv_supported(g)) return MQ_ERR_UNSUPPORTED;
    if (mq::spatial_supported(g))
        return launch_status(
            mq::launch_conv_fwd_spatial(g, x->fmt, operand(x), operand(w), y, stream, amax_ws));
    const hipError_t e = mq::launch_conv_fwd(g, x->fmt, operand(x), operand(w), y, stream);
    if (e != hipSuccess) return launch_status(e);
    return launch_status(
        mq::launch_amax(y, (int64_t)g.Ho * g.Wo * g.Cout * g.N, amax_ws, stream));
}

mq_status mq_conv_backward_amax(const mq_conv *p, const mq_qtensor *w, const mq_qtensor *gy,
                                const mq_qtensor *x, float *gw, float *gx, void *ws,
                                size_t ws_bytes, uint32_t *gx_amax_ws, size_t gx_amax_ws_bytes,
                                hipStream_t stream)
{
    if (!gx_amax_ws) return MQ_ERR_WORKSPACE;
    const mq_status wst = amax_ws_check(gx_amax_ws, gx_amax_ws_bytes);
    if (wst != MQ_OK) return wst;
    const mq_status chk = mq::backward_check(p, w, gy, x, gw, gx);
    if (chk != MQ_OK) return chk;
    mq::ConvGeom g;
    conv_geom(p, &g);
    if (mq::wgrad_fast_supported(g) && mq::spatial_supported(g)) {
        if (!ws || ws_bytes < mq::wgrad_fast_workspace_bytes(g)) return MQ_ERR_WORKSPACE;
        mq::WgradSum sum;
        const hipError_t e = mq::launch_conv_wgrad_partials(g, x->fmt, operand(gy), operand(x),
                                                            gw, ws, ws_bytes, stream, &sum);
        if (e != hipSuccess) return launch_status(e);
        return launch_status(mq::launch_conv_dgrad_spatial(g, w->fmt, operand(w), operand(gy),
                                                           gx, stream, &sum, gx_amax_ws));
    }
    const mq_status st = mq_conv_backward(p, w, gy, x, gw, gx, ws, ws_bytes, stream);
    if (st != MQ_OK) return st;
    return launch_status(mq::launch_amax(gx, (int64_t)g.H * g.W * g.Cin * g.N, gx_amax_ws, stream));
}

} // extern "C"
