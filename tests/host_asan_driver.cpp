// host_asan_driver.cpp -- the C ABI's host-side validation under AddressSanitizer and
// UndefinedBehaviorSanitizer (test infrastructure, CPU only).
//
// Built with g++ together with csrc/mq_api.cpp; the kernel launchers the API calls after its
// checks are replaced by the stubs below (they only count calls), so no GPU is needed. Every
// entry point is called with null, negative, huge, misaligned and mismatched arguments, and with
// valid ones; the sanitizers report any out-of-bounds host access or undefined arithmetic (for
// example a size product that overflows), and the driver checks the status of each call.
#include "../include/mq.h"
#include "../microscaling_quantized_convolution_amd/csrc/mq_kernels.hpp"
#include "../microscaling_quantized_convolution_amd/csrc/mq_wgrad_sum.hpp"

#include <climits>
#include <cstdio>
#include <cstdlib>

static int g_launches = 0;

namespace mq {
hipError_t launch_relayout_cbf(const float *, float *, int, int, int, int, int, uint32_t *, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_relayout_weight(const float *, float *, int, int, int, int, int, uint32_t *, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_quantize(const float *, int64_t, int, int, int, int, uint64_t, uint8_t *, uint8_t *, float *, uint32_t *, bool, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_quantize_nchw(const float *, int, int, int, int, int, int, uint64_t, uint8_t *, uint8_t *, float *, uint32_t *, bool, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_quantize_batch(const QuantJobDesc *jobs, int njobs, int, hipStream_t)
{
    for (int i = 0; i < njobs; ++i) (void)jobs[i].src; // every job descriptor is readable
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_quantize_weight(const float *, int, int, int, int, int, int, uint64_t, uint8_t *, uint8_t *, float *, uint32_t *, hipStream_t) { ++g_launches; return hipSuccess; }
size_t wgrad_workspace_bytes(const ConvGeom &) { return 4096; }
hipError_t launch_conv_fwd(const ConvGeom &, int, QOperand, QOperand, float *, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_conv_wgrad(const ConvGeom &, int, QOperand, QOperand, float *, void *, size_t, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_conv_dgrad(const ConvGeom &, int, QOperand, QOperand, float *, hipStream_t) { ++g_launches; return hipSuccess; }
bool spatial_supported(const ConvGeom &g) { return g.Kh <= 3 && g.Kw <= 3 && g.sh == g.sw; }
hipError_t launch_conv_fwd_spatial(const ConvGeom &, int, QOperand, QOperand, float *, hipStream_t, uint32_t *) { ++g_launches; return hipSuccess; }
hipError_t launch_conv_dgrad_spatial(const ConvGeom &, int, QOperand, QOperand, float *, hipStream_t, const WgradSum *, uint32_t *) { ++g_launches; return hipSuccess; }
hipError_t launch_amax(const float *, int64_t, uint32_t *, hipStream_t) { ++g_launches; return hipSuccess; }
bool wgrad_fast_supported(const ConvGeom &g) { return g.Kw <= 3 && g.sh == g.sw; }
size_t wgrad_fast_workspace_bytes(const ConvGeom &) { return 8192; }
hipError_t launch_conv_wgrad_fast(const ConvGeom &, int, QOperand, QOperand, float *, void *, size_t, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_conv_wgrad_partials(const ConvGeom &, int, QOperand, QOperand, float *, void *, size_t, hipStream_t, WgradSum *sum)
{
    *sum = WgradSum{};
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_wgrad_sum(const WgradSum &, hipStream_t) { ++g_launches; return hipSuccess; }
} // namespace mq

static int g_fail = 0;
#define EXPECT(call, st)                                                                           \
    do {                                                                                           \
        const mq_status got_ = (call);                                                             \
        if (got_ != (st)) {                                                                        \
            std::fprintf(stderr, "line %d: %s -> %d, expected %d\n", __LINE__, #call, (int)got_,   \
                         (int)(st));                                                               \
            ++g_fail;                                                                              \
        }                                                                                          \
    } while (0)

static mq_qtensor qt(int o0, int o1, int r, int s, int fmt, int role, uintptr_t p = 0x10000)
{
    mq_qtensor q;
    q.o0 = o0; q.o1 = o1; q.r = r; q.s = s; q.fmt = fmt; q.role = role;
    q.codes = reinterpret_cast<uint8_t *>(p);
    q.scales = reinterpret_cast<uint8_t *>(p);
    q.tscale = reinterpret_cast<float *>(p);
    return q;
}

int main()
{
    float *f = reinterpret_cast<float *>(0x20000);
    uint32_t *ws = reinterpret_cast<uint32_t *>(0x30000);
    const size_t wsb = MQ_QUANTIZE_WS_BYTES;
    hipStream_t s0 = nullptr;
    const int big[] = {INT_MAX, INT_MAX - 3, 1 << 30, 1 << 16, 65536, -1, 0};

    // status strings of every value, and one outside the enum
    for (int st = -1; st <= 6; ++st)
        if (!mq_status_str(static_cast<mq_status>(st))) ++g_fail;

    // size queries with extreme dimensions
    for (int a : big)
        for (int b : big) {
            (void)mq_codes_bytes(a, b, a, b, MQ_NVFP4);
            (void)mq_codes_bytes(b, 1, a, 3, MQ_NVFP6);
            (void)mq_scales_bytes(a, a, b, b);
        }

    // relayouts
    EXPECT(mq_relayout_cbf(nullptr, f, 1, 1, 1, 1, 0, nullptr, 0, s0), MQ_ERR_ARG);
    EXPECT(mq_relayout_cbf(f, f, 1, 1, 1, 1, 0, ws, wsb - 1, s0), MQ_ERR_WORKSPACE);
    EXPECT(mq_relayout_cbf(f, f, 2, 70000, 3, 3, 0, nullptr, 0, s0), MQ_ERR_UNSUPPORTED);
    EXPECT(mq_relayout_cbf(f, f, 2, 3, 4, 5, 1, ws, wsb, s0), MQ_OK);
    for (int a : big) (void)mq_relayout_cbf(f, f, a, 3, a, 2, 0, nullptr, 0, s0);
    EXPECT(mq_relayout_weight(f, f, 0, 1, 1, 1, 0, nullptr, 0, s0), MQ_ERR_ARG);
    EXPECT(mq_relayout_weight(f, f, 4, 5, 3, 3, 0, nullptr, 0, s0), MQ_OK);

    // quantization of single tensors
    for (int fmt : {(int)MQ_NVFP4, (int)MQ_NVFP6, 5})
        for (int a : big)
            for (int b : big) {
                mq_qtensor q = qt(a, b, a, b, fmt, MQ_ROLE_ACT);
                (void)mq_quantize(f, &q, MQ_RNE, 1, ws, wsb, 0, s0);
                (void)mq_quantize_nchw(f, &q, MQ_SR, 1, ws, wsb, 0, s0);
                q.role = MQ_ROLE_WEIGHT;
                (void)mq_quantize_weight(f, &q, MQ_RNE, 0, ws, wsb, s0);
            }
    mq_qtensor x = qt(8, 8, 16, 2, MQ_NVFP4, MQ_ROLE_ACT);
    EXPECT(mq_quantize(f, &x, MQ_RNE, 0, ws, wsb, 0, s0), MQ_OK);
    EXPECT(mq_quantize(f, &x, 7, 0, ws, wsb, 0, s0), MQ_ERR_ARG);
    EXPECT(mq_quantize(f, nullptr, MQ_RNE, 0, ws, wsb, 0, s0), MQ_ERR_ARG);
    EXPECT(mq_quantize_nchw(f, &x, MQ_SR, 3, ws, wsb, MQ_QUANTIZE_AMAX_READY, s0), MQ_OK);
    mq_qtensor mis = qt(8, 8, 16, 2, MQ_NVFP4, MQ_ROLE_ACT, 0x10008);
    EXPECT(mq_quantize(f, &mis, MQ_RNE, 0, ws, wsb, 0, s0), MQ_ERR_ARG);

    // batched quantization: every job count, including more than the maximum
    mq_quant_job jobs[MQ_QUANTIZE_BATCH_MAX + 2];
    for (int i = 0; i < MQ_QUANTIZE_BATCH_MAX + 2; ++i) {
        jobs[i].src = f;
        jobs[i].layout = MQ_SRC_NCHW;
        jobs[i].rnd = MQ_RNE;
        jobs[i].seed = 0;
        jobs[i].flags = 0;
        jobs[i].dst = x;
        jobs[i].amax_ws = ws + 4096 * i;
        jobs[i].amax_ws_bytes = wsb;
    }
    for (int n = -1; n <= MQ_QUANTIZE_BATCH_MAX + 2; ++n) (void)mq_quantize_batch(jobs, n, s0);
    EXPECT(mq_quantize_batch(jobs, 2, s0), MQ_OK);
    EXPECT(mq_quantize_batch(jobs, MQ_QUANTIZE_BATCH_MAX + 1, s0), MQ_ERR_UNSUPPORTED);
    EXPECT(mq_quantize_batch(nullptr, 1, s0), MQ_ERR_ARG);
    jobs[1].dst = qt(INT_MAX, INT_MAX, INT_MAX, INT_MAX, MQ_NVFP4, MQ_ROLE_ACT);
    (void)mq_quantize_batch(jobs, 2, s0);

    // convolutions: valid, mismatched and extreme geometries
    mq_conv c = {2, 16, 8, 8, 16, 3, 3, 1, 1, 0, 0};
    mq_qtensor w = qt(3, 3, 16, 16, MQ_NVFP4, MQ_ROLE_WEIGHT);
    mq_qtensor g = qt(6, 6, 16, 2, MQ_NVFP4, MQ_ROLE_GRAD);
    EXPECT(mq_conv_fwd(&c, &x, &w, f, s0), MQ_OK);
    EXPECT(mq_conv_fwd(&c, &w, &x, f, s0), MQ_ERR_SHAPE);
    EXPECT(mq_conv_dgrad(&c, &w, &g, f, s0), MQ_OK);
    const size_t need = mq_wgrad_workspace_bytes(&c);
    EXPECT(mq_conv_wgrad(&c, &g, &x, f, ws, need, s0), MQ_OK);
    EXPECT(mq_conv_wgrad(&c, &g, &x, f, ws, need - 1, s0), MQ_ERR_WORKSPACE);
    EXPECT(mq_conv_backward(&c, &w, &g, &x, f, f, ws, need, s0), MQ_OK);
    EXPECT(mq_conv_backward(nullptr, &w, &g, &x, f, f, ws, need, s0), MQ_ERR_ARG);
    EXPECT(mq_conv_fwd_amax(&c, &x, &w, f, ws, wsb, s0), MQ_OK);
    EXPECT(mq_conv_fwd_amax(&c, &x, &w, f, nullptr, wsb, s0), MQ_ERR_WORKSPACE);
    EXPECT(mq_conv_fwd_amax(&c, &x, &w, f, ws, wsb - 4, s0), MQ_ERR_WORKSPACE);
    EXPECT(mq_conv_fwd_amax(&c, &x, &w, f, ws + 1, wsb, s0), MQ_OK); // 4-byte aligned
    EXPECT(mq_conv_fwd_amax(&c, &x, &w, f, reinterpret_cast<uint32_t *>(0x30002), wsb, s0), MQ_ERR_ARG);
    EXPECT(mq_conv_backward_amax(&c, &w, &g, &x, f, f, ws, need, ws, wsb, s0), MQ_OK);
    EXPECT(mq_conv_backward_amax(&c, &w, &g, &x, f, f, ws, need, nullptr, wsb, s0), MQ_ERR_WORKSPACE);
    EXPECT(mq_conv_backward_amax(&c, &x, &g, &x, f, f, ws, need, ws, wsb, s0), MQ_ERR_SHAPE);
    mq_conv c5 = {2, 16, 8, 8, 16, 5, 5, 1, 1, 2, 2}; // generic kernels: the amax pass after
    mq_qtensor w5 = qt(5, 5, 16, 16, MQ_NVFP4, MQ_ROLE_WEIGHT), g5 = qt(8, 8, 16, 2, MQ_NVFP4, MQ_ROLE_GRAD);
    EXPECT(mq_conv_fwd_amax(&c5, &x, &w5, f, ws, wsb, s0), MQ_OK);
    EXPECT(mq_conv_backward_amax(&c5, &w5, &g5, &x, f, f, ws, 1 << 20, ws, wsb, s0), MQ_OK);
    for (int a : big)
        for (int b : big) {
            mq_conv e = {a, b, a, 7, b, 3, a, 1, b, 0, a};
            mq_qtensor ex = qt(a, 7, b, a, MQ_NVFP4, MQ_ROLE_ACT);
            mq_qtensor ew = qt(3, a, b, b, MQ_NVFP4, MQ_ROLE_WEIGHT);
            mq_qtensor eg = qt(a, b, b, a, MQ_NVFP4, MQ_ROLE_GRAD);
            (void)mq_conv_fwd(&e, &ex, &ew, f, s0);
            (void)mq_conv_dgrad(&e, &ew, &eg, f, s0);
            (void)mq_wgrad_workspace_bytes(&e);
            (void)mq_conv_wgrad(&e, &eg, &ex, f, ws, 1 << 20, s0);
            (void)mq_conv_backward(&e, &ew, &eg, &ex, f, f, ws, 1 << 20, s0);
            mq_conv e2 = {b, a, b, a, a, 1, 1, a, a, b, b};
            (void)mq_conv_fwd(&e2, &ex, &ew, f, s0);
            (void)mq_wgrad_workspace_bytes(&e2);
        }

    if (g_launches == 0) ++g_fail;
    std::printf("host validation: %d failures, %d launches\n", g_fail, g_launches);
    return g_fail != 0;
}
