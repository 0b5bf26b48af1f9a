// mq_kernels.hpp -- host-side launch entry points of the library's kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mq.h"

namespace mq {

// Host-side validation of mq_conv_backward's arguments other than the workspace: MQ_OK, or the
// status mq_conv_backward returns for them (mq_api.cpp).
mq_status backward_check(const mq_conv *p, const mq_qtensor *w, const mq_qtensor *gy,
                         const mq_qtensor *x, const float *gw, const float *gx);

// Tensor-amax workspace: word 0 = number of partial maxima P (1..kAmaxParts), words 1..P = the
// partials (max |x| as fp32 bit patterns). Written by the amax pass or by a relayout that is
// given the workspace (amax_ws non-null), read by the quantize kernel.
constexpr int kAmaxParts = 1024;
hipError_t launch_relayout_cbf(const float *src, float *dst, int N, int C, int H, int W,
                               int inverse, uint32_t *amax_ws, hipStream_t st);
hipError_t launch_relayout_weight(const float *src, float *dst, int Cout, int Cin, int Kh,
                                  int Kw, int inverse, uint32_t *amax_ws, hipStream_t st);
hipError_t launch_quantize(const float *src, int64_t planes, int R, int S, int fmt, int rnd,
                           uint64_t seed, uint8_t *codes, uint8_t *scales, float *tscale,
                           uint32_t *amax_ws, bool amax_ready, hipStream_t st);
// NCHW fp32 -> quantized channel-batch-first squares [H][W][C4][N4]: the same codes, scales and
// T as launch_relayout_cbf followed by launch_quantize, without the fp32 copy (the amax pass,
// unless amax_ready, then one launch). hipErrorInvalidValue when the zero-padded tensor
// reaches 2^31 bytes.
hipError_t launch_quantize_nchw(const float *src, int N, int C, int H, int W, int fmt, int rnd,
                                uint64_t seed, uint8_t *codes, uint8_t *scales, float *tscale,
                                uint32_t *amax_ws, bool amax_ready, hipStream_t st);
// One tensor of a batched quantization. layout: 0 = dense [o0][o1][r][s] (channel-batch-first
// activations and gradients, tap-major weights), 1 = NCHW with (o0, o1, r, s) = (H, W, C, N),
// 2 = OIHW weight with (o0, o1, r, s) = (Kh, Kw, Cout, Cin). Dimensions, pointers and workspace
// are validated by the caller; rnd 0 = RNE, 1 = SR.
struct QuantJobDesc {
    const float *src;
    int layout, o0, o1, r, s, rnd;
    uint64_t seed;
    uint8_t *codes, *scales;
    float *tscale;
    uint32_t *amax_ws;
    bool amax_ready;
};
// Up to four tensors of one format: one amax launch (jobs without their amax ready) and one
// quantizing launch. hipErrorInvalidValue for more than four jobs, 2^31 squares or more, or an
// NCHW source whose zero-padded size reaches 2^31 bytes.
hipError_t launch_quantize_batch(const QuantJobDesc *jobs, int njobs, int fmt, hipStream_t st);
// OIHW fp32 weight [Cout][Cin][Kh][Kw] -> quantized tap-major squares [Kh][Kw][Cout][Cin], the
// same codes, scales and T as launch_relayout_weight followed by launch_quantize, without the
// fp32 copy (one launch for a weight of at most 65536 elements, every workgroup reducing the
// whole amax itself; else the amax pass in amax_ws and a quantizer that gathers from OIHW).
hipError_t launch_quantize_weight(const float *src, int Cout, int Cin, int Kh, int Kw, int fmt,
                                  int rnd, uint64_t seed, uint8_t *codes, uint8_t *scales,
                                  float *tscale, uint32_t *amax_ws, hipStream_t st);

// Convolution geometry shared by the GEMM kernels.
struct ConvGeom {
    int N, Cin, H, W, Cout, Kh, Kw, sh, sw, ph, pw, Ho, Wo;
    int N4, Cin4, Cout4; // squares along N, Cin, Cout
};

struct QOperand {
    const uint8_t *codes;
    const uint8_t *scales;
    const float *tscale;
};

size_t wgrad_workspace_bytes(const ConvGeom &g);
hipError_t launch_conv_fwd(const ConvGeom &g, int fmt, QOperand x, QOperand w, float *y,
                           hipStream_t st);
hipError_t launch_conv_wgrad(const ConvGeom &g, int fmt, QOperand gy, QOperand x, float *gw,
                             void *ws, size_t ws_bytes, hipStream_t st);
hipError_t launch_conv_dgrad(const ConvGeom &g, int fmt, QOperand w, QOperand gy, float *gx,
                             hipStream_t st);

struct WgradSum;

// Halo-tiled forward / input-gradient kernels (Kh, Kw <= 3, equal strides 1 or 2).
// launch_conv_dgrad_spatial with a sum: the weight gradient's split sum runs in the same launch,
// on workgroups of its own (a grid row after the input-gradient classes).
// amax_ws (null = none): a tensor-amax workspace that receives the partial maxima of |output|,
// written by the kernel's epilogue (or by the amax pass over the output when the launch has more
// workgroups than partials), so that quantizing the output can pass MQ_QUANTIZE_AMAX_READY.
bool spatial_supported(const ConvGeom &g);
hipError_t launch_conv_fwd_spatial(const ConvGeom &g, int fmt, QOperand x, QOperand w, float *y,
                                   hipStream_t st, uint32_t *amax_ws = nullptr);
hipError_t launch_conv_dgrad_spatial(const ConvGeom &g, int fmt, QOperand w, QOperand gy,
                                     float *gx, hipStream_t st, const struct WgradSum *sum = nullptr,
                                     uint32_t *amax_ws = nullptr);
// The tensor-amax pass over n floats: partial maxima of |x| into ws (count in ws[0]).
hipError_t launch_amax(const float *x, int64_t n, uint32_t *ws, hipStream_t st);

// Split-K weight gradient with all kw taps of one kernel row per workgroup (Kw <= 3,
// equal strides 1 or 2) and a deterministic split sum.
bool wgrad_fast_supported(const ConvGeom &g);
size_t wgrad_fast_workspace_bytes(const ConvGeom &g);
hipError_t launch_conv_wgrad_fast(const ConvGeom &g, int fmt, QOperand gy, QOperand x, float *gw,
                                  void *ws, size_t ws_bytes, hipStream_t st);
// The split-K kernel alone: the partial sums go to ws and *sum describes their sum into gw, to be
// run by launch_wgrad_sum or by workgroups riding along in the input-gradient launch.
hipError_t launch_conv_wgrad_partials(const ConvGeom &g, int fmt, QOperand gy, QOperand x,
                                      float *gw, void *ws, size_t ws_bytes, hipStream_t st,
                                      struct WgradSum *sum);
// The sum of those partials as a kernel of its own (nothing when there is nothing to sum).
hipError_t launch_wgrad_sum(const struct WgradSum &sum, hipStream_t st);

} // namespace mq
