/*
 * mq.h -- C ABI of the microscaling-quantized convolution library for MI355X (gfx950).
 *
 * The library implements the hot path of MicroQonv (onedev.kr paper digest "합성곱 텐서 레이아웃
 * 재배열로 마이크로스케일링 양자화의 이중 연산과 메모리 이동을 줄이는 MicroQonv"): every convolution
 * tensor is quantized exactly once, before any im2col expansion, into a channel-batch-first layout
 * with 4x4 square-block scaling, and all three convolution GEMMs run directly on the quantized
 * data with the im2col matrix formed on chip only.
 *
 * Conventions shared by every call:
 *   - Every pointer argument named *_dev, and every pointer inside mq_qtensor, is device memory
 *     on the current HIP device. The caller allocates and owns all memory; the library
 *     allocates nothing and keeps no state between calls (the one exception is the device
 *     array of mq_conv_backward_noalloc, part of the library's code object on each GPU).
 *   - Every call is asynchronous on `stream` (0 = the null stream). The return value reports
 *     only synchronous host-side argument validation and launch errors; no call synchronizes.
 *   - Data problems are not reported through the status: a tensor containing NaN or Inf
 *     quantizes to T = NaN, scales 0x7F (E4M3 NaN) and codes 0, and any convolution that
 *     consumes it produces NaN.
 *   - Calls that overlap on one stream are ordered; calls on different streams that share a
 *     buffer race.
 */
#ifndef MQ_H
#define MQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MQ_OK = 0,
    MQ_ERR_ARG = 1,         /* null pointer, non-positive size, unknown enum value */
    MQ_ERR_SHAPE = 2,       /* tensor shapes do not match the convolution / each other */
    MQ_ERR_UNSUPPORTED = 3, /* valid request outside the implemented set (see each call) */
    MQ_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required */
    MQ_ERR_LAUNCH = 5       /* a kernel launch failed (hipGetLastError) */
} mq_status;

/* Element formats (onedev.kr digest, sections "How it differs" and "How it is used"):
 * NVFP4 = E2M1 elements, NVFP6 = E2M3 elements; both with one E4M3 scale per 4x4 square and one
 * fp32 tensor scale. */
typedef enum { MQ_NVFP4 = 4, MQ_NVFP6 = 6 } mq_format;

/* Role of a quantized tensor; fixes the meaning of its four dimensions (o0, o1, r, s):
 *   MQ_ROLE_ACT    activation X          (Hin,  Win,  Cin,  N)   channel-batch-first
 *   MQ_ROLE_WEIGHT weight W              (Kh,   Kw,   Cout, Cin) one Cout x Cin matrix per tap
 *   MQ_ROLE_GRAD   output gradient G_Y   (Hout, Wout, Cout, N)   channel-batch-first */
typedef enum { MQ_ROLE_ACT = 0, MQ_ROLE_WEIGHT = 1, MQ_ROLE_GRAD = 2 } mq_role;

/* Element rounding: round-to-nearest-even (weights, activations) or stochastic (gradients),
 * per the onedev.kr digest, section "How it differs". */
typedef enum { MQ_RNE = 0, MQ_SR = 1 } mq_round;

/*
 * A quantized tensor: logical shape [o0][o1][r][s] (s fastest), cut into 4x4 squares over
 * (r, s) with r and s zero-padded up to multiples of 4. With R4 = ceil(r/4), S4 = ceil(s/4):
 *   square t = ((i0*o1 + i1)*R4 + ir/4)*S4 + is/4, element e = (ir%4)*4 + is%4;
 *   codes:  NVFP4 8 bytes per square, element e = nibble (e%2) of byte 8t + e/2 (low first);
 *           NVFP6 12 bytes per square, element e = bits [6e, 6e+6) of the little-endian
 *           96-bit word at byte 12t;
 *           code bits: NVFP4 s|ee|m (bias 1), NVFP6 s|ee|mmm (bias 1); padded slots are 0;
 *   scales: 1 byte per square, E4M3 s|eeee|mmm (bias 7, subnormals, 0x7E = 448, 0x7F = NaN);
 *   tscale: one fp32, the tensor scale T.
 * Value of an element: decode(code) * decode(scale) * T.
 * fmt and role hold mq_format / mq_role values. codes must be 16-byte aligned, scales and tscale
 * 4-byte aligned (device allocations are); other pointers give MQ_ERR_ARG. The convolutions may
 * read the up to 3 bytes that follow the last scale byte in its aligned 4-byte word (never
 * beyond it) and ignore them.
 */
typedef struct {
    int32_t o0, o1, r, s;
    int32_t fmt;
    int32_t role;
    uint8_t *codes;
    uint8_t *scales;
    float *tscale;
} mq_qtensor;

/* One 2-D convolution (groups 1, dilation 1, zero padding). Output size
 * Hout = (H + 2*pad_h - Kh)/stride_h + 1, Wout likewise. */
typedef struct {
    int32_t N, Cin, H, W, Cout, Kh, Kw, stride_h, stride_w, pad_h, pad_w;
} mq_conv;

/* Human-readable name of a status code (static string, never NULL). */
const char *mq_status_str(mq_status st);

/* Bytes needed for the code stream / scale bytes of a quantized tensor with the given logical
 * shape and format: squares * (8 | 12) and squares * 1. Returns 0 for invalid arguments. */
size_t mq_codes_bytes(int32_t o0, int32_t o1, int32_t r, int32_t s, int32_t fmt);
size_t mq_scales_bytes(int32_t o0, int32_t o1, int32_t r, int32_t s);

/*
 * Tensor-amax workspace (mq_quantize, and optionally the relayouts): device scratch of at least
 * MQ_QUANTIZE_WS_BYTES bytes, 4-byte aligned. Word 0 holds the number P of partial maxima,
 * words 1..P the partials (max |x| per part of the tensor, as fp32 bit patterns). Calls on one
 * stream may share a workspace; calls that can run concurrently must not.
 */
#define MQ_QUANTIZE_WS_BYTES 8192

/*
 * mq_relayout_cbf: NCHW fp32 <-> channel-batch-first fp32.
 * Channel-batch-first X_{Cin,N} (onedev.kr digest, section "How it works"): for each pixel
 * (h, w) all channels and all batch elements are contiguous; here [H][W][C][N], N fastest.
 *   inverse = 0: dst[h][w][c][n] = src[n][c][h][w]
 *   inverse = 1: dst[n][c][h][w] = src[h][w][c][n]
 * src_dev, dst_dev: N*C*H*W floats each, must not overlap.
 * amax_ws_dev: null, or a tensor-amax workspace that receives the partial maxima of the tensor
 *          (the relayout reads every element anyway), so that mq_quantize of dst_dev can pass
 *          MQ_QUANTIZE_AMAX_READY and skip its own pass over the tensor. amax_ws_bytes is
 *          ignored when amax_ws_dev is null.
 * Errors: MQ_ERR_ARG for null pointers, non-positive sizes or a misaligned workspace;
 *         MQ_ERR_WORKSPACE for a workspace below MQ_QUANTIZE_WS_BYTES; MQ_ERR_UNSUPPORTED for
 *         C > 65535.
 */
mq_status mq_relayout_cbf(const float *src_dev, float *dst_dev, int32_t N, int32_t C, int32_t H,
                          int32_t W, int32_t inverse, uint32_t *amax_ws_dev, size_t amax_ws_bytes,
                          hipStream_t stream);

/*
 * mq_relayout_weight: OIHW fp32 <-> tap-major [Kh][Kw][Cout][Cin] fp32, the layout of the 2-D
 * weight matrix W_{fCout,Cin} (Cout x Kh*Kw*Cin; onedev.kr digest, section "How it differs")
 * with one Cout x Cin block per tap.
 *   inverse = 0: dst[kh][kw][co][ci] = src[co][ci][kh][kw];  inverse = 1: the reverse.
 * amax_ws_dev, amax_ws_bytes: as for mq_relayout_cbf.
 * Errors: MQ_ERR_ARG for null pointers, non-positive sizes or a misaligned workspace;
 *         MQ_ERR_WORKSPACE for a workspace below MQ_QUANTIZE_WS_BYTES.
 */
mq_status mq_relayout_weight(const float *src_dev, float *dst_dev, int32_t Cout, int32_t Cin,
                             int32_t Kh, int32_t Kw, int32_t inverse, uint32_t *amax_ws_dev,
                             size_t amax_ws_bytes, hipStream_t stream);

/* mq_quantize flag: amax_ws_dev already holds the partial maxima of this tensor's values (from a
 * relayout that wrote src_dev, earlier on the same stream); the amax pass is skipped. */
#define MQ_QUANTIZE_AMAX_READY 1u

/*
 * mq_quantize: quantize one fp32 tensor, exactly once, with the NVFP4 / NVFP6 recipe of the
 * onedev.kr digest, section "How it differs":
 *   amax = max |x| over the tensor;
 *   T    = amax / (448 * Emax)                              (Emax = 6 for E2M1, 7.5 for E2M3)
 *   per 4x4 square: B = CastE4M3(max|x_i| / (T * Emax))    (nearest-even, saturating at 448)
 *   per element:    code = Round(x_i / (B * T))            (RNE, or SR for rnd = MQ_SR)
 * All scale arithmetic is IEEE fp32 in the written order. Stochastic rounding rounds |q| up
 * from its lower grid neighbour lo to hi iff u16 < ((|q|-lo)/(hi-lo)) * 65536, with u16 the
 * (e%2)-th 16-bit half of word (e%8)/2 of Philox4x32-10(counter = (2t + e/8, 0, 0, 0),
 * key = seed) for element e of square t. Codes keep the sign bit of x. Squares with B = 0 hold
 * codes 0; a tensor with T = 0 holds scales 0 and codes 0.
 *
 * src_dev: the tensor as dense fp32 [o0][o1][r][s] (for activations and gradients this is the
 *          channel-batch-first layout).
 * dst:     host struct describing the destination; dst->codes, dst->scales, dst->tscale are
 *          device buffers of mq_codes_bytes / mq_scales_bytes / 4 bytes.
 * amax_ws_dev / amax_ws_bytes: a tensor-amax workspace (overwritten unless flags has
 *          MQ_QUANTIZE_AMAX_READY, then read).
 * flags:   0 or MQ_QUANTIZE_AMAX_READY.
 * Errors: MQ_ERR_ARG (null pointer, bad enum or flag, non-positive dims, misaligned pointer),
 *         MQ_ERR_WORKSPACE (amax_ws_dev null or smaller than MQ_QUANTIZE_WS_BYTES),
 *         MQ_ERR_UNSUPPORTED (2^31 squares or more).
 */
mq_status mq_quantize(const float *src_dev, const mq_qtensor *dst, int32_t rnd, uint64_t seed,
                      uint32_t *amax_ws_dev, size_t amax_ws_bytes, uint32_t flags,
                      hipStream_t stream);

/*
 * mq_quantize_nchw: quantize an NCHW fp32 activation or output gradient straight into its
 * channel-batch-first quantized layout (onedev.kr digest, section "How it works": the layout
 * change happens before quantization, which then runs once, section "How it differs"). The
 * codes, scales and T are those of mq_relayout_cbf (inverse = 0) followed by mq_quantize on its
 * output, with the same recipe, rounding and random draws (square t of the channel-batch-first
 * tensor), without writing the fp32 channel-batch-first copy: an amax pass over src_dev (unless
 * flags has MQ_QUANTIZE_AMAX_READY), then one quantizing pass that reads NCHW and writes squares.
 * src_dev: N*C*H*W floats [n][c][h][w] with (H, W, C, N) = (dst->o0, dst->o1, dst->r, dst->s).
 * dst:     role MQ_ROLE_ACT or MQ_ROLE_GRAD, buffers as for mq_quantize.
 * amax_ws_dev / amax_ws_bytes / flags: as for mq_quantize (the partial maxima may come from any
 *          layout of the same values).
 * Errors: MQ_ERR_ARG (null pointer, bad enum or flag, non-positive dims, misaligned pointer),
 *         MQ_ERR_SHAPE (role MQ_ROLE_WEIGHT), MQ_ERR_WORKSPACE (as for mq_quantize),
 *         MQ_ERR_UNSUPPORTED (the source zero-padded to whole squares, 16*ceil(N/4)*ceil(C/4)*H*W
 *         floats, reaches 2^31 bytes).
 */
mq_status mq_quantize_nchw(const float *src_dev, const mq_qtensor *dst, int32_t rnd, uint64_t seed,
                           uint32_t *amax_ws_dev, size_t amax_ws_bytes, uint32_t flags,
                           hipStream_t stream);

/* Source order of a batched quantization job (mq_quant_job.layout). */
typedef enum {
    MQ_SRC_DENSE = 0, /* [o0][o1][r][s] as stored by the quantized layout (mq_quantize) */
    MQ_SRC_NCHW = 1,  /* NCHW activation or gradient, dst (o0, o1, r, s) = (H, W, C, N) */
    MQ_SRC_OIHW = 2   /* OIHW weight, dst (o0, o1, r, s) = (Kh, Kw, Cout, Cin) */
} mq_source_layout;

#define MQ_QUANTIZE_BATCH_MAX 4

/* One tensor of mq_quantize_batch: what mq_quantize (MQ_SRC_DENSE), mq_quantize_nchw
 * (MQ_SRC_NCHW) or mq_quantize_weight (MQ_SRC_OIHW) would take, with its own workspace. */
typedef struct {
    const float *src;     /* device fp32 source in the order `layout` names */
    int32_t layout;       /* mq_source_layout */
    int32_t rnd;          /* mq_round */
    uint64_t seed;        /* SR seed (ignored for MQ_RNE) */
    uint32_t flags;       /* 0 or MQ_QUANTIZE_AMAX_READY */
    mq_qtensor dst;       /* destination (device buffers) */
    uint32_t *amax_ws;    /* this tensor's amax workspace, device, 4-byte aligned */
    size_t amax_ws_bytes; /* >= MQ_QUANTIZE_WS_BYTES */
} mq_quant_job;

/*
 * mq_quantize_batch: quantize up to MQ_QUANTIZE_BATCH_MAX tensors of one format with one amax
 * launch and one quantizing launch, each exactly as the single-tensor call for its layout would
 * (same recipe of the onedev.kr digest, section "How it differs"; same codes, scales, T and
 * stochastic draws). Batching lets a small tensor share the launches of a large one: the
 * forward pass of a layer quantizes X (NCHW) and W (OIHW) together.
 * jobs: host array of njobs (1..MQ_QUANTIZE_BATCH_MAX) job descriptions; every job needs its own
 *       amax workspace (the same pointer twice is MQ_ERR_ARG).
 * Errors: MQ_ERR_ARG (null pointer, bad enum or flag, misaligned pointer, non-positive dims,
 *         shared workspace), MQ_ERR_SHAPE (formats differ between jobs; an NCHW job with a
 *         weight destination or an OIHW job with another role), MQ_ERR_WORKSPACE (a workspace
 *         missing or below MQ_QUANTIZE_WS_BYTES), MQ_ERR_UNSUPPORTED (more than
 *         MQ_QUANTIZE_BATCH_MAX jobs, 2^31 squares or more, or an NCHW source that reaches 2^31
 *         bytes once zero-padded to whole squares).
 */
mq_status mq_quantize_batch(const mq_quant_job *jobs, int32_t njobs, hipStream_t stream);

/*
 * mq_quantize_weight: quantize an OIHW fp32 weight straight into the tap-major quantized layout
 * [Kh][Kw][Cout][Cin] of the 2-D weight matrix (onedev.kr digest, section "How it differs"),
 * with the same amax, T, square scales and codes as mq_relayout_weight followed by mq_quantize
 * on its output (the recipe above), without writing the fp32 tap-major copy. A weight of at
 * most 65536 elements takes one launch (every workgroup reduces the whole tensor's amax itself,
 * then quantizes its share of the squares); a larger one runs the amax pass into amax_ws_dev and
 * a quantizer that gathers from OIHW.
 * w_oihw_dev: Cout*Cin*Kh*Kw floats, [co][ci][kh][kw].
 * dst:     role MQ_ROLE_WEIGHT with (o0, o1, r, s) = (Kh, Kw, Cout, Cin).
 * rnd, seed: as for mq_quantize.
 * amax_ws_dev / amax_ws_bytes: a tensor-amax workspace (overwritten; untouched for a small
 *          weight, but required either way).
 * Errors: MQ_ERR_ARG (null pointer, bad enum, misaligned pointer), MQ_ERR_SHAPE (dst role not
 *         MQ_ROLE_WEIGHT), MQ_ERR_WORKSPACE (workspace null or smaller than
 *         MQ_QUANTIZE_WS_BYTES), MQ_ERR_UNSUPPORTED (2^31 squares or more).
 */
mq_status mq_quantize_weight(const float *w_oihw_dev, const mq_qtensor *dst, int32_t rnd,
                             uint64_t seed, uint32_t *amax_ws_dev, size_t amax_ws_bytes,
                             hipStream_t stream);

/*
 * mq_conv_fwd: forward GEMM Y = W . X' (onedev.kr digest, section "How it differs") with the
 * im2col matrix X' formed on chip from the channel-batch-first quantized X (section "How it
 * works"):
 *   Y[ho][wo][co][n] = T_W * T_X * sum_{kh,kw,ci} Wq[kh][kw][co][ci]
 *                                               * Xq[ho*sh - ph + kh][wo*sw - pw + kw][ci][n]
 * (zero outside the input), accumulated in fp32 from exact fp16 (or bf16) products.
 * x: MQ_ROLE_ACT tensor of shape (H, W, Cin, N); w: MQ_ROLE_WEIGHT tensor (Kh, Kw, Cout, Cin);
 * same format. y_dev: fp32 channel-batch-first [Hout][Wout][Cout][N], fully overwritten.
 * Errors: MQ_ERR_ARG, MQ_ERR_SHAPE (dims or formats disagree with p), MQ_ERR_UNSUPPORTED.
 */
mq_status mq_conv_fwd(const mq_conv *p, const mq_qtensor *x, const mq_qtensor *w, float *y_dev,
                      hipStream_t stream);

/* Bytes of device workspace mq_conv_wgrad needs for this convolution (0 on invalid input). */
size_t mq_wgrad_workspace_bytes(const mq_conv *p);

/*
 * mq_conv_wgrad: weight-gradient GEMM G_W = G_Y . X'^T (onedev.kr digest, section "How it
 * differs"), reading the quantized G_Y and X along their batch-contiguous direction:
 *   G_W[kh][kw][co][ci] = T_G * T_X * sum_{ho,wo,n} Gq[ho][wo][co][n]
 *                                               * Xq[ho*sh - ph + kh][wo*sw - pw + kw][ci][n]
 * gy: MQ_ROLE_GRAD (Hout, Wout, Cout, N); x: MQ_ROLE_ACT (H, W, Cin, N); same format.
 * gw_dev: fp32 [Kh][Kw][Cout][Cin], fully overwritten.
 * ws_dev / ws_bytes: device scratch of at least mq_wgrad_workspace_bytes(p) bytes (split-K
 * partial sums; summed in a fixed order, so results are deterministic).
 * Errors: MQ_ERR_ARG, MQ_ERR_SHAPE, MQ_ERR_WORKSPACE, MQ_ERR_UNSUPPORTED.
 */
mq_status mq_conv_wgrad(const mq_conv *p, const mq_qtensor *gy, const mq_qtensor *x,
                        float *gw_dev, void *ws_dev, size_t ws_bytes, hipStream_t stream);

/*
 * mq_conv_dgrad: input-gradient GEMM G_X' = W^T . G_Y (onedev.kr digest, section "How it
 * differs") with the col2im sum fused, so the Kh*Kw-inflated G_X' never exists in memory:
 *   G_X[h][w][ci][n] = T_W * T_G * sum_{kh,kw,co} Wq[kh][kw][co][ci] * Gq[ho][wo][co][n]
 *       over (ho, wo) with ho*sh - ph + kh = h and wo*sw - pw + kw = w.
 * w: MQ_ROLE_WEIGHT (Kh, Kw, Cout, Cin); gy: MQ_ROLE_GRAD (Hout, Wout, Cout, N); same format.
 * gx_dev: fp32 channel-batch-first [H][W][Cin][N], fully overwritten.
 * Errors: MQ_ERR_ARG, MQ_ERR_SHAPE, MQ_ERR_UNSUPPORTED.
 */
mq_status mq_conv_dgrad(const mq_conv *p, const mq_qtensor *w, const mq_qtensor *gy,
                        float *gx_dev, hipStream_t stream);

/*
 * mq_conv_backward: both gradients of one convolution, G_W as mq_conv_wgrad and G_X as
 * mq_conv_dgrad compute them (same values, bit for bit), for the backward pass that needs both.
 * For the tuned shapes the weight gradient's split sum runs inside the input-gradient launch, on
 * workgroups of its own (when the CUs that launch leaves idle finish it in a few passes), instead
 * of as a launch between the two GEMMs. gw_dev, gx_dev and ws_dev must not overlap.
 * w: MQ_ROLE_WEIGHT (Kh, Kw, Cout, Cin); gy: MQ_ROLE_GRAD (Hout, Wout, Cout, N);
 * x: MQ_ROLE_ACT (H, W, Cin, N); one format.
 * gw_dev: fp32 [Kh][Kw][Cout][Cin]; gx_dev: fp32 [H][W][Cin][N]; both fully overwritten.
 * ws_dev / ws_bytes: as for mq_conv_wgrad (mq_wgrad_workspace_bytes(p)).
 * Errors: MQ_ERR_ARG, MQ_ERR_SHAPE, MQ_ERR_WORKSPACE, MQ_ERR_UNSUPPORTED.
 */
mq_status mq_conv_backward(const mq_conv *p, const mq_qtensor *w, const mq_qtensor *gy,
                           const mq_qtensor *x, float *gw_dev, float *gx_dev, void *ws_dev,
                           size_t ws_bytes, hipStream_t stream);

/*
 * mq_conv_fwd_amax: mq_conv_fwd (same Y, bit for bit) whose epilogue also writes the tensor-amax
 * partial maxima of |Y| into amax_ws_dev, in the format mq_quantize reads with
 * MQ_QUANTIZE_AMAX_READY. When Y is the next tensor to be quantized (the next layer's activation
 * with nothing elementwise in between), mq_quantize of Y (channel-batch-first, dense source)
 * then skips its own read of Y: the tensor amax of the NVFP4 / NVFP6 recipe (onedev.kr digest,
 * section "How it differs": T = max|X| / (448 * Emax)) comes from the producer of the tensor.
 * The workgroups of the tuned kernels each write one partial; other shapes run the amax pass over
 * Y after the convolution (same partials format, same result).
 * amax_ws_dev / amax_ws_bytes: a tensor-amax workspace (MQ_QUANTIZE_WS_BYTES, 4-byte aligned),
 *          overwritten; pass it to mq_quantize of Y with MQ_QUANTIZE_AMAX_READY, later on the same
 *          stream.
 * Errors: as mq_conv_fwd; MQ_ERR_WORKSPACE (workspace null or below MQ_QUANTIZE_WS_BYTES),
 *         MQ_ERR_ARG (misaligned workspace).
 */
mq_status mq_conv_fwd_amax(const mq_conv *p, const mq_qtensor *x, const mq_qtensor *w,
                           float *y_dev, uint32_t *amax_ws_dev, size_t amax_ws_bytes,
                           hipStream_t stream);

/*
 * mq_conv_backward_amax: mq_conv_backward (same G_W and G_X, bit for bit) whose input-gradient
 * epilogue also writes the tensor-amax partial maxima of |G_X| into gx_amax_ws_dev (format as for
 * mq_conv_fwd_amax). G_X is the output gradient of the layer before when nothing elementwise sits
 * between, so its stochastic quantization (mq_quantize, MQ_QUANTIZE_AMAX_READY) skips its amax
 * pass.
 * gx_amax_ws_dev / gx_amax_ws_bytes: a tensor-amax workspace, overwritten.
 * Errors: as mq_conv_backward; MQ_ERR_WORKSPACE / MQ_ERR_ARG for the amax workspace as above.
 */
mq_status mq_conv_backward_amax(const mq_conv *p, const mq_qtensor *w, const mq_qtensor *gy,
                                const mq_qtensor *x, float *gw_dev, float *gx_dev, void *ws_dev,
                                size_t ws_bytes, uint32_t *gx_amax_ws_dev, size_t gx_amax_ws_bytes,
                                hipStream_t stream);

/*
 * Size of the device array that mq_conv_backward_noalloc keeps the weight gradient's split-K
 * partial sums in (one array per GPU, held until the process ends).
 */
#define MQ_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * mq_conv_backward_noalloc: mq_conv_backward (same kernels, same G_W and G_X bit for bit) for
 * callers that cannot allocate memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid hipMalloc. The weight gradient's split-K partial sums go to a
 * library-owned device array of MQ_NOALLOC_SCRATCH_BYTES on the current device instead of a
 * caller workspace; the call allocates nothing (no hipMalloc, no allocating library routine).
 * The caller still provides every input and output as for mq_conv_backward, on the current HIP
 * device (stream must belong to it).
 * Every call on one GPU shares that GPU's array: calls that can overlap on one GPU (different
 * streams, or threads without ordering between their calls) race and must not be issued;
 * calls ordered on one stream are fine.
 * Errors: as mq_conv_backward; MQ_ERR_UNSUPPORTED when mq_wgrad_workspace_bytes(p) exceeds
 *         MQ_NOALLOC_SCRATCH_BYTES; MQ_ERR_LAUNCH when the device array cannot be located.
 */
mq_status mq_conv_backward_noalloc(const mq_conv *p, const mq_qtensor *w, const mq_qtensor *gy,
                                   const mq_qtensor *x, float *gw_dev, float *gx_dev,
                                   hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MQ_H */
