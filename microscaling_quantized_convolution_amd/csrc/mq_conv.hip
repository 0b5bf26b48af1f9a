// mq_conv.hip -- the three convolution GEMMs on square-block quantized, channel-batch-first data.
//
// onedev.kr MicroQonv digest, section "How it differs": with W_{fCout,Cin} (Cout x Kh*Kw*Cin)
// and G_{YfCout,N} (Cout x Hout*Wout*N) the convolution is three GEMMs,
//   forward  Y   = W . X'          (M = Cout, N = Hout*Wout*N, K = Kh*Kw*Cin)
//   wgrad    G_W = G_Y . X'^T      (M = Cout, N = Kh*Kw*Cin,   K = Hout*Wout*N)
//   dgrad    G_X' = W^T . G_Y      (M = Cin,  N = H*W*N,       K = Kh*Kw*Cout, col2im fused)
// and one side of every 4x4 square lies along each GEMM's reduction direction, so the squares
// quantized once serve all three. Section "How it works": from the channel-batch-first layout
// the im2col operand is gathered on chip (contiguous along Cin in forward, along N in the
// gradients) and never written to memory.
//
// Each workgroup computes a BM x BN tile of C. Per K-step it gathers the quantized squares of the
// A and B blocks (an out-of-image square is zero), decodes them exactly to bf16 (an E2M1/E2M3
// value times an E4M3 scale has at most 8 significant bits) into LDS, and runs bf16
// 32x32x16 MFMAs with fp32 accumulation. The tensor scales multiply in the epilogue (in double,
// one rounding to fp32). The weight gradient splits K over workgroups and sums the partials in a
// fixed order in a second kernel.
#include "mq_device.hpp"
#include "mq_kernels.hpp"

namespace mq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

enum GemmKind { kFwd = 0, kWgrad = 1, kDgrad = 2 };

constexpr int BM = 64, BN = 128, BK = 32;   // workgroup tile, K-step (elements)
constexpr int BK4 = BK / 4;                 // squares per K-step
constexpr int LDK = BK + 8;                 // LDS row length in bf16 (pad against conflicts)

struct GemmArgs {
    ConvGeom g;
    QOperand a, b;
    float *out;       // Y / G_X (fwd, dgrad) or split-K partials (wgrad)
    int M4, N4c, K4;  // squares along M, along the columns, along K
    int k4_per_split; // wgrad only
    int ldp;          // wgrad partial row length (columns, padded to BN)
};

// Square lookups. Return the square index into the operand, or -1 for a zero square.
// ks is set when the square's s-dimension runs along K (else its r-dimension does).
template <int KIND>
__device__ __forceinline__ int64_t a_square(const ConvGeom &g, int m4, int k4)
{
    if (KIND == kFwd) { // W[tap][co][ci]: m = co, k = (tap, ci)
        int tap = k4 / g.Cin4, ci4 = k4 - tap * g.Cin4;
        return ((int64_t)tap * g.Cout4 + m4) * g.Cin4 + ci4;
    } else if (KIND == kWgrad) { // G[pix][co][n]: m = co, k = (pix, n)
        int pix = k4 / g.N4, nb4 = k4 - pix * g.N4;
        return ((int64_t)pix * g.Cout4 + m4) * g.N4 + nb4;
    } else { // W[tap][co][ci]: m = ci, k = (tap, co)
        int tap = k4 / g.Cout4, co4 = k4 - tap * g.Cout4;
        return ((int64_t)tap * g.Cout4 + co4) * g.Cin4 + m4;
    }
}

template <int KIND>
__device__ __forceinline__ int64_t b_square(const ConvGeom &g, int k4, int n4)
{
    if (KIND == kFwd) { // X[hi][wi][ci][n]: k = (tap, ci), column = (pix_out, n)
        int tap = k4 / g.Cin4, ci4 = k4 - tap * g.Cin4;
        int pix = n4 / g.N4, nb4 = n4 - pix * g.N4;
        int ho = pix / g.Wo, wo = pix - ho * g.Wo;
        int kh = tap / g.Kw, kw = tap - kh * g.Kw;
        int hi = ho * g.sh - g.ph + kh, wi = wo * g.sw - g.pw + kw;
        if (hi < 0 || hi >= g.H || wi < 0 || wi >= g.W) return -1;
        return (((int64_t)hi * g.W + wi) * g.Cin4 + ci4) * g.N4 + nb4;
    } else if (KIND == kWgrad) { // X[hi][wi][ci][n]: k = (pix_out, n), column = (tap, ci)
        int pix = k4 / g.N4, nb4 = k4 - pix * g.N4;
        int tap = n4 / g.Cin4, ci4 = n4 - tap * g.Cin4;
        int ho = pix / g.Wo, wo = pix - ho * g.Wo;
        int kh = tap / g.Kw, kw = tap - kh * g.Kw;
        int hi = ho * g.sh - g.ph + kh, wi = wo * g.sw - g.pw + kw;
        if (hi < 0 || hi >= g.H || wi < 0 || wi >= g.W) return -1;
        return (((int64_t)hi * g.W + wi) * g.Cin4 + ci4) * g.N4 + nb4;
    } else { // G[ho][wo][co][n]: k = (tap, co), column = (pix_in, n)
        int tap = k4 / g.Cout4, co4 = k4 - tap * g.Cout4;
        int pix = n4 / g.N4, nb4 = n4 - pix * g.N4;
        int hi = pix / g.W, wi = pix - hi * g.W;
        int kh = tap / g.Kw, kw = tap - kh * g.Kw;
        int th = hi + g.ph - kh, tw = wi + g.pw - kw;
        if (th < 0 || tw < 0) return -1;
        int ho = th / g.sh, wo = tw / g.sw;
        if (ho * g.sh != th || wo * g.sw != tw || ho >= g.Ho || wo >= g.Wo) return -1;
        return (((int64_t)ho * g.Wo + wo) * g.Cout4 + co4) * g.N4 + nb4;
    }
}

// Orientation of the A / B squares: true = the square's s-dimension is the GEMM's K.
template <int KIND> struct Orient;
template <> struct Orient<kFwd> { static constexpr bool a_ks = true, b_ks = false; };
template <> struct Orient<kWgrad> { static constexpr bool a_ks = true, b_ks = true; };
template <> struct Orient<kDgrad> { static constexpr bool a_ks = false, b_ks = false; };

// Decode one square to 16 bf16 bit patterns (element order e = r*4 + s).
template <int FMT>
__device__ __forceinline__ void decode_square(const QOperand &q, int64_t sq, uint32_t (&v)[16])
{
    using F = Fmt<FMT>;
    if (sq < 0) {
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] = 0u;
        return;
    }
    const uint32_t sc = q.scales[sq];
    const float B = ((sc & 0x7Fu) == 0x7Fu) ? __uint_as_float(0x7FC00000u) : e4m3_to_float(sc);
    uint32_t code[16];
    if (FMT == kFP4) {
        const uint2 w = *reinterpret_cast<const uint2 *>(q.codes + 8 * sq);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            code[e] = (w.x >> (4 * e)) & 0xFu;
            code[e + 8] = (w.y >> (4 * e)) & 0xFu;
        }
    } else {
        const uint32_t *p = reinterpret_cast<const uint32_t *>(q.codes + 12 * sq);
        const uint32_t w0 = p[0], w1 = p[1], w2 = p[2];
        const uint64_t lo = ((uint64_t)w1 << 32) | w0;
        const uint64_t hi = ((uint64_t)w2 << 32) | w1;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int bit = 6 * e;
            code[e] = (bit < 58) ? (uint32_t)(lo >> bit) & 0x3Fu
                                 : (uint32_t)(hi >> (bit - 32)) & 0x3Fu;
        }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const uint32_t mag = code[e] & F::kMaxMag;
        const float val = elem_mag_to_float<FMT>(mag) * B;
        v[e] = bf16_bits_exact(val) | ((code[e] & F::kSign) ? 0x8000u : 0u);
    }
}

// Write a decoded square into an LDS operand tile laid out [row][k] (k contiguous).
template <bool KS>
__device__ __forceinline__ void store_square(uint16_t *lds, int row0, int k0,
                                             const uint32_t (&v)[16])
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t p0, p1;
        if (KS) { // square row i -> LDS row row0+i, elements (i,0..3) along k
            p0 = v[4 * i + 0] | (v[4 * i + 1] << 16);
            p1 = v[4 * i + 2] | (v[4 * i + 3] << 16);
        } else { // square column i -> LDS row row0+i, elements (0..3,i) along k
            p0 = v[i] | (v[4 + i] << 16);
            p1 = v[8 + i] | (v[12 + i] << 16);
        }
        *reinterpret_cast<uint2 *>(lds + (row0 + i) * LDK + k0) = make_uint2(p0, p1);
    }
}

template <int FMT, int KIND>
__global__ void __launch_bounds__(256) conv_gemm_kernel(GemmArgs args)
{
    __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDK];
    const ConvGeom &g = args.g;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int m4_0 = blockIdx.y * (BM / 4), n4_0 = blockIdx.x * (BN / 4);

    int k4_beg = 0, k4_end = args.K4;
    if (KIND == kWgrad) {
        k4_beg = blockIdx.z * args.k4_per_split;
        k4_end = min(args.K4, k4_beg + args.k4_per_split);
    }

    f32x16_t acc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;

    for (int k4_0 = k4_beg; k4_0 < k4_end; k4_0 += BK4) {
        // A block: (BM/4) x BK4 = 128 squares, k fastest across threads.
        if (tid < (BM / 4) * BK4) {
            const int kl = tid % BK4, ml = tid / BK4;
            const int m4 = m4_0 + ml, k4 = k4_0 + kl;
            int64_t sq = -1;
            if (m4 < args.M4 && k4 < k4_end) sq = a_square<KIND>(g, m4, k4);
            uint32_t v[16];
            decode_square<FMT>(args.a, sq, v);
            store_square<Orient<KIND>::a_ks>(As, 4 * ml, 4 * kl, v);
        }
        // B block: BK4 x (BN/4) = 256 squares.
        {
            int kl, nl;
            if (KIND == kWgrad) { kl = tid % BK4; nl = tid / BK4; } // K runs along memory
            else { nl = tid % (BN / 4); kl = tid / (BN / 4); }
            const int n4 = n4_0 + nl, k4 = k4_0 + kl;
            int64_t sq = -1;
            if (n4 < args.N4c && k4 < k4_end) sq = b_square<KIND>(g, k4, n4);
            uint32_t v[16];
            decode_square<FMT>(args.b, sq, v);
            store_square<Orient<KIND>::b_ks>(Bs, 4 * nl, 4 * kl, v);
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; kk += 16) {
            const int kofs = kk + 8 * (lane >> 5);
            const bf16x8_t af =
                *reinterpret_cast<const bf16x8_t *>(As + (32 * wm + (lane & 31)) * LDK + kofs);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const bf16x8_t bfr = *reinterpret_cast<const bf16x8_t *>(
                    Bs + (64 * wn + 32 * j + (lane & 31)) * LDK + kofs);
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfr, acc[j], 0, 0, 0);
            }
        }
        __syncthreads();
    }

    // Epilogue. Accumulator r of lane l holds C[8*(r/4) + 4*(l/32) + r%4][l%32] of the 32x32 tile.
    double scale = 1.0;
    if (KIND != kWgrad) scale = (double)*args.a.tscale * (double)*args.b.tscale;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = 4 * m4_0 + 32 * wm + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const int n = 4 * n4_0 + 64 * wn + 32 * j + (lane & 31);
            const float c = acc[j][r];
            if (KIND == kWgrad) {
                // partial [split][m][n]; padded rows/cols are written too (the buffer covers them)
                args.out[((int64_t)blockIdx.z * (gridDim.y * BM) + m) * args.ldp + n] = c;
            } else {
                const int Mreal = (KIND == kFwd) ? g.Cout : g.Cin;
                const int nb = n % (4 * g.N4), pix = n / (4 * g.N4);
                if (m < Mreal && nb < g.N && n < 4 * args.N4c)
                    args.out[((int64_t)pix * Mreal + m) * g.N + nb] = (float)((double)c * scale);
            }
        }
    }
}

// Sum the split-K partials in split order and apply the tensor scales:
// G_W[tap][co][ci] = T_G * T_X * sum_z partial[z][co][tap*4*Cin4 + ci].
__global__ void __launch_bounds__(256) wgrad_reduce_kernel(const float *__restrict__ part,
                                                           int splits, int64_t split_stride,
                                                           int ldp, ConvGeom g, const float *ta,
                                                           const float *tb, float *__restrict__ gw)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)g.Kh * g.Kw * g.Cout * g.Cin;
    if (i >= total) return;
    const int ci = (int)(i % g.Cin);
    const int64_t r = i / g.Cin;
    const int co = (int)(r % g.Cout);
    const int tap = (int)(r / g.Cout);
    const int64_t off = (int64_t)co * ldp + (int64_t)tap * 4 * g.Cin4 + ci;
    // fixed summation order z = 0, 1, ...; loads issued 8 at a time
    float s = 0.0f;
    int z = 0;
    for (; z + 8 <= splits; z += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = part[(z + u) * split_stride + off];
#pragma unroll
        for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; z < splits; ++z) s += part[z * split_stride + off];
    gw[i] = (float)((double)s * ((double)*ta * (double)*tb));
}

// ---- launch helpers ------------------------------------------------------------------------

struct WgradPlan {
    int mtiles, ntiles, splits, k4_per_split, ldp;
    size_t bytes;
};

static WgradPlan plan_wgrad(const ConvGeom &g)
{
    WgradPlan p;
    const int M4 = g.Cout4, N4c = g.Kh * g.Kw * g.Cin4;
    const int64_t K4 = (int64_t)g.Ho * g.Wo * g.N4;
    p.mtiles = (M4 + BM / 4 - 1) / (BM / 4);
    p.ntiles = (N4c + BN / 4 - 1) / (BN / 4);
    // Enough splits to fill the GPU (~1024 workgroups) and to keep each fp32 accumulation chain
    // within 4096 products (1024 squares along K).
    const int64_t tiles = (int64_t)p.mtiles * p.ntiles;
    int64_t want = (512 + tiles - 1) / tiles;
    if (want > 64) want = 64; // partial traffic grows with the split count
    int64_t min_for_chain = (K4 + 1023) / 1024;
    if (want < min_for_chain) want = min_for_chain;
    int64_t kps = (K4 + want - 1) / want;
    kps = ((kps + BK4 - 1) / BK4) * BK4;
    if (kps < BK4) kps = BK4;
    p.k4_per_split = (int)kps;
    p.splits = (int)((K4 + kps - 1) / kps);
    p.ldp = p.ntiles * BN;
    p.bytes = (size_t)p.splits * p.mtiles * BM * p.ldp * sizeof(float);
    return p;
}

size_t wgrad_workspace_bytes(const ConvGeom &g) { return plan_wgrad(g).bytes; }

template <int KIND>
static hipError_t launch_gemm(int fmt, const GemmArgs &a, dim3 grid, hipStream_t st)
{
    if (fmt == kFP4)
        hipLaunchKernelGGL((conv_gemm_kernel<kFP4, KIND>), grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((conv_gemm_kernel<kFP6, KIND>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_conv_fwd(const ConvGeom &g, int fmt, QOperand x, QOperand w, float *y,
                           hipStream_t st)
{
    GemmArgs a;
    a.g = g; a.a = w; a.b = x; a.out = y;
    a.M4 = g.Cout4; a.N4c = g.Ho * g.Wo * g.N4; a.K4 = g.Kh * g.Kw * g.Cin4;
    a.k4_per_split = a.K4; a.ldp = 0;
    dim3 grid((a.N4c + BN / 4 - 1) / (BN / 4), (a.M4 + BM / 4 - 1) / (BM / 4), 1);
    return launch_gemm<kFwd>(fmt, a, grid, st);
}

hipError_t launch_conv_dgrad(const ConvGeom &g, int fmt, QOperand w, QOperand gy, float *gx,
                             hipStream_t st)
{
    GemmArgs a;
    a.g = g; a.a = w; a.b = gy; a.out = gx;
    a.M4 = g.Cin4; a.N4c = g.H * g.W * g.N4; a.K4 = g.Kh * g.Kw * g.Cout4;
    a.k4_per_split = a.K4; a.ldp = 0;
    dim3 grid((a.N4c + BN / 4 - 1) / (BN / 4), (a.M4 + BM / 4 - 1) / (BM / 4), 1);
    return launch_gemm<kDgrad>(fmt, a, grid, st);
}

hipError_t launch_conv_wgrad(const ConvGeom &g, int fmt, QOperand gy, QOperand x, float *gw,
                             void *ws, size_t ws_bytes, hipStream_t st)
{
    const WgradPlan p = plan_wgrad(g);
    if (ws_bytes < p.bytes) return hipErrorInvalidValue;
    GemmArgs a;
    a.g = g; a.a = gy; a.b = x; a.out = reinterpret_cast<float *>(ws);
    a.M4 = g.Cout4; a.N4c = g.Kh * g.Kw * g.Cin4; a.K4 = g.Ho * g.Wo * g.N4;
    a.k4_per_split = p.k4_per_split; a.ldp = p.ldp;
    dim3 grid(p.ntiles, p.mtiles, p.splits);
    hipError_t e = launch_gemm<kWgrad>(fmt, a, grid, st);
    if (e != hipSuccess) return e;
    const int64_t total = (int64_t)g.Kh * g.Kw * g.Cout * g.Cin;
    const int64_t split_stride = (int64_t)p.mtiles * BM * p.ldp;
    hipLaunchKernelGGL(wgrad_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       st, reinterpret_cast<const float *>(ws), p.splits, split_stride, p.ldp, g,
                       gy.tscale, x.tscale, gw);
    return hipGetLastError();
}

} // namespace mq
