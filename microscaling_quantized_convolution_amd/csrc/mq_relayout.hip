// mq_relayout.hip -- fp32 layout changes at the network boundary.
//
// Channel-batch-first activations (onedev.kr MicroQonv digest, section "How it works"): for each
// pixel all channels and all batch elements are contiguous, stored [H][W][C][N]. Per channel c
// the change NCHW <-> CBF is a transpose of an N x (H*W) matrix, done in LDS tiles so that both
// the reads and the writes are coalesced.
//
// Weights (section "How it differs", W_{fCout,Cin}): OIHW <-> [Kh][Kw][Cout][Cin].
//
// A relayout can also produce the tensor-amax partials that quantization needs (it reads every
// element anyway): each workgroup writes the max |x| of the tiles it moved, so the quantizer can
// skip its own amax pass over the tensor.
#include "mq_kernels.hpp"

namespace mq {

typedef float f32x4v __attribute__((ext_vector_type(4)));

// Transpose tiles: dst[c][b][a] = src[c][a][b]; src rows have stride src_ld, dst rows dst_ld,
// channels src_cs / dst_cs. Tiles are numbered (c, a-tile, b-tile) with the b-tile fastest and
// taken grid-stride by the workgroups.
struct TransposeArgs {
    const float *src;
    float *dst;
    int A, B;
    int64_t src_ld, dst_ld, src_cs, dst_cs;
    int tilesA, tilesB;
    int64_t ntiles;
    uint32_t *amax_ws; // null: no amax
};

__device__ __forceinline__ uint32_t abs_bits(float v) { return __float_as_uint(v) & 0x7FFFFFFFu; }

// Workgroup max of m to amax_ws[1 + blockIdx.x] (and the count to amax_ws[0]).
__device__ __forceinline__ void write_partial(uint32_t m, uint32_t *ws, uint32_t *red)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    if (lane == 0) red[wid] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = red[0];
        for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r = max(r, red[w]);
        ws[1 + blockIdx.x] = r;
        if (blockIdx.x == 0) ws[0] = gridDim.x;
    }
}

// Scalar 64 x 64 tiles (any shape).
template <bool AMAX>
__global__ void __launch_bounds__(256) transpose_kernel(TransposeArgs p)
{
    constexpr int kT = 64;
    __shared__ float tile[kT][kT + 1];
    __shared__ uint32_t red[4];
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6; // 64 x 4
    uint32_t m = 0u;
    for (int64_t t = blockIdx.x; t < p.ntiles; t += gridDim.x) {
        const int bt = (int)(t % p.tilesB);
        const int64_t rest = t / p.tilesB;
        const int at = (int)(rest % p.tilesA);
        const int c = (int)(rest / p.tilesA);
        const int a0 = at * kT, b0 = bt * kT;
        const float *s = p.src + c * p.src_cs;
        float *d = p.dst + c * p.dst_cs;
#pragma unroll
        for (int i = 0; i < kT; i += 4) {
            const int a = a0 + ty + i, b = b0 + tx;
            if (a < p.A && b < p.B) {
                const float v = __builtin_nontemporal_load(s + a * p.src_ld + b);
                tile[ty + i][tx] = v;
                if (AMAX) m = max(m, abs_bits(v));
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kT; i += 4) {
            const int b = b0 + ty + i, a = a0 + tx;
            if (a < p.A && b < p.B) d[b * p.dst_ld + a] = tile[tx][ty + i];
        }
        __syncthreads(); // the tile is reused by the next iteration
    }
    if (AMAX) write_partial(m, p.amax_ws, red);
}

// The same transpose with 16-byte global accesses on both sides, for shapes whose rows, strides
// and base addresses are multiples of 4 floats. A tile is TA rows (a) x TB columns (b), 4096
// floats; each of the 256 lanes moves four float4 in and four out. LDS rows are padded by two
// floats, which spreads the column reads of the store phase over distinct banks.
template <int TA, bool AMAX>
__global__ void __launch_bounds__(256) transpose4_kernel(TransposeArgs p)
{
    constexpr int TB = 4096 / TA, PITCH = TB + 2;
    __shared__ float tile[TA * PITCH];
    __shared__ uint32_t red[4];
    const int tid = threadIdx.x;
    uint32_t m = 0u;
    // tile t -> (channel, a0, b0)
    auto coords = [&](int64_t t, int &c, int &a0, int &b0) {
        const int bt = (int)(t % p.tilesB);
        const int64_t rest = t / p.tilesB;
        a0 = (int)(rest % p.tilesA) * TA;
        c = (int)(rest / p.tilesA);
        b0 = bt * TB;
    };
    auto load = [&](int64_t t, f32x4v (&v)[4]) {
        int c, a0, b0;
        coords(t, c, a0, b0);
        const float *s = p.src + c * p.src_cs;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int idx = tid + 256 * k, ra = idx / (TB / 4), cb = idx % (TB / 4);
            const int a = a0 + ra, b = b0 + 4 * cb;
            v[k] = (a < p.A && b < p.B) ? __builtin_nontemporal_load(
                                              reinterpret_cast<const f32x4v *>(s + a * p.src_ld + b))
                                        : f32x4v{0.f, 0.f, 0.f, 0.f};
        }
    };
    // the next tile's loads are issued as soon as this tile is in LDS, so they overlap the
    // LDS reads and global stores of this tile
    f32x4v v[4];
    int64_t t = blockIdx.x;
    if (t < p.ntiles) load(t, v);
    for (; t < p.ntiles; t += gridDim.x) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int idx = tid + 256 * k, ra = idx / (TB / 4), cb = idx % (TB / 4);
            float *tp = tile + ra * PITCH + 4 * cb;
            tp[0] = v[k][0]; tp[1] = v[k][1]; tp[2] = v[k][2]; tp[3] = v[k][3];
            if (AMAX)
                m = max(m, max(max(abs_bits(v[k][0]), abs_bits(v[k][1])),
                               max(abs_bits(v[k][2]), abs_bits(v[k][3]))));
        }
        __syncthreads();
        const int64_t tn = t + gridDim.x;
        if (tn < p.ntiles) load(tn, v);
        int c, a0, b0;
        coords(t, c, a0, b0);
        float *d = p.dst + c * p.dst_cs;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int idx = tid + 256 * k, rb = idx / (TA / 4), ca = idx % (TA / 4);
            const int b = b0 + rb, a = a0 + 4 * ca;
            const float *tp = tile + 4 * ca * PITCH + rb;
            const f32x4v o = {tp[0], tp[PITCH], tp[2 * PITCH], tp[3 * PITCH]};
            if (a < p.A && b < p.B) *reinterpret_cast<f32x4v *>(d + b * p.dst_ld + a) = o;
        }
        __syncthreads(); // the tile is reused by the next iteration
    }
    if (AMAX) write_partial(m, p.amax_ws, red);
}

template <typename K>
static void launch_tiles(K kernel, TransposeArgs &p, int C, int TA, int TB, hipStream_t st)
{
    p.tilesA = (p.A + TA - 1) / TA;
    p.tilesB = (p.B + TB - 1) / TB;
    p.ntiles = (int64_t)p.tilesA * p.tilesB * C;
    // at most kAmaxParts workgroups (one amax partial each), every one with the same number of
    // tiles so that none finishes a whole tile later than the rest
    const int64_t iters = (p.ntiles + kAmaxParts - 1) / kAmaxParts;
    const unsigned grid = (unsigned)((p.ntiles + iters - 1) / iters);
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(256), 0, st, p);
}

// Transposes with few columns (B <= 32, e.g. OIHW weights with B = Kh*Kw): lane a reads row a
// (B contiguous floats; neighbouring lanes read neighbouring rows, so a wave reads one contiguous
// span) and writes column a of dst (coalesced). No LDS.
template <bool AMAX>
__global__ void __launch_bounds__(256) rows_to_columns_kernel(TransposeArgs p)
{
    __shared__ uint32_t red[4];
    uint32_t m = 0u;
    const int64_t rows = (int64_t)p.A * p.tilesA; // tilesA holds the channel count here
    for (int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x; r < rows; r += (int64_t)gridDim.x * 256) {
        const int c = (int)(r / p.A), a = (int)(r - (int64_t)c * p.A);
        const float *s = p.src + c * p.src_cs + a * p.src_ld;
        float *d = p.dst + c * p.dst_cs + a;
        for (int b = 0; b < p.B; ++b) {
            const float v = s[b];
            d[b * p.dst_ld] = v;
            if (AMAX) m = max(m, abs_bits(v));
        }
    }
    if (AMAX) write_partial(m, p.amax_ws, red);
}

// dst[c][b][a] = src[c][a][b] for C channels.
static hipError_t launch_transpose(const float *src, float *dst, int C, int A, int B,
                                   int64_t src_ld, int64_t dst_ld, int64_t src_cs,
                                   int64_t dst_cs, uint32_t *amax_ws, hipStream_t st)
{
    TransposeArgs p;
    p.src = src; p.dst = dst; p.A = A; p.B = B;
    p.src_ld = src_ld; p.dst_ld = dst_ld; p.src_cs = src_cs; p.dst_cs = dst_cs;
    p.amax_ws = amax_ws;
    const bool am = amax_ws != nullptr;
    const bool vec = A % 4 == 0 && B % 4 == 0 && src_ld % 4 == 0 && dst_ld % 4 == 0 &&
                     src_cs % 4 == 0 && dst_cs % 4 == 0 &&
                     (reinterpret_cast<uintptr_t>(src) & 15u) == 0 &&
                     (reinterpret_cast<uintptr_t>(dst) & 15u) == 0;
    if (B <= 32 && src_ld == B) {
        // rows of B contiguous floats: one lane per row
        p.tilesA = C;
        const int64_t rows = (int64_t)A * C;
        const int64_t want = (rows + 255) / 256;
        const unsigned grid = (unsigned)(want < kAmaxParts ? want : kAmaxParts);
        if (am) hipLaunchKernelGGL(rows_to_columns_kernel<true>, dim3(grid), dim3(256), 0, st, p);
        else hipLaunchKernelGGL(rows_to_columns_kernel<false>, dim3(grid), dim3(256), 0, st, p);
    } else if (vec) {
        // tile rows: few rows -> 32 x 128 tiles, few columns -> 128 x 32, else 64 x 64
        if (A <= 32) {
            if (am) launch_tiles(transpose4_kernel<32, true>, p, C, 32, 128, st);
            else launch_tiles(transpose4_kernel<32, false>, p, C, 32, 128, st);
        } else if (B <= 32) {
            if (am) launch_tiles(transpose4_kernel<128, true>, p, C, 128, 32, st);
            else launch_tiles(transpose4_kernel<128, false>, p, C, 128, 32, st);
        } else {
            if (am) launch_tiles(transpose4_kernel<64, true>, p, C, 64, 64, st);
            else launch_tiles(transpose4_kernel<64, false>, p, C, 64, 64, st);
        }
    } else {
        if (am) launch_tiles(transpose_kernel<true>, p, C, 64, 64, st);
        else launch_tiles(transpose_kernel<false>, p, C, 64, 64, st);
    }
    return hipGetLastError();
}

hipError_t launch_relayout_cbf(const float *src, float *dst, int N, int C, int H, int W,
                               int inverse, uint32_t *amax_ws, hipStream_t st)
{
    const int64_t HW = (int64_t)H * W;
    if (!inverse) // per channel: src[n][hw] (ld C*HW) -> dst[hw][n] (ld C*N)
        return launch_transpose(src, dst, C, N, (int)HW, (int64_t)C * HW, (int64_t)C * N, HW,
                                (int64_t)N, amax_ws, st);
    // per channel: src[hw][n] (ld C*N) -> dst[n][hw] (ld C*HW)
    return launch_transpose(src, dst, C, (int)HW, N, (int64_t)C * N, (int64_t)C * HW,
                            (int64_t)N, HW, amax_ws, st);
}

hipError_t launch_relayout_weight(const float *src, float *dst, int Cout, int Cin, int Kh,
                                  int Kw, int inverse, uint32_t *amax_ws, hipStream_t st)
{
    // OIHW is a (Cout*Cin) x (Kh*Kw) matrix; tap-major is its transpose.
    const int64_t P = (int64_t)Cout * Cin;
    const int T = Kh * Kw;
    if (!inverse)
        return launch_transpose(src, dst, 1, (int)P, T, (int64_t)T, P, 0, 0, amax_ws, st);
    return launch_transpose(src, dst, 1, T, (int)P, P, (int64_t)T, 0, 0, amax_ws, st);
}

} // namespace mq
