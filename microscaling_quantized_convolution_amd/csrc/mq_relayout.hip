// mq_relayout.hip -- fp32 layout changes at the network boundary.
//
// Channel-batch-first activations (onedev.kr MicroQonv digest, section "How it works"): for each
// pixel all channels and all batch elements are contiguous, stored [H][W][C][N]. Per channel c
// the change NCHW <-> CBF is a transpose of an N x (H*W) matrix, done in 64x64 LDS tiles so that
// both the reads and the writes are coalesced.
//
// Weights (section "How it differs", W_{fCout,Cin}): OIHW <-> [Kh][Kw][Cout][Cin].
#include "mq_kernels.hpp"

namespace mq {

constexpr int kTile = 64;
typedef float f32x4v __attribute__((ext_vector_type(4)));

// dst[b][a] = src[a][b] for one channel: src is A x B with row stride src_ld, dst is B x A with
// row stride dst_ld; channel c offsets src by c*src_cs and dst by c*dst_cs.
__global__ void __launch_bounds__(256) transpose_kernel(const float *__restrict__ src,
                                                        float *__restrict__ dst, int A, int B,
                                                        int64_t src_ld, int64_t dst_ld,
                                                        int64_t src_cs, int64_t dst_cs)
{
    __shared__ float tile[kTile][kTile + 1];
    const int c = blockIdx.z;
    const int a0 = blockIdx.y * kTile, b0 = blockIdx.x * kTile;
    const float *s = src + c * src_cs;
    float *d = dst + c * dst_cs;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6; // 64 x 4
#pragma unroll
    for (int i = 0; i < kTile; i += 4) {
        int a = a0 + ty + i, b = b0 + tx;
        if (a < A && b < B) tile[ty + i][tx] = __builtin_nontemporal_load(s + a * src_ld + b);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kTile; i += 4) {
        int b = b0 + ty + i, a = a0 + tx;
        if (a < A && b < B) d[b * dst_ld + a] = tile[tx][ty + i];
    }
}

// The same transpose with 16-byte global accesses on both sides, for shapes whose rows, strides
// and base addresses are multiples of 4 floats. A tile is TA rows (a) x TB columns (b), 4096
// floats; each of the 256 lanes moves four float4 in and four out. LDS rows are padded by two
// floats, which spreads the column reads of the store phase over distinct banks.
template <int TA>
__global__ void __launch_bounds__(256) transpose4_kernel(const float *__restrict__ src,
                                                         float *__restrict__ dst, int A, int B,
                                                         int64_t src_ld, int64_t dst_ld,
                                                         int64_t src_cs, int64_t dst_cs)
{
    constexpr int TB = 4096 / TA, PITCH = TB + 2;
    __shared__ float tile[TA * PITCH];
    const int c = blockIdx.z;
    const int a0 = blockIdx.y * TA, b0 = blockIdx.x * TB;
    const float *s = src + c * src_cs;
    float *d = dst + c * dst_cs;
    const int tid = threadIdx.x;
    f32x4v v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int idx = tid + 256 * k, ra = idx / (TB / 4), cb = idx % (TB / 4);
        const int a = a0 + ra, b = b0 + 4 * cb;
        v[k] = (a < A && b < B)
                   ? __builtin_nontemporal_load(reinterpret_cast<const f32x4v *>(s + a * src_ld + b))
                   : f32x4v{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int idx = tid + 256 * k, ra = idx / (TB / 4), cb = idx % (TB / 4);
        float *t = tile + ra * PITCH + 4 * cb;
        t[0] = v[k][0]; t[1] = v[k][1]; t[2] = v[k][2]; t[3] = v[k][3];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int idx = tid + 256 * k, rb = idx / (TA / 4), ca = idx % (TA / 4);
        const int b = b0 + rb, a = a0 + 4 * ca;
        const float *t = tile + 4 * ca * PITCH + rb;
        const f32x4v o = {t[0], t[PITCH], t[2 * PITCH], t[3 * PITCH]};
        if (a < A && b < B) *reinterpret_cast<f32x4v *>(d + b * dst_ld + a) = o;
    }
}

// dst[c][b][a] = src[c][a][b] for C channels (strides as in transpose_kernel).
static hipError_t launch_transpose(const float *src, float *dst, int C, int A, int B,
                                   int64_t src_ld, int64_t dst_ld, int64_t src_cs,
                                   int64_t dst_cs, hipStream_t st)
{
    const bool vec = A % 4 == 0 && B % 4 == 0 && src_ld % 4 == 0 && dst_ld % 4 == 0 &&
                     src_cs % 4 == 0 && dst_cs % 4 == 0 &&
                     (reinterpret_cast<uintptr_t>(src) & 15u) == 0 &&
                     (reinterpret_cast<uintptr_t>(dst) & 15u) == 0;
    if (vec) {
        // tile rows: few rows -> 32 x 128 tiles, few columns -> 128 x 32, else 64 x 64
        if (A <= 32) {
            dim3 grid((unsigned)((B + 127) / 128), (unsigned)((A + 31) / 32), (unsigned)C);
            hipLaunchKernelGGL((transpose4_kernel<32>), grid, dim3(256), 0, st, src, dst, A, B,
                               src_ld, dst_ld, src_cs, dst_cs);
        } else if (B <= 32) {
            dim3 grid((unsigned)((B + 31) / 32), (unsigned)((A + 127) / 128), (unsigned)C);
            hipLaunchKernelGGL((transpose4_kernel<128>), grid, dim3(256), 0, st, src, dst, A, B,
                               src_ld, dst_ld, src_cs, dst_cs);
        } else {
            dim3 grid((unsigned)((B + 63) / 64), (unsigned)((A + 63) / 64), (unsigned)C);
            hipLaunchKernelGGL((transpose4_kernel<64>), grid, dim3(256), 0, st, src, dst, A, B,
                               src_ld, dst_ld, src_cs, dst_cs);
        }
    } else {
        dim3 grid((unsigned)((B + kTile - 1) / kTile), (unsigned)((A + kTile - 1) / kTile),
                  (unsigned)C);
        hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, st, src, dst, A, B, src_ld,
                           dst_ld, src_cs, dst_cs);
    }
    return hipGetLastError();
}

hipError_t launch_relayout_cbf(const float *src, float *dst, int N, int C, int H, int W,
                               int inverse, hipStream_t st)
{
    const int64_t HW = (int64_t)H * W;
    if (!inverse) // per channel: src[n][hw] (ld C*HW) -> dst[hw][n] (ld C*N)
        return launch_transpose(src, dst, C, N, (int)HW, (int64_t)C * HW, (int64_t)C * N, HW,
                                (int64_t)N, st);
    // per channel: src[hw][n] (ld C*N) -> dst[n][hw] (ld C*HW)
    return launch_transpose(src, dst, C, (int)HW, N, (int64_t)C * N, (int64_t)C * HW,
                            (int64_t)N, HW, st);
}

hipError_t launch_relayout_weight(const float *src, float *dst, int Cout, int Cin, int Kh,
                                  int Kw, int inverse, hipStream_t st)
{
    // OIHW is a (Cout*Cin) x (Kh*Kw) matrix; tap-major is its transpose.
    const int64_t P = (int64_t)Cout * Cin;
    const int T = Kh * Kw;
    if (!inverse)
        return launch_transpose(src, dst, 1, (int)P, T, (int64_t)T, P, 0, 0, st);
    return launch_transpose(src, dst, 1, T, (int)P, P, (int64_t)T, 0, 0, st);
}

} // namespace mq
