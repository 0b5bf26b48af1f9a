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

hipError_t launch_relayout_cbf(const float *src, float *dst, int N, int C, int H, int W,
                               int inverse, hipStream_t st)
{
    const int64_t HW = (int64_t)H * W;
    if (!inverse) {
        // per channel: src[n][hw] (ld C*HW) -> dst[hw][n] (ld C*N)
        dim3 grid((unsigned)((HW + kTile - 1) / kTile), (unsigned)((N + kTile - 1) / kTile), C);
        hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, st, src, dst, N, (int)HW,
                           (int64_t)C * HW, (int64_t)C * N, HW, (int64_t)N);
    } else {
        // per channel: src[hw][n] (ld C*N) -> dst[n][hw] (ld C*HW)
        dim3 grid((unsigned)((N + kTile - 1) / kTile), (unsigned)((HW + kTile - 1) / kTile), C);
        hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, st, src, dst, (int)HW, N,
                           (int64_t)C * N, (int64_t)C * HW, (int64_t)N, HW);
    }
    return hipGetLastError();
}

hipError_t launch_relayout_weight(const float *src, float *dst, int Cout, int Cin, int Kh,
                                  int Kw, int inverse, hipStream_t st)
{
    // OIHW is a (Cout*Cin) x (Kh*Kw) matrix; tap-major is its transpose.
    const int64_t P = (int64_t)Cout * Cin;
    const int T = Kh * Kw;
    if (!inverse) {
        dim3 grid((unsigned)((T + kTile - 1) / kTile), (unsigned)((P + kTile - 1) / kTile), 1);
        hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, st, src, dst, (int)P, T,
                           (int64_t)T, P, (int64_t)0, (int64_t)0);
    } else {
        dim3 grid((unsigned)((P + kTile - 1) / kTile), (unsigned)((T + kTile - 1) / kTile), 1);
        hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, st, src, dst, T, (int)P, P,
                           (int64_t)T, (int64_t)0, (int64_t)0);
    }
    return hipGetLastError();
}

} // namespace mq
