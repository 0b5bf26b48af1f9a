// mq_wgrad_sum.hpp -- the weight gradient's deterministic split-K sum (device side).
//
// The weight-gradient kernel leaves one fp32 partial block per split; the output is
// G_W[i] = T_G * T_X * sum_{s = 0..S-1} part[s][i] (onedev.kr MicroQonv digest, section "How it
// differs": the tensor scales stay out of the GEMM and multiply its result). The sum runs in a
// fixed order, so the result does not depend on scheduling. With more than 16 splits, 256 lanes
// own a block of 64 consecutive outputs (16 float4 x 16 split groups); group g adds splits g,
// g + 16, ... in order, and the 16 group sums are added in group order. With at most 16 splits a
// block is 1024 outputs, a float4 per lane, and the lane adds the splits in order from zero: the
// same additions in the same order as the grouped sum, which would add only zeros beyond split
// S - 1 (the running sum is never -0, so those change nothing), in one round of loads. The same
// code serves the standalone sum kernel and workgroups that ride along in the input-gradient
// launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mq {

struct WgradSum {
    const float *part;     // [split][stride] fp32 partial sums
    int S;                 // splits
    int64_t stride;        // floats per split
    int64_t total;         // outputs
    const float *tg, *tx;  // tensor scales T_G, T_X
    float *out;            // G_W, `total` floats
};

// Outputs per block, and blocks of a sum.
__host__ __device__ inline int64_t wgrad_sum_block_outputs(int S) { return S <= 16 ? 1024 : 64; }
__host__ __device__ inline int64_t wgrad_sum_blocks(const WgradSum &w)
{
    const int64_t b = wgrad_sum_block_outputs(w.S);
    return (w.total + b - 1) / b;
}

// Sum the outputs of block blk (those below total) with lanes tid = 0..255 of a workgroup group;
// red is that group's 16 x 17 float4 of LDS. Every lane of the group must call it (one barrier
// inside), also with blk past the end.
__device__ __forceinline__ void wgrad_sum_block(const WgradSum &w, int64_t blk, int tid,
                                                float4 (*red)[17])
{
    if (w.S <= 16) {
        const int64_t i0 = (blk * 256 + tid) * 4; // first of the lane's four outputs
        const double sc = (double)*w.tg * (double)*w.tx;
        if ((w.total % 4 == 0) && (w.stride % 4 == 0)) {
            if (i0 < w.total) {
                float4 p[16];
#pragma unroll
                for (int z = 0; z < 16; ++z)
                    p[z] = z < w.S ? *reinterpret_cast<const float4 *>(w.part + z * w.stride + i0)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
                float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
                for (int z = 0; z < 16; ++z)
                    if (z < w.S) { t.x += p[z].x; t.y += p[z].y; t.z += p[z].z; t.w += p[z].w; }
                *reinterpret_cast<float4 *>(w.out + i0) =
                    make_float4((float)((double)t.x * sc), (float)((double)t.y * sc),
                                (float)((double)t.z * sc), (float)((double)t.w * sc));
            }
        } else {
            for (int q = 0; q < 4; ++q) {
                const int64_t i = i0 + q;
                if (i < w.total) {
                    float e = 0.f;
                    for (int z = 0; z < w.S; ++z) e += w.part[z * w.stride + i];
                    w.out[i] = (float)((double)e * sc);
                }
            }
        }
        __syncthreads();
        return;
    }
    const int v = tid & 15, g = tid >> 4;
    const int64_t i4 = blk * 16 + v; // float4 index
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    const bool vec = (w.total % 4 == 0) && (w.stride % 4 == 0);
    if (vec && i4 * 4 < w.total) {
        // eight loads in flight per batch, added in split order afterwards
        for (int z0 = g; z0 < w.S; z0 += 16 * 8) {
            float4 p[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int z = z0 + 16 * k;
                p[k] = z < w.S ? *reinterpret_cast<const float4 *>(w.part + z * w.stride + i4 * 4)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (z0 + 16 * k < w.S) { s.x += p[k].x; s.y += p[k].y; s.z += p[k].z; s.w += p[k].w; }
        }
    } else if (!vec) {
        float e[4] = {0.f, 0.f, 0.f, 0.f};
        for (int q = 0; q < 4; ++q) {
            const int64_t i = i4 * 4 + q;
            if (i < w.total)
                for (int z = g; z < w.S; z += 16) e[q] += w.part[z * w.stride + i];
        }
        s = make_float4(e[0], e[1], e[2], e[3]);
    }
    red[g][v] = s;
    __syncthreads();
    if (g == 0) {
        float4 t = red[0][v];
        for (int q = 1; q < 16; ++q) {
            const float4 p = red[q][v];
            t.x += p.x; t.y += p.y; t.z += p.z; t.w += p.w;
        }
        const double sc = (double)*w.tg * (double)*w.tx;
        const float r[4] = {t.x, t.y, t.z, t.w};
        for (int q = 0; q < 4; ++q) {
            const int64_t i = i4 * 4 + q;
            if (i < w.total) w.out[i] = (float)((double)r[q] * sc);
        }
    }
}

} // namespace mq
