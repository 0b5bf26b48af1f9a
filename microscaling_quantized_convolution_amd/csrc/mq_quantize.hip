// mq_quantize.hip -- tensor amax and square-block quantization (NVFP4 / NVFP6).
//
// Implements the quantizer of the onedev.kr MicroQonv digest, section "How it differs":
//   T = amax / (448 * Emax); per 4x4 square B = CastE4M3(max|x_i| / (T * Emax));
//   element code = Round(x_i / (B * T)), nearest-even for weights/activations, stochastic for
//   gradients. Each tensor is quantized once; the square shares its scale along 4 elements in
//   both of its dimensions, so the same codes serve the GEMMs that reduce along either one.
//
// Two kernels per tensor: amax (grid-stride max of |x| as uint bit patterns, one partial maximum
// per workgroup) and quantize (each workgroup first reduces the partial maxima to the tensor's
// amax, then one lane per 4x4 square). No atomics and no memset: the workspace holds the number
// of partials in word 0 and the partials after it, all written by the pass that produces them
// (this amax kernel, or a relayout that already moved the tensor, which then saves a full read).
#include "mq_device.hpp"
#include "mq_kernels.hpp"
#include "mq_stage.hpp"

namespace mq {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Max over |x| as unsigned bit patterns: for non-negative floats the order of the bit patterns
// is the numeric order, and NaN patterns sort above +inf, so a NaN anywhere wins.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
    return v;
}

__device__ __forceinline__ uint32_t absmax4(u32x4_t v)
{
    return max(max(v[0] & 0x7FFFFFFFu, v[1] & 0x7FFFFFFFu), max(v[2] & 0x7FFFFFFFu, v[3] & 0x7FFFFFFFu));
}

// Maximum over the 64-lane waves of a workgroup of kThreads lanes (every lane gets it).
template <int kThreads>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t *red)
{
    v = wave_max_u32(v);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    if (lane == 0) red[wid] = v;
    __syncthreads();
    uint32_t r = red[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) r = max(r, red[w]);
    return r;
}

// 1024-lane workgroups with eight 16-byte loads per lane in flight (measured faster than 256 or
// 512 lanes, or 4 or 16 loads, on 26 MB and 103 MB tensors)
constexpr int kAmaxThreads = 1024;
constexpr int kAmaxVec = 8;
constexpr int64_t kQuantBlocks = 1024;

// Partial maxima: workgroup b of P writes max |x| over its grid-stride share to ws[1 + b]; ws[0]
// is P. Eight independent 16-byte loads per lane are in flight at a time, enough to cover HBM
// latency.
__device__ __forceinline__ void amax_body(const float *__restrict__ x, int64_t n,
                                          uint32_t *__restrict__ ws, int b, int P, uint32_t *red)
{
    uint32_t m = 0u;
    const int64_t nt = (int64_t)P * kAmaxThreads;
    const int64_t i = (int64_t)b * kAmaxThreads + threadIdx.x;
    int64_t tail = 0;
    if ((reinterpret_cast<uintptr_t>(x) & 15u) == 0) {
        const int64_t n4 = n >> 2;
        const u32x4_t *x4 = reinterpret_cast<const u32x4_t *>(x);
        // groups of kAmaxVec loads, the last one predicated, so that every load of a group is
        // in flight at once (a lane with fewer loads than a group still pays one round trip)
        for (int64_t j = i; j < n4; j += kAmaxVec * nt) {
            u32x4_t v[kAmaxVec];
#pragma unroll
            for (int k = 0; k < kAmaxVec; ++k) {
                const int64_t jk = j + k * nt;
                v[k] = jk < n4 ? x4[jk] : u32x4_t{0u, 0u, 0u, 0u}; // cached: quantize reads x next
            }
#pragma unroll
            for (int k = 0; k < kAmaxVec; ++k) m = max(m, absmax4(v[k]));
        }
        tail = n4 << 2;
    }
    for (int64_t j = tail + i; j < n; j += nt) m = max(m, __float_as_uint(x[j]) & 0x7FFFFFFFu);
    m = block_max_u32<kAmaxThreads>(m, red);
    if (threadIdx.x == 0) {
        ws[1 + b] = m;
        if (b == 0) ws[0] = (uint32_t)P;
    }
}

__global__ void __launch_bounds__(kAmaxThreads) amax_kernel(const float *__restrict__ x, int64_t n,
                                                            uint32_t *__restrict__ ws)
{
    __shared__ uint32_t red[kAmaxThreads / 64];
    amax_body(x, n, ws, (int)blockIdx.x, (int)gridDim.x, red);
}

// Workgroups of a pass: at least one, at most kAmaxParts, about kAmaxVec 16-byte loads per lane.
inline int amax_parts(int64_t n)
{
    const int64_t want = (n / 4 + kAmaxVec * kAmaxThreads - 1) / (kAmaxVec * kAmaxThreads);
    return (int)(want < 1 ? 1 : (want > kAmaxParts ? kAmaxParts : want));
}

hipError_t launch_amax(const float *x, int64_t n, uint32_t *ws, hipStream_t st)
{
    hipLaunchKernelGGL(amax_kernel, dim3((unsigned)amax_parts(n)), dim3(kAmaxThreads), 0, st, x, n, ws);
    return hipGetLastError();
}

struct QuantArgs {
    const float *src;
    uint8_t *codes;
    uint8_t *scales;
    float *tscale;
    const uint32_t *amax_ws;   // [0]: count P <= kAmaxParts, [1..P]: partial maxima of |x| bits
    int64_t planes; // o0 * o1
    int32_t R, S, R4, S4;
    int64_t nsq;
    uint32_t seed_lo, seed_hi;
};

// Round-to-nearest-even grid codes of 16 finite quotients q (sign | magnitude, packed as stored:
// NVFP4 element e in nibble e of w[0..1], NVFP6 element e at bits 6e .. 6e+5 of w[0..2]). The
// gfx950 conversions with scale 1.0 round to nearest, ties to even, and saturate at the largest
// element (6 or 7.5): the same codes as grid_rne with the sign of q, for every finite fp32 input
// of either sign (checked exhaustively on the device).
template <int FMT>
__device__ __forceinline__ void pack_rne(const float (&q)[16], uint32_t (&w)[3])
{
    if constexpr (FMT == kFP4) {
        // byte k of a word: element 2k in the low nibble, 2k + 1 in the high one
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint32_t v = 0u;
            v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, q[8 * h + 0], q[8 * h + 1], 1.0f, 0);
            v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, q[8 * h + 2], q[8 * h + 3], 1.0f, 1);
            v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, q[8 * h + 4], q[8 * h + 5], 1.0f, 2);
            v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, q[8 * h + 6], q[8 * h + 7], 1.0f, 3);
            w[h] = v;
        }
        w[2] = 0u;
    } else {
        // The 32-value conversion puts a[i] in 6-bit field 2i and b[i] in field 2i + 1: even
        // elements in a, odd ones in b give the fields in element order (fields 16..31, from
        // the zero upper halves, are dropped). Its result may not overlap its sources while it
        // runs, hence the early-clobber output.
        typedef float f32x16_v __attribute__((ext_vector_type(16)));
        typedef uint32_t u32x6_v __attribute__((ext_vector_type(6)));
        f32x16_v a, b;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[i] = q[2 * i];
            b[i] = q[2 * i + 1];
            a[8 + i] = 0.0f;
            b[8 + i] = 0.0f;
        }
        u32x6_v v;
        asm("v_cvt_scalef32_2xpk16_fp6_f32 %0, %1, %2, 1.0" : "=&v"(v) : "v"(a), "v"(b));
        w[0] = v[0]; w[1] = v[1]; w[2] = v[2];
    }
}

// Pack 16 codes (sign | magnitude) as stored, the layout of pack_rne.
template <int FMT>
__device__ __forceinline__ void pack_codes(const uint32_t (&code)[16], uint32_t (&w)[3])
{
    w[0] = w[1] = w[2] = 0u;
    if (FMT == kFP4) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            w[0] |= code[e] << (4 * e);
            w[1] |= code[e + 8] << (4 * e);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int bit = 6 * e;
            w[bit >> 5] |= code[e] << (bit & 31);
            if ((bit & 31) > 26) w[(bit >> 5) + 1] |= code[e] >> (32 - (bit & 31));
        }
    }
}

// One square: 16 values in row-major order (slots outside the tensor hold +0, which always gets
// code 0) -> the E4M3 scale byte (returned) and the square's packed codes w (8 bytes NVFP4,
// 12 bytes NVFP6). T is the tensor scale; nonfinite: the tensor amax is Inf or NaN (scale 0x7F,
// codes 0). r0, r1: the square's Philox draws (SR only).
template <int FMT, bool SR>
__device__ __forceinline__ uint32_t quantize_square(const float (&x)[16], float T, bool nonfinite,
                                                    const Philox4 &r0, const Philox4 &r1,
                                                    uint32_t (&w)[3])
{
    using F = Fmt<FMT>;
    uint32_t bcode;
    if (nonfinite) {
        bcode = 0x7Fu;
        w[0] = w[1] = w[2] = 0u;
    } else {
        float bmax = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) bmax = fmaxf(bmax, fabsf(x[e]));
        const float TE = T * F::kEmax;
        // T == 0 only for an all-zero (or vanishingly small) tensor: scales 0, codes 0.
        bcode = (T == 0.0f) ? 0u : e4m3_rne_sat(bmax / TE);
        const float B = e4m3_to_float(bcode);
        const float D = B * T;
        const bool zero = (bcode == 0u) || (D == 0.0f);
        // x / D for 16 elements from one reciprocal: with rD = RN(1/D), q0 = RN(x * rD) and the
        // exact residual x - q0 * D, RN(q0 + residual * rD) is the correctly rounded quotient
        // (Markstein's theorem) as long as nothing underflows: D within 2^+-64 and
        // |x / D| >= 2^-20 (or x = 0). A square with any other element divides instead under
        // stochastic rounding, where a tiny quotient's code depends on its exact value (the
        // round-up draw). Nearest rounding sends every |q| below 2^-20 to a zero code of q's
        // sign, which the reciprocal form keeps, so there only D's range is checked.
        float q[16];
        if (SR) {
            // Only |q| is used (the code's sign is x's), and a zero scale's codes are cleared
            // below whatever q holds, so the reciprocal form runs for those squares too.
            const float rD = 1.0f / D;
            const float Dlo = D * 0x1p-20f;
            // some 0 < |x| < Dlo: on the bit patterns shifted left once (sign dropped), 2|x|-2
            // wraps for |x| = 0, so its minimum over the square is below 2Dlo-2 exactly then
            uint32_t mn = 0xFFFFFFFFu;
#pragma unroll
            for (int e = 0; e < 16; ++e) mn = min(mn, (__float_as_uint(x[e]) << 1) - 2u);
            const bool slow = !(D >= 0x1p-64f && D <= 0x1p64f) || mn < (__float_as_uint(Dlo) << 1) - 2u;
            if (slow && !zero) {
#pragma unroll
                for (int e = 0; e < 16; ++e) q[e] = x[e] / D; // IEEE division
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float q0 = x[e] * rD;
                    q[e] = __builtin_fmaf(__builtin_fmaf(-q0, D, x[e]), rD, q0);
                }
            }
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) q[e] = 0.0f; // zero scale: +0 codes
            if (!zero) {
                const float rD = 1.0f / D;
                if (!(D >= 0x1p-64f && D <= 0x1p64f)) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) q[e] = x[e] / D; // IEEE division
                } else {
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const float q0 = x[e] * rD;
                        // x = -0 leaves q0 = -0 and a +0 residual, whose sum is +0: the sign of
                        // x is put back (for every other x the quotient already carries it), so
                        // that nearest rounding keeps the code's sign bit equal to x's
                        q[e] = __builtin_copysignf(
                            __builtin_fmaf(__builtin_fmaf(-q0, D, x[e]), rD, q0), x[e]);
                    }
                }
            }
        }
        if (SR) {
            uint32_t code[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const uint32_t rw = (e < 8) ? r0.v[(e & 7) >> 1] : r1.v[(e & 7) >> 1];
                const uint32_t u16 = (rw >> (16 * (e & 1))) & 0xFFFFu;
                const uint32_t c = grid_sr<FMT>(fabsf(q[e]), u16) |
                                   ((__float_as_uint(x[e]) >> 31) ? F::kSign : 0u);
                code[e] = zero ? 0u : c; // a zero scale holds +0 codes
            }
            pack_codes<FMT>(code, w);
        } else {
            pack_rne<FMT>(q, w);
        }
    }
    return bcode;
}

// Store square t's packed codes: 8 bytes (NVFP4) or 12 bytes (NVFP6).
template <int FMT>
__device__ __forceinline__ void store_square_codes(uint8_t *codes, int64_t t, const uint32_t (&w)[3])
{
    if (FMT == kFP4) {
        *reinterpret_cast<uint2 *>(codes + 8 * t) = make_uint2(w[0], w[1]);
    } else {
        uint32_t *dst = reinterpret_cast<uint32_t *>(codes + 12 * t);
        dst[0] = w[0]; dst[1] = w[1]; dst[2] = w[2];
    }
}

// One lane per 4x4 square. FULL = every square lies entirely inside [R][S] and S % 4 == 0, so
// the four rows are aligned float4 loads. OIHW: the source is a weight in OIHW order (plane =
// kh*Kw + kw, R = Cout, S = Cin): element (plane, r, s) is read from src[(r*S + s)*planes +
// plane], so the tap-major fp32 copy is never written.
// Tensor scale T from the partial maxima in ws (every lane of a 256-lane workgroup takes part),
// in two halves: the loads, issued before a lane loads its squares, and the reduction. Vector
// loads complete in issue order, so partial maxima loaded after the squares would hold the
// reduction (and every square's arithmetic) until the lane's last square load had landed. Every
// one of the kAmaxParts words is loaded (the workspace always holds them) and the count masks
// the unused ones afterwards, so no load waits for another.
struct TScaleIn {
    uint32_t np;
    uint32_t v[kAmaxParts / 256];
};

__device__ __forceinline__ TScaleIn load_tscale_in(const uint32_t *ws)
{
    TScaleIn in;
    in.np = ws[0];
#pragma unroll
    for (int k = 0; k < kAmaxParts / 256; ++k) in.v[k] = ws[1 + threadIdx.x + 256u * k];
    return in;
}

template <int FMT>
__device__ __forceinline__ float tensor_scale(const TScaleIn &in, uint32_t *red, bool &nonfinite)
{
    const uint32_t np = min(in.np, (uint32_t)kAmaxParts);
    uint32_t pm = 0u;
#pragma unroll
    for (int k = 0; k < kAmaxParts / 256; ++k) {
        const uint32_t i = threadIdx.x + 256u * k;
        pm = max(pm, i < np ? in.v[k] : 0u);
    }
    const uint32_t abits = block_max_u32<256>(pm, red);
    nonfinite = abits >= 0x7F800000u;
    return __uint_as_float(abits) / (448.0f * Fmt<FMT>::kEmax);
}

__device__ __forceinline__ void store_tscale(float *tscale, float T, bool nonfinite)
{
    *tscale = nonfinite ? __uint_as_float(0x7FC00000u) : T;
}

template <bool OIHW> constexpr int kCbfLanes = OIHW ? 64 : 256;

// Squares of one tensor, grid-stride over the P workgroups of the pass (this is workgroup b).
// The lane's first square is loaded before the tensor scale is reduced (the two do not depend
// on each other), so their memory round trips overlap; workgroup 0 stores T.
template <int FMT, bool SR, bool FULL, bool OIHW>
__device__ __forceinline__ void cbf_body(const QuantArgs &a, uint32_t *red, int b, int P)
{
    // square indices fit in 31 bits (checked at launch). A gathering (OIHW) pass uses 64 lanes
    // per workgroup: its loads are scattered, which the per-CU memory pipeline serves a few
    // lanes at a time, so its squares are spread over four times as many workgroups.
    constexpr int LANES = kCbfLanes<OIHW>;
    const int nsq = (int)a.nsq;
    const int t0 = b * LANES + (int)threadIdx.x;
    const bool active = (int)threadIdx.x < LANES && t0 < nsq;
    const int tl = active ? t0 : 0; // an idle lane loads square 0 and never uses it
    const int stride = P * LANES;

    // Square t = (plane * R4 + r4) * S4 + s4, stepped by `stride` with carries instead of
    // divisions: the step is (dp, dr, ds) in the same mixed radix.
    struct Pos { int plane, r4, s4; };
    const int ds = stride % a.S4, dr = (stride / a.S4) % a.R4, dp = stride / a.S4 / a.R4;
    auto advance = [&](Pos p) {
        p.s4 += ds;
        const int c1 = p.s4 >= a.S4;
        p.s4 -= c1 ? a.S4 : 0;
        p.r4 += dr + c1;
        const int c2 = p.r4 >= a.R4;
        p.r4 -= c2 ? a.R4 : 0;
        p.plane += dp + c2;
        return p;
    };
    // Square p's 16 elements, row-major; slots outside [R][S] read as 0.
    auto load = [&](Pos p, float (&x)[16]) {
        const int s4 = p.s4, r4 = p.r4;
        const int64_t base = ((int64_t)p.plane * a.R + 4 * r4) * (int64_t)a.S + 4 * s4;
        if (OIHW) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 4 * r4 + i, c = 4 * s4 + j;
                    const bool in = r < a.R && c < a.S;
                    x[4 * i + j] = in ? a.src[((int64_t)r * a.S + c) * a.planes + p.plane] : 0.0f;
                }
        } else if (FULL) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f32x4_t v = __builtin_nontemporal_load(
                    reinterpret_cast<const f32x4_t *>(a.src + base + (int64_t)i * a.S));
                x[4 * i + 0] = v[0]; x[4 * i + 1] = v[1]; x[4 * i + 2] = v[2]; x[4 * i + 3] = v[3];
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    bool in = (4 * r4 + i < a.R) && (4 * s4 + j < a.S);
                    x[4 * i + j] = in ? a.src[base + (int64_t)i * a.S + j] : 0.0f;
                }
        }
    };

    // Grid-stride over squares with the next square's loads in flight while this one is
    // quantized (the last step reloads its own square, so every step issues the same loads).
    Pos pos = {tl / a.S4 / a.R4, (tl / a.S4) % a.R4, tl % a.S4};
    const TScaleIn tin = load_tscale_in(a.amax_ws);
    float xn[16];
    load(pos, xn);
    bool nonfinite;
    const float T = tensor_scale<FMT>(tin, red, nonfinite);
    if (b == 0 && threadIdx.x == 0) store_tscale(a.tscale, T, nonfinite);
    if (!active) return;
    if constexpr (OIHW) {
        // one or a few squares per lane: no prefetch (a reload of the last square would double
        // the scattered loads)
        for (int t = t0;;) {
            Philox4 r0 = {}, r1 = {};
            if (SR) {
                const uint64_t j = 2u * (uint64_t)t;
                r0 = philox4x32_10((uint32_t)j, (uint32_t)(j >> 32), 0u, 0u, a.seed_lo, a.seed_hi);
                r1 = philox4x32_10((uint32_t)(j + 1), (uint32_t)((j + 1) >> 32), 0u, 0u,
                                   a.seed_lo, a.seed_hi);
            }
            uint32_t w[3];
            const uint32_t bcode = quantize_square<FMT, SR>(xn, T, nonfinite, r0, r1, w);
            a.scales[t] = (uint8_t)bcode;
            store_square_codes<FMT>(a.codes, t, w);
            t += stride;
            if (t >= nsq) break;
            pos = advance(pos);
            load(pos, xn);
        }
        return;
    }
    // One step: quantize square t from x while the next square's loads go into xnext. The
    // loop is unrolled by two so that the two register sets trade roles instead of being copied.
    auto step = [&](int t, const float (&x)[16], float (&xnext)[16]) {
        const bool more = t + stride < nsq;
        if (more) pos = advance(pos);
        load(pos, xnext); // the last step reloads its own square
        // The square's random bits do not depend on its values: drawn here, the Philox rounds
        // run while the square's loads are still in flight.
        Philox4 r0 = {}, r1 = {};
        if (SR) {
            const uint64_t j = 2u * (uint64_t)t;
            r0 = philox4x32_10((uint32_t)j, (uint32_t)(j >> 32), 0u, 0u, a.seed_lo, a.seed_hi);
            r1 = philox4x32_10((uint32_t)(j + 1), (uint32_t)((j + 1) >> 32), 0u, 0u, a.seed_lo,
                               a.seed_hi);
        }
        uint32_t w[3];
        const uint32_t bcode = quantize_square<FMT, SR>(x, T, nonfinite, r0, r1, w);
        a.scales[t] = (uint8_t)bcode;
        store_square_codes<FMT>(a.codes, t, w);
    };
    float xm[16];
    for (int t = t0; t < nsq; t += 2 * stride) {
        step(t, xn, xm);
        if (t + stride >= nsq) break;
        step(t + stride, xm, xn);
    }
}

template <int FMT, bool SR, bool FULL, bool OIHW = false>
__global__ void __launch_bounds__(256) quantize_kernel(QuantArgs a)
{
    warm_kernel_args<QuantArgs>();
    __shared__ uint32_t red[4];
    cbf_body<FMT, SR, FULL, OIHW>(a, red, (int)blockIdx.x, (int)gridDim.x);
}

template <int FMT, bool SR>
static hipError_t launch_quant(const QuantArgs &a, bool full, hipStream_t st)
{
    // a few grid-stride steps per lane (4 workgroups of 256 lanes per CU) when the tensor is big
    const int64_t want = (a.nsq + 255) / 256;
    const unsigned blocks = (unsigned)(want < kQuantBlocks ? want : kQuantBlocks);
    if (full)
        hipLaunchKernelGGL((quantize_kernel<FMT, SR, true>), dim3(blocks), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((quantize_kernel<FMT, SR, false>), dim3(blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

// ---- NCHW fp32 straight to quantized channel-batch-first squares ----
//
// The same codes, scales and T as the NCHW -> [H][W][C][N] relayout followed by quantize_kernel,
// without the fp32 channel-batch-first copy: square t = ((p*C4 + c4)*N4 + n4) of pixel p holds
// x[4*n4 + j][4*c4 + i][p] at element 4i + j. A lane owns one pixel and NQ consecutive batch
// squares of one channel square; a wave covers 64 consecutive pixels, so each load instruction
// reads 256 contiguous bytes of one (n, c) plane, and the lane's NQ squares (NQ*8 or NQ*12 code
// bytes, NQ scale bytes) are contiguous in the output. Waves are ordered batch group fastest,
// then channel square, so the four waves of a workgroup complete whole output lines.
struct QuantNchwArgs {
    const float *src;        // [N][C][HW]
    uint8_t *codes, *scales;
    float *tscale;
    const uint32_t *amax_ws; // partial maxima of this tensor
    int N, C, HW, C4, N4, NG; // NG = N4 / NQ batch-square groups
    int items;                // waves of work: ceil(HW/64) * C4 * NG
    uint32_t bytes;           // N*C*HW*4 (below 2^31)
    uint32_t seed_lo, seed_hi;
};

template <int FMT, int NQ>
__device__ __forceinline__ void store_group(const QuantNchwArgs &a, int t0, const uint32_t (&w)[NQ][3],
                                            const uint32_t (&bc)[NQ])
{
    if constexpr (NQ % 4 == 0) {
        // t0 is a multiple of 4: per four squares 32 (NVFP4) or 48 (NVFP6) aligned code bytes
        // and one scale word
#pragma unroll
        for (int g = 0; g < NQ / 4; ++g) {
            const int b = 4 * g;
            uint4 *dst = reinterpret_cast<uint4 *>(a.codes + (FMT == kFP4 ? 8 : 12) * (int64_t)(t0 + b));
            if (FMT == kFP4) {
                dst[0] = make_uint4(w[b][0], w[b][1], w[b + 1][0], w[b + 1][1]);
                dst[1] = make_uint4(w[b + 2][0], w[b + 2][1], w[b + 3][0], w[b + 3][1]);
            } else {
                dst[0] = make_uint4(w[b][0], w[b][1], w[b][2], w[b + 1][0]);
                dst[1] = make_uint4(w[b + 1][1], w[b + 1][2], w[b + 2][0], w[b + 2][1]);
                dst[2] = make_uint4(w[b + 2][2], w[b + 3][0], w[b + 3][1], w[b + 3][2]);
            }
            *reinterpret_cast<uint32_t *>(a.scales + t0 + b) =
                bc[b] | (bc[b + 1] << 8) | (bc[b + 2] << 16) | (bc[b + 3] << 24);
        }
    } else {
#pragma unroll
        for (int k = 0; k < NQ; ++k) {
            store_square_codes<FMT>(a.codes, t0 + k, w[k]);
            a.scales[t0 + k] = (uint8_t)bc[k];
        }
    }
}

template <int PX> struct PixelLoad;
template <> struct PixelLoad<1> {
    static __device__ __forceinline__ void get(rsrc_t r, uint32_t v, uint32_t s, float (&o)[1])
    {
        o[0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)v, (int)s, 0));
    }
};
template <> struct PixelLoad<2> {
    static __device__ __forceinline__ void get(rsrc_t r, uint32_t v, uint32_t s, float (&o)[2])
    {
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        const u32x2_t t = __builtin_amdgcn_raw_buffer_load_b64(r, (int)v, (int)s, 0);
        o[0] = __uint_as_float(t[0]); o[1] = __uint_as_float(t[1]);
    }
};
template <> struct PixelLoad<4> {
    static __device__ __forceinline__ void get(rsrc_t r, uint32_t v, uint32_t s, float (&o)[4])
    {
        const u32x4_t t = __builtin_amdgcn_raw_buffer_load_b128(r, (int)v, (int)s, 0);
        o[0] = __uint_as_float(t[0]); o[1] = __uint_as_float(t[1]);
        o[2] = __uint_as_float(t[2]); o[3] = __uint_as_float(t[3]);
    }
};

// PX: consecutive pixels per lane, read as one PX-float load per (n, c) plane (H*W a multiple
// of PX and the source PX*4-byte aligned, so a lane's pixels are all inside or all past H*W).
// The lane's loads are issued before the tensor scale is reduced (their round trips overlap);
// workgroup 0 stores T.
template <int FMT, bool SR, int NQ, int PX>
__device__ __forceinline__ void nchw_body(const QuantNchwArgs &a, uint32_t *red, int b)
{
    const int witem = wave_uniform(b * 4 + (int)(threadIdx.x >> 6));
    const bool act = witem < a.items; // an idle wave loads nothing (out-of-range offsets)
    const int item = act ? witem : 0;
    const int lane = threadIdx.x & 63;
    const int ng = item % a.NG, c4 = (item / a.NG) % a.C4, pb = item / a.NG / a.C4;
    const int p = (pb * 64 + lane) * PX;
    const bool pin = p < a.HW;
    // lane offset of element (n, c) = (4*ng*NQ, 4*c4); the others add a wave-uniform offset.
    // Rows n >= N lie past the end of the tensor and read as zero through the range check;
    // channels c >= C and pixels past HW are masked to an out-of-range offset.
    const rsrc_t src = make_rsrc(a.src, a.bytes);
    const uint32_t CHW4 = (uint32_t)a.C * (uint32_t)a.HW * 4u, HW4 = (uint32_t)a.HW * 4u;
    const uint32_t lane_off = (uint32_t)(4 * ng * NQ) * CHW4 + (uint32_t)(4 * c4) * HW4 + 4u * (uint32_t)p;
    const TScaleIn tin = load_tscale_in(a.amax_ws);
    // square by square, so that the first square's arithmetic can start while the later
    // squares' loads are still in flight
    float x[PX][NQ][16];
#pragma unroll
    for (int k = 0; k < NQ; ++k) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool cin = 4 * c4 + i < a.C;
            const uint32_t voff = (act && pin && cin) ? lane_off : kBad;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float v[PX];
                PixelLoad<PX>::get(src, voff, (uint32_t)(4 * k + j) * CHW4 + (uint32_t)i * HW4, v);
#pragma unroll
                for (int q = 0; q < PX; ++q) x[q][k][4 * i + j] = v[q];
            }
        }
        __builtin_amdgcn_sched_barrier(0); // keep the squares' loads in this order
    }
    bool nonfinite;
    const float T = tensor_scale<FMT>(tin, red, nonfinite);
    if (b == 0 && threadIdx.x == 0) store_tscale(a.tscale, T, nonfinite);
    if (!act || !pin) return;
#pragma unroll
    for (int q = 0; q < PX; ++q) {
        const int t0 = ((p + q) * a.C4 + c4) * a.N4 + ng * NQ; // square indices fit in 31 bits
        uint32_t w[NQ][3], bc[NQ];
#pragma unroll
        for (int k = 0; k < NQ; ++k) {
            Philox4 r0 = {}, r1 = {};
            if (SR) {
                const uint64_t jj = 2u * (uint64_t)(t0 + k);
                r0 = philox4x32_10((uint32_t)jj, (uint32_t)(jj >> 32), 0u, 0u, a.seed_lo, a.seed_hi);
                r1 = philox4x32_10((uint32_t)(jj + 1), (uint32_t)((jj + 1) >> 32), 0u, 0u,
                                   a.seed_lo, a.seed_hi);
            }
            bc[k] = quantize_square<FMT, SR>(x[q][k], T, nonfinite, r0, r1, w[k]);
        }
        store_group<FMT, NQ>(a, t0, w, bc);
    }
}

template <int FMT, bool SR, int NQ, int PX>
__global__ void __launch_bounds__(256) quantize_nchw_kernel(QuantNchwArgs a)
{
    warm_kernel_args<QuantNchwArgs>();
    __shared__ uint32_t red[4];
    nchw_body<FMT, SR, NQ, PX>(a, red, (int)blockIdx.x);
}

template <int FMT, bool SR, int NQ, int PX>
static void launch_nchw_shape(QuantNchwArgs a, hipStream_t st)
{
    const int pbs = (a.HW + 64 * PX - 1) / (64 * PX);
    a.NG = a.N4 / NQ;
    a.items = pbs * a.C4 * a.NG;
    hipLaunchKernelGGL((quantize_nchw_kernel<FMT, SR, NQ, PX>), dim3((a.items + 3) / 4), dim3(256),
                       0, st, a);
}

// Batch squares per lane: four (64 loads in flight per lane, the fastest shape on large tensors)
// when that still gives every CU a workgroup; one otherwise, so that a small tensor spreads over
// four times as many workgroups and each lane's chain of loads is a quarter as long.
static int nchw_nq(int N4, int HW, int C4)
{
    const int64_t wgs4 = ((int64_t)(HW + 63) / 64) * C4 * (N4 / 4) / 4;
    return (N4 % 4 == 0 && wgs4 >= 256) ? 4 : 1;
}

template <int FMT, bool SR>
static hipError_t launch_quant_nchw(const QuantNchwArgs &a, hipStream_t st)
{
    const bool al16 = (reinterpret_cast<uintptr_t>(a.src) & 15u) == 0;
    if (nchw_nq(a.N4, a.HW, a.C4) == 4) launch_nchw_shape<FMT, SR, 4, 1>(a, st);
    else if (a.N4 % 4 != 0 && al16 && a.HW % 4 == 0) launch_nchw_shape<FMT, SR, 1, 4>(a, st);
    else launch_nchw_shape<FMT, SR, 1, 1>(a, st);
    return hipGetLastError();
}

// ---- several tensors in one amax launch and one quantizing launch ----
//
// Each job is one tensor with its own source order (channel-batch-first or any [o0][o1][r][s]
// array, NCHW, or an OIHW weight), rounding, seed, amax workspace and destination; the codes,
// scales and T are those of the single-tensor calls. The amax pass runs every job's workgroups
// in one grid (one grid row per job; jobs with the amax ready take none), and so does the
// quantizing pass, so small tensors ride along with a large one instead of paying a launch and
// a memory round trip of their own.
enum { kJobCbf = 0, kJobNchw = 1, kJobOihw = 2 };
constexpr int kMaxJobs = 4;

struct QuantJob {
    int kind, sr, full, nq;
    int a_P;       // amax pass workgroups (0: partial maxima already in the workspace)
    int q_P;       // quantizing pass workgroups
    int64_t an;    // elements (amax pass; the source and workspace are the kind's own)
    union {
        QuantArgs cbf;      // kJobCbf, kJobOihw
        QuantNchwArgs nchw; // kJobNchw
    };
};

// NJ job slots: the kernel arguments are read by every workgroup, so a batch of one or two
// tensors takes the two-slot variant (measured 0.4 us faster per launch pair than four slots).
template <int NJ> struct QuantBatchArgs {
    QuantJob job[NJ];
    int njobs;
};

// Grid (workgroups of the largest job, jobs): workgroup (b, j) is block b of job j, and blocks
// past a job's own count leave at once. The job comes from the grid, not from a search over the
// arguments, which would put a chain of dependent argument loads before every workgroup's
// first memory access (measured 0.5 us per launch pair).
template <int NJ>
__global__ void __launch_bounds__(kAmaxThreads) amax_batch_kernel(QuantBatchArgs<NJ> a)
{
    warm_kernel_args<QuantBatchArgs<NJ>>();
    __shared__ uint32_t red[kAmaxThreads / 64];
    const QuantJob &jb = a.job[blockIdx.y];
    const int b = (int)blockIdx.x;
    if (b >= jb.a_P) return;
    const bool nchw = jb.kind == kJobNchw;
    amax_body(nchw ? jb.nchw.src : jb.cbf.src, jb.an,
              const_cast<uint32_t *>(nchw ? jb.nchw.amax_ws : jb.cbf.amax_ws), b, jb.a_P, red);
}

template <int FMT, int NJ>
__global__ void __launch_bounds__(256) quantize_batch_kernel(QuantBatchArgs<NJ> a)
{
    warm_kernel_args<QuantBatchArgs<NJ>>();
    __shared__ uint32_t red[4];
    const QuantJob &jb = a.job[blockIdx.y];
    const int lb = (int)blockIdx.x;
    if (lb >= jb.q_P) return; // (a whole workgroup: before any barrier)
    if (jb.kind == kJobNchw) {
        if (jb.nq == 4) {
            if (jb.sr) nchw_body<FMT, true, 4, 1>(jb.nchw, red, lb);
            else nchw_body<FMT, false, 4, 1>(jb.nchw, red, lb);
        } else {
            if (jb.sr) nchw_body<FMT, true, 1, 1>(jb.nchw, red, lb);
            else nchw_body<FMT, false, 1, 1>(jb.nchw, red, lb);
        }
    } else if (jb.kind == kJobOihw) {
        if (jb.sr) cbf_body<FMT, true, false, true>(jb.cbf, red, lb, jb.q_P);
        else cbf_body<FMT, false, false, true>(jb.cbf, red, lb, jb.q_P);
    } else if (jb.full) {
        if (jb.sr) cbf_body<FMT, true, true, false>(jb.cbf, red, lb, jb.q_P);
        else cbf_body<FMT, false, true, false>(jb.cbf, red, lb, jb.q_P);
    } else {
        if (jb.sr) cbf_body<FMT, true, false, false>(jb.cbf, red, lb, jb.q_P);
        else cbf_body<FMT, false, false, false>(jb.cbf, red, lb, jb.q_P);
    }
}

// A small weight (at most kSmallWeight floats), from OIHW fp32 to quantized tap-major squares in
// one launch: every workgroup reduces the whole tensor's amax itself (1024 lanes, a few 16-byte
// loads each; no step across workgroups, no workspace), then its first kSmallSquares lanes
// quantize one square each, gathered from OIHW, with the same arithmetic as quantize_kernel.
constexpr int kSmallWeight = 65536;
constexpr int kSmallThreads = 1024;
constexpr int kSmallSquares = 64;

template <int FMT, bool SR>
__global__ void __launch_bounds__(kSmallThreads) quantize_weight_small_kernel(QuantArgs a)
{
    using F = Fmt<FMT>;
    __shared__ uint32_t red[kSmallThreads / 64];
    const int n = (int)(a.planes * a.R * a.S);
    // The square's own 16 values and the whole-tensor amax reads do not depend on each other:
    // all of them are issued before any is used, so the launch costs one memory round trip.
    const int t = (int)blockIdx.x * kSmallSquares + (int)threadIdx.x;
    const bool mine = threadIdx.x < kSmallSquares && t < (int)a.nsq;
    const int tt = mine ? t : 0;
    const int planes = (int)a.planes;
    const int s4 = tt % a.S4, r4 = (tt / a.S4) % a.R4, plane = tt / a.S4 / a.R4;
    float x[16];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * r4 + i, c = 4 * s4 + j;
            const bool in = mine && r < a.R && c < a.S;
            x[4 * i + j] = in ? a.src[(r * a.S + c) * planes + plane] : 0.0f;
        }
    uint32_t m = 0u;
    if ((reinterpret_cast<uintptr_t>(a.src) & 15u) == 0) {
        // n <= kSmallWeight: at most kSmallWeight / 4 / kSmallThreads 16-byte loads per lane
        constexpr int kV = kSmallWeight / 4 / kSmallThreads;
        const int n4 = n >> 2;
        const u32x4_t *x4 = reinterpret_cast<const u32x4_t *>(a.src);
        u32x4_t v[kV];
#pragma unroll
        for (int k = 0; k < kV; ++k) {
            const int j = (int)threadIdx.x + k * kSmallThreads;
            v[k] = j < n4 ? x4[j] : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int k = 0; k < kV; ++k) m = max(m, absmax4(v[k]));
        const int tail = (n4 << 2) + (int)threadIdx.x; // n % 4 trailing floats
        if (tail < n) m = max(m, __float_as_uint(a.src[tail]) & 0x7FFFFFFFu);
    } else {
        for (int j = threadIdx.x; j < n; j += kSmallThreads)
            m = max(m, __float_as_uint(a.src[j]) & 0x7FFFFFFFu);
    }
    const uint32_t abits = block_max_u32<kSmallThreads>(m, red);
    const bool nonfinite = abits >= 0x7F800000u;
    const float T = __uint_as_float(abits) / (448.0f * F::kEmax);
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.tscale = nonfinite ? __uint_as_float(0x7FC00000u) : T;
    if (!mine) return;
    Philox4 r0 = {}, r1 = {};
    if (SR) {
        const uint64_t jj = 2u * (uint64_t)t;
        r0 = philox4x32_10((uint32_t)jj, (uint32_t)(jj >> 32), 0u, 0u, a.seed_lo, a.seed_hi);
        r1 = philox4x32_10((uint32_t)(jj + 1), (uint32_t)((jj + 1) >> 32), 0u, 0u, a.seed_lo,
                           a.seed_hi);
    }
    uint32_t w[3];
    const uint32_t bcode = quantize_square<FMT, SR>(x, T, nonfinite, r0, r1, w);
    a.scales[t] = (uint8_t)bcode;
    store_square_codes<FMT>(a.codes, t, w);
}

template <int FMT, bool SR>
static hipError_t launch_quant_weight(const QuantArgs &a, uint32_t *amax_ws, hipStream_t st)
{
    const int64_t n = a.planes * a.R * a.S;
    if (n <= kSmallWeight) {
        hipLaunchKernelGGL((quantize_weight_small_kernel<FMT, SR>),
                           dim3((unsigned)((a.nsq + kSmallSquares - 1) / kSmallSquares)),
                           dim3(kSmallThreads), 0, st, a);
        return hipGetLastError();
    }
    // larger: the amax pass over the OIHW array (same values), then the gathering quantizer
    const int parts = amax_parts(n);
    hipLaunchKernelGGL(amax_kernel, dim3(parts), dim3(kAmaxThreads), 0, st, a.src, n, amax_ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    QuantArgs b = a;
    b.amax_ws = amax_ws;
    const int64_t wantq = (a.nsq + kCbfLanes<true> - 1) / kCbfLanes<true>;
    const unsigned blocks = (unsigned)(wantq < kQuantBlocks ? wantq : kQuantBlocks);
    hipLaunchKernelGGL((quantize_kernel<FMT, SR, false, true>), dim3(blocks), dim3(256), 0, st, b);
    return hipGetLastError();
}

hipError_t launch_quantize_weight(const float *src, int Cout, int Cin, int Kh, int Kw, int fmt,
                                  int rnd, uint64_t seed, uint8_t *codes, uint8_t *scales,
                                  float *tscale, uint32_t *amax_ws, hipStream_t st)
{
    QuantArgs a;
    a.src = src; a.codes = codes; a.scales = scales; a.tscale = tscale;
    a.amax_ws = amax_ws;
    a.planes = (int64_t)Kh * Kw; a.R = Cout; a.S = Cin; a.R4 = (Cout + 3) / 4; a.S4 = (Cin + 3) / 4;
    a.nsq = a.planes * a.R4 * a.S4;
    if (a.nsq >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    a.seed_lo = (uint32_t)seed; a.seed_hi = (uint32_t)(seed >> 32);
    if (fmt == kFP4)
        return rnd ? launch_quant_weight<kFP4, true>(a, amax_ws, st)
                   : launch_quant_weight<kFP4, false>(a, amax_ws, st);
    return rnd ? launch_quant_weight<kFP6, true>(a, amax_ws, st)
               : launch_quant_weight<kFP6, false>(a, amax_ws, st);
}

hipError_t launch_quantize(const float *src, int64_t planes, int R, int S, int fmt, int rnd,
                           uint64_t seed, uint8_t *codes, uint8_t *scales, float *tscale,
                           uint32_t *amax_ws, bool amax_ready, hipStream_t st)
{
    if (planes * ((R + 3) / 4) * (int64_t)((S + 3) / 4) >= ((int64_t)1 << 31))
        return hipErrorInvalidValue; // square indices are 31-bit
    const int64_t n = planes * (int64_t)R * S;
    // at least 8 float4 per lane where the tensor allows, at most kAmaxParts workgroups
    const int parts = amax_parts(n);
    if (!amax_ready) {
        hipLaunchKernelGGL(amax_kernel, dim3(parts), dim3(kAmaxThreads), 0, st, src, n, amax_ws);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }

    QuantArgs a;
    a.src = src; a.codes = codes; a.scales = scales; a.tscale = tscale;
    a.amax_ws = amax_ws;
    a.planes = planes; a.R = R; a.S = S; a.R4 = (R + 3) / 4; a.S4 = (S + 3) / 4;
    a.nsq = planes * a.R4 * a.S4; // below 2^31 (the API rejects larger tensors)
    a.seed_lo = (uint32_t)seed; a.seed_hi = (uint32_t)(seed >> 32);
    const bool full = (R % 4 == 0) && (S % 4 == 0) &&
                      ((reinterpret_cast<uintptr_t>(src) & 15u) == 0);
    if (fmt == kFP4)
        return rnd ? launch_quant<kFP4, true>(a, full, st) : launch_quant<kFP4, false>(a, full, st);
    return rnd ? launch_quant<kFP6, true>(a, full, st) : launch_quant<kFP6, false>(a, full, st);
}

hipError_t launch_quantize_nchw(const float *src, int N, int C, int H, int W, int fmt, int rnd,
                                uint64_t seed, uint8_t *codes, uint8_t *scales, float *tscale,
                                uint32_t *amax_ws, bool amax_ready, hipStream_t st)
{
    const int64_t n = (int64_t)N * C * H * W;
    const int64_t HW = (int64_t)H * W;
    const int64_t C4 = (C + 3) / 4, N4 = (N + 3) / 4;
    // 32-bit byte offsets below 2^31 even for the zero-padded rows and channels (4*N4 x 4*C4
    // planes); 31-bit square and work-item indices
    if (16 * N4 * C4 * HW * 4 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    if (!amax_ready) {
        const int parts = amax_parts(n);
        hipLaunchKernelGGL(amax_kernel, dim3(parts), dim3(kAmaxThreads), 0, st, src, n, amax_ws);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    QuantNchwArgs a;
    a.src = src; a.codes = codes; a.scales = scales; a.tscale = tscale; a.amax_ws = amax_ws;
    a.N = N; a.C = C; a.HW = (int)HW; a.C4 = (int)C4; a.N4 = (int)N4;
    a.NG = 0; a.items = 0;
    a.bytes = (uint32_t)(n * 4);
    a.seed_lo = (uint32_t)seed; a.seed_hi = (uint32_t)(seed >> 32);
    if (fmt == kFP4)
        return rnd ? launch_quant_nchw<kFP4, true>(a, st) : launch_quant_nchw<kFP4, false>(a, st);
    return rnd ? launch_quant_nchw<kFP6, true>(a, st) : launch_quant_nchw<kFP6, false>(a, st);
}

template <int NJ>
static hipError_t launch_batch_nj(const QuantJobDesc *jobs, int njobs, int fmt, hipStream_t st)
{
    QuantBatchArgs<NJ> a = {};
    a.njobs = njobs;
    for (int i = 0; i < njobs; ++i) {
        const QuantJobDesc &d = jobs[i];
        QuantJob &jb = a.job[i];
        jb.sr = d.rnd != 0;
        const int64_t n = (int64_t)d.o0 * d.o1 * d.r * d.s;
        const int64_t R4 = (d.r + 3) / 4, S4 = (d.s + 3) / 4;
        const int64_t nsq = (int64_t)d.o0 * d.o1 * R4 * S4;
        if (nsq >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
        jb.an = n;
        jb.a_P = d.amax_ready ? 0 : amax_parts(n);
        if (d.layout == kJobNchw) {
            // dims (o0, o1, r, s) = (H, W, C, N)
            const int64_t HW = (int64_t)d.o0 * d.o1;
            if (16 * S4 * R4 * HW * 4 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
            jb.kind = kJobNchw;
            QuantNchwArgs &q = jb.nchw;
            q.src = d.src; q.codes = d.codes; q.scales = d.scales; q.tscale = d.tscale;
            q.amax_ws = d.amax_ws;
            q.N = d.s; q.C = d.r; q.HW = (int)HW; q.C4 = (int)R4; q.N4 = (int)S4;
            jb.nq = nchw_nq(q.N4, q.HW, q.C4);
            q.NG = q.N4 / jb.nq;
            q.items = (int)((HW + 63) / 64) * q.C4 * q.NG;
            q.bytes = (uint32_t)(n * 4);
            q.seed_lo = (uint32_t)d.seed; q.seed_hi = (uint32_t)(d.seed >> 32);
            jb.q_P = (q.items + 3) / 4;
        } else {
            // kJobCbf: [o0*o1][r][s]; kJobOihw: weight [r=Cout][s=Cin][o0*o1 taps]
            jb.kind = d.layout;
            QuantArgs &q = jb.cbf;
            q.src = d.src; q.codes = d.codes; q.scales = d.scales; q.tscale = d.tscale;
            q.amax_ws = d.amax_ws;
            q.planes = (int64_t)d.o0 * d.o1; q.R = d.r; q.S = d.s; q.R4 = (int)R4; q.S4 = (int)S4;
            q.nsq = nsq;
            q.seed_lo = (uint32_t)d.seed; q.seed_hi = (uint32_t)(d.seed >> 32);
            jb.full = d.layout == kJobCbf && d.r % 4 == 0 && d.s % 4 == 0 &&
                      (reinterpret_cast<uintptr_t>(d.src) & 15u) == 0;
            const int lanes = d.layout == kJobOihw ? 64 : 256;
            const int64_t want = (nsq + lanes - 1) / lanes;
            jb.q_P = (int)(want < kQuantBlocks ? want : kQuantBlocks);
        }
    }
    // largest job in grid row 0: the hardware dispatches row by row, so the small jobs' empty
    // columns come after the large job's workgroups instead of before them (job order is free:
    // each job carries its own pointers)
    for (int i = 1; i < njobs; ++i)
        for (int k = i; k > 0 && a.job[k].q_P > a.job[k - 1].q_P; --k) {
            const QuantJob t = a.job[k];
            a.job[k] = a.job[k - 1];
            a.job[k - 1] = t;
        }
    int amax_max = 0, q_max = 0;
    for (int i = 0; i < njobs; ++i) {
        amax_max = a.job[i].a_P > amax_max ? a.job[i].a_P : amax_max;
        q_max = a.job[i].q_P > q_max ? a.job[i].q_P : q_max;
    }
    if (amax_max > 0) {
        hipLaunchKernelGGL((amax_batch_kernel<NJ>), dim3((unsigned)amax_max, (unsigned)njobs),
                           dim3(kAmaxThreads), 0, st, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (fmt == kFP4)
        hipLaunchKernelGGL((quantize_batch_kernel<kFP4, NJ>), dim3((unsigned)q_max, (unsigned)njobs),
                           dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((quantize_batch_kernel<kFP6, NJ>), dim3((unsigned)q_max, (unsigned)njobs),
                           dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_quantize_batch(const QuantJobDesc *jobs, int njobs, int fmt, hipStream_t st)
{
    if (njobs < 1 || njobs > kMaxJobs) return hipErrorInvalidValue;
    return njobs <= 2 ? launch_batch_nj<2>(jobs, njobs, fmt, st)
                      : launch_batch_nj<kMaxJobs>(jobs, njobs, fmt, st);
}

} // namespace mq
