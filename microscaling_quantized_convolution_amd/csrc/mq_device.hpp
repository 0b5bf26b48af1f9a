// mq_device.hpp -- device helpers shared by the library's kernels (gfx950 only).
//
// Number formats of the NVFP4 / NVFP6 recipe (onedev.kr MicroQonv digest, section "How it
// differs": E4M3 block scale, E2M1 elements; section "How it is used": E2M3 elements):
//   E2M1 s|ee|m     bias 1, subnormal 0.5*m, largest 6
//   E2M3 s|ee|mmm   bias 1, subnormal m/8,   largest 7.5
//   E4M3 s|eeee|mmm bias 7, subnormal m*2^-9, largest 448 (0x7E), 0x7F = NaN
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mq {

constexpr int kFP4 = 4;
constexpr int kFP6 = 6;

template <int FMT> struct Fmt;
template <> struct Fmt<kFP4> {
    static constexpr int kBits = 4;        // bits per code
    static constexpr int kMant = 1;        // mantissa bits
    static constexpr uint32_t kSign = 0x8; // sign bit of a code
    static constexpr uint32_t kMaxMag = 7; // largest magnitude code
    static constexpr int kBytesPerSquare = 8;
    static constexpr float kEmax = 6.0f;
    // Grid rounding on [0,2): code = 2a; [2,4): a + 2; [4, inf): a/2 + 4 (see quantize).
    static constexpr float kScale0 = 2.0f;
    static constexpr float kAdd1 = 2.0f, kAdd2 = 4.0f;
};
template <> struct Fmt<kFP6> {
    static constexpr int kBits = 6;
    static constexpr int kMant = 3;
    static constexpr uint32_t kSign = 0x20;
    static constexpr uint32_t kMaxMag = 31;
    static constexpr int kBytesPerSquare = 12;
    static constexpr float kEmax = 7.5f;
    // [0,2): code = 8a; [2,4): 4a + 8; [4, inf): 2a + 16.
    static constexpr float kScale0 = 8.0f;
    static constexpr float kAdd1 = 8.0f, kAdd2 = 16.0f;
};

// Value of an E4M3 code (finite codes only; callers handle 0x7F separately).
__device__ __forceinline__ float e4m3_to_float(uint32_t c)
{
    // Place eeee.mmm right below the fp32 exponent LSB: as a float this is the E4M3 value times
    // 2^(1-127) * 2^(7-1)... i.e. value * 2^-120, exact also for E4M3 subnormals (they become fp32
    // denormals). Rescale by 2^120.
    uint32_t mag = c & 0x7Fu;
    float v = __uint_as_float(mag << 20) * 0x1p120f;
    return (c & 0x80u) ? -v : v;
}

// CastE4M3 of a non-negative, non-NaN fp32: round to nearest, ties to even, subnormals kept,
// saturating at 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_rne_sat(float s)
{
    if (!(s < 448.0f)) return 0x7Eu;          // also +inf
    if (s < 0x1p-6f) {                        // E4M3 subnormal range: m * 2^-9, m = 0..8
        return (uint32_t)__builtin_rintf(s * 512.0f); // 8 -> code 8 = 2^-6, the first normal
    }
    uint32_t b = __float_as_uint(s);
    // keep 3 mantissa bits, round-to-nearest-even on the 20 dropped bits
    b += 0x7FFFFu + ((b >> 20) & 1u);
    uint32_t e = (b >> 23) - 127u + 7u;
    uint32_t m = (b >> 20) & 7u;
    uint32_t c = (e << 3) | m;
    return c > 0x7Eu ? 0x7Eu : c;
}

// Value of an element magnitude code: the code placed right under the fp32 exponent field is
// the element value times 2^-126 (subnormal codes become fp32 denormals), so rescale by 2^126.
template <int FMT>
__device__ __forceinline__ float elem_mag_to_float(uint32_t mag)
{
    return __uint_as_float(mag << (23 - Fmt<FMT>::kMant)) * 0x1p126f;
}

// Nearest-even grid code of a = |q| (a >= 0, finite), saturating at the largest element.
// On each of [0,2), [2,4), [4,inf) the grid is uniform, so the code is an affine function of
// a rounded with rint (ties to even integer = ties to even code).
template <int FMT>
__device__ __forceinline__ uint32_t grid_rne(float a)
{
    using F = Fmt<FMT>;
    float sc = a < 2.0f ? F::kScale0 : (a < 4.0f ? 0.5f * F::kScale0 : 0.25f * F::kScale0);
    float ad = a < 2.0f ? 0.0f : (a < 4.0f ? F::kAdd1 : F::kAdd2);
    float c = __builtin_rintf(a * sc) + ad;
    c = fminf(c, (float)F::kMaxMag);
    return (uint32_t)c;
}

// Stochastic grid rounding of a = |q|: from the lower neighbour up iff u16 < frac * 65536,
// frac = (a - lo) / step (lo is the grid value at or below a, step a power of two).
// With x = a / step (exact) that is ceil(x - u16 / 65536): for x < 2^8 the difference is exact
// or keeps its sign and integer part (for x below 1 with a draw far above it), so its ceiling
// is floor(x) + 1 exactly when the fractional part exceeds the draw. Codes past the largest
// element saturate (the min). Checked on the device against the threshold form for every fp32
// magnitude below 12, with the draws at and next to each threshold.
template <int FMT>
__device__ __forceinline__ uint32_t grid_sr(float a, uint32_t u16)
{
    using F = Fmt<FMT>;
    // binade of the grid step: m = 1 below 2 (one step size down to zero), 2 on [2,4), 3 from 4
    // up (frexp's exponent of a, clamped); x = a / step and the code offset follow from m
    constexpr int kL = FMT == kFP4 ? 1 : 3; // log2(kScale0) = log2(kAdd1)
    const int e = __builtin_amdgcn_frexp_expf(a);
    const int m = min(max(e, 1), 3);
    const float nx = __builtin_amdgcn_ldexpf(-a, kL + 1 - m); // -x, exact
    // z = RN(u - x) = -RN(x - u) (nearest rounding is symmetric), and ceil(x - u) = -floor(z):
    // v_cvt_flr_i32_f32 takes the floor and the conversion in one instruction, where the
    // compiler emits a ceiling and a conversion
    const float z = __builtin_fmaf((float)u16, 0x1p-16f, nx);
    int fl;
    asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(fl) : "v"(z));
    // the code offset of the binade in one shift-and-add (left to itself, the compiler
    // reassociates the two subtractions into three instructions)
    uint32_t base = ((uint32_t)m << kL) - (1u << kL);
    asm("" : "+v"(base));
    const uint32_t c = base - (uint32_t)fl;
    return c < F::kMaxMag ? c : F::kMaxMag;
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): multipliers 0xD2511F53 / 0xCD9E8D57,
// Weyl increments 0x9E3779B9 / 0xBB67AE85.
struct Philox4 {
    uint32_t v[4];
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1)
{
    // each 32 x 32 -> 64-bit product is one v_mad_u64_u32 (high and low halves together), and
    // each three-way exclusive or one v_bitop3_b32 (truth table 0x96)
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
        const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
        c0 = n0;
        c1 = (uint32_t)p1;
        c2 = n2;
        c3 = (uint32_t)p0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    Philox4 r;
    r.v[0] = c0; r.v[1] = c1; r.v[2] = c2; r.v[3] = c3;
    return r;
}

// bf16 bit pattern of an fp32 value that is exactly representable in bf16.
__device__ __forceinline__ uint32_t bf16_bits_exact(float v) { return __float_as_uint(v) >> 16; }

// Bring a kernel's argument block into the scalar cache in one round trip: one load per 64-byte
// line, all in flight together, and one wait. Left to the compiler, each argument is loaded next
// to its first use, and the lines of a large argument block (per-job or per-class tables
// indexed by the grid) then arrive one dependent miss after another before the first memory
// access of the kernel. The loads wait inside the asm block, so no load is in flight once it
// ends.
template <typename Args>
__device__ __forceinline__ void warm_kernel_args()
{
    static_assert(sizeof(Args) >= 4 && sizeof(Args) <= 640, "argument block of 1 to 10 lines");
    constexpr uint32_t kLast = ((uint32_t)sizeof(Args) - 4u) & ~3u; // last dword of the block
#define MQ_LINE(k) ((64u * (k)) < kLast ? 64u * (k) : kLast)
    const uint64_t kp = (uint64_t)__builtin_amdgcn_kernarg_segment_ptr();
    uint32_t d0, d1, d2, d3, d4, d5, d6, d7, d8, d9;
    asm volatile("s_load_dword %0, %10, 0\n\t"
                 "s_load_dword %1, %10, %11\n\t"
                 "s_load_dword %2, %10, %12\n\t"
                 "s_load_dword %3, %10, %13\n\t"
                 "s_load_dword %4, %10, %14\n\t"
                 "s_load_dword %5, %10, %15\n\t"
                 "s_load_dword %6, %10, %16\n\t"
                 "s_load_dword %7, %10, %17\n\t"
                 "s_load_dword %8, %10, %18\n\t"
                 "s_load_dword %9, %10, %19\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&s"(d0), "=&s"(d1), "=&s"(d2), "=&s"(d3), "=&s"(d4), "=&s"(d5), "=&s"(d6),
                   "=&s"(d7), "=&s"(d8), "=&s"(d9)
                 : "s"(kp), "i"(MQ_LINE(1)), "i"(MQ_LINE(2)), "i"(MQ_LINE(3)), "i"(MQ_LINE(4)),
                   "i"(MQ_LINE(5)), "i"(MQ_LINE(6)), "i"(MQ_LINE(7)), "i"(MQ_LINE(8)),
                   "i"(MQ_LINE(9)));
#undef MQ_LINE
    asm volatile("" ::"s"(d0), "s"(d1), "s"(d2), "s"(d3), "s"(d4), "s"(d5), "s"(d6), "s"(d7),
                 "s"(d8), "s"(d9));
}

} // namespace mq
