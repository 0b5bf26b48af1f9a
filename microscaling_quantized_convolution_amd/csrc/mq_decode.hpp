// mq_decode.hpp -- exact decode of quantized 4x4 squares to fp16 pairs (gfx950).
//
// An element value is E * B with E an E2M1 / E2M3 value and B an E4M3 scale; E*B has at most 6
// (NVFP4) or 8 (NVFP6) significant bits and lies in [2^-12, 3360], so fp16 holds it exactly and
// fp16 MFMA products are exact in fp32. The tensor scale T stays out (applied in the epilogue).
//
// NVFP4: v_cvt_scalef32_pk_f16_fp4 converts the two E2M1 codes of a byte and multiplies them by
// the power of two of its fp32 scale operand (only the exponent is used), so E4M3 = 2^k * mant
// splits into one convert with 2^k and one packed fp16 multiply by mant.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mq_device.hpp"

namespace mq {

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// E4M3 scale -> (power of two as fp32, mantissa factor as fp16 pair). mant * pow2 = B exactly.
// NaN scale (0x7F) gives a NaN factor so that every decoded value is NaN.
struct SplitScale {
    float pow2;
    f16x2_t mant;
};

__device__ __forceinline__ SplitScale split_e4m3(uint32_t sc)
{
    const uint32_t e = (sc >> 3) & 15u, m = sc & 7u;
    SplitScale r;
    // normal: (1 + m/8) * 2^(e-7); subnormal (e = 0): m * 2^-9. Branch-free selects.
    const uint32_t mnorm = 0x3C00u | (m << 7);
    const uint32_t msub = __builtin_bit_cast(uint16_t, (_Float16)(float)m);
    uint32_t mbits = e ? mnorm : msub;
    r.pow2 = __uint_as_float((e ? e + 120u : 118u) << 23);
    mbits = ((sc & 0x7Fu) == 0x7Fu) ? 0x7E00u : mbits;
    r.mant = __builtin_bit_cast(f16x2_t, mbits | (mbits << 16));
    return r;
}

// NVFP4 square (two code words, element e = nibble e of the 64-bit pair) -> d[j] = fp16 pair of
// elements (2j, 2j+1), i.e. d[2r], d[2r+1] hold square row r.
__device__ __forceinline__ void decode_fp4_square(uint32_t w0, uint32_t w1, uint32_t sc,
                                                  uint32_t (&d)[8])
{
    const SplitScale s = split_e4m3(sc);
    f16x2_t h[8];
    h[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, s.pow2, 0);
    h[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, s.pow2, 1);
    h[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, s.pow2, 2);
    h[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, s.pow2, 3);
    h[4] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, s.pow2, 0);
    h[5] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, s.pow2, 1);
    h[6] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, s.pow2, 2);
    h[7] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, s.pow2, 3);
#pragma unroll
    for (int j = 0; j < 8; ++j) d[j] = __builtin_bit_cast(uint32_t, h[j] * s.mant);
}

// NVFP6 square (three code words, element e = bits [6e, 6e+6) of the 96-bit word) -> d as above.
// A code s|ee|mmm placed as fp16 bits s<<15 | eemmm<<7 is E * 2^-14 (subnormal codes become
// fp16 subnormals), so E*B = that * 2^14 * B with both products exact.
__device__ __forceinline__ void decode_fp6_square(uint32_t w0, uint32_t w1, uint32_t w2,
                                                  uint32_t sc, uint32_t (&d)[8])
{
    const SplitScale s = split_e4m3(sc);
    const _Float16 bscale = (_Float16)s.pow2 * s.mant[0]; // exact: B is an fp16 value
    const f16x2_t b2 = {bscale, bscale};
    const f16x2_t k14 = {(_Float16)16384.0f, (_Float16)16384.0f};
    const uint64_t lo = ((uint64_t)w1 << 32) | w0;
    const uint64_t hi = ((uint64_t)w2 << 32) | w1;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t f[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int e = 2 * j + u, bit = 6 * e;
            const uint32_t c = (bit < 58) ? (uint32_t)(lo >> bit) & 0x3Fu
                                          : (uint32_t)(hi >> (bit - 32)) & 0x3Fu;
            f[u] = ((c & 31u) << 7) | ((c & 32u) << 10);
        }
        const f16x2_t v = __builtin_bit_cast(f16x2_t, f[0] | (f[1] << 16));
        d[j] = __builtin_bit_cast(uint32_t, (v * k14) * b2);
    }
}

// Column c (0..3) of a decoded square as two fp16-pair words: (row0,row1), (row2,row3).
__device__ __forceinline__ void square_column(const uint32_t (&d)[8], int c, uint32_t &p0,
                                              uint32_t &p1)
{
    // v_perm_b32: selector bytes 0-3 take the second operand, 4-7 the first.
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
    p0 = __builtin_amdgcn_perm(d[2 + (c >> 1)], d[c >> 1], sel);
    p1 = __builtin_amdgcn_perm(d[6 + (c >> 1)], d[4 + (c >> 1)], sel);
}

} // namespace mq
