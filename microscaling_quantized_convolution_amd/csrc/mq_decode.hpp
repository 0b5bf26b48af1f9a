// mq_decode.hpp -- exact decode of quantized 4x4 squares to fp16 pairs (gfx950).
//
// An element value is E * B with E an E2M1 / E2M3 value and B an E4M3 scale; E*B has at most 6
// (NVFP4) or 8 (NVFP6) significant bits and lies in [2^-12, 3360], so fp16 holds it exactly and
// fp16 MFMA products are exact in fp32. The tensor scale T stays out (applied in the epilogue).
//
// The E4M3 scale converts to fp16 in hardware (exact), the E2M1 codes too (two per byte), the
// E2M3 codes 32 at a time, and one packed fp16 multiply per element pair applies the scale.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mq_device.hpp"

namespace mq {

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Scale bytes -> fp16. v_cvt_scalef32_pk_f16_fp8 converts two E4M3 bytes (OCP e4m3fn: subnormals,
// 0x7F/0xFF NaN) to fp16 exactly: every E4M3 value is an fp16 value.
template <bool HIGH_PAIR>
__device__ __forceinline__ f16x2_t e4m3_pair_to_f16(uint32_t four_bytes)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(four_bytes, 1.0f, HIGH_PAIR);
}

// NVFP4 square (two code words, element e = nibble e of the 64-bit pair) with scale B (fp16) ->
// d[j] = fp16 pair of elements (2j, 2j+1), i.e. d[2r], d[2r+1] hold square row r. The convert
// gives the E2M1 values exactly (scale 1); one packed multiply applies B. A NaN scale makes every
// element NaN, a zero scale every element +-0.
__device__ __forceinline__ void decode_fp4_square(uint32_t w0, uint32_t w1, _Float16 B,
                                                  uint32_t (&d)[8])
{
    const f16x2_t b2 = {B, B};
    f16x2_t h[8];
    h[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 0);
    h[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 1);
    h[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 2);
    h[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 3);
    h[4] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 0);
    h[5] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 1);
    h[6] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 2);
    h[7] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 3);
#pragma unroll
    for (int j = 0; j < 8; ++j) d[j] = __builtin_bit_cast(uint32_t, h[j] * b2);
}

// Two NVFP6 squares (six code words: the first square's three, then the second's; element e of
// a square = bits [6e, 6e+6) of its 96-bit word) with scales B0, B1 -> d0, d1 as above. One
// v_cvt_scalef32_pk32_f16_fp6 converts the 32 E2M3 codes (code i = bits [6i, 6i+6) of the
// 192-bit word, which is the two squares' packing) to their fp16 values exactly (scale 1: every
// E2M3 value is an fp16 value); one packed multiply per pair applies the square's scale. A NaN
// scale makes every element NaN, a zero scale every element +-0.
__device__ __forceinline__ void decode_fp6_square_pair(const uint32_t (&w)[6], _Float16 B0,
                                                       _Float16 B1, uint32_t (&d0)[8],
                                                       uint32_t (&d1)[8])
{
    typedef uint32_t u32x6_t __attribute__((ext_vector_type(6)));
    typedef _Float16 f16x32_t __attribute__((ext_vector_type(32)));
    const u32x6_t v = {w[0], w[1], w[2], w[3], w[4], w[5]};
    const f16x32_t h = __builtin_amdgcn_cvt_scalef32_pk32_f16_fp6(v, 1.0f);
    const f16x2_t b0 = {B0, B0}, b1 = {B1, B1};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const f16x2_t e0 = {h[2 * j], h[2 * j + 1]}, e1 = {h[16 + 2 * j], h[17 + 2 * j]};
        d0[j] = __builtin_bit_cast(uint32_t, e0 * b0);
        d1[j] = __builtin_bit_cast(uint32_t, e1 * b1);
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
