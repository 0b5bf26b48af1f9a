// mq_stage.hpp -- register staging of quantized squares for the convolution kernels.
//
// A staging item is four squares that are consecutive along a GEMM's reduction dimension
// (16 reduction elements) and share one 4-element column or row block. Items are loaded into
// registers one stage ahead (so the global-load latency hides behind the current stage's MFMAs),
// then decoded exactly to fp16 and written to LDS as four 16-element reduction rows.
#pragma once

#include "mq_decode.hpp"

namespace mq {

template <int FMT> struct RawItem {
    static constexpr int kW = (FMT == kFP4) ? 2 : 3; // code words per square
    uint32_t w[4][kW];
    uint32_t sc, sh; // scale bytes: square k is byte k + b of the 64-bit pair (sh:sc)
    uint32_t m;      // bits 0-3: square k is real (a clear bit decodes as zeros whatever was
                     // loaded); bits 8-9: the byte offset b
};

// Buffer resources: raw (stride 0) descriptors whose range check makes every load at an offset
// >= the buffer size return zero. kBad is such an offset for every buffer this library builds
// (all are below 2^31 bytes).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kBad = 0x80000000u;
// cache-policy operand of buffer stores: the non-temporal bit (gfx950)
constexpr int kStoreNT = 2;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// Scale bytes are read as aligned 4-byte words. The range check drops a whole word that reaches
// past the end, which would lose the last real scales, so the range is rounded up to whole
// words: the scale array is 4-byte aligned, so its last word lies inside the memory page of its
// last byte, and the extra bytes only ever belong to squares that are masked off.
__device__ __forceinline__ rsrc_t make_scale_rsrc(const uint8_t *base, uint32_t nsquares)
{
    return make_rsrc(base, (nsquares + 3u) & ~3u);
}

// Load the four squares sq0 + k*step (k = 0..3) whose bit k of `mask` is set; the others read as
// zero codes with a zero scale (out-of-range buffer offsets).
template <int FMT>
__device__ __forceinline__ void load_item(RawItem<FMT> &r, rsrc_t codes, rsrc_t scales,
                                          uint32_t sq0, uint32_t step, uint32_t mask)
{
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));
    r.sc = 0u;
    r.sh = 0u;
    r.m = 0xFu;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const bool on = (mask >> k) & 1u;
        const uint32_t sq = sq0 + k * step;
        const uint32_t coff = on ? sq * (uint32_t)(RawItem<FMT>::kW * 4) : kBad;
        const uint32_t soff = on ? sq : kBad;
        if constexpr (FMT == kFP4) {
            const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(codes, (int)coff, 0, 0);
            r.w[k][0] = v[0];
            r.w[k][1] = v[1];
        } else {
            const u32x3_t v = __builtin_amdgcn_raw_buffer_load_b96(codes, (int)coff, 0, 0);
            r.w[k][0] = v[0];
            r.w[k][1] = v[1];
            r.w[k][2] = v[2];
        }
        r.sc |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(scales, (int)soff, 0, 0) << (8 * k);
    }
}

// Load four squares that are consecutive in memory (sq0 .. sq0+3) with wide loads: 32 (NVFP4) or
// 48 (NVFP6) code bytes, and the four scale bytes as the two aligned words that hold them.
// Squares whose bit of `mask` is clear decode as zeros (their scale is replaced by 0 at decode
// time). The code has no branch and never touches the loaded data, so no load waits before its
// value is decoded (a data-dependent select or a branch join would make the compiler wait).
template <int FMT>
__device__ __forceinline__ void load_item_contig(RawItem<FMT> &r, rsrc_t codes, rsrc_t scales,
                                                 uint32_t sq0, uint32_t mask)
{
    const uint32_t coff = mask ? sq0 * (uint32_t)(RawItem<FMT>::kW * 4) : kBad;
    if constexpr (FMT == kFP4) {
        const u32x4_t v0 = __builtin_amdgcn_raw_buffer_load_b128(codes, (int)coff, 0, 0);
        const u32x4_t v1 = __builtin_amdgcn_raw_buffer_load_b128(codes, (int)(coff + 16u), 0, 0);
        r.w[0][0] = v0[0]; r.w[0][1] = v0[1]; r.w[1][0] = v0[2]; r.w[1][1] = v0[3];
        r.w[2][0] = v1[0]; r.w[2][1] = v1[1]; r.w[3][0] = v1[2]; r.w[3][1] = v1[3];
    } else {
        const u32x4_t v0 = __builtin_amdgcn_raw_buffer_load_b128(codes, (int)coff, 0, 0);
        const u32x4_t v1 = __builtin_amdgcn_raw_buffer_load_b128(codes, (int)(coff + 16u), 0, 0);
        const u32x4_t v2 = __builtin_amdgcn_raw_buffer_load_b128(codes, (int)(coff + 32u), 0, 0);
        r.w[0][0] = v0[0]; r.w[0][1] = v0[1]; r.w[0][2] = v0[2];
        r.w[1][0] = v0[3]; r.w[1][1] = v1[0]; r.w[1][2] = v1[1];
        r.w[2][0] = v1[2]; r.w[2][1] = v1[3]; r.w[2][2] = v2[0];
        r.w[3][0] = v2[1]; r.w[3][1] = v2[2]; r.w[3][2] = v2[3];
    }
    const uint32_t a4 = sq0 & ~3u;
    r.sc = __builtin_amdgcn_raw_buffer_load_b32(scales, (int)(mask ? a4 : kBad), 0, 0);
    r.sh = __builtin_amdgcn_raw_buffer_load_b32(scales, (int)(mask ? a4 + 4u : kBad), 0, 0);
    r.m = mask | ((sq0 & 3u) << 8);
}

// load_item_contig in two steps: the offsets and mask of an item (plan_item), then its loads
// (issue_item). A caller that plans the next chunk's loads before decoding the current one
// leaves the loads nothing to compute, so the compiler takes no register that a load still in
// flight will write as a temporary for them (such a reuse made it wait for loads of later
// chunks too).
struct ItemPlan {
    uint32_t coff, soff, m;
};
template <int FMT>
__device__ __forceinline__ ItemPlan plan_item(uint32_t sq0, uint32_t mask)
{
    ItemPlan p;
    p.coff = mask ? sq0 * (uint32_t)(RawItem<FMT>::kW * 4) : kBad;
    p.soff = mask ? (sq0 & ~3u) : kBad;
    p.m = mask | ((sq0 & 3u) << 8);
    return p;
}
template <int FMT>
__device__ __forceinline__ void issue_item(RawItem<FMT> &r, rsrc_t codes, rsrc_t scales,
                                           const ItemPlan &p)
{
    const u32x4_t v0 = __builtin_amdgcn_raw_buffer_load_b128(codes, (int)p.coff, 0, 0);
    const u32x4_t v1 = __builtin_amdgcn_raw_buffer_load_b128(codes, (int)(p.coff + 16u), 0, 0);
    if constexpr (FMT == kFP4) {
        r.w[0][0] = v0[0]; r.w[0][1] = v0[1]; r.w[1][0] = v0[2]; r.w[1][1] = v0[3];
        r.w[2][0] = v1[0]; r.w[2][1] = v1[1]; r.w[3][0] = v1[2]; r.w[3][1] = v1[3];
    } else {
        const u32x4_t v2 = __builtin_amdgcn_raw_buffer_load_b128(codes, (int)(p.coff + 32u), 0, 0);
        r.w[0][0] = v0[0]; r.w[0][1] = v0[1]; r.w[0][2] = v0[2];
        r.w[1][0] = v0[3]; r.w[1][1] = v1[0]; r.w[1][2] = v1[1];
        r.w[2][0] = v1[2]; r.w[2][1] = v1[3]; r.w[2][2] = v2[0];
        r.w[3][0] = v2[1]; r.w[3][1] = v2[2]; r.w[3][2] = v2[3];
    }
    // (an item outside the tensor has soff = kBad; kBad + 4 is out of range too)
    r.sc = __builtin_amdgcn_raw_buffer_load_b32(scales, (int)p.soff, 0, 0);
    r.sh = __builtin_amdgcn_raw_buffer_load_b32(scales, (int)(p.soff + 4u), 0, 0);
    r.m = p.m;
}

// The four squares' scales as fp16 (squares 0,1 in sc[0], 2,3 in sc[1]); a square whose bit of
// the item mask is clear gets scale 0, so it decodes to zeros whatever codes were loaded.
template <int FMT>
__device__ __forceinline__ void item_scales(const RawItem<FMT> &r, f16x2_t (&sc)[2])
{
    const uint32_t s4 = __builtin_amdgcn_alignbyte(r.sh, r.sc, (r.m >> 8) & 3u);
    // bit k of the mask -> 0xFF in byte k
    const uint32_t keep = (((r.m & 0xFu) * 0x00204081u) & 0x01010101u) * 0xFFu;
    sc[0] = e4m3_pair_to_f16<false>(s4 & keep);
    sc[1] = e4m3_pair_to_f16<true>(s4 & keep);
}

// Squares k0 and k0 + 1 (k0 even) of an item, decoded (d[0], d[1]).
template <int FMT>
__device__ __forceinline__ void decode_pair(const RawItem<FMT> &r, const f16x2_t (&sc)[2], int k0,
                                            uint32_t (&d)[2][8])
{
    const _Float16 B0 = sc[k0 >> 1][0], B1 = sc[k0 >> 1][1];
    if constexpr (FMT == kFP4) {
        decode_fp4_square(r.w[k0][0], r.w[k0][1], B0, d[0]);
        decode_fp4_square(r.w[k0 + 1][0], r.w[k0 + 1][1], B1, d[1]);
    } else {
        const uint32_t w[6] = {r.w[k0][0],     r.w[k0][1],     r.w[k0][2],
                               r.w[k0 + 1][0], r.w[k0 + 1][1], r.w[k0 + 1][2]};
        decode_fp6_square_pair(w, B0, B1, d[0], d[1]);
    }
}

// LDS operand rows: 16 fp16 (32 bytes, two 16-byte units). Bits 0-2 of the unit index
// row*2 + chunk are XORed with a function of the row (a permutation inside each aligned group of
// four rows) chosen so that every access pattern of the convolution kernels spreads over distinct
// banks: MFMA operand reads (16 consecutive rows per group of 16 lanes need 16 distinct units
// modulo 16), 16-byte staging writes of rows four apart (8 lanes, distinct units modulo 8) and
// 8-byte staging writes of rows 16 and 32 apart.
__device__ __forceinline__ int lds_row_off(int row, int chunk)
{
    const int x = ((row >> 3) & 1) | ((((row >> 2) ^ (row >> 5)) & 1) << 1) |
                  ((((row >> 4) ^ (row >> 6)) & 1) << 2);
    return ((row * 2 + chunk) ^ x) << 4;
}

// The same offset for row R + r with R a multiple of 32, from lane_off = lds_row_off(r, chunk)
// (r < 32): the swizzle is linear over XOR, and R contributes only through its bits 5 and 6.
__device__ __forceinline__ int lds_row_off32(int R, int lane_off)
{
    return (R << 5) + (lane_off ^ (R & 96));
}

// LDS offset of row P*16 + r for operands laid out in 16-row slots (a pixel of a 16-batch halo,
// or of a layer with at most 16 channels), from lane_off16 = lds_row_off(r, chunk), r < 16: the
// swizzle of lds_row_off takes bits 2 and 3 of the row from r and bits 4-6 from P.
__device__ __forceinline__ int lds_row_off16(int P, int lane_off16)
{
    return (P << 9) + (lane_off16 ^ (((P << 4) & 32) | (((P ^ (P >> 2)) & 1) << 6)));
}

// The hardware hands workgroups to the 8 XCDs in turn (linear id mod 8), and each XCD has an L2
// of its own. A launch renumbers its P workgroups so that the XCD running linear id n holds a
// contiguous range of numbers: the first P8 = P - P % 8 ids map to (n mod 8) * P8 / 8 + n / 8,
// the rest stay. Work items that share input (neighbouring pixel tiles of a convolution, whose
// halos overlap) then run under one L2 instead of eight: the forward and input-gradient
// kernels of a 56x56 ResNet layer fetch less and run 5-11 % faster. (The weight gradient's
// splits measured no better grouped this way.) A bijection of [0, P), so the work a number owns
// does not depend on it.
__device__ __forceinline__ int xcd_number(int n, int P)
{
    const int P8 = P & ~7;
    return n < P8 ? (n & 7) * (P8 >> 3) + (n >> 3) : n;
}

// A value the caller knows to be equal across the wave, made visibly uniform to the compiler
// (so that branches on it stay scalar and buffer descriptors chosen by it stay in SGPRs).
__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Decode an item and write it as four LDS rows (row0 .. row0+3). KR: the squares' first
// dimension is the reduction, so LDS row i takes square column i (a register transpose);
// otherwise LDS row i takes square row i.
template <int FMT, bool KR>
__device__ __forceinline__ void store_item(const RawItem<FMT> &r, uint8_t *lds, int row0)
{
    uint32_t rows[4][8];
    f16x2_t sc[2];
    item_scales<FMT>(r, sc);
#pragma unroll
    for (int k0 = 0; k0 < 4; k0 += 2) {
        uint32_t dd[2][8];
        decode_pair<FMT>(r, sc, k0, dd);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int k = k0 + kk;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (KR) {
                    square_column(dd[kk], i, rows[i][2 * k], rows[i][2 * k + 1]);
                } else {
                    rows[i][2 * k] = dd[kk][2 * i];
                    rows[i][2 * k + 1] = dd[kk][2 * i + 1];
                }
            }
        }
    }
    // rows row0 .. row0+3 share one swizzle (row0 is a multiple of 4): unit u of row i is at
    // P ^ ((2i + u) << 4)
    const int P = lds_row_off(row0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<uint4 *>(lds + (P ^ ((2 * i) << 4))) =
            make_uint4(rows[i][0], rows[i][1], rows[i][2], rows[i][3]);
        *reinterpret_cast<uint4 *>(lds + (P ^ ((2 * i + 1) << 4))) =
            make_uint4(rows[i][4], rows[i][5], rows[i][6], rows[i][7]);
    }
}

// Decode an item whose four squares lie side by side along the rows of the LDS operand (the
// reduction block kb = 4 elements is shared): square j fills LDS rows row0 + 4j .. row0 + 4j + 3
// at reduction elements 4*kb .. 4*kb + 3 (8 bytes each). row0 is a multiple of 16. KR as in
// store_item.
template <int FMT, bool KR>
__device__ __forceinline__ void store_item_rows(const RawItem<FMT> &r, uint8_t *lds, int row0, int kb)
{
    f16x2_t sc[2];
    item_scales<FMT>(r, sc);
    const int Q = lds_row_off(row0, kb >> 1) + 8 * (kb & 1);
#pragma unroll
    for (int j0 = 0; j0 < 4; j0 += 2) {
        uint32_t dd[2][8];
        decode_pair<FMT>(r, sc, j0, dd);
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int j = j0 + jj;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t p0, p1;
                if (KR) {
                    square_column(dd[jj], i, p0, p1);
                } else {
                    p0 = dd[jj][2 * i];
                    p1 = dd[jj][2 * i + 1];
                }
                // row0 is a multiple of 16: rows row0 + s differ from row0 in the swizzle only
                // by the bits that s sets (bit 3 and bit 2 of the row move unit bits 0 and 1)
                const int s4 = 4 * j + i;
                const int K = (2 * s4) ^ ((s4 >> 3) & 1) ^ (((s4 >> 2) & 1) << 1);
                *reinterpret_cast<uint2 *>(lds + (Q ^ (K << 4))) = make_uint2(p0, p1);
            }
        }
    }
}

// fp32 epilogue scale T_a * T_b: one float when the product is a normal float (or zero / NaN /
// inf), else the caller falls back to double arithmetic.
__device__ __forceinline__ bool scale_is_float_safe(double s)
{
    const double a = s < 0 ? -s : s;
    return a == 0.0 || !(a == a) || (a >= 1.1754943508222875e-38 && a <= 3.4028234663852886e38);
}

} // namespace mq
