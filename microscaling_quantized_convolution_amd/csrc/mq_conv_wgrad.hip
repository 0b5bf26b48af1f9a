// mq_conv_wgrad.hip -- weight-gradient GEMM G_W = G_Y . X'^T on channel-batch-first data.
//
// onedev.kr MicroQonv digest, section "How it differs": with G_{YfCout,N} (Cout x Hout*Wout*N)
// the weight gradient is a GEMM whose reduction runs over output pixels and batch elements; in
// the channel-batch-first layout (section "How it works") both operands are read along the batch
// dimension N, which is the second side of every 4x4 square of G_Y and X, so neither operand
// needs a transpose: a decoded square row is four consecutive reduction elements.
//
//   G_W[kh][kw][co][ci] = T_G * T_X * sum_{oh, ow, n} Gq[oh][ow][co][n]
//                                        * Xq[oh*s - ph + kh][ow*s - pw + kw][ci][n]
//
// A workgroup owns one kernel row kh, 64 output channels, 64 input channels and every kw, and a
// contiguous range of reduction stages; a stage is PW output pixels of one output row and 32 batch
// elements (eight batch squares, 256 contiguous code bytes per pixel and channel square for NVFP4).
// Per stage it decodes the G_Y strip (PW pixels) and the X row segment it meets
// ((PW-1)*s + Kw pixels) once into LDS as fp16; each wave runs 32x32x16 fp16 MFMAs for a
// 32 x 32 x Kw block. The fp32 partial block goes to the workspace, and a second kernel sums the
// splits in a fixed order (deterministic) and applies the tensor scales. A reduction that is not
// split (one split) writes G_W itself, scaled, with no partial block and no sum.
#include <type_traits>

#include "mq_kernels.hpp"
#include "mq_stage.hpp"
#include "mq_wgrad_sum.hpp"

namespace mq {

namespace {

constexpr int kRowBytes = 32; // 16 fp16 (one 16-element reduction step) per LDS row
constexpr int kNPItems = 512;  // staging items per stage: one per producer lane

struct WgradArgs {
    const uint8_t *g_codes, *g_scales; // squares [Ho][Wo][Cout4][N4]
    const uint8_t *x_codes, *x_scales; // squares [H][W][Cin4][N4]
    float *part;                       // [split][Kh*Kw][Cout][Cin] fp32 partial sums
    float *gw;                         // G_W [Kh*Kw][Cout][Cin] (written here when direct)
    const float *tg, *tx;              // tensor scales T_G, T_X
    int direct;                        // one split: scale and write G_W, no partials
    int H, W, Ho, Wo, Cin, Cout, Cin4, Cout4, N4;
    int Kh, Kw, sh, sw, ph, pw;
    int owb, nch;          // pixel blocks per output row, 32-element batch chunks
    int stages, per_split; // total stages, stages per split
    int cot, cit;          // Cout / Cin tiles of 64
    int splits, tiles;     // reduction splits, (kh, Cout tile, Cin tile) tiles
    int64_t split_stride;  // floats per split
};

// Waves 0..3 consume (MFMAs on one LDS buffer); waves 4..11 produce (load the squares of the
// stage after next, decode the next stage into the other buffer); one barrier per stage.
// KS: 16-element reduction steps per stage and pixel: 2 (32 batch elements, eight batch
// squares) when the batch has at least eight squares, else 1 (four squares: the whole batch of a
// pixel and channel square is then 32 contiguous bytes, so neighbouring lanes stay contiguous).
// Output pixels per stage: 16 / KS for stride 1, 8 / KS for stride 2 (twice as wide an X
// segment), so that two stage buffers fit in LDS.
// GL (the batch has a multiple of 16 elements, so every item is four real squares or none): the
// stage width is chosen so that the stage has at most 512 items, one per producer lane (with
// 64-channel slots, stride 1: 7 pixels for KS = 2, 15 for KS = 1; stride 2: 5 and 10), so that
// no SIMD decodes more than two items per stage. A wave may then hold G_Y and X items at once,
// so items are loaded through per-lane global addresses instead of buffer descriptors.
// SC: LDS rows per pixel (channel slots). 64 in general; a layer with at most 32 (16) input and
// output channels takes 32-row (16-row) slots with GL, so that a stage carries two (four) times
// the pixels for the same items and LDS, and each barrier, stage prologue and decode round
// serves that much more MFMA work (with 64-row slots such a layer's stages were mostly fixed
// costs). A 16-row slot is read as a 32-row MFMA operand whose rows 16-31 repeat rows 0-15:
// those output rows and columns lie past the channels and are never written.
__host__ __device__ constexpr int stage_pixels(int si, int ks, bool gl, int sc)
{
    return gl ? ((kNPItems / ((sc / 4) * ks)) - (3 - si)) / (1 + si) : (si == 1 ? 16 : 8) / ks;
}
// Producer threads: two waves per SIMD, so that one wave's decode overlaps the other's LDS
// writes and load issue (one producer wave per SIMD left each stage producer-bound).
constexpr int kNP = 512;
constexpr int kWgradThreads = 256 + kNP;
static_assert(kNP == kNPItems, "one staging item per producer lane");
inline int stage_ks(int N4) { return N4 >= 8 ? 2 : 1; }
inline bool stage_gl(int N4, int si) { return N4 % 4 == 0 && (si == 1 || si == 2); }
inline int stage_sc(const ConvGeom &g)
{
    if (!stage_gl(g.N4, g.sh)) return 64;
    const int c = g.Cout > g.Cin ? g.Cout : g.Cin;
    return c <= 16 ? 16 : c <= 32 ? 32 : 64;
}

// KF: the kernel width Kw when fixed at compile time (1 or 3), 0 = read at run time.
template <int FMT, int SI, int KF, int kKS, bool GL, int SC>
__global__ void __launch_bounds__(kWgradThreads) conv_wgrad_kernel(WgradArgs a)
{
    warm_kernel_args<WgradArgs>();
    static_assert(SC == 64 || (GL && (SC == 32 || SC == 16)), "narrow slots with GL only");
    constexpr int kPWg = stage_pixels(SI, kKS, GL, SC);
    constexpr int KWM = KF ? KF : 3;
    constexpr int HCM = (kPWg - 1) * SI + KWM;
    constexpr int C4S = SC / 4; // channel squares per pixel slot
    constexpr int GBYTES = kPWg * kKS * SC * kRowBytes, XBYTES = HCM * kKS * SC * kRowBytes;
    constexpr int ITEMS = (kPWg * C4S * kKS + HCM * C4S * kKS + kNP - 1) / kNP;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][GBYTES + XBYTES];
    static_assert(3 * KWM * 16 * 64 * 4 <= GBYTES + XBYTES, "small-tile sums fit one stage buffer");

    const int tid = threadIdx.x, lane = tid & 63, wave = wave_uniform(tid >> 6);
    const int split = blockIdx.x;
    int tile = blockIdx.y;
    const int cit_i = tile % a.cit; tile /= a.cit;
    const int cot_i = tile % a.cot;
    const int kh = tile / a.cot;
    const int co4_0 = cot_i * 16, ci4_0 = cit_i * 16;
    const int kw = KF ? KF : a.Kw;
    const int HC = (kPWg - 1) * SI + kw;
    const int st0 = split * a.per_split;
    const int st1 = min(a.stages, st0 + a.per_split);
    const int nst = st1 > st0 ? st1 - st0 : 0;
    // A tile with at most 32 output and 32 input channels (a layer of 16 or 32 channels) has one
    // 32x32 MFMA block of real outputs: all four consumer waves then compute that block, each
    // over every fourth pixel of a stage, and their sums meet in LDS at the end (in wave order,
    // so the result stays deterministic). Otherwise three waves would run padding only while one
    // carried the stage's every MFMA.
    const bool small = SC < 64 || (a.Cout - co4_0 * 4 <= 32 && a.Cin - ci4_0 * 4 <= 32);

    if (wave >= 4) {
        // ================= producer =================
        const int ptid = tid - 256;
        const int nG = kPWg * C4S * kKS, nGX = nG + HC * C4S * kKS;
        constexpr int CB = (FMT == kFP4) ? 8 : 12;
        const uint32_t g_sq = (uint32_t)a.Ho * a.Wo * a.Cout4 * a.N4;
        const uint32_t x_sq = (uint32_t)a.H * a.W * a.Cin4 * a.N4;
        const rsrc_t g_c = make_rsrc(a.g_codes, g_sq * CB), g_s = make_scale_rsrc(a.g_scales, g_sq);
        const rsrc_t x_c = make_rsrc(a.x_codes, x_sq * CB), x_s = make_scale_rsrc(a.x_scales, x_sq);
        // Producer items: it < nG -> G_Y strip (pixel, co4, batch half); else X segment (column,
        // ci4, batch half). With KS = 2 bit 0 picks the half of the stage's eight batch squares,
        // four squares (consecutive in memory) per item, so neighbouring lanes read neighbouring
        // 32-byte pieces of one pixel's [channel square][batch square] block. Without GL, nG is a
        // whole number of waves, so no wave mixes the two kinds.
        // Two register stages: stage c + 3 is loaded into the slot stage c + 1 was just decoded
        // from (two stage times ahead of its use). The loop is unrolled by two so that slots are
        // never copied, which keeps the compiler's waits down to the stage being decoded.
        RawItem<FMT> raw[2][ITEMS];
        // (batch chunk, pixel block, output row) of the next load's stage: loads go through the
        // stages in order, so the position is stepped with carries instead of divided out
        int l_nc = st0 % a.nch, l_ob = (st0 / a.nch) % a.owb, l_oh = st0 / a.nch / a.owb;
        // GL: one item per lane (ITEMS == 1), the same (pixel or column, channel square, batch
        // half) at every stage; its square offset within the stage, its validity along the
        // channels and its arrays are fixed
        static_assert(!GL || ITEMS == 1, "one staging item per producer lane");
        constexpr int SHg = kKS == 2 ? 1 : 0;
        constexpr int SHc = SC == 64 ? 4 : SC == 32 ? 3 : 2; // log2(C4S)
        const bool gl_isG = ptid < nG;
        const int gl_i2 = gl_isG ? ptid : ptid - nG;
        const int gl_pix = gl_i2 >> (SHc + SHg), gl_c4 = (gl_i2 >> SHg) & (C4S - 1),
                  gl_nh = gl_i2 & (kKS - 1);
        const bool gl_inv = ptid < nGX && (gl_isG ? co4_0 + gl_c4 < a.Cout4 : ci4_0 + gl_c4 < a.Cin4);
        const int gl_lsq = (gl_pix * (gl_isG ? a.Cout4 : a.Cin4) + (gl_isG ? co4_0 : ci4_0) + gl_c4) * a.N4 +
                           4 * gl_nh;
        const uint8_t *gl_cb = gl_isG ? a.g_codes : a.x_codes;
        const uint8_t *gl_sb = gl_isG ? a.g_scales : a.x_scales;
        const int gl_row = (gl_pix * kKS + gl_nh) * SC + 4 * gl_c4;
        auto load = [&](int st, RawItem<FMT>(&dst)[ITEMS]) {
            const int nc = l_nc, ob = l_ob, oh = l_oh;
            if constexpr (GL) {
                {
                    const bool c1 = l_nc + 1 >= a.nch;
                    l_nc = c1 ? 0 : l_nc + 1;
                    const bool c2 = c1 && l_ob + 1 >= a.owb;
                    l_ob = c1 ? (c2 ? 0 : l_ob + 1) : l_ob;
                    l_oh += c2 ? 1 : 0;
                }
                // the stage moves a wave-uniform base; the lane's part is fixed (gl_*)
                const int ow0 = ob * kPWg;
                const int ih = oh * SI - a.ph + kh;
                const int iw0 = ow0 * SI - a.pw;
                const int bg = ((oh * a.Wo + ow0) * a.Cout4) * a.N4 + 4 * kKS * nc;
                const int bx = ((ih * a.W + iw0) * a.Cin4) * a.N4 + 4 * kKS * nc;
                // every item is four real squares or none (N4 % 4 == 0); an empty item reads
                // the array's first squares and decodes them as zeros (mask 0)
                const bool nok = st < st1 && 4 * gl_nh < a.N4 - 4 * kKS * nc;
                const bool pok = gl_isG ? gl_pix < a.Wo - ow0
                                        : (ih >= 0 && ih < a.H && gl_pix >= -iw0 && gl_pix < a.W - iw0);
                const bool ok = gl_inv && nok && pok;
                const uint32_t sq = ok ? (uint32_t)((gl_isG ? bg : bx) + gl_lsq) : 0u;
                const uint8_t *cp = gl_cb + (size_t)sq * CB;
                const uint8_t *sp = gl_sb + sq;
                RawItem<FMT> &r = dst[0];
                const u32x4_t v0 = *reinterpret_cast<const u32x4_t *>(cp);
                const u32x4_t v1 = *reinterpret_cast<const u32x4_t *>(cp + 16);
                if constexpr (FMT == kFP4) {
                    r.w[0][0] = v0[0]; r.w[0][1] = v0[1]; r.w[1][0] = v0[2]; r.w[1][1] = v0[3];
                    r.w[2][0] = v1[0]; r.w[2][1] = v1[1]; r.w[3][0] = v1[2]; r.w[3][1] = v1[3];
                } else {
                    const u32x4_t v2 = *reinterpret_cast<const u32x4_t *>(cp + 32);
                    r.w[0][0] = v0[0]; r.w[0][1] = v0[1]; r.w[0][2] = v0[2];
                    r.w[1][0] = v0[3]; r.w[1][1] = v1[0]; r.w[1][2] = v1[1];
                    r.w[2][0] = v1[2]; r.w[2][1] = v1[3]; r.w[2][2] = v2[0];
                    r.w[3][0] = v2[1]; r.w[3][1] = v2[2]; r.w[3][2] = v2[3];
                }
                r.sc = *reinterpret_cast<const uint32_t *>(sp); // sq % 4 == 0: one word
                r.sh = 0u;
                r.m = ok ? 0xFu : 0u;
                return;
            }
            {
                const bool c1 = l_nc + 1 >= a.nch;
                l_nc = c1 ? 0 : l_nc + 1;
                const bool c2 = c1 && l_ob + 1 >= a.owb;
                l_ob = c1 ? (c2 ? 0 : l_ob + 1) : l_ob;
                l_oh += c2 ? 1 : 0;
            }
            const int ow0 = ob * kPWg;
            const int ih = oh * SI - a.ph + kh;
            const int iw0 = ow0 * SI - a.pw;
            constexpr int SH = kKS == 2 ? 1 : 0; // item index bits below the channel square
    #pragma unroll
            for (int q = 0; q < ITEMS; ++q) {
                const int it = ptid + q * kNP;
                const bool isG = wave_uniform(it & ~63) < nG;
                const int nh = it & (kKS - 1); // nG is even, so X items keep the same bit
                // a stage past the end of this split loads nothing (mask 0), so that every stage
                // issues the same loads without branches and each decode waits for its own stage
                const int nvalid = a.N4 - 4 * (kKS * nc + nh);
                const uint32_t nmask =
                    st >= st1 || nvalid <= 0 ? 0u : nvalid >= 4 ? 0xFu : ((1u << nvalid) - 1u);
                const int ow = ow0 + (it >> (4 + SH)), co4 = co4_0 + ((it >> SH) & 15);
                const uint32_t sqg =
                    (((uint32_t)oh * a.Wo + ow) * a.Cout4 + co4) * a.N4 + 4 * (kKS * nc + nh);
                const uint32_t mg = (ow < a.Wo && co4 < a.Cout4) ? nmask : 0u;
                const int j = it - nG;
                const int iw = iw0 + (j >> (4 + SH)), ci4 = ci4_0 + ((j >> SH) & 15);
                const uint32_t sqx =
                    (((uint32_t)ih * a.W + iw) * a.Cin4 + ci4) * a.N4 + 4 * (kKS * nc + nh);
                const bool in = it < nGX && ih >= 0 && ih < a.H && iw >= 0 && iw < a.W &&
                                ci4 < a.Cin4;
                load_item_contig<FMT>(dst[q], isG ? g_c : x_c, isG ? g_s : x_s, isG ? sqg : sqx,
                                      isG ? mg : (in ? nmask : 0u));
            }
        };
        auto store = [&](int buf, const RawItem<FMT>(&src)[ITEMS]) {
            if constexpr (GL) {
                // LDS rows: [pixel or column][reduction step][64 channels]
                if (ptid < nGX)
                    store_item<FMT, false>(src[0], lds[buf] + (gl_isG ? 0 : GBYTES), gl_row);
                return;
            }
    #pragma unroll
            for (int q = 0; q < ITEMS; ++q) {
                const int it = ptid + q * kNP;
                const int wit = wave_uniform(it & ~63);
                // LDS rows: [pixel or column][reduction step][64 channels]
                constexpr int SH = kKS == 2 ? 1 : 0;
                if (wit < nG)
                    store_item<FMT, false>(src[q], lds[buf],
                                           ((it >> (4 + SH)) * kKS + (it & (kKS - 1))) * 64 +
                                               4 * ((it >> SH) & 15));
                else if (wit < nGX && it < nGX) {
                    const int j = it - nG;
                    store_item<FMT, false>(src[q], lds[buf] + GBYTES,
                                           ((j >> (4 + SH)) * kKS + (j & (kKS - 1))) * 64 +
                                               4 * ((j >> SH) & 15));
                }
            }
        };

        load(st0, raw[0]);
        load(st0 + 1, raw[1]);
        store(0, raw[0]);
        load(st0 + 2, raw[0]);
        __syncthreads();
        int c = 0;
        for (; c + 1 < nst; c += 2) {
            store(1, raw[1]);
            load(st0 + c + 3, raw[1]);
            __syncthreads();
            if (c + 2 < nst) store(0, raw[0]);
            load(st0 + c + 4, raw[0]);
            __syncthreads();
        }
        if (c < nst) __syncthreads(); // last stage: nothing left to decode
        if (small) __syncthreads();   // the consumers' cross-wave sum
        return;
    }

    // ================= consumer =================
    // (the two roles take wave-uniform branches and pass the same number of barriers)
    const int wm = wave & 1, wc = wave >> 1;
    f32x16_t acc[KWM];
#pragma unroll
    for (int t = 0; t < KWM; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] = 0.0f;
    const int half = lane >> 5, l32 = lane & 31;
    const int loff = lds_row_off(l32, half);
    // LDS offset of this lane's operand row in slot P (SC rows per slot; with 16-row slots,
    // lanes 16-31 read rows 0-15 again)
    const int loff16 = lds_row_off(l32 & 15, half);
    auto slot = [&](int P) {
        if constexpr (SC == 16) return lds_row_off16(P, loff16);
        else return lds_row_off32(P * SC, loff);
    };
    __syncthreads();
    if (small) {
        for (int c = 0; c < nst; ++c) {
            const uint8_t *Gs = lds[c & 1], *Xs = lds[c & 1] + GBYTES;
#pragma unroll
            for (int ks = 0; ks < kKS; ++ks) {
                if constexpr (SC == 16) {
                    // Two pixels per MFMA: lanes 0-15 carry pixel 2j (operand rows and columns
                    // 0-15), lanes 16-31 pixel 2j + 1 (rows and columns 16-31), so the two
                    // diagonal 16x16 blocks of the product are the two pixels' terms (the others
                    // are cross terms, never used). A pair past the stage's last pixel reads an
                    // in-range slot with a zero G_Y operand.
                    constexpr int NPAIR = (kPWg + 1) / 2;
                    const int hi = l32 >> 4;
#pragma unroll
                    for (int i = 0; i < (NPAIR + 3) / 4; ++i) {
                        const int j = wave + 4 * i;
                        if (j < NPAIR) {
                            const int pxl = 2 * j + hi;
                            const bool real = pxl < kPWg;
                            const int px = real ? pxl : 2 * j;
                            u32x4_t gu = *reinterpret_cast<const u32x4_t *>(Gs + slot(px * kKS + ks));
                            if (!real) gu = u32x4_t{0u, 0u, 0u, 0u};
                            const f16x8_t gf = __builtin_bit_cast(f16x8_t, gu);
#pragma unroll
                            for (int t = 0; t < KWM; ++t)
                                if (t < kw) {
                                    const f16x8_t xb = __builtin_bit_cast(
                                        f16x8_t, *reinterpret_cast<const u32x4_t *>(
                                                     Xs + slot((px * SI + t) * kKS + ks)));
                                    acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(gf, xb, acc[t], 0, 0, 0);
                                }
                        }
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < (kPWg + 3) / 4; ++i) {
                        const int px = wave + 4 * i;
                        if (px < kPWg) {
                            const f16x8_t gf = __builtin_bit_cast(
                                f16x8_t, *reinterpret_cast<const u32x4_t *>(
                                             Gs + slot(px * kKS + ks)));
#pragma unroll
                            for (int t = 0; t < KWM; ++t)
                                if (t < kw) {
                                    const f16x8_t xb = __builtin_bit_cast(
                                        f16x8_t, *reinterpret_cast<const u32x4_t *>(
                                                     Xs + slot((px * SI + t) * kKS + ks)));
                                    acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(gf, xb, acc[t], 0, 0, 0);
                                }
                        }
                    }
                }
            }
            __syncthreads();
        }
        // the four waves' sums: waves 1-3 through LDS (the stage buffers are free after the last
        // barrier), added by wave 0 in wave order
        float *red = reinterpret_cast<float *>(&lds[0][0]);
        if (wave > 0) {
#pragma unroll
            for (int t = 0; t < KWM; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) red[(((wave - 1) * KWM + t) * 16 + r) * 64 + lane] = acc[t][r];
        }
        __syncthreads();
        if (wave != 0) return;
        // one wave's sums at a time (unrolled over the waves, the compiler loaded all three
        // sets ahead of the additions and spilled)
#pragma unroll 1
        for (int w = 0; w < 3; ++w)
#pragma unroll
            for (int t = 0; t < KWM; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[t][r] += red[((w * KWM + t) * 16 + r) * 64 + lane];
        if constexpr (SC == 16) {
            // the second pixel's block (rows and columns 16-31: lane l32 + 16, registers 8-15)
            // onto the first's (rows and columns 0-15, which the epilogue writes)
#pragma unroll
            for (int t = 0; t < KWM; ++t)
#pragma unroll
                for (int r = 0; r < 8; ++r) acc[t][r] += __shfl_down(acc[t][r + 8], 16);
        }
    } else if constexpr (SC == 64) {
    for (int c = 0; c < nst; ++c) {
        const uint8_t *Gs = lds[c & 1], *Xs = lds[c & 1] + GBYTES;
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks) {
            // every X column of the buffer is read (columns past HC are never used)
            u32x4_t xf[HCM];
#pragma unroll
            for (int cc = 0; cc < HCM; ++cc)
                xf[cc] = *reinterpret_cast<const u32x4_t *>(
                    Xs + lds_row_off32((cc * kKS + ks) * 64 + wc * 32, loff));
#pragma unroll
            for (int px = 0; px < kPWg; ++px) {
                const f16x8_t gf = __builtin_bit_cast(
                    f16x8_t, *reinterpret_cast<const u32x4_t *>(
                                 Gs + lds_row_off32((px * kKS + ks) * 64 + wm * 32, loff)));
#pragma unroll
                for (int t = 0; t < KWM; ++t)
                    if (t < kw)
                        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            gf, __builtin_bit_cast(f16x8_t, xf[px * SI + t]), acc[t], 0, 0, 0);
            }
        }
        __syncthreads();
    }
    }

    // ---- partial block part[split][kh*Kw + kw][co][ci], or (one split) G_W itself, scaled
    // as the split sum scales a sum of one partial: (float)(acc * (double)T_G * T_X) ----
    // (a copy per form, chosen by a wave-uniform branch: with one loop the compiler computed the
    // scaled form for every partial too)
    const int ci = ci4_0 * 4 + wc * 32 + l32;
    auto write = [&](auto direct) {
        constexpr bool D = decltype(direct)::value != 0;
        float *out = D ? a.gw : a.part + (int64_t)split * a.split_stride;
        const double sc = D ? (double)*a.tg * (double)*a.tx : 1.0;
#pragma unroll
        for (int t = 0; t < KWM; ++t) {
            if (t >= kw) continue;
            float *o = out + (int64_t)(kh * kw + t) * a.Cout * a.Cin;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int co = co4_0 * 4 + wm * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                const float v = D ? (float)((double)acc[t][r] * sc) : acc[t][r];
                if (co < a.Cout && ci < a.Cin) o[(int64_t)co * a.Cin + ci] = v;
            }
        }
    };
    if (a.direct) write(std::integral_constant<int, 1>{});
    else write(std::integral_constant<int, 0>{});
}

// The split sum as a kernel of its own: blocks grid-stride over the 256-lane workgroups (a
// workgroup per block made launches of tens of thousands of tiny workgroups).
__global__ void __launch_bounds__(256) wgrad_sum_kernel(WgradSum w)
{
    __shared__ float4 red[16][17];
    const int64_t nb = wgrad_sum_blocks(w);
    for (int64_t blk = blockIdx.x; blk < nb; blk += gridDim.x) {
        wgrad_sum_block(w, blk, (int)threadIdx.x, red);
        __syncthreads(); // the next block reuses red
    }
}

struct Plan {
    int owb, nch, stages, cot, cit, tiles, splits, per_split;
    int64_t split_stride;
    size_t bytes;
};

Plan plan(const ConvGeom &g)
{
    Plan p;
    const int ks = stage_ks(g.N4);
    const int kPWg = stage_pixels(g.sh, ks, stage_gl(g.N4, g.sh), stage_sc(g));
    p.owb = (g.Wo + kPWg - 1) / kPWg;
    p.nch = (g.N4 + 4 * ks - 1) / (4 * ks);
    p.stages = g.Ho * p.owb * p.nch;
    p.cot = (g.Cout4 + 15) / 16;
    p.cit = (g.Cin4 + 15) / 16;
    p.tiles = g.Kh * p.cot * p.cit;
    p.split_stride = (int64_t)g.Kh * g.Kw * g.Cout * g.Cin;
    // Split count: a workgroup holds one CU (its LDS), so tiles * splits workgroups run in
    // ceil(tiles * splits / 256) rounds of per_split stages. Pick the count with the least
    // modelled time: rounds * per_split stages (about 1.9 us each) plus the partial sums that
    // every split writes and the sum kernel reads back (at about 5 TB/s); at most ~16 MB of
    // partial sums. Ties keep the smaller count.
    const int64_t out_bytes = p.split_stride * 4;
    int64_t cap = (16ll << 20) / (out_bytes > 0 ? out_bytes : 1);
    if (cap < 1) cap = 1;
    if (cap > p.stages) cap = p.stages;
    int64_t best_per = p.stages;
    double best = -1.0;
    for (int64_t s = 1; s <= cap; ++s) {
        const int64_t per = (p.stages + s - 1) / s;
        const int64_t splits = (p.stages + per - 1) / per;
        if (splits != s) continue; // the same split as a smaller s
        const int64_t rounds = (p.tiles * splits + 255) / 256;
        // one split writes G_W directly: no partials to write and read back, no sum launch
        const double t = 1.9 * (double)(rounds * per) +
                         (splits > 1 ? 2.0 * (double)(splits * out_bytes) / 5e6 + 3.0 : 0.0);
        if (best < 0.0 || t < best) {
            best = t;
            best_per = per;
        }
    }
    p.per_split = (int)best_per;
    p.splits = (p.stages + p.per_split - 1) / p.per_split;
    // one split needs no partials (a token workspace keeps 0 meaning "invalid convolution")
    p.bytes = p.splits > 1 ? (size_t)p.splits * (size_t)p.split_stride * 4 : 256;
    return p;
}

} // namespace

bool wgrad_fast_supported(const ConvGeom &g)
{
    if (g.Kw > 3 || g.sh != g.sw || (g.sh != 1 && g.sh != 2)) return false;
    // 32-bit byte offsets below 2^31 for the operands and one split's partial block
    const uint64_t lim = 1ull << 31;
    const uint64_t xs = (uint64_t)g.H * g.W * g.Cin4 * g.N4 * 12,
                   gs = (uint64_t)g.Ho * g.Wo * g.Cout4 * g.N4 * 12,
                   ps = (uint64_t)g.Kh * g.Kw * g.Cout * g.Cin * 4;
    return xs < lim && gs < lim && ps < lim;
}

size_t wgrad_fast_workspace_bytes(const ConvGeom &g) { return plan(g).bytes; }

template <int FMT, int SI, int KS, bool GL, int SC>
static void launch_wgrad_ks(const ConvGeom &g, dim3 grid, const WgradArgs &a, hipStream_t st)
{
    if (g.Kw == 3)
        hipLaunchKernelGGL((conv_wgrad_kernel<FMT, SI, 3, KS, GL, SC>), grid, dim3(kWgradThreads), 0, st, a);
    else if (g.Kw == 1)
        hipLaunchKernelGGL((conv_wgrad_kernel<FMT, SI, 1, KS, GL, SC>), grid, dim3(kWgradThreads), 0, st, a);
    else hipLaunchKernelGGL((conv_wgrad_kernel<FMT, SI, 0, KS, GL, SC>), grid, dim3(kWgradThreads), 0, st, a);
}

template <int FMT, int SI, int KS>
static void launch_wgrad_gl(const ConvGeom &g, dim3 grid, const WgradArgs &a, hipStream_t st)
{
    const int sc = stage_sc(g); // below 64 with GL only
    if (sc == 16) launch_wgrad_ks<FMT, SI, KS, true, 16>(g, grid, a, st);
    else if (sc == 32) launch_wgrad_ks<FMT, SI, KS, true, 32>(g, grid, a, st);
    else if (stage_gl(g.N4, SI)) launch_wgrad_ks<FMT, SI, KS, true, 64>(g, grid, a, st);
    else launch_wgrad_ks<FMT, SI, KS, false, 64>(g, grid, a, st);
}

template <int FMT, int SI>
static void launch_wgrad_si(const ConvGeom &g, dim3 grid, const WgradArgs &a, hipStream_t st)
{
    if (stage_ks(g.N4) == 2) launch_wgrad_gl<FMT, SI, 2>(g, grid, a, st);
    else launch_wgrad_gl<FMT, SI, 1>(g, grid, a, st);
}

template <int FMT>
static void launch_wgrad_fmt(const ConvGeom &g, dim3 grid, const WgradArgs &a, hipStream_t st)
{
    if (g.sh == 1) launch_wgrad_si<FMT, 1>(g, grid, a, st);
    else launch_wgrad_si<FMT, 2>(g, grid, a, st);
}

hipError_t launch_conv_wgrad_partials(const ConvGeom &g, int fmt, QOperand gy, QOperand x,
                                      float *gw, void *ws, size_t ws_bytes, hipStream_t st,
                                      WgradSum *sum)
{
    const Plan p = plan(g);
    if (ws_bytes < p.bytes) return hipErrorInvalidValue;
    WgradArgs a;
    a.g_codes = gy.codes; a.g_scales = gy.scales; a.x_codes = x.codes; a.x_scales = x.scales;
    a.part = reinterpret_cast<float *>(ws);
    a.gw = gw; a.tg = gy.tscale; a.tx = x.tscale;
    a.direct = p.splits == 1 ? 1 : 0;
    a.H = g.H; a.W = g.W; a.Ho = g.Ho; a.Wo = g.Wo; a.Cin = g.Cin; a.Cout = g.Cout;
    a.Cin4 = g.Cin4; a.Cout4 = g.Cout4; a.N4 = g.N4;
    a.Kh = g.Kh; a.Kw = g.Kw; a.sh = g.sh; a.sw = g.sw; a.ph = g.ph; a.pw = g.pw;
    a.owb = p.owb; a.nch = p.nch; a.stages = p.stages; a.per_split = p.per_split;
    a.cot = p.cot; a.cit = p.cit; a.split_stride = p.split_stride;
    a.splits = p.splits; a.tiles = p.tiles;
    dim3 grid((unsigned)p.splits, (unsigned)p.tiles, 1);
    if (fmt == kFP4) launch_wgrad_fmt<kFP4>(g, grid, a, st);
    else launch_wgrad_fmt<kFP6>(g, grid, a, st);
    sum->part = reinterpret_cast<const float *>(ws);
    sum->S = p.splits;
    sum->stride = p.split_stride;
    sum->total = a.direct ? 0 : p.split_stride; // nothing to sum after a direct write
    sum->tg = gy.tscale;
    sum->tx = x.tscale;
    sum->out = gw;
    return hipGetLastError();
}

hipError_t launch_conv_wgrad_fast(const ConvGeom &g, int fmt, QOperand gy, QOperand x, float *gw,
                                  void *ws, size_t ws_bytes, hipStream_t st)
{
    WgradSum w;
    const hipError_t e = launch_conv_wgrad_partials(g, fmt, gy, x, gw, ws, ws_bytes, st, &w);
    if (e != hipSuccess) return e;
    return launch_wgrad_sum(w, st);
}

hipError_t launch_wgrad_sum(const WgradSum &w, hipStream_t st)
{
    if (w.total <= 0) return hipSuccess;
    const int64_t nb = wgrad_sum_blocks(w);
    hipLaunchKernelGGL(wgrad_sum_kernel, dim3((unsigned)(nb < 2048 ? nb : 2048)), dim3(256), 0, st, w);
    return hipGetLastError();
}

} // namespace mq
